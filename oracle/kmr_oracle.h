/*
 * CPU oracle for the int4 weight-only decode step -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may load
 * this library.  It shares no code with the HIP library: its own header, its own
 * bf16 helpers, its own loops.  Host pointers only; fp64 arithmetic except where
 * the quantizer's definition fixes fp32 steps.
 *
 * Sources (the kaminari page, "kaminari - a single-GPU Qwen3-VL inference engine,
 * explained"; and "The Ghost in the Batch: How vLLM Silently Switches Algorithms"):
 *   - decoder structure: kaminari section 03 (model/modules.py: TextModel,
 *     DecoderLayer, TextAttention with fused QKV, MLP, Mrope) and section 05;
 *   - the one-token decode step with ids (batch,1), positions (3,batch,1),
 *     cache_position and the static KV buffers: kaminari section 04, "3 . decode";
 *   - int4 weight-only decoder linears, bf16 lm_head / embeddings / norms:
 *     kaminari section 07;
 *   - attention softmax(Q K^T / sqrt(d)) V: Ghost in the Batch, "What Attention
 *     Does (60 Seconds)".
 * Where the pages leave a step open, the reading taken is stated beside it.
 */
#ifndef KMR_ORACLE_H
#define KMR_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab, n_layers, group_size;
  double rms_eps;
  double rope_theta;
  int32_t mrope_section[3];
  int32_t mrope_interleaved;
  int32_t pad_id;
  int32_t eos_id;
} ora_dims;

typedef struct {            /* one int4 matrix: codes u8 [N][K/2], (scale, zero) bf16 [N][K/G][2] */
  const uint8_t* packed;
  const uint16_t* sz;
  int64_t N, K;
} ora_qmat;

typedef struct {
  const uint16_t *in_norm, *q_norm, *k_norm, *post_norm;   /* bf16 gains */
  ora_qmat qkv, o, gate_up, down;
} ora_layer;

typedef struct {
  const uint16_t *embed, *final_norm, *lm_head;             /* bf16 [V][H], [H], [V][H] */
  const ora_layer* layers;                                  /* [n_layers] */
} ora_model;

#define ORA_ADVANCE 1u

void ora_quantize_int4(const uint16_t* w, int64_t N, int64_t K, int64_t G,
                       uint8_t* packed, uint16_t* sz);
void ora_dequant(const uint8_t* packed, const uint16_t* sz, int64_t N, int64_t K, int64_t G,
                 double* out);
void ora_gemv_int4(const uint8_t* packed, const uint16_t* sz, int64_t N, int64_t K, int64_t G,
                   const double* x, int64_t B, double* y);
void ora_rmsnorm(const double* x, const uint16_t* gain, int64_t n, double eps, double* out);
int32_t ora_mrope_axis(int64_t pair, int64_t half_dim, const int32_t* sections, int32_t interleaved);
void ora_mrope(double* v, int64_t D, const int32_t* pos3, const int32_t* sections,
               int32_t interleaved, double theta);
void ora_attend(const double* q, const uint16_t* k, const uint16_t* v, int64_t n_pos,
                int64_t D, double* out);
double ora_bf16_round(double x);
double ora_silu(double a);   /* a / (1 + e^-a), the MLP's gate activation */
int ora_decode_layer(const ora_dims* d, const ora_layer* w, int64_t layer,
                     uint16_t* kcache, uint16_t* vcache, int64_t B, int64_t M,
                     double* x, const int32_t* pos, const int32_t* cpos);
int ora_decode_step(const ora_dims* d, const ora_model* m, uint16_t* kcache, uint16_t* vcache,
                    int64_t B, int64_t M, const int32_t* ids, int32_t* pos, int32_t* cpos,
                    uint8_t* finished, uint32_t flags, int32_t* next, double* logits,
                    double* margin, double* hidden_out);
int ora_threads(void);

#ifdef __cplusplus
}
#endif
#endif
