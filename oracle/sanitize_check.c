/*
 * sanitize_check.c -- TEST INFRASTRUCTURE: a standalone driver that runs every
 * entry point of the CPU oracle (kmr_oracle.c) on a small model, so that the
 * oracle can be built with AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_oracle_sanitize.py).  Exits 0 when every result is finite and
 * every call accepted its arguments; the sanitizers abort on any memory or
 * undefined-behaviour error.  The model: 2 layers, hidden 64, 4 q / 2 kv heads of
 * head_dim 16, intermediate 128, vocab 97, group 32, with weights from a fixed
 * linear congruential sequence rounded to bf16.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kmr_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double next_uniform(void) {   /* in [-1, 1) */
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(g_state >> 11) / 4503599627370496.0 - 1.0;
}

static uint16_t to_bf16(double x) {   /* round to nearest even through fp32 */
  float f = (float)x;
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static uint16_t* bf16_array(int64_t n, double scale, double offset) {
  uint16_t* a = malloc((size_t)n * sizeof *a);
  for (int64_t i = 0; i < n; ++i) a[i] = to_bf16(offset + scale * next_uniform());
  return a;
}

static ora_qmat quantized(int64_t N, int64_t K, int64_t G, double scale) {
  uint16_t* w = bf16_array(N * K, scale, 0.0);
  uint8_t* packed = malloc((size_t)(N * K / 2));
  uint16_t* sz = malloc((size_t)(N * (K / G) * 2) * sizeof *sz);
  ora_quantize_int4(w, N, K, G, packed, sz);
  free(w);
  ora_qmat q = {packed, sz, N, K};
  return q;
}

static int all_finite(const double* a, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) return 0;
  return 1;
}

int main(void) {
  ora_dims d = {64, 4, 2, 16, 128, 97, 2, 32, 1e-6, 5e6, {3, 3, 2}, 1, 0, -1};
  const int64_t H = d.hidden, D = d.head_dim, I = d.intermediate, V = d.vocab, G = d.group_size;
  const int64_t NQKV = (d.n_heads + 2 * d.n_kv_heads) * D, B = 3, M = 12;
  ora_layer layers[2];
  for (int l = 0; l < 2; ++l) {
    layers[l].in_norm = bf16_array(H, 0.5, 1.0);
    layers[l].q_norm = bf16_array(D, 0.5, 1.0);
    layers[l].k_norm = bf16_array(D, 0.5, 1.0);
    layers[l].post_norm = bf16_array(H, 0.5, 1.0);
    layers[l].qkv = quantized(NQKV, H, G, 0.05);
    layers[l].o = quantized(H, d.n_heads * D, G, 0.05);
    layers[l].gate_up = quantized(2 * I, H, G, 0.05);
    layers[l].down = quantized(H, I, G, 0.05);
  }
  ora_model m = {bf16_array(V * H, 0.05, 0.0), bf16_array(H, 0.5, 1.0), bf16_array(V * H, 0.05, 0.0), layers};
  const int64_t cache_n = d.n_layers * B * d.n_kv_heads * M * D;
  uint16_t* kc = bf16_array(cache_n, 1.0, 0.0);
  uint16_t* vc = bf16_array(cache_n, 1.0, 0.0);

  /* one layer on a hidden state, then advancing steps (row 2 finished, row 1 reaching max_len) */
  double x[3 * 64];
  for (int64_t i = 0; i < B * H; ++i) x[i] = next_uniform();
  int32_t pos[9] = {0, 5, 9, 1, 2, 3, 0, 5, 9}, cpos[3] = {0, 10, 4};
  if (ora_decode_layer(&d, &layers[1], 1, kc, vc, B, M, x, pos, cpos) || !all_finite(x, B * H)) return 1;
  int32_t ids[3] = {5, 96, 0}, next[3];
  uint8_t fin[3] = {0, 0, 1};
  double logits[3 * 97], margin[3], hidden[3 * 64];
  for (int s = 0; s < 4; ++s) {
    if (ora_decode_step(&d, &m, kc, vc, B, M, ids, pos, cpos, fin, ORA_ADVANCE, next, logits, margin, hidden))
      return 2;
    if (!all_finite(logits, B * V) || !all_finite(hidden, B * H) || !all_finite(margin, B)) return 3;
    for (int b = 0; b < B; ++b) {
      if (next[b] < 0 || next[b] >= V) return 4;
      ids[b] = next[b];
    }
  }
  /* out-of-range inputs are rejected, not read */
  int32_t bad_cpos[3] = {0, (int32_t)M, 1};
  if (ora_decode_layer(&d, &layers[0], 0, kc, vc, B, M, x, pos, bad_cpos) == 0) return 5;
  /* the standalone pieces */
  double y[2 * 64], dq[64 * 64];
  ora_gemv_int4(layers[0].o.packed, layers[0].o.sz, H, d.n_heads * D, G, x, 2, y);
  ora_dequant(layers[0].o.packed, layers[0].o.sz, H, d.n_heads * D, G, dq);
  ora_rmsnorm(x, layers[0].in_norm, H, d.rms_eps, y);
  ora_mrope(y, D, pos, d.mrope_section, 0, d.rope_theta);
  ora_attend(y, kc, vc, M, D, y + 64);
  if (!all_finite(y, 2 * H) || !all_finite(dq, 64 * 64) || !isfinite(ora_silu(-3.0))) return 6;
  printf("oracle sanitize check ok: next = %d %d %d\n", next[0], next[1], next[2]);
  return 0;
}
