/*
 * CPU oracle for the int4 weight-only decode step -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct: every matrix-vector product is one fp64
 * dot product per output in ascending k; every weight is dequantized on the fly
 * from its code, scale and zero; attention is the textbook softmax over all
 * cached positions.  OpenMP only hands independent outputs (rows of a product,
 * heads of attention) to different threads; it changes no arithmetic.
 *
 * Nothing here is shared with the HIP library.  Only the tests, the smoke check
 * and the benchmark's CPU-baseline leg may load it.
 *
 * Page references are to "kaminari - a single-GPU Qwen3-VL inference engine,
 * explained" (section numbers as printed there) and to "The Ghost in the Batch:
 * How vLLM Silently Switches Algorithms".
 */
#include "kmr_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- bf16 helpers */

static float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static double bf16_to_f64(uint16_t h) { return (double)bf16_to_f32(h); }

/* fp32 -> bf16, round to nearest, ties to even (the reading taken for every
 * narrowing: the pages fix no rounding rule). */
static uint16_t f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  uint32_t keep = u >> 16;
  uint32_t rest = u & 0xffffu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;
  return (uint16_t)keep;
}

/* fp64 -> bf16 with a single round-to-nearest-even (no detour through fp32). */
static uint16_t f64_to_bf16(double x) {
  if (isnan(x)) return 0x7fc0;
  if (x == 0.0) return signbit(x) ? 0x8000 : 0x0000;
  double a = fabs(x);
  int e;
  double m = frexp(a, &e); /* a = m * 2^e, 0.5 <= m < 1 */
  int bits = 8;            /* significant bits of a normal bf16 */
  if (e - 1 < -126) bits = 8 - (-126 - (e - 1));
  double r = nearbyint(ldexp(m, bits)); /* default rounding mode: ties to even */
  float f = (float)ldexp(r, e - bits);  /* exact in bf16 (or inf on overflow) */
  uint32_t u;
  memcpy(&u, &f, 4);
  uint16_t h = (uint16_t)(u >> 16);
  if (signbit(x)) h |= 0x8000u;
  return h;
}

double ora_bf16_round(double x) { return bf16_to_f64(f64_to_bf16(x)); }

int ora_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------ int4 quantizer
 * Kaminari section 07: decoder attention/MLP linears become weight-only int4;
 * everything else stays bf16.  The pages give no formula.  Reading taken: per
 * row, groups of G consecutive k; asymmetric affine codes with a float-domain
 * zero at mid-code 8, the convention of the weight-only int4 library the page
 * names:
 *     s = bf16(max((hi - lo) / 15, 2^-24))
 *     z = bf16(lo + 8 s)
 *     q = clamp(rne((w - z) / s) + 8, 0, 15),   w_hat = (q - 8) s + z
 * Each line is IEEE fp32 in exactly this order, with no fused multiply-add
 * (the build passes -ffp-contract=off), so the codes are reproducible bit for
 * bit.  Layout: codes u8 [N][K/2], even k in the low nibble; (scale, zero) as an
 * interleaved bf16 pair per (row, group).
 */
void ora_quantize_int4(const uint16_t* w, int64_t N, int64_t K, int64_t G, uint8_t* packed,
                       uint16_t* sz) {
  const int64_t ng = K / G;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < ng; ++g) {
      const uint16_t* src = w + n * K + g * G;
      float lo = bf16_to_f32(src[0]), hi = lo;
      for (int64_t i = 1; i < G; ++i) {
        float v = bf16_to_f32(src[i]);
        if (v < lo) lo = v;
        if (v > hi) hi = v;
      }
      float range = hi - lo;
      float s32 = range / 15.0f;
      if (!(s32 >= 0x1p-24f)) s32 = 0x1p-24f;
      uint16_t sb = f32_to_bf16(s32);
      float s = bf16_to_f32(sb);
      float eight_s = 8.0f * s;
      float z32 = lo + eight_s;
      uint16_t zb = f32_to_bf16(z32);
      float z = bf16_to_f32(zb);
      sz[(n * ng + g) * 2 + 0] = sb;
      sz[(n * ng + g) * 2 + 1] = zb;
      for (int64_t i = 0; i < G; ++i) {
        int64_t k = g * G + i;
        float diff = bf16_to_f32(src[i]) - z;
        float t = diff / s;
        float r = nearbyintf(t); /* ties to even */
        int q = (int)r + 8;
        if (q < 0) q = 0;
        if (q > 15) q = 15;
        uint8_t* byte = packed + n * (K / 2) + k / 2;
        if ((k & 1) == 0)
          *byte = (uint8_t)((*byte & 0xf0u) | (uint8_t)q);
        else
          *byte = (uint8_t)((*byte & 0x0fu) | (uint8_t)(q << 4));
      }
    }
  }
}

static inline int code_at(const uint8_t* packed, int64_t K, int64_t n, int64_t k) {
  uint8_t b = packed[n * (K / 2) + k / 2];
  return (k & 1) ? (b >> 4) : (b & 0x0f);
}

/* w_hat = (q - 8) s + z.  Both s and z are bf16, so the product and the sum are
 * exact in fp64 for any realistic exponent spread. */
static inline double dequant_at(const uint8_t* packed, const uint16_t* sz, int64_t K, int64_t G,
                                int64_t n, int64_t k) {
  int64_t ng = K / G, g = k / G;
  double s = bf16_to_f64(sz[(n * ng + g) * 2 + 0]);
  double z = bf16_to_f64(sz[(n * ng + g) * 2 + 1]);
  return (double)(code_at(packed, K, n, k) - 8) * s + z;
}

void ora_dequant(const uint8_t* packed, const uint16_t* sz, int64_t N, int64_t K, int64_t G,
                 double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) out[n * K + k] = dequant_at(packed, sz, K, G, n, k);
}

/* y[b][n] = sum_k w_hat[n][k] x[b][k]: the weight-only int4 linear of kaminari
 * section 07, one fp64 dot product per output, ascending k. */
void ora_gemv_int4(const uint8_t* packed, const uint16_t* sz, int64_t N, int64_t K, int64_t G,
                   const double* x, int64_t B, double* y) {
#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)(B > 0 ? B : 1));
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t b = 0; b < B; ++b) acc[b] = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double wv = dequant_at(packed, sz, K, G, n, k);
        for (int64_t b = 0; b < B; ++b) acc[b] += wv * x[b * K + k];
      }
      for (int64_t b = 0; b < B; ++b) y[b * N + n] = acc[b];
    }
    free(acc);
  }
}

/* bf16 x bf16-weight product for the untied lm_head (kept bf16, kaminari section 07). */
static void gemv_bf16(const uint16_t* w, int64_t N, int64_t K, const double* x, int64_t B,
                      double* y) {
#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * (size_t)(B > 0 ? B : 1));
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t b = 0; b < B; ++b) acc[b] = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double wv = bf16_to_f64(w[n * K + k]);
        for (int64_t b = 0; b < B; ++b) acc[b] += wv * x[b * K + k];
      }
      for (int64_t b = 0; b < B; ++b) y[b * N + n] = acc[b];
    }
    free(acc);
  }
}

/* RMSNorm (the decoder's norms, kaminari section 03 modules):
 * out = x / sqrt(mean(x^2) + eps) * gain.  eps is a parameter (1e-6 read). */
void ora_rmsnorm(const double* x, const uint16_t* gain, int64_t n, double eps, double* out) {
  double ss = 0.0;
  for (int64_t i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / (double)n + eps);
  for (int64_t i = 0; i < n; ++i) out[i] = x[i] * inv * bf16_to_f64(gain[i]);
}

/* 3D M-RoPE (kaminari sections 03 and 04: positions (3, batch, 1)).  The pages
 * do not say which frequency pair follows which axis.  Reading taken: the
 * interleaved layout (pair j on axis h when j%3==1 and j<3*s_h, on axis w when
 * j%3==2 and j<3*s_w, else t); the contiguous layout ([0,s_t) t, then s_h pairs
 * h, then w) is kept as the alternative. */
int32_t ora_mrope_axis(int64_t j, int64_t half_dim, const int32_t* sec, int32_t interleaved) {
  (void)half_dim;
  if (interleaved) {
    if (j % 3 == 1 && j < 3 * (int64_t)sec[1]) return 1;
    if (j % 3 == 2 && j < 3 * (int64_t)sec[2]) return 2;
    return 0;
  }
  if (j < sec[0]) return 0;
  if (j < (int64_t)sec[0] + sec[1]) return 1;
  return 2;
}

/* Rotate-half pairing (j, j + D/2), angle = pos[axis(j)] * theta^(-2j/D). */
void ora_mrope(double* v, int64_t D, const int32_t* pos3, const int32_t* sec,
               int32_t interleaved, double theta) {
  int64_t half = D / 2;
  for (int64_t j = 0; j < half; ++j) {
    int32_t ax = ora_mrope_axis(j, half, sec, interleaved);
    double inv_freq = pow(theta, -2.0 * (double)j / (double)D);
    double ang = (double)pos3[ax] * inv_freq;
    double c = cos(ang), s = sin(ang);
    double a = v[j], b = v[j + half];
    v[j] = a * c - b * s;
    v[j + half] = b * c + a * s;
  }
}

/* softmax(q . K^T / sqrt(D)) V over n_pos stored bf16 rows (Ghost in the Batch,
 * "What Attention Does (60 Seconds)"). */
void ora_attend(const double* q, const uint16_t* k, const uint16_t* v, int64_t n_pos, int64_t D,
                double* out) {
  double* sc = (double*)malloc(sizeof(double) * (size_t)(n_pos > 0 ? n_pos : 1));
  double inv_sqrt_d = 1.0 / sqrt((double)D);
  double mx = -INFINITY;
  for (int64_t j = 0; j < n_pos; ++j) {
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += q[d] * bf16_to_f64(k[j * D + d]);
    sc[j] = dot * inv_sqrt_d;
    if (sc[j] > mx) mx = sc[j];
  }
  double den = 0.0;
  for (int64_t j = 0; j < n_pos; ++j) {
    sc[j] = exp(sc[j] - mx);
    den += sc[j];
  }
  for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
  for (int64_t j = 0; j < n_pos; ++j) {
    double p = sc[j] / den;
    for (int64_t d = 0; d < D; ++d) out[d] += p * bf16_to_f64(v[j * D + d]);
  }
  free(sc);
}

static double silu(double a) { return a / (1.0 + exp(-a)); }

/* SiLU as the MLP uses it, exported so that tests can pin it to closed forms. */
double ora_silu(double a) { return silu(a); }

/* One decoder layer for B independent rows, in place on x [B][H].
 * Order (kaminari section 03: TextAttention with fused QKV, Mrope, MLP; the
 * standard Qwen3 decoder block, which the pages name but do not spell out):
 *   h = RMSNorm(x; in_norm);  [q|k|v] = W_qkv h
 *   per head: q <- MRoPE(RMSNorm_D(q; q_norm)),  k <- MRoPE(RMSNorm_D(k; k_norm))
 *   K[l][b][g][c_b] = bf16(k), V[l][b][g][c_b] = bf16(v)   (static cache written in
 *       place at cache_position, kaminari sections 03 and 04)
 *   o_h = attention over stored rows 0..c_b of kv head g = h / (Hq/Hkv)
 *   x += W_o o;  h = RMSNorm(x; post_norm);  x += W_down(silu(gate) * up)
 * Returns -1 (and touches nothing) when a cache position is outside [0, M). */
int ora_decode_layer(const ora_dims* d, const ora_layer* w, int64_t layer, uint16_t* kcache,
                     uint16_t* vcache, int64_t B, int64_t M, double* x, const int32_t* pos,
                     const int32_t* cpos) {
  const int64_t H = d->hidden, Hq = d->n_heads, Hkv = d->n_kv_heads, D = d->head_dim;
  const int64_t I = d->intermediate, G = d->group_size;
  const int64_t NQKV = (Hq + 2 * Hkv) * D;
  for (int64_t b = 0; b < B; ++b)
    if (cpos[b] < 0 || cpos[b] >= M) return -1;

  double* h = (double*)calloc((size_t)(B * H), sizeof(double));
  double* qkv = (double*)malloc(sizeof(double) * (size_t)(B * NQKV));
  double* o = (double*)malloc(sizeof(double) * (size_t)(B * Hq * D));
  double* y = (double*)malloc(sizeof(double) * (size_t)(B * H));
  double* gu = (double*)malloc(sizeof(double) * (size_t)(B * 2 * I));
  double* a = (double*)malloc(sizeof(double) * (size_t)(B * I));

  for (int64_t b = 0; b < B; ++b) ora_rmsnorm(x + b * H, w->in_norm, H, d->rms_eps, h + b * H);
  ora_gemv_int4(w->qkv.packed, w->qkv.sz, NQKV, H, G, h, B, qkv);

  for (int64_t b = 0; b < B; ++b) {
    double* row = qkv + b * NQKV;
    int32_t p3[3] = {pos[0 * B + b], pos[1 * B + b], pos[2 * B + b]};
    double* tmp = (double*)malloc(sizeof(double) * (size_t)D);
    for (int64_t hh = 0; hh < Hq; ++hh) {
      ora_rmsnorm(row + hh * D, w->q_norm, D, d->rms_eps, tmp);
      memcpy(row + hh * D, tmp, sizeof(double) * (size_t)D);
      ora_mrope(row + hh * D, D, p3, d->mrope_section, d->mrope_interleaved, d->rope_theta);
    }
    for (int64_t g = 0; g < Hkv; ++g) {
      double* kk = row + (Hq + g) * D;
      double* vv = row + (Hq + Hkv + g) * D;
      ora_rmsnorm(kk, w->k_norm, D, d->rms_eps, tmp);
      memcpy(kk, tmp, sizeof(double) * (size_t)D);
      ora_mrope(kk, D, p3, d->mrope_section, d->mrope_interleaved, d->rope_theta);
      int64_t base = ((((layer * B) + b) * Hkv + g) * M + cpos[b]) * D;
      for (int64_t dd = 0; dd < D; ++dd) {
        kcache[base + dd] = f64_to_bf16(kk[dd]);
        vcache[base + dd] = f64_to_bf16(vv[dd]);
      }
    }
    free(tmp);
  }

  const int64_t qpg = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t hh = 0; hh < Hq; ++hh) {
      int64_t g = hh / qpg;
      int64_t base = (((layer * B) + b) * Hkv + g) * M * D;
      ora_attend(qkv + b * NQKV + hh * D, kcache + base, vcache + base, (int64_t)cpos[b] + 1, D,
                 o + (b * Hq + hh) * D);
    }

  ora_gemv_int4(w->o.packed, w->o.sz, H, Hq * D, G, o, B, y);
  for (int64_t i = 0; i < B * H; ++i) x[i] += y[i];

  for (int64_t b = 0; b < B; ++b) ora_rmsnorm(x + b * H, w->post_norm, H, d->rms_eps, h + b * H);
  ora_gemv_int4(w->gate_up.packed, w->gate_up.sz, 2 * I, H, G, h, B, gu);
  for (int64_t b = 0; b < B; ++b)
    for (int64_t i = 0; i < I; ++i)
      a[b * I + i] = silu(gu[b * 2 * I + i]) * gu[b * 2 * I + I + i];
  ora_gemv_int4(w->down.packed, w->down.sz, H, I, G, a, B, y);
  for (int64_t i = 0; i < B * H; ++i) x[i] += y[i];

  free(h); free(qkv); free(o); free(y); free(gu); free(a);
  return 0;
}

/* One greedy decode step (kaminari section 04, "3 . decode"): embedding of the
 * row's token (pad id for finished rows, whose batch slot stays in the step),
 * all layers, final RMSNorm, bf16 lm_head, argmax (lowest index among equal
 * maxima).  margin[b] = top-1 minus top-2 logit.  With ORA_ADVANCE, a live row
 * takes its token; EOS or reaching the last cache slot marks it finished,
 * otherwise its cache position and all three position axes move on by one.
 * Finished rows emit the pad id and keep their positions. */
int ora_decode_step(const ora_dims* d, const ora_model* m, uint16_t* kcache, uint16_t* vcache,
                    int64_t B, int64_t M, const int32_t* ids, int32_t* pos, int32_t* cpos,
                    uint8_t* finished, uint32_t flags, int32_t* next, double* logits,
                    double* margin, double* hidden_out) {
  const int64_t H = d->hidden, V = d->vocab;
  for (int64_t b = 0; b < B; ++b) {
    if (cpos[b] < 0 || cpos[b] >= M) return -1;
    int32_t id = (finished && finished[b]) ? d->pad_id : ids[b];
    if (id < 0 || id >= V) return -2;
  }
  double* x = (double*)malloc(sizeof(double) * (size_t)(B * H));
  double* hf = (double*)malloc(sizeof(double) * (size_t)(B * H));
  double* lg = logits ? logits : (double*)malloc(sizeof(double) * (size_t)(B * V));

  for (int64_t b = 0; b < B; ++b) {
    int32_t id = (finished && finished[b]) ? d->pad_id : ids[b];
    for (int64_t i = 0; i < H; ++i) x[b * H + i] = bf16_to_f64(m->embed[(int64_t)id * H + i]);
  }
  for (int64_t l = 0; l < d->n_layers; ++l) {
    int rc = ora_decode_layer(d, &m->layers[l], l, kcache, vcache, B, M, x, pos, cpos);
    if (rc) { free(x); free(hf); if (!logits) free(lg); return rc; }
  }
  if (hidden_out) memcpy(hidden_out, x, sizeof(double) * (size_t)(B * H));
  for (int64_t b = 0; b < B; ++b) ora_rmsnorm(x + b * H, m->final_norm, H, d->rms_eps, hf + b * H);
  gemv_bf16(m->lm_head, V, H, hf, B, lg);

  for (int64_t b = 0; b < B; ++b) {
    const double* r = lg + b * V;
    int64_t best = 0;
    for (int64_t n = 1; n < V; ++n)
      if (r[n] > r[best]) best = n;
    double second = -INFINITY;
    for (int64_t n = 0; n < V; ++n)
      if (n != best && r[n] > second) second = r[n];
    if (margin) margin[b] = r[best] - second;
    int fin = finished ? finished[b] : 0;
    next[b] = fin ? d->pad_id : (int32_t)best;
    if ((flags & ORA_ADVANCE) && !fin) {
      if (d->eos_id >= 0 && best == d->eos_id) {
        if (finished) finished[b] = 1;
      } else if ((int64_t)cpos[b] + 1 >= M) {
        if (finished) finished[b] = 1;
      } else {
        cpos[b] += 1;
        for (int ax = 0; ax < 3; ++ax) pos[ax * B + b] += 1;
      }
    }
  }
  free(x); free(hf);
  if (!logits) free(lg);
  return 0;
}
