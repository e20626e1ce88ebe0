// HIP kernels of the int4 weight-only decode step (gfx950, wave64).
//
// Decode step as on the kaminari page ("kaminari - a single-GPU Qwen3-VL
// inference engine, explained", section 04 "3 . decode"; model structure in
// section 03; int4 weight-only decoder linears in section 07); attention and its
// split merge as in "The Ghost in the Batch" ("What Attention Does", "The merge
// math").
#pragma once
#include "kmr_device.h"

namespace kmr {

constexpr int kAttnSplit = 64;     // cache positions per attention item of the device-wide
                                   // persistent kernel, and ...
constexpr int kAttnSplitPP = 256;  // ... per work-group of the per-phase kernels (both fixed,
                                   // so a row's result never depends on the batch size)
constexpr int kGemvRowsPerWave = 2;
constexpr int kLmRowsPerWave = 4;
constexpr int kLmRowsPerBlock = 4 * kLmRowsPerWave;

constexpr uint32_t kStatusRange = 16u;   // a staged GEMV input overflowed fp16

__device__ __forceinline__ void raise_status(uint32_t* st, uint32_t bit) {
  __hip_atomic_fetch_or(st, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ read probe
// Streams `words` 16-byte words with the 16-byte non-temporal loads the GEMVs use,
// eight loads in flight per thread, and writes one XOR word per thread so that no
// load can be dropped: the achievable streaming-read rate of the device.
__global__ __launch_bounds__(256) void k_read_probe(const uint4* __restrict__ src, size_t words,
                                                    uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x, nt = (size_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + 7 * nt < words; i += 8 * nt) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = load_stream16(src + i + u * nt);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < words; i += nt) {
    const uint4 v = load_stream16(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = acc;
}

// ------------------------------------------------------------------ fill

// Clears every status bit outside `keep` (one thread).
__global__ void k_status_keep(uint32_t* st, uint32_t keep) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *st &= keep;
}

__global__ void k_fill_zero(uint32_t* __restrict__ p, size_t words) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < words; i += stride) p[i] = 0u;
}

// ------------------------------------------------------------------ slots
// One cache row copy: blockIdx.y = 2 * (layer * Hkv + head) + (0: K, 1: V) picks a
// contiguous run of n * D bf16 in each cache; 16-byte words along x.
struct KvCopyArgs {
  const uint16_t *sk, *sv;
  uint16_t *dk, *dv;
  int Hkv, D, n;
  int sB, sM, srow, dB, dM, drow;
};

__global__ __launch_bounds__(256) void k_kv_copy_row(KvCopyArgs a) {
  const int s = blockIdx.y >> 1, which = blockIdx.y & 1;
  const int l = s / a.Hkv, g = s - l * a.Hkv;
  const uint4* src = reinterpret_cast<const uint4*>(
      (which ? a.sv : a.sk) + (((size_t)l * a.sB + a.srow) * a.Hkv + g) * a.sM * a.D);
  uint4* dst = reinterpret_cast<uint4*>((which ? a.dv : a.dk) +
                                        (((size_t)l * a.dB + a.drow) * a.Hkv + g) * a.dM * a.D);
  const size_t words = (size_t)a.n * a.D / 8;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256)
    dst[i] = src[i];
}

// Admit (admit != 0) or retire one slot: single-thread stores of its step state.
__global__ void k_slot_set(int32_t* ids, int32_t* pos, int32_t* cpos, uint8_t* fin, int B, int row,
                           int admit, int token, int p0, int p1, int p2, int c) {
  if (threadIdx.x != 0) return;
  if (admit) {
    ids[row] = token;
    pos[row] = p0;
    pos[B + row] = p1;
    pos[2 * B + row] = p2;
    cpos[row] = c;
    fin[row] = 0;
  } else {
    fin[row] = 1;
  }
}

// ------------------------------------------------------------------ int4 quantizer
// Per (row, group): s = bf16(max((hi-lo)/15, 2^-24)), z = bf16(lo + 8 s),
// q = clamp(rne((w - z)/s) + 8, 0, 15); IEEE fp32, each operation rounded on its
// own (no contraction), divisions correctly rounded.  One thread per group: this
// runs once per model and is not on the decode path.
__global__ void k_quantize_int4(const uint16_t* __restrict__ w, int N, int K, int G,
                                uint8_t* __restrict__ packed, uint32_t* __restrict__ sz) {
#pragma clang fp contract(off)
  const int ng = K / G;
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long long)N * ng) return;
  const int n = (int)(idx / ng), g = (int)(idx % ng);
  const uint16_t* src = w + (size_t)n * K + (size_t)g * G;
  float lo = bf16_to_f32(src[0]), hi = lo;
  for (int i = 1; i < G; ++i) {
    float v = bf16_to_f32(src[i]);
    lo = v < lo ? v : lo;
    hi = v > hi ? v : hi;
  }
  float range = hi - lo;
  float s32 = range / 15.0f;
  if (!(s32 >= 0x1p-24f)) s32 = 0x1p-24f;
  const uint16_t sb = f32_to_bf16(s32);
  const float s = bf16_to_f32(sb);
  const float eight_s = 8.0f * s;
  const float z32 = lo + eight_s;
  const uint16_t zb = f32_to_bf16(z32);
  const float z = bf16_to_f32(zb);
  sz[idx] = (uint32_t)sb | ((uint32_t)zb << 16);
  uint8_t* dst = packed + (size_t)n * (K / 2) + (size_t)g * (G / 2);
  for (int i = 0; i < G; i += 2) {
    int q2[2];
    for (int t = 0; t < 2; ++t) {
      float diff = bf16_to_f32(src[i + t]) - z;
      float r = __builtin_rintf(diff / s);
      int q = (int)r + 8;
      q2[t] = q < 0 ? 0 : (q > 15 ? 15 : q);
    }
    dst[i / 2] = (uint8_t)(q2[0] | (q2[1] << 4));
  }
}

// ------------------------------------------------------------------ step prologue
// Embedding gather (bf16 row -> fp32 residual stream; finished rows read pad_id)
// and the RoPE cos/sin of each row's three-axis position, in fp64 then rounded
// to fp32: pair j uses axis(j) and angle pos[axis] * theta^(-2j/D).
struct PrepArgs {
  const uint16_t* embed;   // [V][H] or null (layer-only call)
  const int32_t* ids;      // [B]
  const uint8_t* finished; // [B] or null
  const int32_t* pos;      // [3][B]
  float* x;                // [B][H]
  float2* cs;              // [B][D/2]
  uint32_t* status;
  int B, H, V, D, pad_id;
  double theta;
  int sec0, sec1, sec2, interleaved;
};

__device__ __forceinline__ int mrope_axis(int j, int s0, int s1, int s2, int interleaved) {
  if (interleaved) {
    if (j % 3 == 1 && j < 3 * s1) return 1;
    if (j % 3 == 2 && j < 3 * s2) return 2;
    return 0;
  }
  (void)s2;
  return j < s0 ? 0 : (j < s0 + s1 ? 1 : 2);
}

__global__ __launch_bounds__(256) void k_prep(PrepArgs a) {
  const int b = blockIdx.x, tid = threadIdx.x;
  if (a.embed) {
    int id = (a.finished && a.finished[b]) ? a.pad_id : a.ids[b];
    const bool ok = id >= 0 && id < a.V;
    if (!ok && tid == 0) raise_status(a.status, 2u);
    const uint16_t* row = a.embed + (size_t)(ok ? id : 0) * a.H;
    for (int k = tid; k < a.H; k += blockDim.x) a.x[(size_t)b * a.H + k] = ok ? bf16_to_f32(row[k]) : 0.0f;
  }
  const int half = a.D / 2;
  for (int j = tid; j < half; j += blockDim.x) {
    const int ax = mrope_axis(j, a.sec0, a.sec1, a.sec2, a.interleaved);
    const double p = (double)a.pos[ax * a.B + b];
    const double inv_freq = pow(a.theta, -2.0 * (double)j / (double)a.D);
    double sn, cn;
    sincos(p * inv_freq, &sn, &cn);
    a.cs[(size_t)b * half + j] = make_float2((float)cn, (float)sn);
  }
}

// ------------------------------------------------------------------ attention partials
// A split of kAttnSplitPP cache positions leaves, per q head, the running max m
// (log2 domain), the sum l of 2^(s - m) and the unnormalised o~ = sum 2^(s - m) v.
// Splits merge with log-sum-exp weights, in split order:
//     o = sum_s 2^(m_s - M) o~_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s.
// The same device function serves the fused O-projection prologue and the
// stand-alone combine kernel, so both give identical bits.
struct AttnPart {
  const float* part_o;     // [B][Hkv][NS][QPG][D]
  const float2* part_ml;   // [B][Hkv][NS][QPG]
  const int32_t* cpos;     // [B]
  int Hkv, NS, QPG, D, M;
};

__device__ __forceinline__ int attn_splits(int c, int M) {
  return (c < 0 || c >= M) ? 1 : c / kAttnSplit + 1;
}
__device__ __forceinline__ int attn_splits_pp(int c, int M) {
  return (c < 0 || c >= M) ? 1 : c / kAttnSplitPP + 1;
}

// Log-sum-exp merge of two partial states (m, l, o[ND]) into the first; an empty
// state has m = -inf.  The fused multiply-adds are explicit so that every caller
// rounds alike; `a` is always the state of the lower split class.
template <int ND>
__device__ __forceinline__ void lse_pair(float& ma, float& la, float* oa, float mb, float lb, const float* ob) {
  if (mb == -INFINITY) return;
  if (ma == -INFINITY) {
    ma = mb;
    la = lb;
#pragma unroll
    for (int i = 0; i < ND; ++i) oa[i] = ob[i];
    return;
  }
  const float mn = fmaxf(ma, mb), ca = exp2f(ma - mn), cb = exp2f(mb - mn);
  la = __builtin_fmaf(la, ca, lb * cb);
#pragma unroll
  for (int i = 0; i < ND; ++i) oa[i] = __builtin_fmaf(oa[i], ca, ob[i] * cb);
  ma = mn;
}

// Partial state of split class j (splits t = j, j + 8, ... in order) of dims
// [d0, d0 + ND) of q head h of batch row b.
template <int ND>
__device__ __forceinline__ void merge_class(const AttnPart& p, int b, int h, int d0, int j, float& m, float& l,
                                            float* o) {
  const int g = h / p.QPG, hh = h - g * p.QPG;
  const int ns = attn_splits_pp(p.cpos[b], p.M);
  const size_t base = ((size_t)b * p.Hkv + g) * p.NS;
  m = -INFINITY;
  l = 0.f;
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = 0.f;
  for (int t = j; t < ns; t += 8) {
    const size_t slot = (base + t) * p.QPG + hh;
    const float2 ml = p.part_ml[slot];
    float ov[ND];
    const float4* src = reinterpret_cast<const float4*>(p.part_o + slot * p.D + d0);
#pragma unroll
    for (int i = 0; i < ND / 4; ++i) {
      const float4 v = src[i];
      ov[4 * i] = v.x; ov[4 * i + 1] = v.y; ov[4 * i + 2] = v.z; ov[4 * i + 3] = v.w;
    }
    lse_pair<ND>(m, l, o, ml.x, ml.y, ov);
  }
}

// Merges dims [d0, d0 + ND) of q head h of batch row b: the 8 split classes, then
// the fixed tree ((0 1)(2 3))((4 5)(6 7)).  k_attn_combine runs the classes on 8
// lanes and the tree with lane exchanges: the same operations in the same order.
template <int ND>
__device__ __forceinline__ void merge_head(const AttnPart& p, int b, int h, int d0, float* out) {
  float m[8], l[8], o[8][ND];
#pragma unroll
  for (int j = 0; j < 8; ++j) merge_class<ND>(p, b, h, d0, j, m[j], l[j], o[j]);
#pragma unroll
  for (int k = 1; k < 8; k <<= 1)
#pragma unroll
    for (int j = 0; j < 8; j += 2 * k) lse_pair<ND>(m[j], l[j], o[j], m[j + k], l[j + k], o[j + k]);
  const float inv = 1.0f / l[0];
#pragma unroll
  for (int i = 0; i < ND; ++i) out[i] = o[0][i] * inv;
}

// Stand-alone merge: 8 lanes per (batch row, q head, 4 dims), lane j taking split
// class j -> o fp32 [B][Hq*D].
__global__ __launch_bounds__(256) void k_attn_combine(AttnPart p, float* __restrict__ out, int B,
                                                      int Hq) {
  const int quads = p.D / 4;
  const int t = blockIdx.x * blockDim.x + threadIdx.x, j = t & 7, idx = t >> 3;
  const bool live = idx < B * Hq * quads;   // (whole 8-lane groups: live is uniform in a group)
  const int b = live ? idx / (Hq * quads) : 0, r = idx - b * Hq * quads;
  const int h = live ? r / quads : 0, dq = live ? r - h * quads : 0;
  float m, l, o[4];
  merge_class<4>(p, b, h, 4 * dq, j, m, l, o);
#pragma unroll
  for (int k = 1; k < 8; k <<= 1) {
    const float mp = __shfl_xor(m, k), lp = __shfl_xor(l, k);
    float op[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) op[i] = __shfl_xor(o[i], k);
    if (j & k) {   // the partner holds the lower class: it is the first operand
      float ml = mp, ll = lp, ol[4] = {op[0], op[1], op[2], op[3]};
      lse_pair<4>(ml, ll, ol, m, l, o);
      m = ml; l = ll;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = ol[i];
    } else {
      lse_pair<4>(m, l, o, mp, lp, op);
    }
  }
  if (live && j == 0) {
    const float inv = 1.0f / l;
    *reinterpret_cast<float4*>(out + (size_t)b * Hq * p.D + h * p.D + 4 * dq) =
        make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  }
}

// ------------------------------------------------------------------ int4 GEMV
// y[b][n] = sum_k w_hat[n][k] x[b][k] with w_hat = (q - 8) s + z per (row, group),
// for batch rows b < B (compile-time tile BT >= B).  Prologues: plain input,
// RMSNorm (x <- x / sqrt(mean x^2 + eps) * gain), or the attention merge above
// (the O projection reads the split partials directly).  Epilogues: store,
// residual add, SiLU(gate) * up over row pairs (n, n + N).
//
// Each wave owns kGemvRowsPerWave rows and lane l covers columns
// [32 (l + 64 j), +32) for j < CPL; its weight loads are issued before the
// prologue so that their latency overlaps the input staging.
//
// Dequantization stays in registers: a 32-bit word of 8 codes becomes four fp16
// pairs with one shift and four and-or operations, using the exponent of 1024
// as a magic bias (0x6400 | q is 1024 + q; codes in bits 4..7 of a half read as
// 1024 + 16 q).  The input is staged in LDS as matching fp16 pairs (odd columns
// pre-divided by 16), so v_dot2_f32_f16 accumulates sum q x plus a known bias in
// fp32; per 32-column chunk the bias and sum x are precomputed, folding scale
// and zero into two multiply-adds per chunk:
//     sum_k ((q_k - 8) s + z) x_k = s (dot - C1) + z C2.
enum { EPI_STORE = 0, EPI_ADD = 1, EPI_SILU = 2 };
enum { PRO_PLAIN = 0, PRO_RMSNORM = 1, PRO_ATTN = 2 };

struct GemvArgs {
  const uint8_t* packed;  // [rows][K/2]
  const uint32_t* sz;     // [rows][K/G] (scale | zero << 16)
  const float* x;         // [B][ldx]   (PRO_PLAIN, PRO_RMSNORM)
  const uint16_t* gain;   // [K]        (PRO_RMSNORM)
  float* y;               // [B][ldy]
  int N;                  // outputs per batch row (EPI_SILU: weight rows are 2N)
  int K, G, B, ldx, ldy;
  float eps;
  AttnPart ap;            // PRO_ATTN; ap.cpos is indexed from batch row b0
  int b0;                 // first batch row of this tile (PRO_ATTN)
  uint4* xsg;             // staged input of a 16-row tile in memory: [16][4][K/32] ...
  float2* ccg;            // ... its chunk constants [16][K/32] ...
  float2* cbg;            // ... and their sums per 128-column block [16][K/128] (k_gemv_stage16)
  float* kpart;           // split-K partials [2][kpart_rows][N] of an EPI_ADD product (or null),
  int kpart_rows, kpart_n;   // for N <= kpart_n
  uint32_t* status;       // sticky status word (KMR_STATUS_RANGE when a staged input overflows fp16)
};

// LDS layout of k_gemv_int4 (byte offsets, 16-byte aligned).
struct GemvLds {
  size_t xs, cc, xm, red, total;
};
__host__ __device__ inline GemvLds gemv_lds(int BT, int K, bool merged_input) {
  GemvLds l{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 15) & ~(size_t)15; return r; };
  const size_t CH = (size_t)K / 32;
  l.xs = take((size_t)BT * 4 * CH * 16);
  l.cc = take((size_t)BT * CH * 8);
  l.xm = take(merged_input ? (size_t)BT * K * 4 : 0);
  l.red = take((size_t)BT * 5 * 4);
  l.total = o;
  return l;
}

// One 32-column chunk e of a staged GEMV input: its four 16-byte words of fp16
// magic-bias pairs (h[8j+i], h[8j+i+4]), odd columns divided by 16, to dst[j * CH]
// for j < 4, and the chunk constants (1024 sum h + 8 sum u, sum u) returned.  A
// value past the fp16 range (the sums then turn infinite or NaN) raises
// KMR_STATUS_RANGE in *status when status is not null.
__device__ __forceinline__ float2 stage_chunk(const float (&e)[32], uint4* dst, int CH, uint32_t* status) {
  float bsum = 0.f, usum = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float* f = e + 8 * j;
    _Float16 h0 = (_Float16)f[0], h4 = (_Float16)f[4], h2 = (_Float16)f[2], h6 = (_Float16)f[6];
    _Float16 h1 = (_Float16)(f[1] * 0.0625f), h5 = (_Float16)(f[5] * 0.0625f);
    _Float16 h3 = (_Float16)(f[3] * 0.0625f), h7 = (_Float16)(f[7] * 0.0625f);
    uint4 pk;
    pk.x = __builtin_bit_cast(uint32_t, half2_t{h0, h4});
    pk.y = __builtin_bit_cast(uint32_t, half2_t{h1, h5});
    pk.z = __builtin_bit_cast(uint32_t, half2_t{h2, h6});
    pk.w = __builtin_bit_cast(uint32_t, half2_t{h3, h7});
    dst[j * CH] = pk;
    const float ev = ((float)h0 + (float)h4) + ((float)h2 + (float)h6);
    const float od = ((float)h1 + (float)h5) + ((float)h3 + (float)h7);
    bsum += ev + od;
    usum += ev + 16.0f * od;
  }
  if (status && !(fabsf(bsum) + fabsf(usum) <= 3.0e38f)) raise_status(status, kStatusRange);
  return make_float2(1024.0f * bsum + 8.0f * usum, usum);
}

// Stages the B <= BT input rows of a GEMV in LDS after its prologue (plain input,
// RMSNorm of it, or the attention merge): the fp16 magic-bias pairs xs [BT][4][CH]
// (h[8w+i], h[8w+i+4]) with odd columns divided by 16, and the per-chunk constants
// cc [BT][CH] = (1024 sum h + 8 sum u, sum u).  Rows b >= B are zero.  Every
// thread of the block must call this; the data is in LDS for all on return.
template <int BT, int PRO>
__device__ __forceinline__ void gemv_stage(const GemvArgs& a, unsigned char* smem) {
  const int K = a.K, CH = K >> 5, B = a.B;
  const GemvLds lay = gemv_lds(BT, K, PRO == PRO_ATTN);
  uint4* xs = reinterpret_cast<uint4*>(smem + lay.xs);            // [BT][4][CH]
  float2* cc = reinterpret_cast<float2*>(smem + lay.cc);          // [BT][CH]
  float* xm = reinterpret_cast<float*>(smem + lay.xm);            // [BT][K] (PRO_ATTN)
  float* red = reinterpret_cast<float*>(smem + lay.red);          // [BT][4]
  float* sinv = red + BT * 4;                                     // [BT]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (PRO == PRO_ATTN) {
    for (int idx = tid; idx < BT * (K / 4); idx += 256) {
      const int b = idx / (K / 4), k4 = 4 * (idx - b * (K / 4));
      float o4[4] = {0.f, 0.f, 0.f, 0.f};
      if (b < B) merge_head<4>(a.ap, a.b0 + b, k4 / a.ap.D, k4 % a.ap.D, o4);
      *reinterpret_cast<float4*>(xm + b * K + k4) = make_float4(o4[0], o4[1], o4[2], o4[3]);
    }
    __syncthreads();
  }
  if (PRO == PRO_RMSNORM) {
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      float ss = 0.f;
      if (b < B)
        for (int k = tid * 4; k < K; k += 1024) {
          float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)b * a.ldx + k);
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
      ss = wave_sum(ss);
      if (lane == 0) red[b * 4 + wave] = ss;
    }
    __syncthreads();
    if (tid < BT) {
      float ss = (red[tid * 4 + 0] + red[tid * 4 + 1]) + (red[tid * 4 + 2] + red[tid * 4 + 3]);
      sinv[tid] = 1.0f / sqrtf(ss / (float)K + a.eps);
    }
    __syncthreads();
  }
  for (int idx = tid; idx < BT * CH; idx += 256) {
    const int b = idx / CH, c = idx - b * CH;
    float e[32];
    if (b < B) {
      if (PRO == PRO_ATTN) {
#pragma unroll
        for (int i = 0; i < 32; ++i) e[i] = xm[b * K + 32 * c + i];
      } else {
        const float4* src = reinterpret_cast<const float4*>(a.x + (size_t)b * a.ldx + 32 * c);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float4 v = src[i];
          e[4 * i] = v.x; e[4 * i + 1] = v.y; e[4 * i + 2] = v.z; e[4 * i + 3] = v.w;
        }
      }
      if (PRO == PRO_RMSNORM) {
        const float iv = sinv[b];
        const uint32_t* gw = reinterpret_cast<const uint32_t*>(a.gain + 32 * c);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          uint32_t gg = gw[i];
          e[2 * i] = (e[2 * i] * iv) * bf16_lo(gg);
          e[2 * i + 1] = (e[2 * i + 1] * iv) * bf16_hi(gg);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) e[i] = 0.f;
    }
    cc[b * CH + c] = stage_chunk(e, xs + b * 4 * CH + c, CH, a.status);
  }
  __syncthreads();

}

template <int BT, int EPI, int PRO, int CPL>
__global__ __launch_bounds__(256) void k_gemv_int4(GemvArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int K = a.K, CH = K >> 5, NG = K / a.G, B = a.B;
  const GemvLds lay = gemv_lds(BT, K, PRO == PRO_ATTN);
  uint4* xs = reinterpret_cast<uint4*>(smem + lay.xs);            // [BT][4][CH]
  float2* cc = reinterpret_cast<float2*>(smem + lay.cc);          // [BT][CH]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  constexpr int RPW = kGemvRowsPerWave;
  constexpr int NR = (EPI == EPI_SILU ? 2 : 1) * RPW;
  const int n0 = (blockIdx.x * 4 + wave) * RPW;
  int wrow[NR];
  bool ok[NR];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int n = n0 + r;
    ok[r] = n < a.N;
    wrow[r] = ok[r] ? n : 0;
    if (EPI == EPI_SILU) {
      ok[RPW + r] = ok[r];
      wrow[RPW + r] = ok[r] ? n + a.N : 0;
    }
  }
  // ---- weight stream first
  uint4 w[NR][CPL];
  uint32_t sw[NR][CPL];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (ok[i] && c < CH) {
        w[i][j] = load_stream16(a.packed + (size_t)wrow[i] * (K / 2) + 16 * c);
        sw[i][j] = a.sz[(size_t)wrow[i] * NG + (32 * c) / a.G];
      } else {
        w[i][j] = make_uint4(0, 0, 0, 0);
        sw[i][j] = 0;
      }
    }

  // ---- prologue: input staging
  gemv_stage<BT, PRO>(a, smem);

  // ---- dequantize and multiply
  float acc[NR][BT];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[i][b] = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    if (c < CH) {
      uint32_t p[NR][16];
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const uint32_t ww[4] = {w[i][j].x, w[i][j].y, w[i][j].z, w[i][j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t t = ww[q] >> 8;
          p[i][4 * q + 0] = and_or(ww[q], 0x000F000Fu, 0x64006400u);
          p[i][4 * q + 1] = and_or(ww[q], 0x00F000F0u, 0x64006400u);
          p[i][4 * q + 2] = and_or(t, 0x000F000Fu, 0x64006400u);
          p[i][4 * q + 3] = and_or(t, 0x00F000F0u, 0x64006400u);
        }
      }
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        uint4 xv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[q] = xs[(b * 4 + q) * CH + c];
        const float2 C = cc[b * CH + c];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          float d = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            d = fdot2(p[i][4 * q + 0], xv[q].x, d);
            d = fdot2(p[i][4 * q + 1], xv[q].y, d);
            d = fdot2(p[i][4 * q + 2], xv[q].z, d);
            d = fdot2(p[i][4 * q + 3], xv[q].w, d);
          }
          // explicit fused ops: the same arithmetic in every instantiation and row
          acc[i][b] = __builtin_fmaf(bf16_lo(sw[i][j]), d - C.x, __builtin_fmaf(bf16_hi(sw[i][j]), C.y, acc[i][b]));
        }
      }
    }
  }

  float v[NR][BT];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int b = 0; b < BT; ++b) v[i][b] = wave_sum(acc[i][b]);

  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if (!ok[r]) continue;
      const int n = n0 + r;
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        if (b >= B) break;
        float* dst = a.y + (size_t)b * a.ldy + n;
        if (EPI == EPI_STORE) {
          *dst = v[r][b];
        } else if (EPI == EPI_ADD) {
          *dst += v[r][b];
        } else {
          const float g = v[r][b], u = v[RPW + r][b];
          *dst = g / (1.0f + expf(-g)) * u;
        }
      }
    }
  }
}

// The staged input of a 16-row batch tile written once to memory (a.xsg, a.ccg, and
// the chunk constants summed per 128-column block in a.cbg), in the layout
// gemv_stage gives LDS, for k_gemv_int4_mfma with GS set.  Grid (16 rows, K/2048):
// one wave per row and 64 chunks, lane = chunk; rows b >= B are zero.  Plain input
// or its RMSNorm (each wave sums the squares of its whole row).
template <int PRO>
__global__ __launch_bounds__(64) void k_gemv_stage16(GemvArgs a) {
  static_assert(PRO == PRO_PLAIN || PRO == PRO_RMSNORM, "plain or RMSNorm input");
  const int b = blockIdx.x, K = a.K, CH = K >> 5, lane = threadIdx.x, c = blockIdx.y * 64 + lane;
  const bool live = b < a.B;
  const float* xr = a.x + (size_t)(live ? b : 0) * a.ldx;
  // this lane's chunk (and gains) first, in flight during the sum of squares
  float e[32];
  uint32_t gw[16];
  const bool own = live && c < CH;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 v = own ? reinterpret_cast<const float4*>(xr + 32 * c)[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    e[4 * i] = v.x; e[4 * i + 1] = v.y; e[4 * i + 2] = v.z; e[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)
    gw[i] = (PRO == PRO_RMSNORM && own) ? reinterpret_cast<const uint32_t*>(a.gain + 32 * c)[i] : 0u;
  if (PRO == PRO_RMSNORM) {
    float ss = 0.f;
    if (live)
      for (int k = lane * 4; k < K; k += 256) {
        const float4 v = *reinterpret_cast<const float4*>(xr + k);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    const float iv = 1.0f / sqrtf(wave_sum(ss) / (float)K + a.eps);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      e[2 * i] = (e[2 * i] * iv) * bf16_lo(gw[i]);
      e[2 * i + 1] = (e[2 * i + 1] * iv) * bf16_hi(gw[i]);
    }
  }
  uint4 scratch[4];
  const float2 C = stage_chunk(e, c < CH ? a.xsg + b * 4 * CH + c : scratch, c < CH ? CH : 1, a.status);
  if (c < CH) a.ccg[b * CH + c] = C;
  // block constants: the 4 chunks of a 128-column block are lanes 4m .. 4m + 3
  float c1 = C.x, c2 = C.y;
  c1 += dpp<0xB1>(c1); c2 += dpp<0xB1>(c2);   // lane ^ 1
  c1 += dpp<0x4E>(c1); c2 += dpp<0x4E>(c2);   // lane ^ 2
  if ((lane & 3) == 0 && c < CH) a.cbg[b * (CH >> 2) + (c >> 2)] = make_float2(c1, c2);
}

// Batch tiles of up to BT = 16 rows on the matrix cores (group size a multiple of
// 128).  A block takes 16 weight rows (EPI_SILU: 16 gate rows and their 16 up
// rows) and its 4 waves split K by 128-column blocks (wave w: blocks w, w + 4, ...).
// Per block, lane (n, gq) = (lane % 16, lane / 16) holds the codes of weight row n
// over chunk 4 kb + gq and the staged batch row n over the same chunk; four
// v_mfma_f32_16x16x32_f16 with the staged rows as the first operand leave in lane
// (n, gq) the dots of batch rows 4 gq + e with weight row n, and the block's scale
// and zero point apply as s (d - C1) + z C2 with the staged constants summed over
// its four chunks (the same algebra as k_gemv_int4, per 128 columns instead of 32).
// Wave partials are summed through LDS in wave order before the epilogue.
constexpr int kMfmaBlocksPerWave = 16;   // K <= 4 * 16 * 128 = 8192
// GS: the staged input comes from memory (k_gemv_stage16) instead of being built in
// this group's LDS.
template <int BT, int EPI, int PRO, bool GS>
__global__ __launch_bounds__(256) void k_gemv_int4_mfma(GemvArgs a) {
  static_assert(BT == 16, "one 16-row operand of batch rows");
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NT = EPI == EPI_SILU ? 2 : 1;   // 16-row weight tiles per block
  // staged in memory (GS): blockIdx.y picks a 16-row tile of the staged rows and of y
  const int tr = GS ? 16 * (int)blockIdx.y : 0;
  const int K = a.K, CH = K >> 5, NG = K / a.G, NB = K >> 7;
  const int B = GS ? (a.B - tr < 16 ? a.B - tr : 16) : a.B;
  const GemvLds lay = gemv_lds(BT, K, PRO == PRO_ATTN);
  const uint4* xs = GS ? a.xsg + (size_t)tr * 4 * CH : reinterpret_cast<const uint4*>(smem + lay.xs);   // [BT][4][CH]
  const float2* cc = GS ? a.ccg + (size_t)tr * CH : reinterpret_cast<const float2*>(smem + lay.cc);     // [BT][CH]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, gq = lane >> 4;
  const int r0 = blockIdx.x * 16;
  const bool rok = r0 + n < a.N;
  // split K (GS, EPI_ADD): blockIdx.z takes the z-th of gridDim.z equal runs of 128-column blocks
  const int KZ = GS ? (int)gridDim.z : 1, kz = GS ? (int)blockIdx.z : 0, NBz = NB / KZ, kb0 = kz * NBz;
  const int nbw = NBz > wave ? (NBz - wave + 3) >> 2 : 0;   // this wave's 128-column blocks

  // ---- weight stream first (in flight while the input is staged)
  uint4 w[NT][kMfmaBlocksPerWave];
  uint32_t sw[NT][kMfmaBlocksPerWave];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int row = rok ? r0 + n + t * a.N : 0;
#pragma unroll
    for (int i = 0; i < kMfmaBlocksPerWave; ++i) {
      const int kb = kb0 + wave + 4 * i;
      if (i < nbw && rok) {
        w[t][i] = load_stream16(a.packed + (size_t)row * (K / 2) + 16 * (4 * kb + gq));
        sw[t][i] = a.sz[(size_t)row * NG + ((kb << 7) / a.G)];
      } else {
        w[t][i] = make_uint4(0, 0, 0, 0);
        sw[t][i] = 0;
      }
    }
  }
  if constexpr (!GS) gemv_stage<BT, PRO>(a, smem);

  // ---- dequantize and multiply
  const int bn = n < B ? n : 0;   // staged row of this lane's operand (padding repeats row 0)
  float acc[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[t][e] = 0.f;
#pragma unroll
  for (int i = 0; i < kMfmaBlocksPerWave; ++i) {
    if (i >= nbw) continue;   // (not break: the loop unrolls, w and sw stay in registers)
    const int kb = kb0 + wave + 4 * i, c = 4 * kb + gq;
    uint4 xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[q] = xs[(bn * 4 + q) * CH + c];
    // the block's input sums of batch rows 4 gq + e
    float C2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = 4 * gq + e < BT ? 4 * gq + e : 0;
      if constexpr (GS) {
        C2[e] = a.cbg[(tr + b) * NB + kb].y;
      } else {
        const float2* cp = cc + b * CH + 4 * kb;
        C2[e] = (cp[0].y + cp[1].y) + (cp[2].y + cp[3].y);
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint32_t p[16];
      dequant16(w[t][i], p);
      // the bias off before the product: even words 1024 + q -> q - 8, odd words
      // 1024 + 16 q -> 16 (q - 8), all exact in fp16.  The matrix core then never
      // sums the 1024-sized terms whose cancellation against the block constant
      // lost ~1e-3 of the result (the VALU path's fp32 sums do not).
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const half2_t h = __builtin_bit_cast(half2_t, p[j]);
        const _Float16 off = (j & 1) ? (_Float16)1152.0f : (_Float16)1032.0f;
        p[j] = __builtin_bit_cast(uint32_t, half2_t{h[0] - off, h[1] - off});
      }
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        d = mfma16x16x32(xv[kt], make_uint4(p[4 * kt], p[4 * kt + 1], p[4 * kt + 2], p[4 * kt + 3]), d);
      const float sc = bf16_lo(sw[t][i]), zp = bf16_hi(sw[t][i]);
      // a weight is sc (q - 8) + zp: sum x w = sc d + zp sum x, with C2 = sum x
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] += __builtin_fmaf(sc, d[e], zp * C2[e]);
    }
  }

  // ---- wave partials -> LDS [4 waves][NT][16 batch rows][16 weight rows], then the epilogue
  __syncthreads();   // (LDS staging: the input is no longer read, its space takes the partials)
  float* part = reinterpret_cast<float*>(smem + (GS ? 0 : lay.xs));
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (4 * gq + e < BT) part[((wave * NT + t) * 16 + 4 * gq + e) * 16 + n] = acc[t][e];
  __syncthreads();
  {
    const int b = tid >> 4, r = tid & 15, nr = r0 + r;
    if (b < B && nr < a.N) {
      float v[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float s = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; ++wv) s += part[((wv * NT + t) * 16 + b) * 16 + r];
        v[t] = s;
      }
      float* dst = a.y + (size_t)(tr + b) * a.ldy + nr;
      if (KZ > 1) {   // (EPI_ADD only) this half's partial; k_gemv_kreduce adds both to y
        a.kpart[((size_t)kz * a.kpart_rows + tr + b) * a.N + nr] = v[0];
      } else if (EPI == EPI_STORE) {
        *dst = v[0];
      } else if (EPI == EPI_ADD) {
        *dst += v[0];
      } else {
        const float g = v[0], u = v[NT - 1];
        *dst = g / (1.0f + expf(-g)) * u;
      }
    }
  }
}

// y[b][n] += (p0 + p1) for the two split-K partials of an EPI_ADD product (fixed order).
__global__ void k_gemv_kreduce(float* y, int ldy, const float* kpart, int rows, int N, int B) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * N) return;
  const int b = i / N, n = i - b * N;
  y[(size_t)b * ldy + n] += kpart[(size_t)b * N + n] + kpart[((size_t)rows + b) * N + n];
}

// ------------------------------------------------------------------ attention
// One work-group per (split of kAttnSplitPP positions, kv head g, batch row b).
// Each 16-lane row of a wave takes one cache position per step (head_dim/16
// dims per lane, so the four rows of a wave read four consecutive cache rows),
// and all of a lane's cache reads are issued first, before the prologue:
// per-head RMSNorm of q and k over head_dim, M-RoPE on both, bf16 rounding of
// the new k and v (their storage precision).  The group owning slot
// cache_position writes them to the cache and attends to them directly.  An
// online softmax per q head of the GQA group runs over the split; the 16 row
// states merge in LDS into this split's partial (m, l, o~), written to the
// workspace for merge_head.
struct AttnArgs {
  const float* qkv;        // [B][ldqkv]
  const uint16_t* q_norm;  // [D]
  const uint16_t* k_norm;  // [D]
  const float2* cs;        // [B][D/2]
  uint16_t* kc;            // layer slice [cacheB][Hkv][M][D]
  uint16_t* vc;
  const int32_t* cpos;     // [B]
  float* part_o;           // [B][Hkv][NS][QPG][D]
  float2* part_ml;         // [B][Hkv][NS][QPG]
  uint32_t* status;
  int ldqkv, Hq, Hkv, M, NS;
  float eps, scale_log2;   // log2(e) / sqrt(D)
  int B;                   // rows
  int first_split;         // shared-prefix splits (0: none) ...
  int prefix_row;          // ... and the cache row that holds the prefix
};

// The attention of split s of kv head g for batch row b (cache position c), given
// this lane's K/V words of the split (kr, vr: positions s*kAttnSplitPP +
// (kAttnSplitPP/4) wave + 4 it + lane/16, dims DPL*(lane%16) ..): q/k norm and RoPE of the row's new token,
// its cache write (last split), the block softmax of each 16-lane row, the 16 row
// states merged, and the split's partial stored.  Every thread of the group calls
// this; it ends after the partial stores (a caller that calls it again must first
// wait at a barrier).
template <int D, int QPG>
__device__ __forceinline__ void attn_split(const AttnArgs& a, int b, int g, int s, int c,
                                           const uint32_t (&kr)[kAttnSplitPP / 16][D / 32],
                                           const uint32_t (&vr)[kAttnSplitPP / 16][D / 32],
                                           float (&s_o)[16][QPG][D], float (&s_m)[16][QPG],
                                           float (&s_l)[16][QPG], float (&s_w)[QPG][16],
                                           float (&s_ML)[QPG][2]) {
  constexpr int DPL = D / 16;   // dims per lane
  constexpr int HALF = D / 2;
  constexpr int IT = kAttnSplitPP / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = lane >> 4, li = lane & 15;
  const int row = wave * 4 + rr;    // 0..15
  const int d0 = li * DPL;
  const int ns = c / kAttnSplitPP + 1;
  const size_t head_base = ((size_t)b * a.Hkv + g) * a.M;   // in rows of D
  const size_t pidx = ((size_t)b * a.Hkv + g) * a.NS + s;      // partial slot
  // ---- prologue: q', k', v of the current token for this lane's dims
  const float* qrow = a.qkv + (size_t)b * a.ldqkv;
  float q[QPG][DPL], kf[DPL], vf[DPL];
#pragma unroll
  for (int h = 0; h < QPG; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) q[h][e] = qrow[(g * QPG + h) * D + d0 + e];
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    kf[e] = qrow[(a.Hq + g) * D + d0 + e];
    vf[e] = qrow[(a.Hq + a.Hkv + g) * D + d0 + e];
  }
  float cs_c[DPL], cs_s[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    const float2 t = a.cs[(size_t)b * HALF + ((d0 + e) % HALF)];
    cs_c[e] = t.x;
    cs_s[e] = (d0 < HALF) ? -t.y : t.y;   // lower half: x c - x' s; upper: x c + x' s
  }
  auto norm_rope = [&](float* vals, const uint16_t* gain) {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) ss += vals[e] * vals[e];
    ss = row16_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
#pragma unroll
    for (int e = 0; e < DPL; ++e) vals[e] = (vals[e] * inv) * bf16_to_f32(gain[d0 + e]);
    float other[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) other[e] = row16_swap8(vals[e]);
#pragma unroll
    for (int e = 0; e < DPL; ++e) vals[e] = vals[e] * cs_c[e] + other[e] * cs_s[e];
  };
#pragma unroll
  for (int h = 0; h < QPG; ++h) norm_rope(q[h], a.q_norm);
  norm_rope(kf, a.k_norm);
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    kf[e] = round_bf16(kf[e]);
    vf[e] = round_bf16(vf[e]);
  }
  if (s == ns - 1 && row == 0) {
    uint16_t* kd = a.kc + (head_base + c) * D + d0;
    uint16_t* vd = a.vc + (head_base + c) * D + d0;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      kd[e] = f32_to_bf16(kf[e]);
      vd[e] = f32_to_bf16(vf[e]);
    }
  }

  // ---- online softmax over this split's positions
  float m[QPG], l[QPG], o[QPG][DPL];
#pragma unroll
  for (int h = 0; h < QPG; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
  }
  // the row's IT positions as one block: their scores (log2 units; -inf past the
  // cache position), one running-max update and rescale per head, then the
  // weighted value rows (hardware exp2)
  float sc[QPG][IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int p = s * kAttnSplitPP + wave * (kAttnSplitPP / 4) + it * 4 + rr;
    float kk[DPL];
    if (p == c) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) kk[e] = kf[e];
    } else {
#pragma unroll
      for (int e = 0; e < DPL / 2; ++e) { kk[2 * e] = bf16_lo(kr[it][e]); kk[2 * e + 1] = bf16_hi(kr[it][e]); }
    }
#pragma unroll
    for (int h = 0; h < QPG; ++h) {
      float t = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) t += q[h][e] * kk[e];
      t = row16_sum(t) * a.scale_log2;
      sc[h][it] = p <= c ? t : -INFINITY;
    }
  }
#pragma unroll
  for (int h = 0; h < QPG; ++h) {
    float mb = m[h];
#pragma unroll
    for (int it = 0; it < IT; ++it) mb = fmaxf(mb, sc[h][it]);
    m[h] = mb;   // (-inf: no valid position, the state stays empty)
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int p = s * kAttnSplitPP + wave * (kAttnSplitPP / 4) + it * 4 + rr;
    float vv[DPL];
    if (p == c) {
#pragma unroll
      for (int e = 0; e < DPL; ++e) vv[e] = vf[e];
    } else {
#pragma unroll
      for (int e = 0; e < DPL / 2; ++e) { vv[2 * e] = bf16_lo(vr[it][e]); vv[2 * e + 1] = bf16_hi(vr[it][e]); }
    }
#pragma unroll
    for (int h = 0; h < QPG; ++h) {
      const float pe = sc[h][it] != -INFINITY ? exp2_fast(sc[h][it] - m[h]) : 0.f;
      l[h] += pe;
#pragma unroll
      for (int e = 0; e < DPL; ++e) o[h][e] += pe * vv[e];
    }
  }

  // ---- merge the 16 row states into this split's partial
#pragma unroll
  for (int h = 0; h < QPG; ++h) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) s_o[row][h][d0 + e] = o[h][e];
    if (li == 0) {
      s_m[row][h] = m[h];
      s_l[row][h] = l[h];
    }
  }
  __syncthreads();
  // the log-sum-exp weight of each (row, head) once, by the first wave: lane
  // 16 h + r holds row r of head h (QPG <= 4); rows that saw nothing have m = -inf
  if (wave == 0) {
    const int h = lane >> 4, r = lane & 15;
    const float mr = h < QPG ? s_m[r][h] : -INFINITY;
    float M = mr;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    const float w = mr == -INFINITY ? 0.f : exp2_fast(mr - M);
    float L = h < QPG ? w * s_l[r][h] : 0.f;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) L += __shfl_xor(L, off);
    if (h < QPG) {
      s_w[h][r] = w;
      if (r == 0) { s_ML[h][0] = M; s_ML[h][1] = L; }
    }
  }
  __syncthreads();
  for (int i = tid; i < QPG * D; i += 256) {
    const int h = i / D, d = i - h * D;
    float O = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) O += s_w[h][r] * s_o[r][h][d];
    a.part_o[(pidx * QPG + h) * D + d] = O;
    if (d == 0) a.part_ml[pidx * QPG + h] = make_float2(s_ML[h][0], s_ML[h][1]);
  }
}

// Shared-prefix (cascade) attention: the first a.first_split splits of every row
// whose cache position is past them, when all rows hold the same K/V there (the
// caller's promise; row a.prefix_row is read).  One work-group per (prefix split,
// kv head, kPrefixRows rows) reads the split's K/V once and runs attn_split for each
// such row, the same operations on the same values as k_attn would, so the partials
// -- and the step's results -- are bit for bit those of the plain path; only the
// prefix K/V reads shrink, by up to kPrefixRows.  (A separate launch: folded into
// k_attn's grid, its code cost every plain work-group registers and occupancy.)
constexpr int kPrefixRows = 4;
template <int D, int QPG>
__global__ __launch_bounds__(256) void k_attn_prefix(AttnArgs a) {
  constexpr int DPL = D / 16;
  constexpr int IT = kAttnSplitPP / 16;
  __shared__ float s_o[16][QPG][D];
  __shared__ float s_m[16][QPG];
  __shared__ float s_l[16][QPG];
  __shared__ float s_w[QPG][16], s_ML[QPG][2];
  const int s = blockIdx.x, g = blockIdx.y, b0 = blockIdx.z * kPrefixRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, rr = lane >> 4, d0 = (lane & 15) * DPL;
  const size_t head_base = ((size_t)a.prefix_row * a.Hkv + g) * a.M;
  // every position of a prefix split lies before the cache position of the rows
  // served here (c >= first_split * kAttnSplitPP), as k_attn's masked loads find
  uint32_t kr[IT][DPL / 2], vr[IT][DPL / 2];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int p = s * kAttnSplitPP + wave * (kAttnSplitPP / 4) + it * 4 + rr;
    const uint32_t* ks = reinterpret_cast<const uint32_t*>(a.kc + (head_base + p) * D + d0);
    const uint32_t* vs = reinterpret_cast<const uint32_t*>(a.vc + (head_base + p) * D + d0);
#pragma unroll
    for (int e = 0; e < DPL / 2; ++e) {
      kr[it][e] = ks[e];
      vr[it][e] = vs[e];
    }
  }
  const int b1 = b0 + kPrefixRows < a.B ? b0 + kPrefixRows : a.B;
  for (int b = b0; b < b1; ++b) {
    const int c = a.cpos[b];
    if (c < a.first_split * kAttnSplitPP || c >= a.M) continue;   // (uniform in the group)
    attn_split<D, QPG>(a, b, g, s, c, kr, vr, s_o, s_m, s_l, s_w, s_ML);
    __syncthreads();   // s_o and the weights are rewritten for the next row
  }
}

template <int D, int QPG>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
  constexpr int DPL = D / 16;   // dims per lane
  constexpr int IT = kAttnSplitPP / 16;
  __shared__ float s_o[16][QPG][D];
  __shared__ float s_m[16][QPG];
  __shared__ float s_l[16][QPG];
  __shared__ float s_w[QPG][16], s_ML[QPG][2];

  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = lane >> 4, li = lane & 15;
  const int d0 = li * DPL;
  const int c = a.cpos[b];
  const size_t head_base = ((size_t)b * a.Hkv + g) * a.M;   // in rows of D
  const size_t pidx = ((size_t)b * a.Hkv + g) * a.NS + s;      // partial slot

  if (c < 0 || c >= a.M) {
    if (s == 0) {   // zero attention for this row: partial (m, l, o~) = (0, 1, 0)
      if (tid == 0 && g == 0) raise_status(a.status, 1u);
      for (int i = tid; i < QPG * D; i += 256) a.part_o[pidx * QPG * D + i] = 0.f;
      if (tid < QPG) a.part_ml[pidx * QPG + tid] = make_float2(0.f, 1.f);
    }
    return;
  }
  if (s * kAttnSplitPP > c) return;
  // a split of the shared prefix of a row past it: k_attn_prefix writes its partial
  if (s < a.first_split && c >= a.first_split * kAttnSplitPP) return;

  // ---- cache reads first
  uint32_t kr[IT][DPL / 2], vr[IT][DPL / 2];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int p = s * kAttnSplitPP + wave * (kAttnSplitPP / 4) + it * 4 + rr;
    if (p < c) {
      const uint32_t* ks = reinterpret_cast<const uint32_t*>(a.kc + (head_base + p) * D + d0);
      const uint32_t* vs = reinterpret_cast<const uint32_t*>(a.vc + (head_base + p) * D + d0);
#pragma unroll
      for (int e = 0; e < DPL / 2; ++e) {
        kr[it][e] = ks[e];
        vr[it][e] = vs[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < DPL / 2; ++e) kr[it][e] = vr[it][e] = 0u;
    }
  }
  attn_split<D, QPG>(a, b, g, s, c, kr, vr, s_o, s_m, s_l, s_w, s_ML);
}


// Positions and cache positions of the prompt tokens [t0, t0 + C) in the per-row
// layouts of the decode kernels: pos_c[a][b] = pos[a][t0 + b] (pos is [3][T]) and
// cpos_c[b] = start + t0 + b.  One group of KMR_PREFILL_CHUNK threads, C <= that.
__global__ void k_prefill_rows(const int32_t* pos, int T, int t0, int C, int start, int32_t* pos_c,
                               int32_t* cpos_c) {
  const int b = threadIdx.x;
  if (b >= C) return;
#pragma unroll
  for (int ax = 0; ax < 3; ++ax) pos_c[ax * C + b] = pos[(size_t)ax * T + t0 + b];
  cpos_c[b] = start + t0 + b;
}

// ------------------------------------------------------------------ lm_head + argmax
// logits[b][n] = sum_k W[n][k] h[b][k] with h = RMSNorm(x; final_norm), bf16 W
// widened to fp32 in registers, fp32 accumulation.  Each group leaves the best
// (value, lowest index) per batch row; k_lm_finish reduces those partials in a
// fixed order, writes next_ids, and applies the finished/advance rules.
struct LmArgs {
  const float* x;            // [B][K]
  const uint16_t* gain;      // [K]
  const uint16_t* W;         // [V][K]
  float* logits;             // [B][V] or null
  float2* part;              // [B][nblk] (value, index as float bits)
  int V, K, B, nblk;
  float eps;
};

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

template <int BT, int CPL>
__global__ __launch_bounds__(256) void k_lmhead(LmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* hs = reinterpret_cast<float*>(smem);       // [BT][K]
  __shared__ float red[BT * 4];
  __shared__ float s_bv[4][BT];
  __shared__ int s_bi[4][BT];
  const int K = a.K, B = a.B, CH = K >> 3;   // 8-column chunks
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int RPW = kLmRowsPerWave;

  // h = RMSNorm(x; gain) into LDS once per group; the group then takes row blocks
  // blockIdx.x, blockIdx.x + gridDim.x, ... (one argmax partial per row block)
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    float ss = 0.f;
    if (b < B)
      for (int k = tid * 4; k < K; k += 1024) {
        float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)b * K + k);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    ss = wave_sum(ss);
    if (lane == 0) red[b * 4 + wave] = ss;
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    const float ss = (red[b * 4 + 0] + red[b * 4 + 1]) + (red[b * 4 + 2] + red[b * 4 + 3]);
    const float inv = 1.0f / sqrtf(ss / (float)K + a.eps);
    for (int k = tid; k < K; k += 256)
      hs[b * K + k] = b < B ? (a.x[(size_t)b * K + k] * inv) * bf16_to_f32(a.gain[k]) : 0.f;
  }
  __syncthreads();

  for (int blk = blockIdx.x; blk < a.nblk; blk += gridDim.x) {
    const int n0 = blk * kLmRowsPerBlock + wave * RPW;
    uint4 w[RPW][CPL];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int n = n0 + r, c = lane + 64 * j;
        w[r][j] = (n < a.V && c < CH)
                      ? load_stream16(a.W + (size_t)n * K + 8 * c)
                      : make_uint4(0, 0, 0, 0);
      }
    float acc[RPW][BT];
#pragma unroll
    for (int r = 0; r < RPW; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (c < CH) {
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          const float4 h0 = *reinterpret_cast<const float4*>(hs + b * K + 8 * c);
          const float4 h1 = *reinterpret_cast<const float4*>(hs + b * K + 8 * c + 4);
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            float t = acc[r][b];
            t = __builtin_fmaf(bf16_lo(w[r][j].x), h0.x, t); t = __builtin_fmaf(bf16_hi(w[r][j].x), h0.y, t);
            t = __builtin_fmaf(bf16_lo(w[r][j].y), h0.z, t); t = __builtin_fmaf(bf16_hi(w[r][j].y), h0.w, t);
            t = __builtin_fmaf(bf16_lo(w[r][j].z), h1.x, t); t = __builtin_fmaf(bf16_hi(w[r][j].z), h1.y, t);
            t = __builtin_fmaf(bf16_lo(w[r][j].w), h1.z, t); t = __builtin_fmaf(bf16_hi(w[r][j].w), h1.w, t);
            acc[r][b] = t;
          }
        }
      }
    }
    float bv[BT];
    int bi[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) { bv[b] = -INFINITY; bi[b] = 0x7fffffff; }
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int n = n0 + r;
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const float v = wave_sum(acc[r][b]);
        if (n < a.V && b < B) {
          if (a.logits && lane == 0) a.logits[(size_t)b * a.V + n] = v;
          if (better(v, n, bv[b], bi[b])) { bv[b] = v; bi[b] = n; }
        }
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < BT; ++b) { s_bv[wave][b] = bv[b]; s_bi[wave][b] = bi[b]; }
    }
    __syncthreads();
    if (tid < B) {
      float v = s_bv[0][tid];
      int i = s_bi[0][tid];
      for (int w2 = 1; w2 < 4; ++w2)
        if (better(s_bv[w2][tid], s_bi[w2][tid], v, i)) { v = s_bv[w2][tid]; i = s_bi[w2][tid]; }
      a.part[(size_t)tid * a.nblk + blk] = make_float2(v, __int_as_float(i));
    }
    __syncthreads();   // s_bv / s_bi are rewritten by the next row block
  }
}

// The lm_head of a 9..16-row batch tile on the matrix cores, for K = 32 NK.  Each
// group stages h = RMSNorm(x; gain) of the tile once in LDS as bf16 h_hi = bf16(h)
// and h_lo = bf16(h - h_hi) (rows padded by 16 bytes: the 16 rows of an operand
// read fall in distinct banks); bf16 weights times both parts are exact in fp32,
// so two v_mfma_f32_16x16x32_bf16 per 32 columns give the fp32 product to about
// 2^-16 of |h|.  Each wave takes 16-row vocabulary blocks (block t = rows 16 t..)
// in a grid-stride loop, streaming its lane's 16-byte weight pieces through a
// ring of kLmRing loads over the unrolled K loop; lane (n, gq) receives batch rows
// 4 gq + e of vocabulary row 16 t + n.  The argmax of each batch row is kept per
// lane over all of the wave's blocks and written, with empty entries for its other
// blocks, after the loop (a store in flight would make every later load wait; so
// the logits stores are a separate instantiation, LG, used only when asked for).
constexpr int kLmRing = 16;
template <int NK, bool LG>
__global__ __launch_bounds__(256) void k_lmhead_mfma(LmArgs a) {
  constexpr int K = 32 * NK, KS = K + 8;   // LDS row stride in bf16
  static_assert(NK >= kLmRing, "the ring is filled from the first K columns");
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* hhi = reinterpret_cast<uint16_t*>(smem);   // [16][KS]
  uint16_t* hlo = hhi + 16 * KS;                        // [16][KS]
  __shared__ float s_inv[16];
  const int B = a.B, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, gq = lane >> 4;

  // ---- h of the tile's rows (rows >= B zero), split into two bf16 parts
  for (int b = wave; b < 16; b += 4) {
    float ss = 0.f;
    if (b < B)
      for (int k = lane * 4; k < K; k += 256) {
        const float4 v = *reinterpret_cast<const float4*>(a.x + (size_t)b * K + k);
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
      }
    ss = wave_sum(ss);
    if (lane == 0) s_inv[b] = b < B ? 1.0f / sqrtf(ss / (float)K + a.eps) : 0.f;
  }
  __syncthreads();
  // 8 consecutive columns per thread and step, the loads of 4 steps issued together
  constexpr int STEPS = 16 * K / (8 * 256), SB = 4;
  static_assert(STEPS % SB == 0, "whole batches of steps");
  for (int j0 = 0; j0 < STEPS; j0 += SB) {
  float4 xv[SB][2];
  uint4 gv[SB];
#pragma unroll
  for (int jj = 0; jj < SB; ++jj) {
    const int j = j0 + jj, i = (j * 256 + tid) * 8, b = i / K, k = i - b * K;
    const float* xp = a.x + (size_t)(b < B ? b : 0) * K + k;
    xv[jj][0] = *reinterpret_cast<const float4*>(xp);
    xv[jj][1] = *reinterpret_cast<const float4*>(xp + 4);
    gv[jj] = *reinterpret_cast<const uint4*>(a.gain + k);
  }
#pragma unroll
  for (int jj = 0; jj < SB; ++jj) {
    const int j = j0 + jj, i = (j * 256 + tid) * 8, b = i / K, k = i - b * K;
    const float xs[8] = {xv[jj][0].x, xv[jj][0].y, xv[jj][0].z, xv[jj][0].w,
                         xv[jj][1].x, xv[jj][1].y, xv[jj][1].z, xv[jj][1].w};
    const uint32_t gw[4] = {gv[jj].x, gv[jj].y, gv[jj].z, gv[jj].w};
    uint32_t ph[4], pl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float h0 = (xs[2 * q] * s_inv[b]) * bf16_lo(gw[q]);
      float h1 = (xs[2 * q + 1] * s_inv[b]) * bf16_hi(gw[q]);
      if (b >= B) h0 = h1 = 0.f;
      const uint16_t a0 = f32_to_bf16(h0), a1 = f32_to_bf16(h1);
      ph[q] = (uint32_t)a0 | ((uint32_t)a1 << 16);
      pl[q] = (uint32_t)f32_to_bf16(h0 - bf16_to_f32(a0)) | ((uint32_t)f32_to_bf16(h1 - bf16_to_f32(a1)) << 16);
    }
    *reinterpret_cast<uint4*>(hhi + b * KS + k) = make_uint4(ph[0], ph[1], ph[2], ph[3]);
    *reinterpret_cast<uint4*>(hlo + b * KS + k) = make_uint4(pl[0], pl[1], pl[2], pl[3]);
  }
  }
  __syncthreads();

  const int ntile = (a.V + 15) >> 4;
  float bv[4];
  int bi[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { bv[e] = -INFINITY; bi[e] = 0x7fffffff; }
  const uint16_t* ahi = hhi + n * KS + 8 * gq;
  const uint16_t* alo = hlo + n * KS + 8 * gq;
  for (int t = blockIdx.x * 4 + wave; t < ntile; t += gridDim.x * 4) {
    const int r = 16 * t + n;
    const bool rok = r < a.V;
    const uint16_t* wr = a.W + (size_t)(rok ? r : 0) * K + 8 * gq;
    uint4 ring[kLmRing];
#pragma unroll
    for (int i = 0; i < kLmRing; ++i) ring[i] = load_stream16(wr + 32 * i);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < NK; ++kt) {
      const uint4 w = ring[kt % kLmRing];
      if (kt + kLmRing < NK) ring[kt % kLmRing] = load_stream16(wr + 32 * (kt + kLmRing));
      const uint4 xh = *reinterpret_cast<const uint4*>(ahi + 32 * kt);
      const uint4 xl = *reinterpret_cast<const uint4*>(alo + 32 * kt);
      acc = mfma16x16x32_bf16(xh, w, acc);
      acc = mfma16x16x32_bf16(xl, w, acc);
      // keeps each step's loads in its step: the ring's loads stay kLmRing steps
      // ahead of their use instead of being moved next to it
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = 4 * gq + e;
      if (b < B && rok) {
        if constexpr (LG) a.logits[(size_t)b * a.V + r] = acc[e];
        if (better(acc[e], r, bv[e], bi[e])) { bv[e] = acc[e]; bi[e] = r; }
      }
    }
  }
  // best of each batch row over the 16 lanes of a row group, then the partials:
  // the wave's first block holds its best, its other blocks empty entries
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const float ov = __shfl_xor(bv[e], off);
      const int oi = __shfl_xor(bi[e], off);
      if (better(ov, oi, bv[e], bi[e])) { bv[e] = ov; bi[e] = oi; }
    }
  const int t0 = blockIdx.x * 4 + wave;
  for (int t = t0; t < ntile; t += gridDim.x * 4)
    if (n == 0)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int b = 4 * gq + e;
        if (b < B)
          a.part[(size_t)b * a.nblk + t] = t == t0 ? make_float2(bv[e], __int_as_float(bi[e]))
                                                   : make_float2(-INFINITY, __int_as_float(0x7fffffff));
      }
}

struct LmFinishArgs {
  const float2* part;        // [B][nblk]
  const uint8_t* finished_in;
  uint8_t* finished;         // may be null
  int32_t* next;
  int32_t* cpos;
  int32_t* pos;              // [3][B]
  int B, nblk, M, pad_id, eos_id;
  uint32_t flags;
};

// One group per batch row: argmax over the lm_head partials (ties to the lowest
// index), then the greedy-step bookkeeping of that row.
__global__ __launch_bounds__(256) void k_lm_finish(LmFinishArgs a) {
  __shared__ float t_v[256];
  __shared__ int t_i[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  float v = -INFINITY;
  int i = 0x7fffffff;
  for (int t = tid; t < a.nblk; t += 256) {
    const float2 pv = a.part[(size_t)b * a.nblk + t];
    if (better(pv.x, __float_as_int(pv.y), v, i)) { v = pv.x; i = __float_as_int(pv.y); }
  }
  t_v[tid] = v;
  t_i[tid] = i;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w && better(t_v[tid + w], t_i[tid + w], t_v[tid], t_i[tid])) {
      t_v[tid] = t_v[tid + w];
      t_i[tid] = t_i[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const int best = t_i[0];
    const int fin = a.finished_in ? a.finished_in[b] : 0;
    a.next[b] = fin ? a.pad_id : best;
    if ((a.flags & 1u) && !fin) {
      if (a.eos_id >= 0 && best == a.eos_id) {
        if (a.finished) a.finished[b] = 1;
      } else if (a.cpos[b] + 1 >= a.M) {
        if (a.finished) a.finished[b] = 1;
      } else {
        a.cpos[b] += 1;
        a.pos[0 * a.B + b] += 1;
        a.pos[1 * a.B + b] += 1;
        a.pos[2 * a.B + b] += 1;
      }
    }
  }
}

}  // namespace kmr
