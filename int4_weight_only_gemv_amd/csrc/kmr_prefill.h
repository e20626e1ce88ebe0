// Prefill kernels: the decoder linears of a prompt chunk as int4 x fp16 matrix-core
// GEMMs that read each weight once per 128 tokens, and causal attention over the
// static cache on the matrix cores with each K/V block shared by the queries of a
// tile (kaminari page, section 04 "Request lifecycle", stage 2: one forward over the
// prompt fills the cache; the first token is the argmax at the last prompt token).
#pragma once
#include "kmr_kernels.h"

namespace kmr {

// 16-byte load and store as one vector access (a uint4 struct copy between address
// spaces becomes a memcpy, which keeps register arrays out of registers).
__device__ __forceinline__ u32x4_t load_vec16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void store_vec16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ uint4 as_uint4(u32x4_t v) { return make_uint4(v.x, v.y, v.z, v.w); }

// ------------------------------------------------------------------ staging
// A chunk's GEMM input, token-major: row t of x (plain, or its RMSNorm with `gain`)
// as fp16 magic-bias pairs (h[8w+i], h[8w+i+4]) with odd columns divided by 16, one
// 16-byte word per 8 columns, xs[t][K/8] (so the 128 columns of a quantization block
// are 256 contiguous bytes per token), and the per-token sums of the staged values
// over each 128-column block, c2[t][K/128] (the zero-point term's input).
// With kp set, x first takes the two split-K partials of the projection that wrote it,
// x += kp[0][t] + kp[1][t] (written back), the same sum k_gemv_kreduce forms.
// One work-group of 256 threads per token; thread i takes the words i, i + 256, ...
struct PfStageArgs {
  float* x;               // [M][ldx]
  const uint16_t* gain;   // [K] (PRO_RMSNORM)
  const float* kp;        // null, or split-K partials [2][M][K] to add to x first
  uint4* xs;              // [M][K/8]
  float* c2;              // [M][K/128]
  uint32_t* status;       // KMR_STATUS_RANGE when a staged value leaves the fp16 range
  int M, K, ldx;
  float eps;
};

constexpr int kPfStageWords = 4;   // words per thread: K <= 8192

template <int PRO>
__global__ __launch_bounds__(256) void k_pf_stage(PfStageArgs a) {
  static_assert(PRO == PRO_PLAIN || PRO == PRO_RMSNORM, "plain or RMSNorm input");
  __shared__ float s_ss[4];
  const int t = blockIdx.x, K = a.K, NW = K >> 3, tid = threadIdx.x, lane = tid & 63;
  float* xr = a.x + (size_t)t * a.ldx;
  float v[kPfStageWords][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kPfStageWords; ++i) {
    const int w = tid + 256 * i;
    if (w < NW) {
      const float4 lo = *reinterpret_cast<const float4*>(xr + 8 * w);
      const float4 hi = *reinterpret_cast<const float4*>(xr + 8 * w + 4);
      float f[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      if (a.kp) {
        const float* p0 = a.kp + (size_t)t * K + 8 * w;
        const float* p1 = a.kp + ((size_t)a.M + t) * K + 8 * w;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] += p0[e] + p1[e];
        *reinterpret_cast<float4*>(xr + 8 * w) = make_float4(f[0], f[1], f[2], f[3]);
        *reinterpret_cast<float4*>(xr + 8 * w + 4) = make_float4(f[4], f[5], f[6], f[7]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[i][e] = f[e];
        ss += f[e] * f[e];
      }
    }
  }
  float iv = 1.f;
  if (PRO == PRO_RMSNORM) {
    ss = wave_sum(ss);
    if (lane == 0) s_ss[tid >> 6] = ss;
    __syncthreads();
    iv = 1.0f / sqrtf(((s_ss[0] + s_ss[1]) + (s_ss[2] + s_ss[3])) / (float)K + a.eps);
  }
#pragma unroll
  for (int i = 0; i < kPfStageWords; ++i) {
    const int w = tid + 256 * i;
    if (i * 256 >= NW) break;   // (uniform: whole rounds of 256 words)
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = w < NW ? v[i][e] : 0.f;
    if (PRO == PRO_RMSNORM && w < NW) {
      const uint4 gw = *reinterpret_cast<const uint4*>(a.gain + 8 * w);
      const uint32_t g[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = (f[2 * e] * iv) * bf16_lo(g[e]);
        f[2 * e + 1] = (f[2 * e + 1] * iv) * bf16_hi(g[e]);
      }
    }
    const _Float16 h0 = (_Float16)f[0], h4 = (_Float16)f[4], h2 = (_Float16)f[2], h6 = (_Float16)f[6];
    const _Float16 h1 = (_Float16)(f[1] * 0.0625f), h5 = (_Float16)(f[5] * 0.0625f);
    const _Float16 h3 = (_Float16)(f[3] * 0.0625f), h7 = (_Float16)(f[7] * 0.0625f);
    const float ev = ((float)h0 + (float)h4) + ((float)h2 + (float)h6);
    const float od = ((float)h1 + (float)h5) + ((float)h3 + (float)h7);
    const float usum = ev + 16.0f * od;
    if (w < NW) {
      store_vec16(a.xs + (size_t)t * NW + w,
                  u32x4_t{__builtin_bit_cast(uint32_t, half2_t{h0, h4}), __builtin_bit_cast(uint32_t, half2_t{h1, h5}),
                          __builtin_bit_cast(uint32_t, half2_t{h2, h6}), __builtin_bit_cast(uint32_t, half2_t{h3, h7})});
      if (!(fabsf(ev + od) + fabsf(usum) <= 3.0e38f)) raise_status(a.status, kStatusRange);
    }
    // a 128-column block is 16 consecutive words: one 16-lane row
    const float bs = row16_sum(usum);
    if ((lane & 15) == 0 && w < NW) a.c2[(size_t)t * (K >> 7) + (w >> 4)] = bs;
  }
}

// ------------------------------------------------------------------ GEMM
// y[t][r] (EPI) = sum_k x[t][k] w[r][k] for the M tokens of a chunk, w = s (q - 8) + z
// per group of G columns (G a multiple of 128).
//
// Work-group tile: 128 tokens x 64 weight rows (EPI_SILU: 32 gate rows and their 32
// up rows), four waves in a 2 x 2 grid, each 64 tokens x two 16-row blocks (for
// EPI_SILU the gate block and the up block of the same 16 outputs).  The K loop runs
// over 128-column blocks: the tile's staged input block (128 tokens x 256 bytes)
// goes to LDS, double-buffered, the next block's loads in flight during this one's
// products; each lane dequantizes the codes of its weight row over chunk 4 kb + gq to
// exact operands (even words q - 8, odd words 16 (q - 8), the odd input columns
// being staged / 16), and 4 x 4 x 2 v_mfma_f32_16x16x32_f16 per block give the
// block's dots d; acc += s d per block.  The zero-point term sum_kb z[r][kb] c2[t][kb]
// is one more product over the K/128 blocks, on the fp32 matrix path
// (v_mfma_f32_16x16x4_f32, four blocks per instruction), after the loop.
// Each weight is thus read once per 128 tokens; a token's input once per 64 rows.
// The loads run two blocks ahead of the products (two register sets), so a block's
// global loads have the products of the block before to complete.  An EPI_ADD
// product may split K in two (gridDim.z = 2), for outputs too few to give every
// compute unit a tile: its partials go to kpart, and the next staging of y adds them.
constexpr int kPfTileM = 128;
constexpr int kPfTileN = 64;

struct PfGemmArgs {
  const uint4* xs;         // staged input [M][K/8] (k_pf_stage)
  const float* c2;         // [M][K/128]
  const uint8_t* packed;   // [rows][K/2]
  const uint32_t* sz;      // [rows][K/G] (scale | zero << 16, bf16)
  float* y;                // [M][ldy]
  float* kpart;            // split K (gridDim.z = 2, EPI_ADD): partials [2][M][N], for k_pf_stage to add
  int M, N, K, G, ldy;     // N outputs per token (EPI_SILU: weight rows are 2N)
};

__host__ __device__ inline size_t pf_gemm_lds() { return (size_t)2 * kPfTileM * 16 * 16; }


__device__ __forceinline__ f32x4_t mfma16x16x4_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int EPI>
__global__ __launch_bounds__(256, 2) void k_pf_gemm(PfGemmArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  // [2][128 tokens][16 slots]: slot j of token t at t * 16 + (j ^ (t & 15))
  uint4* sA = reinterpret_cast<uint4*>(smem);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, gq = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;
  const int K = a.K, CH = K >> 5, NB = K >> 7, NG = K / a.G;
  const int m0 = blockIdx.y * kPfTileM;
  // this wave's weight rows; rows past N (and tokens past M) read row 0 (token M - 1)
  // and are never stored
  int wrow[2];
  bool wok[2];
  if (EPI == EPI_SILU) {
    const int o = blockIdx.x * (kPfTileN / 2) + 16 * wn + n;
    wok[0] = wok[1] = o < a.N;
    wrow[0] = wok[0] ? o : 0;
    wrow[1] = wok[0] ? a.N + o : 0;
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = blockIdx.x * kPfTileN + 32 * wn + 16 * j + n;
      wok[j] = r < a.N;
      wrow[j] = wok[j] ? r : 0;
    }
  }
  // split K: blockIdx.z takes the z-th of gridDim.z equal runs of 128-column blocks
  const int nbz = NB / (int)gridDim.z, kb0 = (int)blockIdx.z * nbz;
  // staging: thread tid moves slot lj of tokens lt + 16 i (i < 8) of the tile
  const int lj = tid & 15, lt = tid >> 4;
  const uint4* asrc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = m0 + lt + 16 * i;
    asrc[i] = a.xs + (size_t)(t < a.M ? t : a.M - 1) * CH * 4 + lj;
  }
  const uint8_t* bsrc[2];
  const uint32_t* ssrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bsrc[j] = a.packed + (size_t)wrow[j] * (K / 2) + 16 * gq;
    ssrc[j] = a.sz + (size_t)wrow[j] * NG;
  }
#define KMR_PF_LOAD(KB, RA, CW, SW)                                                    \
  {                                                                                   \
    const int kbl = (KB);                                                             \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) RA[i] = load_vec16(asrc[i] + 16 * kbl); \
    _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                   \
      CW[j] = load_vec16(bsrc[j] + 64 * kbl);                                         \
      SW[j] = ssrc[j][(kbl << 7) / a.G];                                              \
    }                                                                                 \
  }
#define KMR_PF_STORE(BUF, RA)                                                          \
  {                                                                                   \
    uint4* dst = sA + (BUF) * (kPfTileM * 16);                                        \
    _Pragma("unroll") for (int i = 0; i < 8; ++i) store_vec16(dst + (lt + 16 * i) * 16 + (lj ^ lt), RA[i]); \
  }
  f32x4_t acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[mb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // block kb: products from LDS buffer BUF and the codes in (CW, SW); the loads of
  // block kb + 2 go to (RA, CW, SW) once the codes are dequantized, and block kb + 1
  // (in RN since the block before) is written to the other buffer at the end.  The
  // loads are unconditional (the last block again at the end): loads under a branch
  // would make the compiler wait for every load in flight before the next store.
  // (Written out twice for the two register sets: register arrays selected by an
  // index, or passed by reference into a shared body, ended up in scratch memory.)
#define KMR_PF_BLOCK(BUF, RA, CW, SW, RN)                                                             \
  {                                                                                                  \
    uint32_t p[2][16];                                                                               \
    _Pragma("unroll") for (int j = 0; j < 2; ++j) {                                                  \
      dequant16(as_uint4(CW[j]), p[j]);                                                              \
      _Pragma("unroll") for (int i = 0; i < 16; ++i) {                                               \
        const half2_t hv = __builtin_bit_cast(half2_t, p[j][i]);                                     \
        const _Float16 off = (i & 1) ? (_Float16)1152.0f : (_Float16)1032.0f;                        \
        p[j][i] = __builtin_bit_cast(uint32_t, half2_t{hv[0] - off, hv[1] - off});                   \
      }                                                                                              \
    }                                                                                                \
    const float sc0 = bf16_lo(SW[0]), sc1 = bf16_lo(SW[1]);                                          \
    KMR_PF_LOAD(kb + 2 < kb0 + nbz ? kb + 2 : kb0 + nbz - 1, RA, CW, SW)                             \
    __builtin_amdgcn_sched_barrier(0); /* (the loads stay ahead of the products) */               \
    const uint4* At = sA + (BUF) * (kPfTileM * 16) + (64 * wm) * 16;                                 \
    f32x4_t d[4][2];                                                                                 \
    _Pragma("unroll") for (int mb = 0; mb < 4; ++mb)                                                 \
      _Pragma("unroll") for (int j = 0; j < 2; ++j) d[mb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};          \
    _Pragma("unroll") for (int kt = 0; kt < 4; ++kt)                                                 \
      _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) {                                             \
        const uint4 xv = At[(16 * mb + n) * 16 + ((4 * gq + kt) ^ n)];                               \
        _Pragma("unroll") for (int j = 0; j < 2; ++j) d[mb][j] =                                     \
            mfma16x16x32(xv, make_uint4(p[j][4 * kt], p[j][4 * kt + 1], p[j][4 * kt + 2], p[j][4 * kt + 3]), \
                         d[mb][j]);                                                                  \
      }                                                                                              \
    _Pragma("unroll") for (int mb = 0; mb < 4; ++mb)                                                 \
      _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                                \
        acc[mb][0][e] = __builtin_fmaf(sc0, d[mb][0][e], acc[mb][0][e]);                             \
        acc[mb][1][e] = __builtin_fmaf(sc1, d[mb][1][e], acc[mb][1][e]);                             \
      }                                                                                              \
    KMR_PF_STORE((BUF) ^ 1, RN)                                                                      \
    __syncthreads();                                                                                 \
  }
  u32x4_t ra0[8], ra1[8], cw0[2], cw1[2];
  uint32_t sw0[2], sw1[2];
  KMR_PF_LOAD(kb0, ra0, cw0, sw0)
  KMR_PF_LOAD(kb0 + 1, ra1, cw1, sw1)
  KMR_PF_STORE(0, ra0)
  __syncthreads();
  // (nbz is a multiple of 4: the blocks go in pairs)
  for (int kb = kb0; kb < kb0 + nbz; ++kb) {
    KMR_PF_BLOCK(0, ra0, cw0, sw0, ra1)
    ++kb;
    KMR_PF_BLOCK(1, ra1, cw1, sw1, ra0)
  }
#undef KMR_PF_BLOCK
#undef KMR_PF_STORE
#undef KMR_PF_LOAD
  // zero points: acc[t][r] += sum_kb c2[t][kb] z[r][kb], four blocks per product
  // (lane (n, gq) supplies c2 of token n and z of weight row n at block 4 s + gq)
  for (int s = kb0; s < kb0 + nbz; s += 4) {
    float zb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) zb[j] = bf16_hi(ssrc[j][((s + gq) << 7) / a.G]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int t = m0 + 64 * wm + 16 * mb + n;
      const float za = a.c2[(size_t)(t < a.M ? t : a.M - 1) * NB + s + gq];
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[mb][j] = mfma16x16x4_f32(za, zb[j], acc[mb][j]);
    }
  }
  // epilogue: lane (n, gq) holds tokens 16 mb + 4 gq + e of its wave for weight row n
  const bool split = gridDim.z > 1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = m0 + 64 * wm + 16 * mb + 4 * gq + e;
      if (t >= a.M) continue;
      float* yr = a.y + (size_t)t * a.ldy;
      if (EPI == EPI_SILU) {
        if (wok[0]) {
          const float g = acc[mb][0][e], u = acc[mb][1][e];
          yr[wrow[0]] = g / (1.0f + expf(-g)) * u;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (wok[j]) {
            if (EPI == EPI_ADD && split) a.kpart[((size_t)blockIdx.z * a.M + t) * a.N + wrow[j]] = acc[mb][j][e];
            else if (EPI == EPI_STORE) yr[wrow[j]] = acc[mb][j][e];
            else yr[wrow[j]] += acc[mb][j][e];
          }
      }
    }
}

// ------------------------------------------------------------------ q/k/v of a chunk
// Per token and head (one wave; lane i < D/2 holds dims i and i + D/2): q heads and
// k heads RMSNorm over head_dim with their gains, then M-RoPE from the chunk's
// cos/sin table (rotate-half pairs (i, i + D/2)); q is written back in place (fp32),
// k and v (bf16, their storage precision) go to the token's cache slot.
struct PfQkArgs {
  float* qkv;              // [M][ldqkv]: Hq q heads, Hkv k heads, Hkv v heads of D
  const uint16_t* q_norm;  // [D]
  const uint16_t* k_norm;  // [D]
  const float2* cs;        // [M][D/2]
  uint16_t* kc;            // layer slice [cache rows][Hkv][max_len][D]
  uint16_t* vc;
  const int32_t* cpos;     // [M]
  int M, ldqkv, Hq, Hkv, D, max_len, crow;
  float eps;
};

__global__ __launch_bounds__(256) void k_pf_qk(PfQkArgs a) {
  const int lane = threadIdx.x & 63, h = blockIdx.x * 4 + (threadIdx.x >> 6), t = blockIdx.y;
  if (h >= a.Hq + 2 * a.Hkv) return;
  const int half = a.D >> 1;
  const bool on = lane < half;
  float* row = a.qkv + (size_t)t * a.ldqkv + (size_t)h * a.D;
  float lo = on ? row[lane] : 0.f, hi = on ? row[lane + half] : 0.f;
  const int c = a.cpos[t];
  if (h >= a.Hq + a.Hkv) {   // v
    const int g = h - a.Hq - a.Hkv;
    uint16_t* vd = a.vc + (((size_t)a.crow * a.Hkv + g) * a.max_len + c) * a.D;
    if (on) {
      vd[lane] = f32_to_bf16(lo);
      vd[lane + half] = f32_to_bf16(hi);
    }
    return;
  }
  const bool isq = h < a.Hq;
  const uint16_t* gain = isq ? a.q_norm : a.k_norm;
  const float inv = 1.0f / sqrtf(wave_sum(lo * lo + hi * hi) / (float)a.D + a.eps);
  if (!on) return;
  lo = (lo * inv) * bf16_to_f32(gain[lane]);
  hi = (hi * inv) * bf16_to_f32(gain[lane + half]);
  const float2 r = a.cs[(size_t)t * half + lane];
  const float nlo = lo * r.x - hi * r.y, nhi = hi * r.x + lo * r.y;
  if (isq) {
    row[lane] = nlo;
    row[lane + half] = nhi;
  } else {
    uint16_t* kd = a.kc + (((size_t)a.crow * a.Hkv + (h - a.Hq)) * a.max_len + c) * a.D;
    kd[lane] = f32_to_bf16(nlo);
    kd[lane + half] = f32_to_bf16(nhi);
  }
}

// ------------------------------------------------------------------ attention
// Causal attention of a chunk's tokens (cache positions consecutive, cpos[t]) over
// slots 0 .. cpos[t] of cache row crow, after k_pf_qk wrote the chunk's slots.
// Work-group: kv head g and 16 tokens; NGRP groups of QPG waves, wave = one q head of
// the GQA group x the 16 tokens.  Group j takes the 32-slot K/V blocks j, j + NGRP,
// ..., staging each in its own LDS buffers once for its QPG waves (double-buffered;
// V transposed), and the groups' softmax states merge in LDS at the end.  Per block,
// S^T = K Q^T on the matrix cores leaves lane (n, gq) the scores of token n at slots
// 16 pb + 4 gq + e, so each lane's running max, sum and output column belong to one
// token; the online softmax rescales by 2^(m - m'), and O^T += V^T P^T takes the
// lane's own probabilities as its operand (the product's k order is the slots the
// lane holds).  Operands are bf16 (the cache's precision for K and V); q and the
// probabilities enter as a bf16 high part plus a bf16 low part, two products each,
// so that their rounding stays near fp32.  Output o[t][h D + d] fp32, divided by the
// softmax sum.
constexpr int kPfKvBlock = 32;
constexpr int kPfAttnTokens = 16;

struct PfAttnArgs {
  const float* q;          // [M][ldq], q head h at h * D (after k_pf_qk)
  const uint16_t* kc;      // layer slice
  const uint16_t* vc;
  const int32_t* cpos;     // [M], consecutive
  float* o;                // [M][ldo]
  int M, ldq, ldo, Hkv, max_len, crow;
  float scale_log2;        // log2(e) / sqrt(D)
};

// Groups per work-group (each QPG waves) and the LDS the kernel takes.
__host__ __device__ constexpr int pf_attn_groups(int QPG) { return QPG == 4 ? 2 : 4; }
__host__ __device__ constexpr int pf_attn_vs() { return kPfKvBlock + 4; }   // V^T row stride (bf16)
__host__ __device__ constexpr size_t pf_attn_group_lds(int D) {
  return (size_t)2 * kPfKvBlock * D * 2 + (size_t)2 * D * pf_attn_vs() * 2;
}
// (the K/V buffers of every group, or the merge area [groups][QPG][D / 4 + 2][64]
// floats that reuses them, whichever is larger)
__host__ __device__ constexpr size_t pf_attn_lds(int D, int QPG) {
  return pf_attn_groups(QPG) * pf_attn_group_lds(D) > (size_t)pf_attn_groups(QPG) * QPG * (D / 4 + 2) * 64 * 4
             ? pf_attn_groups(QPG) * pf_attn_group_lds(D)
             : (size_t)pf_attn_groups(QPG) * QPG * (D / 4 + 2) * 64 * 4;
}

template <int D, int QPG>
__global__ __launch_bounds__(64 * QPG * pf_attn_groups(QPG)) void k_pf_attn(PfAttnArgs a) {
  constexpr int NGRP = pf_attn_groups(QPG);
  constexpr int GT = 64 * QPG;            // threads per group
  constexpr int SL = D / 8;               // 16-byte slots per K row
  constexpr int KS = D / 32;              // k steps of S^T
  constexpr int DB = D / 16;              // 16-dim blocks of O^T
  constexpr int VS = pf_attn_vs();        // 8-byte reads of 16 V^T rows hit distinct banks
  constexpr int KN = kPfKvBlock * SL;     // 16-byte K words per block
  constexpr int VN = (kPfKvBlock / 2) * SL;   // V items per block (two slots x 8 dims)
  constexpr int KI = (KN + GT - 1) / GT, VI = (VN + GT - 1) / GT;
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n = lane & 15, gq = lane >> 4;
  const int grp = wave / QPG, gw = wave % QPG, gt = tid - grp * GT;
  uint4* sK = reinterpret_cast<uint4*>(smem + grp * pf_attn_group_lds(D));        // [2][KN]
  uint16_t* sV = reinterpret_cast<uint16_t*>(smem + grp * pf_attn_group_lds(D) + (size_t)2 * KN * 16);   // [2][D][VS]
  const int g = blockIdx.y, hq = g * QPG + gw;
  const int t0 = blockIdx.x * kPfAttnTokens, tq = t0 + n;
  const bool qok = tq < a.M;
  const int cq = a.cpos[qok ? tq : a.M - 1];
  const int cmax = a.cpos[(t0 + kPfAttnTokens < a.M ? t0 + kPfAttnTokens : a.M) - 1];
  const int nblk = cmax / kPfKvBlock + 1;
  const int iters = (nblk + NGRP - 1) / NGRP;   // the same for every group (uniform barriers)
  const size_t head = ((size_t)a.crow * a.Hkv + g) * a.max_len;   // cache row of slot 0 of this kv head

  // q of token tq, head hq: dims 32 ks + 8 gq + i as bf16 high and low parts
  uint4 qh[KS], ql[KS];
  {
    const float* qr = a.q + (size_t)(qok ? tq : 0) * a.ldq + (size_t)hq * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float4 f0 = *reinterpret_cast<const float4*>(qr + 32 * ks + 8 * gq);
      const float4 f1 = *reinterpret_cast<const float4*>(qr + 32 * ks + 8 * gq + 4);
      const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split_bf16x2(f[2 * i], f[2 * i + 1], wh[i], wl[i]);
      qh[ks] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
      ql[ks] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    }
  }

  // staging of block kb by the group: K rows as 16-byte slots (slot c of slot row p at
  // p * SL + (c ^ (p % SL))); V transposed, two slots per 32-bit word (item: slot pair
  // pp, dims 8 c ..; consecutive threads take consecutive pairs, so their LDS words are
  // adjacent).  A slot past cmax is loaded from slot cmax instead: a slot past the
  // tile's last position may hold anything (a NaN there would reach the sums as
  // 0 * NaN), while slot cmax holds finite data that every token's mask then gives
  // weight 0.  Every load is issued unconditionally (a load under a branch makes the
  // compiler wait for every load in flight before the next LDS store).
  auto load_kv = [&](int kb, u32x4_t (&kr)[KI], u32x4_t (&vr)[VI][2]) {
    const int p0 = kb * kPfKvBlock;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int it = gt + GT * i, p = it / SL, c = it % SL, q = p0 + p <= cmax ? p0 + p : cmax;
      kr[i] = load_vec16(a.kc + (head + q) * D + 8 * (it < KN ? c : 0));
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int it = gt + GT * i, pp = it % (kPfKvBlock / 2), c = it / (kPfKvBlock / 2);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = p0 + 2 * pp + u, q = p <= cmax ? p : cmax;
        vr[i][u] = load_vec16(a.vc + (head + q) * D + 8 * (it < VN ? c : 0));
      }
    }
  };
  auto store_kv = [&](int buf, const u32x4_t (&kr)[KI], const u32x4_t (&vr)[VI][2]) {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int it = gt + GT * i, p = it / SL, c = it % SL;
      if (it < KN) store_vec16(sK + buf * KN + p * SL + (c ^ (p % SL)), kr[i]);
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int it = gt + GT * i, pp = it % (kPfKvBlock / 2), c = it / (kPfKvBlock / 2);
      if (it < VN) {
        uint16_t* vb = sV + buf * (D * VS);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x0 = vr[i][0][w], x1 = vr[i][1][w];
          *reinterpret_cast<uint32_t*>(vb + (8 * c + 2 * w) * VS + 2 * pp) = (x0 & 0xffffu) | (x1 << 16);
          *reinterpret_cast<uint32_t*>(vb + (8 * c + 2 * w + 1) * VS + 2 * pp) = (x0 >> 16) | (x1 & 0xffff0000u);
        }
      }
    }
  };

  float m = -INFINITY, l = 0.f;
  f32x4_t ot[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) ot[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the group's blocks kb = grp + NGRP it, two in flight ahead of the products: block it
  // is in LDS buffer it & 1, block it + 1 in the other register set since the block
  // before, block it + 2's loads are issued into this set at the start of block it
  u32x4_t kra[KI], vra[VI][2], krb[KI], vrb[VI][2];
  load_kv(grp, kra, vra);
  load_kv(grp + NGRP, krb, vrb);
  store_kv(0, kra, vra);
  __syncthreads();
  auto block = [&](int it, int buf, u32x4_t (&kc)[KI], u32x4_t (&vc)[VI][2], const u32x4_t (&kn)[KI],
                   const u32x4_t (&vn)[VI][2]) {
    const int kb = grp + NGRP * it;
    const bool live = kb < nblk;
    load_kv(kb + 2 * NGRP, kc, vc);
    if (live) {
      // S^T = K Q^T: lane (n, gq) gets slots 16 pb + 4 gq + e of token n
      f32x4_t st[2];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb) {
        st[pb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int p = 16 * pb + n;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const uint4 kf = as_uint4(load_vec16(sK + buf * KN + p * SL + ((4 * ks + gq) ^ (p % SL))));
          st[pb] = mfma16x16x32_bf16(kf, qh[ks], st[pb]);
          st[pb] = mfma16x16x32_bf16(kf, ql[ks], st[pb]);
        }
      }
      const int p0 = kb * kPfKvBlock;
      float s[2][4], bm = -INFINITY;
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = p0 + 16 * pb + 4 * gq + e;
          s[pb][e] = p <= cq ? st[pb][e] * a.scale_log2 : -INFINITY;
          bm = fmaxf(bm, s[pb][e]);
        }
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      // a token's first block may hold none of its slots (the block past cq, for a
      // token before the group's slots): m stays -inf and nothing is added
      const float mn = fmaxf(m, bm);
      const float al = mn == -INFINITY ? 1.f : exp2_fast(m - mn);
      m = mn;
      l *= al;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) ot[db][e] *= al;
      // (with mn = -inf every score here is -inf too: subtracting 0 keeps exp2(-inf) = 0)
      const float mref = mn == -INFINITY ? 0.f : mn;
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int pb = 0; pb < 2; ++pb)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float e0 = exp2_fast(s[pb][2 * i] - mref), e1 = exp2_fast(s[pb][2 * i + 1] - mref);
          l += e0 + e1;
          split_bf16x2(e0, e1, ph[2 * pb + i], pl[2 * pb + i]);
        }
      const uint4 PH = make_uint4(ph[0], ph[1], ph[2], ph[3]), PL = make_uint4(pl[0], pl[1], pl[2], pl[3]);
      // O^T += V^T P^T: lane (n, gq) supplies V^T row 16 db + n at slots 4 gq .. + 3, 16 + 4 gq .. + 3
      const uint16_t* vb = sV + buf * (D * VS);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = vb + (16 * db + n) * VS;
        const uint2 w0 = *reinterpret_cast<const uint2*>(vrow + 4 * gq);
        const uint2 w1 = *reinterpret_cast<const uint2*>(vrow + 16 + 4 * gq);
        const uint4 vf = make_uint4(w0.x, w0.y, w1.x, w1.y);
        ot[db] = mfma16x16x32_bf16(vf, PH, ot[db]);
        ot[db] = mfma16x16x32_bf16(vf, PL, ot[db]);
      }
    }
    store_kv(buf ^ 1, kn, vn);   // (after the group's last block: a buffer no one reads again)
    __syncthreads();
  };
  for (int it = 0; it < iters; it += 2) {
    block(it, 0, kra, vra, krb, vrb);
    if (it + 1 < iters) block(it + 1, 1, krb, vrb, kra, vra);   // (iters is the same for every group)
  }
  // merge the groups' states: groups 1.. write (m, l, O^T) per lane, group 0 combines
  // (a group that saw no slot of a token has m = -inf and weight 0)
  float* sm = reinterpret_cast<float*>(smem);   // [NGRP][QPG][DB * 4 + 2][64]
  constexpr int F = DB * 4 + 2;
  if (grp > 0) {
    float* d = sm + ((size_t)(grp * QPG + gw) * F) * 64 + lane;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) d[(4 * db + e) * 64] = ot[db][e];
    d[(F - 2) * 64] = m;
    d[(F - 1) * 64] = l;
  }
  __syncthreads();
  if (grp == 0) {
    float mg[NGRP], wg[NGRP];
    mg[0] = m;
#pragma unroll
    for (int j = 1; j < NGRP; ++j) mg[j] = sm[((size_t)(j * QPG + gw) * F + F - 2) * 64 + lane];
    float M = mg[0];
#pragma unroll
    for (int j = 1; j < NGRP; ++j) M = fmaxf(M, mg[j]);
#pragma unroll
    for (int j = 0; j < NGRP; ++j) wg[j] = mg[j] == -INFINITY ? 0.f : exp2_fast(mg[j] - M);
    float L = wg[0] * l;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int e = 0; e < 4; ++e) ot[db][e] *= wg[0];
#pragma unroll
    for (int j = 1; j < NGRP; ++j) {
      const float* src = sm + ((size_t)(j * QPG + gw) * F) * 64 + lane;
      L += wg[j] * src[(F - 1) * 64];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 4; ++e) ot[db][e] += wg[j] * src[(4 * db + e) * 64];
    }
    L += __shfl_xor(L, 16);
    L += __shfl_xor(L, 32);
    if (qok) {
      const float il = 1.0f / L;
      float* orow = a.o + (size_t)tq * a.ldo + (size_t)hq * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float4*>(orow + 16 * db + 4 * gq) =
            make_float4(ot[db][0] * il, ot[db][1] * il, ot[db][2] * il, ot[db][3] * il);
    }
  }
}

}  // namespace kmr
