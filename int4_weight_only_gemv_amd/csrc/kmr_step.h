// Persistent decode-step kernel: the whole greedy step (embedding, every layer,
// final norm, lm_head, argmax, advance) in one cooperative launch.
//
// Why: the step is a chain of ~6 dependent phases per layer (fused QKV,
// attention splits, split merge, O projection, gate-up, down), each moving only
// a few MB.  A kernel boundary costs about 1.5 us on this GPU and a fenced grid
// barrier several us, while a one-way signal between two work-groups through
// device-scope (sc1) stores and loads costs about 0.4 us.  So every phase
// publishes its outputs as tagged 64-bit words (tag in the high half, fp32 value
// in the low half) with device-scope stores, and each consumer polls the words it
// needs until all carry the tag of the phase that produced them: one hop per
// dependency, no barrier, no cache flush.
//
// Latency is the budget, so a phase does as little as possible after its input
// arrives: weight rows (and the norm gains) are loaded and dequantized to fp16
// pairs while the input is still being polled; after one work-group-level gather
// into LDS every wave works alone (its lanes read their own columns, the RMSNorm
// sum is a wave reduction, the dot products use the pre-dequantized weights).
//
// Tags: (step << 9) | phase, where step counts decode steps on this workspace
// and phase numbers the published vectors of a step, so a stale word from any
// earlier phase or step never matches.  Buffers are reused every layer without
// double buffering: each phase's output feeds every work-group of the next
// phase (directly or through the split merge), so no producer can overwrite a
// buffer before all consumers of its previous contents have read them.
//
// All waits are bounded: a wait that exceeds kSpinLimit polls raises
// KMR_STATUS_TIMEOUT and the work-group returns, so the grid always drains.
#pragma once
#include "kmr_kernels.h"

namespace kmr {

#ifndef KMR_POLL_SLEEP
#define KMR_POLL_SLEEP 1   // s_sleep units (64 clocks) between polls of a tagged buffer
#endif
constexpr int kStepThreads = 512;
constexpr int kStepWaves = kStepThreads / 64;
constexpr int kMaxStepLayers = 32;
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr uint32_t kStatusTimeout = 4u;
constexpr int kMergeChunk = 16;   // attention splits merged per gather

#ifdef KMR_TRACE
// Diagnostic builds only: per-group timestamps of phase boundaries.
// (a.trace is a kernel argument: recording a mark waits on nothing but the clock)
#define KMR_TRACE_MARK(ev)                                                              \
  do {                                                                                   \
    if (a.trace && threadIdx.x == 0 && (ev) < 64)                                        \
      a.trace[(size_t)blockIdx.x * 64 + (ev)] = wall_clock64();                          \
  } while (0)
#else
#define KMR_TRACE_MARK(ev) do { } while (0)
#endif

struct StepLayer {
  const uint16_t *in_norm, *q_norm, *k_norm, *post_norm;
  const uint8_t *qkv_p, *o_p, *gu_p, *d_p;
  const uint32_t *qkv_s, *o_s, *gu_s, *d_s;
};

struct StepArgs {
  const uint16_t* embed;
  const uint16_t* final_norm;
  const uint16_t* lm_head;
  const int32_t* ids;
  int32_t* pos;             // [3][B]
  int32_t* cpos;            // [B]
  uint8_t* finished;        // [B] or null
  int32_t* next;            // [B]
  float* logits;            // [B][V] or null
  uint16_t* kc;             // [L][cacheB][Hkv][M][D]
  uint16_t* vc;
  // workspace
  uint32_t* status;
  uint32_t* step_ctr;
  uint32_t* lm_cnt;
  uint32_t* xarr;           // [8] per-XCD arrival counters of the XCD-local kernel
  uint64_t* tx;             // [B][H]       tagged residual stream
  uint64_t* tqkv;           // [B][NQKV]
  uint64_t* to;             // [B][Hq*D]    attention output
  uint64_t* tact;           // [B][I]
  uint64_t* tpart;          // [B][Hkv][NS][QPG][D+2]  split partials (o~, m, l)
  float2* lm_part;          // [B][nwg]
  // XCD-local exchange buffers (k_stepx only); "per XCD" regions are strided by
  // the x_* strides (in 64-bit words)
  uint64_t* lx;             // per XCD [B][H]          x after the last layer
  uint64_t* sx;             // per XCD [2][B][srow_x]  staged x: entering a layer, after O
  uint64_t* lqkv;           // per XCD [B][QX]         q/k/v of the XCD's kv heads
  uint64_t* lpart;          // per XCD [B][GPX][NSX][PW] attention split partials
  uint64_t* lact;           // per XCD [B][srow_a]     staged SiLU(gate)*up of the XCD's slice
  uint64_t* pO;             // [NX][B][H]              O split-K partials
  uint64_t* pD;             // [NX][B][H]              down split-K partials
  long long x_lx, x_sx, x_lqkv, x_lpart, x_lact, srow_x, srow_a;
  int intra_plain;          // 1: XCD-local stores stay in the XCD's L2 (placement verified)
  // dims
  int B, H, Hq, Hkv, I, V, L, G, lgG, M, cacheB, NS, pad_id, eos_id;   // lgG = log2(G)
  uint32_t flags;
  uint32_t tag_xor;         // 0; a test hook sets a phase bit no producer writes, so every wait gives up
  uint32_t spin_limit;      // polls before a wait gives up
  uint64_t* trace;          // per-group phase timestamps (diagnostic builds only) or null
  float eps, scale_log2;
  double theta;
  int sec0, sec1, sec2, interleaved;
  StepLayer layers[kMaxStepLayers];
};

__device__ __forceinline__ uint64_t ld_dev64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_devf(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_devf(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void publish(uint64_t* p, uint32_t tag, float v) {
  st_dev64(p, ((uint64_t)tag << 32) | __float_as_uint(v));
}

// LDS position of float i of a gathered vector: 16-byte granules of each
// 32-float chunk are rotated by the chunk index, so that 64 lanes reading one
// chunk each (granule by granule) hit distinct banks.
__device__ __forceinline__ int swz(int i) {
  const int g = i >> 2, c = g >> 3, col = g & 7;
  return (((c << 3) | (col ^ (c & 7))) << 2) | (i & 3);
}

// Whether any thread of the work-group failed a bounded wait, with one barrier:
// a failing thread sets a flag in LDS before the barrier and every thread reads
// it after.  The flag is cleared once at kernel start (group_fail_reset, followed
// by a barrier) and never again: a failure ends the group, and any wave that sees
// it leaves (a wave that has ended no longer holds up the others' barriers).
__device__ __forceinline__ int* group_fail_flag() {
  __shared__ int flag;
  return &flag;
}
__device__ __forceinline__ void group_fail_reset() {
  if (threadIdx.x == 0) *group_fail_flag() = 0;
}
__device__ __forceinline__ bool group_failed(bool bad) {
  int* f = group_fail_flag();
  if (bad) *f = 1;
  __syncthreads();
  return *f != 0;
}

// Polls `total` tagged words until all carry `tag`, then stores their values in
// LDS at dst[place(i)] (at most `lim` polls per pass).  Word i lives at src + addr(i).  Each thread issues all
// its loads of a pass before checking any, so a poll costs one memory round
// trip; `pre` runs after the first loads are issued (to overlap other work with
// them).  Returns false, for the whole work-group, on timeout.
template <int PT, typename Addr, typename Place, typename Pre, int NT = kStepThreads>
__device__ __forceinline__ bool gather_tagged(const uint64_t* src, int total, uint32_t tag,
                                              float* dst, Addr addr, Place place, Pre pre, uint32_t lim) {
  const int tid = otid();
  bool ok = true;
  bool first = true;
  for (int base = 0; base < total && ok; base += NT * PT) {
    uint64_t v[PT];
    int idx[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) idx[j] = base + tid + NT * j;
    uint32_t spins = 0;
    bool fresh;
    do {
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (idx[j] < total) v[j] = ld_dev64(src + addr(idx[j]));
      if (first) {
        pre();
        first = false;
      }
      fresh = true;
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (idx[j] < total) fresh &= (uint32_t)(v[j] >> 32) == tag;
      if (!fresh) {
        if (++spins > lim) { ok = false; break; }
        __builtin_amdgcn_s_sleep(KMR_POLL_SLEEP);
      }
    } while (!fresh);
    if (ok)
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (idx[j] < total) dst[place(idx[j])] = __uint_as_float((uint32_t)v[j]);
  }
  if (first) pre();
  return !group_failed(!ok);
}

struct NoPre {
  __device__ void operator()() const {}
};

// The pair (value of the lower lane, value of the upper lane) of lanes l and
// l ^ 16 (BIT = 16) or l ^ 32 (BIT = 32), the same on both lanes.
template <int BIT>
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
  const uint32_t u = __float_as_uint(v);
  const auto r = BIT == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                           : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// ------------------------------------------------------------------ GEMV input staging
// Value of lane l ^ 4 (the other half of an 8-lane group), from two DPP
// rotations within each 16-lane row: banks 0 and 2 take lane + 4, banks 1 and 3
// take lane - 4.
__device__ __forceinline__ float lane_xor4(float v) {
  const float up = dpp<0x12C, 0xf, 0x5>(v);   // row_ror 12: lane i <- lane i + 4
  const float dn = dpp<0x124, 0xf, 0xA>(v);   // row_ror 4:  lane i <- lane i - 4
  return (otid() & 4) ? dn : up;
}

// Converts this thread's PT values of a [B][K] input (value j is element
// base + 512 j + tid, row wb[j], column wk[j]) into the LDS layout the dot
// products read: xs[(b*4 + w)*CH + c] holds the fp16 pairs of word w (8 columns)
// of 32-column chunk c, and cc[b*CH + c] its (C1, C2) = (1024 sum h + 8 sum x,
// sum x) over the values actually used (odd columns pre-divided by 16, matching
// the magic-bias weight pairs).  An 8-column word lives in 8 consecutive lanes
// (pairs formed with lane ^ 4), a 32-column chunk in 32 consecutive lanes, so K
// must be a multiple of 32.  Every lane of the wave must call this (DPP).
// Returns whether one of this thread's values overflowed fp16 (the caller raises
// KMR_STATUS_RANGE).
template <int PT>
__device__ __forceinline__ bool stage_values(const float (&e)[PT], const bool (&has)[PT],
                                             const int (&wb)[PT], const int (&wk)[PT], int K,
                                             uint4* xs, float2* cc) {
  const int lane = otid() & 63, CH = K >> 5, i8 = lane & 7;
  uint32_t* xs32 = reinterpret_cast<uint32_t*>(xs);
  bool over = false;
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const _Float16 h = (_Float16)((i8 & 1) ? e[j] * 0.0625f : e[j]);
    const float hf = (float)h;
    over |= has[j] && !(fabsf(hf) <= 65504.f);
    const float uf = (i8 & 1) ? 16.0f * hf : hf;
    const float other = lane_xor4(hf);
    // chunk sums over the 32 lanes of the chunk
    float bs = row16_sum(hf), us = row16_sum(uf), blo, bhi, ulo, uhi;
    lane_pair<16>(bs, blo, bhi);
    lane_pair<16>(us, ulo, uhi);
    if (has[j]) {
      const int c = wk[j] >> 5, w = (wk[j] >> 3) & 3;
      if (i8 < 4)
        xs32[((wb[j] * 4 + w) * CH + c) * 4 + i8] =
            __builtin_bit_cast(uint32_t, half2_t{h, (_Float16)other});
      if ((lane & 31) == 0) {
        const float bsum = blo + bhi, usum = ulo + uhi;
        cc[wb[j] * CH + c] = make_float2(1024.0f * bsum + 8.0f * usum, usum);
      }
    }
  }
  return over;
}

// Gathers a tagged [B][K] input (PT words per thread per pass, consecutive lanes
// polling consecutive words), optionally RMS-normalises it with `gain`, and
// stages it with stage_values.
template <int BT, int PT, int NT = kStepThreads>
__device__ __forceinline__ bool gather_stage(const uint64_t* src, int K, int B, uint32_t tag,
                                             const uint16_t* gain, float eps, uint4* xs, float2* cc,
                                             float* red, uint32_t lim, uint32_t* status) {
  const int tid = otid(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int total = B * K;
  float inv[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) inv[b] = 1.f;
  for (int base = 0; base < total; base += NT * PT) {
    int idx[PT], wb[PT], wk[PT];
    bool has[PT];
    uint16_t graw[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      idx[j] = base + NT * j + tid;
      has[j] = idx[j] < total;
      wb[j] = 0;
#pragma unroll
      for (int b = 1; b < BT; ++b) wb[j] += idx[j] >= b * K ? 1 : 0;
      wk[j] = idx[j] - wb[j] * K;
    }
    if (gain) {
      // raw loads with in-range addresses and no use before the polls below, so
      // nothing waits on them until the values are needed
#pragma unroll
      for (int j = 0; j < PT; ++j) graw[j] = gain[wk[j] < K ? wk[j] : K - 1];
    }
    uint64_t v[PT];
    uint32_t spins = 0;
    bool fresh, ok = true;
    do {
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (has[j]) v[j] = ld_dev64(src + idx[j]);
      fresh = true;
#pragma unroll
      for (int j = 0; j < PT; ++j)
        if (has[j]) fresh &= (uint32_t)(v[j] >> 32) == tag;
      if (!fresh) {
        if (++spins > lim) { ok = false; break; }
        __builtin_amdgcn_s_sleep(KMR_POLL_SLEEP);
      }
    } while (!fresh);
    if (group_failed(!ok)) return false;
    float x[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) x[j] = has[j] ? __uint_as_float((uint32_t)v[j]) : 0.f;
    if (gain) {
      // one pass holds every value (checked on the host): per-row sum of squares
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < PT; ++j)
          if (has[j] && wb[j] == b) ss += x[j] * x[j];
        ss = wave_sum(ss);
        if (lane == 0) red[b * (NT / 64) + wave] = ss;
      }
      __syncthreads();
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        float ss = 0.f;
#pragma unroll
        for (int w = 0; w < (NT / 64); ++w) ss += red[b * (NT / 64) + w];
        inv[b] = rsqrt_f(ss / (float)K + eps);
      }
    }
    float e[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      float iv = inv[0];
#pragma unroll
      for (int b = 1; b < BT; ++b) if (wb[j] == b) iv = inv[b];
      e[j] = gain ? (x[j] * iv) * bf16_to_f32(graw[j]) : x[j];
    }
    if (stage_values<PT>(e, has, wb, wk, K, xs, cc)) raise_status(status, kStatusRange);
  }
  __syncthreads();
  return true;
}

// ------------------------------------------------------------------ per-wave GEMV pieces
// NR weight rows for this lane's CPL 32-column chunks (codes and scale/zero).
template <int NR, int CPL>
struct WRows {
  uint4 raw[NR][CPL];
  uint32_t sz[NR][CPL];
};

template <int NR, int CPL>
__device__ __forceinline__ void wrows_load(WRows<NR, CPL>& w, const uint8_t* packed,
                                           const uint32_t* sz, int K, int lgG, const int* row,
                                           const bool* ok) {
  const int lane = otid() & 63, CH = K >> 5, NG = K >> lgG;
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (ok[i] && c < CH) {
        w.raw[i][j] = load_stream16(packed + (size_t)row[i] * (K / 2) + 16 * c);
        w.sz[i][j] = sz[(size_t)row[i] * NG + ((32 * c) >> lgG)];
      } else {
        w.raw[i][j] = make_uint4(0, 0, 0, 0);
        w.sz[i][j] = 0;
      }
    }
}

// Per-chunk constants (C1, C2) = (1024 sum(h) + 8 sum(u), sum(u)) of a staged input
// row, from a precomputed array ...
struct ChunkCC {
  const float2* cc;
  int CH;   // chunks per row
  __device__ float2 get(int b, int c) const { return cc[b * CH + c]; }
};
// ... or from the per-8-column-word sums (sum h, sum u) of a staged vector, 16-byte
// aligned rows of K/4 floats
struct ChunkSums {
  const float* sum;
  int K4;
  __device__ float2 get(int b, int c) const {
    const float4* p = reinterpret_cast<const float4*>(sum + b * K4 + 8 * c);
    const float4 lo = p[0], hi = p[1];
    const float sh = (lo.x + lo.z) + (hi.x + hi.z), su = (lo.y + lo.w) + (hi.y + hi.w);
    return make_float2(1024.0f * sh + 8.0f * su, su);
  }
};

// out[i][b] = dot of weight row i with staged input row b (uniform across the wave).
template <int BT, int NR, int CPL, typename CS>
__device__ __forceinline__ void wave_dot_c(const WRows<NR, CPL>& w, int K, int B, const uint4* xs,
                                           const CS& cs, float (&out)[NR][BT]) {
  const int lane = otid() & 63, CH = K >> 5;
  float acc[NR][BT];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[i][b] = 0.f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = lane + 64 * j;
    if (c < CH) {
      // the input chunk of every row first, then one row of weights at a time:
      // each row is dequantized once and only its 16 words are live
      uint4 xv[BT][4];
      float2 C[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const int bb = b < B ? b : 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[b][q] = xs[(bb * 4 + q) * CH + c];
        C[b] = cs.get(bb, c);
      }
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        uint32_t p[16];
        dequant16(w.raw[i][j], p);
        const float s = bf16_lo(w.sz[i][j]), z = bf16_hi(w.sz[i][j]);
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          if (BT > 1 && b >= B) break;   // (a batch-1 instantiation runs only at B == 1)
          float d = 0.f;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            d = fdot2(p[4 * q + 0], xv[b][q].x, d);
            d = fdot2(p[4 * q + 1], xv[b][q].y, d);
            d = fdot2(p[4 * q + 2], xv[b][q].z, d);
            d = fdot2(p[4 * q + 3], xv[b][q].w, d);
          }
          // explicit fused ops: the same arithmetic in every instantiation and row
          acc[i][b] = __builtin_fmaf(s, d - C[b].x, __builtin_fmaf(z, C[b].y, acc[i][b]));
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int b = 0; b < BT; ++b) out[i][b] = wave_sum(acc[i][b]);
}

template <int BT, int NR, int CPL>
__device__ __forceinline__ void wave_dot(const WRows<NR, CPL>& w, int K, int B, const uint4* xs,
                                         const float2* cc, float (&out)[NR][BT]) {
  wave_dot_c<BT, NR, CPL>(w, K, B, xs, ChunkCC{cc, K >> 5}, out);
}

struct AttnItem {
  int b, g, s, ns;
};

// Attention work items are (batch row, kv head, split), enumerated row by row.
__device__ __forceinline__ AttnItem attn_item(int item, const int* cpos, int B, int Hkv, int M) {
  AttnItem r{0, 0, 0, 1};
  int rem = item;
  for (r.b = 0; r.b < B; ++r.b) {
    r.ns = attn_splits(cpos[r.b], M);
    if (rem < Hkv * r.ns) break;
    rem -= Hkv * r.ns;
  }
  r.g = rem / r.ns;
  r.s = rem - r.g * r.ns;
  return r;
}

// Per-head RMSNorm over head_dim (16 lanes x DPL dims) then rotate-half RoPE,
// the partner dim sitting 8 lanes away in the same 16-lane row.
template <int DPL>
__device__ __forceinline__ void norm_rope(float (&vals)[DPL], const float (&gain)[DPL],
                                          const float (&c)[DPL], const float (&sn)[DPL], int D,
                                          float eps) {
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) ss += vals[e] * vals[e];
  ss = row16_sum(ss);
  const float inv = rsqrt_f(ss / (float)D + eps);
#pragma unroll
  for (int e = 0; e < DPL; ++e) vals[e] = (vals[e] * inv) * gain[e];
  float other[DPL];
#pragma unroll
  for (int e = 0; e < DPL; ++e) other[e] = row16_swap8(vals[e]);
#pragma unroll
  for (int e = 0; e < DPL; ++e) vals[e] = vals[e] * c[e] + other[e] * sn[e];
}

// Log-sum-exp merge of (m2, l2, o2) into (m, l, o); an empty state has m = -inf.
__device__ __forceinline__ void lse_merge(float& m, float& l, float* o, float m2, float l2,
                                          const float* o2, int n) {
  const float M = fmaxf(m, m2);
  const float c1 = m == -INFINITY ? 0.f : exp2_fast(m - M);
  const float c2 = m2 == -INFINITY ? 0.f : exp2_fast(m2 - M);
  l = l * c1 + l2 * c2;
  for (int i = 0; i < n; ++i) o[i] = o[i] * c1 + o2[i] * c2;
  m = M;
}


// LDS layout of the step kernel (dynamic shared memory, byte offsets):
//   xs    uint4 [BT][4][KMAX/32]  staged fp16 input pairs
//   cc    float2 [BT][KMAX/32]    per-chunk (C1, C2)
//   xin   fp32 scratch            attention q/k/v, wave states, split merge,
//                                 lm_head input
//   xown  fp32 [BT][RPBX]         this group's rows of the residual stream
//   cs    float2 [BT][D/2]        RoPE cos/sin of each row
//   red   float [128]
struct StepLds {
  size_t xs, cc, xin, xown, cs, red, total;
};

__host__ __device__ inline StepLds step_lds(int BT, int KMAX, int RPBX, int H, int D, int QPG) {
  StepLds s{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 15) & ~(size_t)15; return r; };
  const size_t merge_bytes = (size_t)kMergeChunk * QPG * (D + 2) * 4;
  const size_t attn_bytes = (size_t)kStepWaves * QPG * (D + 2) * 4 + (size_t)(QPG + 2) * D * 4;
  size_t xin_bytes = (size_t)BT * H * 4;
  if (xin_bytes < merge_bytes) xin_bytes = merge_bytes;
  if (xin_bytes < attn_bytes) xin_bytes = attn_bytes;
  s.xs = take((size_t)BT * 4 * (KMAX / 32) * 16);
  s.cc = take((size_t)BT * (KMAX / 32) * 8);
  s.xin = take(xin_bytes);
  s.xown = take((size_t)BT * RPBX * 4);
  s.cs = take((size_t)BT * (D / 2) * 8);
  s.red = take(128 * 4);
  s.total = o;
  return s;
}

// A step that cannot complete (a wait gave up, or an earlier call on this
// workspace did): KMR_STATUS_TIMEOUT is raised and every row's next id becomes
// -1, so a caller that feeds next_ids back without reading the status decodes
// nothing further.  Cache positions and positions stay unadvanced (the advance
// belongs to the last group's tail, which no group reaches once one has given
// up).  Any thread may call this; threads 0..B-1 write.
__device__ __forceinline__ void step_abandon(const StepArgs& a) {
  const int tid = threadIdx.x;
  if (tid == 0) raise_status(a.status, kStatusTimeout);
  if (tid < a.B) a.next[tid] = -1;
}

// Whether the workspace carries KMR_STATUS_TIMEOUT from an earlier call: its
// arrival counter and tags are then stale, and the step refuses to run until the
// workspace is re-initialised (the bit survives kmr_status).  Called by every
// thread with the same result: thread 0 reads the word, the barrier shares it.
__device__ __forceinline__ bool step_refused(const StepArgs& a, int* s_flag) {
  if (threadIdx.x == 0)
    *s_flag = (__hip_atomic_load(a.status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & kStatusTimeout) != 0;
  __syncthreads();
  return *s_flag != 0;
}

// Final RMSNorm, lm_head rows of this group with the argmax of each batch row,
// and (in the last group to finish) the argmax over all groups, the greedy-step
// bookkeeping and the step counter.  xin holds the gathered fp32 [B][H] input.
template <int BT, int NT = kStepThreads>
__device__ __forceinline__ void step_tail(const StepArgs& a, float* xin, float* red, int* s_last_p,
                                          uint32_t step) {
  const int tid = otid(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int B = a.B, M = a.M, K = a.H;
  int& s_last = *s_last_p;
  {
    // h = RMSNorm(x; final_norm), same association order as k_lmhead
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      float ss = 0.f;
      if (tid < 256 && b < B)
        for (int k = tid * 4; k < K; k += 1024) {
          const float4 v = *reinterpret_cast<const float4*>(xin + b * K + k);
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
        }
      ss = wave_sum(ss);
      if ((tid & 63) == 0 && tid < 256) red[b * 4 + (tid >> 6)] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const float ss = (red[b * 4 + 0] + red[b * 4 + 1]) + (red[b * 4 + 2] + red[b * 4 + 3]);
      const float inv = rsqrt_f(ss / (float)K + a.eps);
      for (int k = tid; k < K; k += NT)
        xin[b * K + k] = b < B ? (xin[b * K + k] * inv) * bf16_to_f32(a.final_norm[k]) : 0.f;
    }
    __syncthreads();
  }
  constexpr int LR = 4;            // rows per wave per pass
  constexpr int LCPL = 4;          // 8-column chunks per lane (K <= 2048)
  const int RPBL = (a.V + nwg - 1) / nwg;
  const int CH8 = K >> 3;
  float bv[BT]; int bi[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) { bv[b] = -INFINITY; bi[b] = 0x7fffffff; }
  for (int r0 = wave * LR; r0 < RPBL; r0 += (NT / 64) * LR) {
    uint4 w[LR][LCPL];
#pragma unroll
    for (int r = 0; r < LR; ++r)
#pragma unroll
      for (int j = 0; j < LCPL; ++j) {
        const int rr = r0 + r, n = wg * RPBL + rr, c = lane + 64 * j;
        w[r][j] = (rr < RPBL && n < a.V && c < CH8) ? load_stream16(a.lm_head + (size_t)n * K + 8 * c)
                                                    : make_uint4(0, 0, 0, 0);
      }
    float acc[LR][BT];
#pragma unroll
    for (int r = 0; r < LR; ++r)
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;
#pragma unroll
    for (int j = 0; j < LCPL; ++j) {
      const int c = lane + 64 * j;
      if (c < CH8) {
#pragma unroll
        for (int b = 0; b < BT; ++b) {
          const float4 h0 = *reinterpret_cast<const float4*>(xin + b * K + 8 * c);
          const float4 h1 = *reinterpret_cast<const float4*>(xin + b * K + 8 * c + 4);
#pragma unroll
          for (int r = 0; r < LR; ++r) {
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
#pragma unroll
    for (int r = 0; r < LR; ++r) {
      const int rr = r0 + r, n = wg * RPBL + rr;
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        const float v = wave_sum(acc[r][b]);
        if (rr < RPBL && n < a.V && b < B) {
          if (a.logits && lane == 0) a.logits[(size_t)b * a.V + n] = v;
          if (better(v, n, bv[b], bi[b])) { bv[b] = v; bi[b] = n; }
        }
      }
    }
  }
  KMR_TRACE_MARK(57);
  float* s_bv = red;                                  // [8][BT]
  int* s_bi = reinterpret_cast<int*>(red + 64);       // [8][BT]
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int b = 0; b < BT; ++b) { s_bv[wave * BT + b] = bv[b]; s_bi[wave * BT + b] = bi[b]; }
  }
  __syncthreads();
  if (tid < B) {
    float v = s_bv[tid];
    int i = s_bi[tid];
    for (int w2 = 1; w2 < (NT / 64); ++w2)
      if (better(s_bv[w2 * BT + tid], s_bi[w2 * BT + tid], v, i)) { v = s_bv[w2 * BT + tid]; i = s_bi[w2 * BT + tid]; }
    st_devf(&a.lm_part[(size_t)tid * nwg + wg].x, v);
    st_devf(&a.lm_part[(size_t)tid * nwg + wg].y, __int_as_float(i));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    // release: this group's argmax partial is visible before its arrival counts;
    // the last group to arrive acquires (the fence) before it reads every partial
    const uint32_t prev = __hip_atomic_fetch_add(a.lm_cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)(nwg - 1);
    if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  KMR_TRACE_MARK(58);
  if (!s_last) return;
  // last group: argmax over all groups' partials (fixed tree order), then the
  // greedy-step bookkeeping, then the step counter
  float* t_v = xin;
  int* t_i = reinterpret_cast<int*>(xin + NT);
  for (int b = 0; b < B; ++b) {
    float v = -INFINITY;
    int i = 0x7fffffff;
    for (int t = tid; t < nwg; t += NT) {
      const float pv = ld_devf(&a.lm_part[(size_t)b * nwg + t].x);
      const int pi = __float_as_int(ld_devf(&a.lm_part[(size_t)b * nwg + t].y));
      if (better(pv, pi, v, i)) { v = pv; i = pi; }
    }
    __syncthreads();
    t_v[tid] = v;
    t_i[tid] = i;
    __syncthreads();
    for (int wdt = NT / 2; wdt > 0; wdt >>= 1) {
      if (tid < wdt && better(t_v[tid + wdt], t_i[tid + wdt], t_v[tid], t_i[tid])) {
        t_v[tid] = t_v[tid + wdt];
        t_i[tid] = t_i[tid + wdt];
      }
      __syncthreads();
    }
    if (tid == 0) {
      const int best = t_i[0];
      const int fin = a.finished ? a.finished[b] : 0;
      a.next[b] = fin ? a.pad_id : best;
      if ((a.flags & 1u) && !fin) {
        if (a.eos_id >= 0 && best == a.eos_id) {
          if (a.finished) a.finished[b] = 1;
        } else if (a.cpos[b] + 1 >= M) {
          if (a.finished) a.finished[b] = 1;
        } else {
          a.cpos[b] += 1;
          a.pos[0 * B + b] += 1;
          a.pos[1 * B + b] += 1;
          a.pos[2 * B + b] += 1;
        }
      }
    }
  }
  if (tid == 0) {
    __hip_atomic_store(a.lm_cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    a.step_ctr[0] = step;
  }
}

template <int BT, int D, int QPG>
__global__ __launch_bounds__(kStepThreads) void k_step(const StepArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int DPL = D / 16, HALF = D / 2, PW = QPG * (D + 2);   // partial words per split
  const int tid = otid(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x, nwg = gridDim.x;
  const int B = BT == 1 ? 1 : a.B;   // (a batch-1 instantiation runs only at B == 1)
  const int H = a.H, Hq = a.Hq, Hkv = a.Hkv, I = a.I, M = a.M;
  const int NQKV = (Hq + 2 * Hkv) * D, QD = Hq * D;
  const int KMAX = H > I ? (H > QD ? H : QD) : (I > QD ? I : QD);
  const int RPBX = (H + nwg - 1) / nwg;                     // residual rows owned per group
  const StepLds L = step_lds(BT, KMAX, RPBX, H, D, QPG);
  group_fail_reset();
  __syncthreads();
  uint4* xs = reinterpret_cast<uint4*>(smem + L.xs);
  float2* cc = reinterpret_cast<float2*>(smem + L.cc);
  float* xin = reinterpret_cast<float*>(smem + L.xin);
  float* xown = reinterpret_cast<float*>(smem + L.xown);
  float2* cs = reinterpret_cast<float2*>(smem + L.cs);
  float* red = reinterpret_cast<float*>(smem + L.red);
  __shared__ int s_last;
  __shared__ int s_c[16];

  if (step_refused(a, &s_last)) {
    step_abandon(a);
    return;
  }
  const uint32_t step = (a.step_ctr[0] + 1u) & 0x7fffffu;
  auto tag = [&](int phase) -> uint32_t { return (step << 9) | (uint32_t)phase; };
  // the tag a consumer waits for (the producer's, unless a test hook skews it)
  auto ctag = [&](int phase) -> uint32_t { return tag(phase) ^ a.tag_xor; };
  const uint32_t lim = a.spin_limit;
  bool alive = true;

  // ---- step prologue: cache positions, RoPE tables, embedding rows of this group
  if (tid < B) s_c[tid] = a.cpos[tid];
  for (int i = tid; i < B * HALF; i += kStepThreads) {
    const int b = i / HALF, j = i - b * HALF;
    const int ax = mrope_axis(j, a.sec0, a.sec1, a.sec2, a.interleaved);
    const double p = (double)a.pos[ax * B + b];
    const double inv_freq = pow(a.theta, -2.0 * (double)j / (double)D);
    double sn, cn;
    sincos(p * inv_freq, &sn, &cn);
    cs[b * HALF + j] = make_float2((float)cn, (float)sn);
  }
  for (int i = tid; i < B * RPBX; i += kStepThreads) {
    const int b = i / RPBX, r = i - b * RPBX, n = wg * RPBX + r;
    if (n >= H) continue;
    int id = (a.finished && a.finished[b]) ? a.pad_id : a.ids[b];
    const bool ok = id >= 0 && id < a.V;
    if (!ok && n == 0) raise_status(a.status, 2u);
    const float v = ok ? bf16_to_f32(a.embed[(size_t)id * H + n]) : 0.f;
    xown[b * RPBX + r] = v;
    publish(a.tx + (size_t)b * H + n, tag(1), v);
  }
  __syncthreads();
  KMR_TRACE_MARK(0);

  for (int l = 0; l < a.L && alive; ++l) {
    const StepLayer& Ly = a.layers[l];
    const int ph = 1 + 6 * l;   // tag of this layer's input x; +1 qkv, +2 partials,
                                // +3 o, +4 x after O, +5 act, +6 x after down
    [[maybe_unused]] const int tev = l < 5 ? 1 + 11 * l : 63;
    // ================= fused QKV: RPB rows per group, NR per wave
    {
      constexpr int NR = 2;
      const int RPB = (NQKV + nwg - 1) / nwg;
      for (int r0 = 0; r0 < RPB || r0 == 0; r0 += kStepWaves * NR) {
        int row[NR]; bool ok[NR];
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          const int rr = r0 + wave * NR + i, n = wg * RPB + rr;
          ok[i] = rr < RPB && n < NQKV;
          row[i] = ok[i] ? n : 0;
        }
        WRows<NR, 1> w;
        wrows_load(w, Ly.qkv_p, Ly.qkv_s, H, a.lgG, row, ok);
        if (r0 == 0) {
          if (!gather_stage<BT, 4 * BT>(a.tx, H, B, ctag(ph), Ly.in_norm, a.eps, xs, cc, red, lim, a.status)) { alive = false; break; }
        }
        KMR_TRACE_MARK(tev + 0);
        float out[NR][BT];
        wave_dot<BT, NR, 1>(w, H, B, xs, cc, out);
        if (lane < B) {
#pragma unroll
          for (int i = 0; i < NR; ++i)
            if (ok[i]) {
              float v = out[i][0];
#pragma unroll
              for (int b = 1; b < BT; ++b) if (lane == b) v = out[i][b];
              publish(a.tqkv + (size_t)lane * NQKV + row[i], tag(ph + 1), v);
            }
        }
        if (RPB <= kStepWaves * NR) break;
      }
      if (group_failed(!alive)) break;
    }
    KMR_TRACE_MARK(tev + 1);
    // ================= attention splits: items (b, g, split)
    uint16_t* kc = a.kc + (size_t)l * a.cacheB * Hkv * M * D;
    uint16_t* vc = a.vc + (size_t)l * a.cacheB * Hkv * M * D;
    int total = 0;
    for (int b = 0; b < B; ++b) total += Hkv * attn_splits(s_c[b], M);
    for (int item = wg; item < total; item += nwg) {
      const AttnItem it_ = attn_item(item, s_c, B, Hkv, M);
      const int b = it_.b, g = it_.g, s = it_.s, ns = it_.ns;
      const int c = s_c[b];
      const int rr = lane >> 4, li = lane & 15, row = wave * 4 + rr, d0 = li * DPL;
      uint64_t* odst = a.to + (size_t)b * QD + (size_t)g * QPG * D;
      if (c < 0 || c >= M) {
        if (tid == 0 && g == 0) raise_status(a.status, 1u);
        for (int i = tid; i < QPG * D; i += kStepThreads) publish(odst + i, tag(ph + 3), 0.f);
        continue;
      }
      const size_t head_base = ((size_t)b * Hkv + g) * M;
      // cache reads first: row `row` takes positions s*64 + 2*row + {0, 1}
      uint32_t kr[2][DPL / 2], vr[2][DPL / 2];
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int p = s * kAttnSplit + 2 * row + it;
        if (p < c) {
          const uint32_t* ks = reinterpret_cast<const uint32_t*>(kc + (head_base + p) * D + d0);
          const uint32_t* vs = reinterpret_cast<const uint32_t*>(vc + (head_base + p) * D + d0);
#pragma unroll
          for (int e = 0; e < DPL / 2; ++e) { kr[it][e] = ks[e]; vr[it][e] = vs[e]; }
        } else {
#pragma unroll
          for (int e = 0; e < DPL / 2; ++e) kr[it][e] = vr[it][e] = 0u;
        }
      }
      float gq[DPL], gk[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) { gq[e] = bf16_to_f32(Ly.q_norm[d0 + e]); gk[e] = bf16_to_f32(Ly.k_norm[d0 + e]); }
      // q heads g*QPG.. (contiguous), then k head g, then v head g, in one poll
      float* qv = xin;                                   // [(QPG + 2) * D]
      {
        const uint64_t* rowp = a.tqkv + (size_t)b * NQKV;
        const int qo = g * QPG * D, ko = (Hq + g) * D - QPG * D, vo = (Hq + Hkv + g) * D - (QPG + 1) * D;
        auto addr = [=](int i) { return (size_t)(i < QPG * D ? qo + i : (i < (QPG + 1) * D ? ko + i : vo + i)); };
        auto place = [](int i) { return i; };
        if (!gather_tagged<(QPG + 2) * D / kStepThreads + 1>(rowp, (QPG + 2) * D, ctag(ph + 1), qv, addr,
                                                            place, NoPre(), lim)) {
          alive = false;
          break;
        }
      }
      KMR_TRACE_MARK(tev + 2);
      float q[QPG][DPL], kf[DPL], vf[DPL];
#pragma unroll
      for (int h = 0; h < QPG; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e) q[h][e] = qv[h * D + d0 + e];
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        kf[e] = qv[QPG * D + d0 + e];
        vf[e] = qv[(QPG + 1) * D + d0 + e];
      }
      float cs_c[DPL], cs_s[DPL];
#pragma unroll
      for (int e = 0; e < DPL; ++e) {
        const float2 t = cs[b * HALF + ((d0 + e) % HALF)];
        cs_c[e] = t.x;
        cs_s[e] = (d0 < HALF) ? -t.y : t.y;
      }
#pragma unroll
      for (int h = 0; h < QPG; ++h) norm_rope<DPL>(q[h], gq, cs_c, cs_s, D, a.eps);
      norm_rope<DPL>(kf, gk, cs_c, cs_s, D, a.eps);
#pragma unroll
      for (int e = 0; e < DPL; ++e) { kf[e] = round_bf16(kf[e]); vf[e] = round_bf16(vf[e]); }
      if (s == ns - 1 && row == 0) {
        uint16_t* kd = kc + (head_base + c) * D + d0;
        uint16_t* vd = vc + (head_base + c) * D + d0;
#pragma unroll
        for (int e = 0; e < DPL; ++e) { kd[e] = f32_to_bf16(kf[e]); vd[e] = f32_to_bf16(vf[e]); }
      }
      float m[QPG], lsum[QPG], o[QPG][DPL];
#pragma unroll
      for (int h = 0; h < QPG; ++h) {
        m[h] = -INFINITY; lsum[h] = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[h][e] = 0.f;
      }
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int p = s * kAttnSplit + 2 * row + it;
        const bool valid = p <= c;
        float kk[DPL], vv[DPL];
        if (p == c) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) { kk[e] = kf[e]; vv[e] = vf[e]; }
        } else {
#pragma unroll
          for (int e = 0; e < DPL / 2; ++e) {
            kk[2 * e] = bf16_lo(kr[it][e]); kk[2 * e + 1] = bf16_hi(kr[it][e]);
            vv[2 * e] = bf16_lo(vr[it][e]); vv[2 * e + 1] = bf16_hi(vr[it][e]);
          }
        }
#pragma unroll
        for (int h = 0; h < QPG; ++h) {
          float sc = 0.f;
#pragma unroll
          for (int e = 0; e < DPL; ++e) sc += q[h][e] * kk[e];
          sc = row16_sum(sc) * a.scale_log2;
          if (valid) {
            const float mn = fmaxf(m[h], sc);
            const float corr = exp2_fast(m[h] - mn);
            const float pe = exp2_fast(sc - mn);
            lsum[h] = lsum[h] * corr + pe;
#pragma unroll
            for (int e = 0; e < DPL; ++e) o[h][e] = o[h][e] * corr + pe * vv[e];
            m[h] = mn;
          }
        }
      }
      KMR_TRACE_MARK(l == 1 ? 59 : 64);
      // merge the 4 rows of each wave: rows (0,1) and (2,3), then (01, 23); both
      // lanes of a pair merge (lower, upper) in that order, so all rows agree
#pragma unroll
      for (int h = 0; h < QPG; ++h) {
        float mlo, mhi, llo, lhi, olo[DPL], ohi[DPL];
        lane_pair<16>(m[h], mlo, mhi);
        lane_pair<16>(lsum[h], llo, lhi);
#pragma unroll
        for (int e = 0; e < DPL; ++e) lane_pair<16>(o[h][e], olo[e], ohi[e]);
        lse_merge(mlo, llo, olo, mhi, lhi, ohi, DPL);
        lane_pair<32>(mlo, m[h], mhi);
        lane_pair<32>(llo, lsum[h], lhi);
#pragma unroll
        for (int e = 0; e < DPL; ++e) lane_pair<32>(olo[e], o[h][e], ohi[e]);
        lse_merge(m[h], lsum[h], o[h], mhi, lhi, ohi, DPL);
      }
      __syncthreads();   // q/k/v scratch is reused below
      float* s_w = xin;                                  // [8 waves][QPG][D + 2]
      if (rr == 0) {
#pragma unroll
        for (int h = 0; h < QPG; ++h) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) s_w[(wave * QPG + h) * (D + 2) + d0 + e] = o[h][e];
          if (li == 0) {
            s_w[(wave * QPG + h) * (D + 2) + D] = m[h];
            s_w[(wave * QPG + h) * (D + 2) + D + 1] = lsum[h];
          }
        }
      }
      __syncthreads();
      uint64_t* pdst = a.tpart + (((size_t)b * Hkv + g) * a.NS + s) * PW;
      for (int i = tid; i < QPG * D; i += kStepThreads) {
        const int h = i / D, d = i - h * D;
        float Mx = -INFINITY, Ls = 0.f, Os = 0.f;
        for (int wv = 0; wv < kStepWaves; ++wv) {
          const float* st = s_w + (wv * QPG + h) * (D + 2);
          lse_merge(Mx, Ls, &Os, st[D], st[D + 1], st + d, 1);
        }
        if (ns == 1) {
          publish(odst + i, tag(ph + 3), Os * (1.0f / Ls));
        } else {
          publish(pdst + h * (D + 2) + d, tag(ph + 2), Os);
          if (d == 0) {
            publish(pdst + h * (D + 2) + D, tag(ph + 2), Mx);
            publish(pdst + h * (D + 2) + D + 1, tag(ph + 2), Ls);
          }
        }
      }
      __syncthreads();
      KMR_TRACE_MARK(l == 1 ? 60 : 64);
    }
    if (group_failed(!alive)) break;
    // ================= split merge: the group of each head's last split merges all
    for (int item = wg; item < total && alive; item += nwg) {
      const AttnItem it_ = attn_item(item, s_c, B, Hkv, M);
      const int b = it_.b, g = it_.g, s = it_.s, ns = it_.ns;
      const int c = s_c[b];
      if (ns == 1 || s != ns - 1 || c < 0 || c >= M) continue;
      const uint64_t* psrc = a.tpart + ((size_t)b * Hkv + g) * a.NS * PW;
      uint64_t* odst = a.to + (size_t)b * QD + (size_t)g * QPG * D;
      float Mx[2], Ls[2], Os[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) { Mx[k] = -INFINITY; Ls[k] = 0.f; Os[k] = 0.f; }
      for (int t0 = 0; t0 < ns && alive; t0 += kMergeChunk) {
        const int nt = ns - t0 < kMergeChunk ? ns - t0 : kMergeChunk;
        auto addr = [=](int i) { return (size_t)t0 * PW + i; };
        auto place = [](int i) { return i; };
        if (!gather_tagged<kMergeChunk * PW / kStepThreads + 1>(psrc, nt * PW, ctag(ph + 2), xin, addr,
                                                               place, NoPre(), lim)) {
          alive = false;
          break;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int i = tid + kStepThreads * k;
          if (i < QPG * D) {
            const int h = i / D, d = i - h * D;
            for (int t = 0; t < nt; ++t) {
              const float* pt = xin + t * PW + h * (D + 2);
              lse_merge(Mx[k], Ls[k], &Os[k], pt[D], pt[D + 1], pt + d, 1);
            }
          }
        }
        __syncthreads();
      }
      if (!alive) break;
      KMR_TRACE_MARK(l == 1 ? 61 : 64);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int i = tid + kStepThreads * k;
        if (i < QPG * D) publish(odst + i, tag(ph + 3), Os[k] * (1.0f / Ls[k]));
      }
      KMR_TRACE_MARK(l == 1 ? 62 : 64);
    }
    if (group_failed(!alive)) break;
    KMR_TRACE_MARK(tev + 3);
    // ================= O projection + residual: this group's RPBX rows of x
    for (int r2 = 0; r2 < RPBX || r2 == 0; r2 += kStepWaves) {
      constexpr int NR = 1;
      const int rr = r2 + wave, n = wg * RPBX + rr;
      int row[NR] = {0};
      bool ok[NR] = {rr < RPBX && n < H};
      if (ok[0]) row[0] = n;
      WRows<NR, 1> w;
      wrows_load(w, Ly.o_p, Ly.o_s, QD, a.lgG, row, ok);
      if (r2 == 0) {
        if (!gather_stage<BT, 4 * BT>(a.to, QD, B, ctag(ph + 3), nullptr, a.eps, xs, cc, red, lim, a.status)) { alive = false; break; }
      }
      KMR_TRACE_MARK(tev + 4);
      float out[NR][BT];
      wave_dot<BT, NR, 1>(w, QD, B, xs, cc, out);
      if (lane < B && ok[0]) {
        float v = out[0][0];
#pragma unroll
        for (int b = 1; b < BT; ++b) if (lane == b) v = out[0][b];
        const float xn = xown[lane * RPBX + rr] + v;
        xown[lane * RPBX + rr] = xn;
        publish(a.tx + (size_t)lane * H + n, tag(ph + 4), xn);
      }
      if (RPBX <= kStepWaves) break;
    }
    if (group_failed(!alive)) break;
    KMR_TRACE_MARK(tev + 5);
    // ================= gate-up + SiLU: RPB pairs per group, NP per wave
    {
      constexpr int NP = 3;
      const int RPB = (I + nwg - 1) / nwg;
      for (int r0 = 0; r0 < RPB || r0 == 0; r0 += kStepWaves * NP) {
        int row[2 * NP]; bool ok[2 * NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int rr = r0 + wave * NP + i, n = wg * RPB + rr;
          ok[i] = ok[NP + i] = rr < RPB && n < I;
          row[i] = ok[i] ? n : 0;
          row[NP + i] = ok[i] ? n + I : 0;
        }
        WRows<2 * NP, 1> w;
        wrows_load(w, Ly.gu_p, Ly.gu_s, H, a.lgG, row, ok);
        if (r0 == 0) {
          if (!gather_stage<BT, 4 * BT>(a.tx, H, B, ctag(ph + 4), Ly.post_norm, a.eps, xs, cc, red, lim, a.status)) { alive = false; break; }
        }
        KMR_TRACE_MARK(tev + 6);
        float out[2 * NP][BT];
        wave_dot<BT, 2 * NP, 1>(w, H, B, xs, cc, out);
        if (lane < B) {
#pragma unroll
          for (int i = 0; i < NP; ++i)
            if (ok[i]) {
              float gt = out[i][0], up = out[NP + i][0];
#pragma unroll
              for (int b = 1; b < BT; ++b) if (lane == b) { gt = out[i][b]; up = out[NP + i][b]; }
              publish(a.tact + (size_t)lane * I + row[i], tag(ph + 5), gt / (1.0f + expf(-gt)) * up);
            }
        }
        if (RPB <= kStepWaves * NP) break;
      }
      if (group_failed(!alive)) break;
    }
    KMR_TRACE_MARK(tev + 7);
    // ================= down + residual
    for (int r2 = 0; r2 < RPBX || r2 == 0; r2 += kStepWaves) {
      constexpr int NR = 1, CPL = 3;
      const int rr = r2 + wave, n = wg * RPBX + rr;
      int row[NR] = {0};
      bool ok[NR] = {rr < RPBX && n < H};
      if (ok[0]) row[0] = n;
      WRows<NR, CPL> w;
      wrows_load(w, Ly.d_p, Ly.d_s, I, a.lgG, row, ok);
      if (r2 == 0) {
        if (!gather_stage<BT, 12>(a.tact, I, B, ctag(ph + 5), nullptr, a.eps, xs, cc, red, lim, a.status)) { alive = false; break; }
      }
      KMR_TRACE_MARK(tev + 8);
      float out[NR][BT];
      wave_dot<BT, NR, CPL>(w, I, B, xs, cc, out);
      if (lane < B && ok[0]) {
        float v = out[0][0];
#pragma unroll
        for (int b = 1; b < BT; ++b) if (lane == b) v = out[0][b];
        const float xn = xown[lane * RPBX + rr] + v;
        xown[lane * RPBX + rr] = xn;
        publish(a.tx + (size_t)lane * H + n, tag(ph + 6), xn);
      }
      if (RPBX <= kStepWaves) break;
    }
    if (group_failed(!alive)) break;
    KMR_TRACE_MARK(tev + 9);
  }

  if (!alive) {
    step_abandon(a);
    return;
  }

  // ================= final RMSNorm + lm_head + argmax partial of this group
  const int K = H;
  {
    auto addr = [](int i) { return (size_t)i; };
    auto place = [](int i) { return i; };
    const bool ok = B * K <= kStepThreads * 4
                        ? gather_tagged<4>(a.tx, B * K, ctag(1 + 6 * a.L), xin, addr, place, NoPre(), lim)
                        : gather_tagged<12>(a.tx, B * K, ctag(1 + 6 * a.L), xin, addr, place, NoPre(), lim);
    if (!ok) {
      step_abandon(a);
      return;
    }
  }
  KMR_TRACE_MARK(56);
  step_tail<BT>(a, xin, red, &s_last, step);
}

}  // namespace kmr
