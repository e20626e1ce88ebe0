// kmr_stepx.h -- the persistent decode step with XCD-local exchanges.
//
// Same computation as k_step (kaminari page, section 04 "3 . decode": one greedy
// token per row from fixed-rank inputs and the static KV buffers), arranged
// around the chip's 8 XCDs instead of treating the 256 work-groups as one pool.
// Each work-group reads its XCD from the hardware and takes its index among that
// XCD's 32 groups from a per-XCD arrival counter, so the arrangement holds however
// the dispatcher deals the groups out; the 32 groups of one XCD share its L2, where
// a hand-off costs about half of a device-wide one.  Per layer, with XCD x owning kv heads [x*GPX, (x+1)*GPX) and
// the intermediate slice [x*IX, (x+1)*IX):
//   QKV      every XCD holds the whole residual stream x; its groups compute the
//            q/k/v rows of its own kv heads                       (XCD-local)
//   attn     split-KV items (row, kv head, 128-position split) of those heads,
//            partials published inside the XCD                    (XCD-local)
//   O        every group merges all split partials of its XCD (log-sum-exp, the
//            merge of "The Ghost in the Batch", "The merge math"), then computes
//            its RPW rows of W_o over the XCD's head columns only (split-K)
//   RS_O     each group sums the 8 XCD partials of its RPW rows (fixed order),
//            adds them to its residual rows, and publishes them   (device-wide)
//   GU       gate/up rows of the XCD's intermediate slice         (XCD-local x)
//   down     W_down rows of the group over the XCD's slice columns (split-K,
//            XCD-local act), then RS_D as RS_O                    (device-wide)
// so two of the six hand-offs of a layer cross XCDs.  Every XCD keeps its own
// bit-identical copy of the residual stream: the same sums in the same order.
#pragma once

#include <type_traits>

#include "kmr_step.h"

namespace kmr {

constexpr int kXcds = 8;            // XCDs of the device
constexpr int kXSplit = 128;        // attention positions per split item
constexpr int kXMergeChunk = 8;     // split partials merged per LDS pass
constexpr int kXNarrowCpl = 3;      // max 32-column chunks per lane in the split-K GEMVs
constexpr uint32_t kStatusTopology = 8u;
constexpr int kXMaxPerXcd = 64;     // work-groups per XCD
constexpr int kXSsSlots = kXMaxPerXcd * 2;   // sums-of-squares slots of a staged row (<= 2 per group)
constexpr int kXGuRows = 6;         // gate/up rows per wave (3 act values)
// s_sleep(8) rounds (512 clocks each) between a group's q/k/v publish and its early
// gate/up request when it has no attention item (batch 1): 6 to 10 measured alike
// at the workload's positions, 4 and 12 measured as no early request at all.
constexpr int kEarlyGuSleeps = 8;

// Store of a tagged word that only groups of this XCD read.  A work-group-scope
// store stays in the XCD's L2, where the device-scope polls of the XCD's other
// groups find it; without verified placement the device-scope store is used,
// which every group sees wherever it runs.
__device__ __forceinline__ void publish_l(uint64_t* p, uint32_t tag, float v, int plain) {
  const uint64_t w = ((uint64_t)tag << 32) | __float_as_uint(v);
  if (plain)
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else
    st_dev64(p, w);
}

// Row b, local kv head gl and split s of attention item `item` (items run row by
// row, then kv head, then split); s_ns in LDS holds each row's split count.
__device__ __forceinline__ void xitem(int item, const int* s_ns, int GPX, int& b, int& gl, int& s) {
  int rem = item;
  b = 0;
  while (rem >= GPX * s_ns[b]) { rem -= GPX * s_ns[b]; ++b; }
  const int ns = s_ns[b];
  gl = GPX == 1 ? 0 : rem / ns;   // one kv head per XCD: no division
  s = rem - gl * ns;
}

// K/V rows of attention item `item` (row b, local kv head, 128-position split), laid
// out for the matrix-core products of the attention loop.  Wave w takes positions
// s*128 + 16 w + {0..15}; lane (r, i) = (lane / 16, lane % 16) loads
//   K: position s*128 + 16 w + i, dims 32 t + 8 r .. + 7 for t < D/32 (the first
//      operand of the score product: row i, columns 8 r .. of each 32-dim step)
//   V: positions s*128 + 16 w + 4 r + e, e < 4, dims DPL i .. + DPL - 1.
// The loads are unconditional (slot clamped into the cache) so that nothing waits
// for them here; the attention loop ignores slots past the row's cache position
// and takes the new slot's k/v from the QKV phase.
template <int DPL, bool LK = true, bool LV = true>
__device__ __forceinline__ void attn_load_kv(uint32_t (&kr)[DPL / 2][4], uint32_t (&vr)[4][DPL / 2],
                                             const uint16_t* kc, const uint16_t* vc, int item,
                                             const int* s_ns, const int* s_c, int GPX, int x, int Hkv,
                                             int M, int D, int wave) {
  static_assert(DPL == 4 || DPL == 8, "head_dim 64 or 128");
  int b, gl, s;
  xitem(item, s_ns, GPX, b, gl, s);
  const int g = x * GPX + gl;
  const int lane = otid() & 63, rr = lane >> 4, li = lane & 15;
  const size_t head_base = ((size_t)b * Hkv + g) * M;
  const int p0 = s * kXSplit + 16 * wave;
  if constexpr (LK) {
    const int p = p0 + li < M ? p0 + li : M - 1;
#pragma unroll
    for (int t = 0; t < DPL / 2; ++t) {
      const uint4 k4 = *reinterpret_cast<const uint4*>(kc + (head_base + p) * D + 32 * t + 8 * rr);
      kr[t][0] = k4.x; kr[t][1] = k4.y; kr[t][2] = k4.z; kr[t][3] = k4.w;
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (!LV) break;
    int p = p0 + 4 * rr + e;
    p = p < M ? p : M - 1;
    // DPL bf16 = DPL * 2 bytes per lane, aligned to that size (DPL * li)
    if constexpr (DPL == 8) {
      const uint4 v4 = *reinterpret_cast<const uint4*>(vc + (head_base + p) * D + DPL * li);
      vr[e][0] = v4.x; vr[e][1] = v4.y; vr[e][2] = v4.z; vr[e][3] = v4.w;
    } else {
      const uint2 v2 = *reinterpret_cast<const uint2*>(vc + (head_base + p) * D + DPL * li);
      vr[e][0] = v2.x; vr[e][1] = v2.y;
    }
  }
}

// ------------------------------------------------------------------ split-K GEMV
// One weight row per 8-lane group, restricted to a KS-column slice: lane
// (lane & 7) of the group takes 32-column chunks (lane & 7) + 8 t, t < kXNarrowCpl.
struct WNarrow {
  uint4 raw[kXNarrowCpl];
  uint32_t sz[kXNarrowCpl];
};

__device__ __forceinline__ void wnarrow_load(WNarrow& w, const uint8_t* packed, const uint32_t* sz,
                                             int K, int lgG, int k0, int KS, int row, bool ok) {
  const int sub = otid() & 7, CHs = KS >> 5, NG = K >> lgG;
#pragma unroll
  for (int t = 0; t < kXNarrowCpl; ++t) {
    const int c = sub + 8 * t;
    if (ok && c < CHs) {
      w.raw[t] = load_stream16(packed + (size_t)row * (K / 2) + (k0 >> 1) + 16 * c);
      w.sz[t] = sz[(size_t)row * NG + ((k0 + 32 * c) >> lgG)];
    } else {
      w.raw[t] = make_uint4(0, 0, 0, 0);
      w.sz[t] = 0;
    }
  }
}

// The same weights streamed into LDS instead of registers: chunk t of thread i at
// raw[t * kStepThreads + i] and sz[t * kStepThreads + i] (each wave's 64 lanes
// contiguous, as the LDS DMA writes them).  Slots of chunks a lane does not load keep
// stale data, which narrow_dot never uses for a published row.
__device__ __forceinline__ void wnarrow_to_lds(const uint8_t* packed, const uint32_t* sz, int K, int lgG,
                                               int k0, int KS, int row, bool ok, uint4* raw_l,
                                               uint32_t* sz_l) {
  const int tid = otid(), sub = tid & 7, wave = tid >> 6, CHs = KS >> 5, NG = K >> lgG;
#pragma unroll
  for (int t = 0; t < kXNarrowCpl; ++t) {
    const int c = sub + 8 * t;
    if (ok && c < CHs) {
      __builtin_amdgcn_global_load_lds(packed + (size_t)row * (K / 2) + (k0 >> 1) + 16 * c,
                                       raw_l + t * kStepThreads + wave * 64, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(sz + (size_t)row * NG + ((k0 + 32 * c) >> lgG),
                                       sz_l + t * kStepThreads + wave * 64, 4, 0, 0);
    }
  }
}
__device__ __forceinline__ void wnarrow_from_lds(WNarrow& w, const uint4* raw_l, const uint32_t* sz_l) {
  const int tid = otid();
#pragma unroll
  for (int t = 0; t < kXNarrowCpl; ++t) {
    w.raw[t] = raw_l[t * kStepThreads + tid];
    w.sz[t] = sz_l[t * kStepThreads + tid];
  }
}

// out[b] = dot of the group's row with staged input row b over the slice; every
// lane of the 8-lane group receives the sums.
template <int BT, typename CS>
__device__ __forceinline__ void narrow_dot(const WNarrow& w, int KS, int B, const uint4* xs,
                                           const CS& cs, float (&out)[BT]) {
  const int sub = otid() & 7, CHs = KS >> 5;
  float acc[BT];
#pragma unroll
  for (int b = 0; b < BT; ++b) acc[b] = 0.f;
#pragma unroll
  for (int t = 0; t < kXNarrowCpl; ++t) {
    const int c = sub + 8 * t;
    if (c < CHs) {
      uint32_t p[16];
      dequant16(w.raw[t], p);
      const float s = bf16_lo(w.sz[t]), z = bf16_hi(w.sz[t]);
#pragma unroll
      for (int b = 0; b < BT; ++b) {
        if (BT > 1 && b >= B) break;   // (a batch-1 instantiation runs only at B == 1)
        uint4 xv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[q] = xs[(b * 4 + q) * CHs + c];
        const float2 C = cs.get(b, c);
        float d = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          d = fdot2(p[4 * q + 0], xv[q].x, d);
          d = fdot2(p[4 * q + 1], xv[q].y, d);
          d = fdot2(p[4 * q + 2], xv[q].z, d);
          d = fdot2(p[4 * q + 3], xv[q].w, d);
        }
        acc[b] = __builtin_fmaf(s, d - C.x, __builtin_fmaf(z, C.y, acc[b]));
      }
    }
  }
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    float v = acc[b];
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
    v += lane_xor4(v);
    out[b] = v;
  }
}

// ------------------------------------------------------------------ reduce-scatter
// Sums the kXcds split-K partials of this group's RPW residual rows in XCD order
// 0..7 and adds the sum to the owned rows.  Thread i < B*RPW gets element
// (b, r) = (i / RPW, i % RPW) in xn (has: a row below H).  Returns false, for the
// whole group, on timeout.
// RPW is a power of two (checked on the host): row and column by shifts.
template <int BT>
__device__ __forceinline__ bool reduce_rows(const uint64_t* part, uint32_t ptag, int B, int H,
                                            int RPW, int row0, float* xown, float* buf, float& xn,
                                            bool& has_x, uint32_t lim) {
  constexpr int PT = 4;
  const int tid = otid(), per = B * RPW, words = kXcds * per, lgR = __builtin_ctz((unsigned)RPW);
  bool ok = true;
  for (int base = 0; base < words && ok; base += kStepThreads * PT) {
    uint64_t v[PT];
    uint32_t off[PT];
    bool has[PT];
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int i = base + kStepThreads * q + tid;
      const int y = BT == 1 ? i >> lgR : i / per, rem = i - y * per, b = rem >> lgR, r = rem & (RPW - 1);
      has[q] = i < words && row0 + r < H;
      off[q] = has[q] ? (uint32_t)((y * B + b) * H + row0 + r) : 0u;
    }
    uint32_t spins = 0;
    bool fresh;
    do {
#pragma unroll
      for (int q = 0; q < PT; ++q)
        if (has[q]) v[q] = ld_dev64(part + off[q]);
      fresh = true;
#pragma unroll
      for (int q = 0; q < PT; ++q)
        if (has[q]) fresh &= (uint32_t)(v[q] >> 32) == ptag;
      if (!fresh) {
        if (++spins > lim) { ok = false; break; }
        __builtin_amdgcn_s_sleep(KMR_POLL_SLEEP);
      }
    } while (!fresh);
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int i = base + kStepThreads * q + tid;
      if (i < words) buf[i] = has[q] ? __uint_as_float((uint32_t)v[q]) : 0.f;
    }
  }
  if (group_failed(!ok)) return false;
  // per <= kStepThreads (checked on the host): one element per thread
  const int b = tid >> lgR, r = tid & (RPW - 1);
  has_x = tid < per && row0 + r < H;
  xn = 0.f;
  if (has_x) {
    // (the partials and the owned value read first: one after another each read
    // would be waited for before the next)
    float pv[kXcds];
#pragma unroll
    for (int y = 0; y < kXcds; ++y) pv[y] = buf[((BT == 1 ? y : y * B + b)) * RPW + r];
    const float xo = xown[b * RPW + r];
    float sum = 0.f;
#pragma unroll
    for (int y = 0; y < kXcds; ++y) sum += pv[y];
    xn = xo + sum;
    xown[b * RPW + r] = xn;
  }
  return true;
}

// ------------------------------------------------------------------ staged vectors
// A GEMV input published already in the layout the dot products read, so that
// each consumer only copies it: per row b of K columns, at src + b * stride,
//   [0, K/2)        fp16 pairs: word 4w + i (i < 4) of 8-column word w holds
//                   (h[8w + i], h[8w + i + 4]), h = fp16(u) for even columns and
//                   fp16(u / 16) for odd ones (matching the magic-bias weight pairs)
//   [K/2, 3K/4)     per 8-column word: sum of h, then sum of the used values
//                   (16 h for odd columns)
//   [3K/4, 3K/4+n)  optional sums of squares of the unscaled input, one per producer
//                   part (a wave's share of the row)
// For an RMSNorm input, u = x * gain and the consumer scales its dot products by
// 1/sqrt(sum of squares / K + eps): the norm's scale is common to the row.
// Residual-stream and MLP values are not normalised before staging, so they are
// staged as u * 2^-3 (kStageScale, an exact power of two) and the consumers
// multiply their dot products back by 2^3: the fp16 pairs then stay finite for
// |u| < 65504 * 8 (about 5.2e5; even columns, the narrower ones).  A producer
// that meets a larger or non-finite value raises KMR_STATUS_RANGE.
constexpr float kStageScale = 0.125f, kStageUnscale = 8.0f;

// Raises KMR_STATUS_RANGE (once per wave) when some lane's staged value u (already
// scaled by kStageScale) is outside the fp16 range.  Every lane of the wave calls this.
__device__ __forceinline__ void stage_range_check(float u, uint32_t* status) {
  if (__builtin_amdgcn_ballot_w64(!(fabsf(u) < 65504.f)) != 0 && (otid() & 63) == 0)
    raise_status(status, kStatusRange);
}

__device__ __forceinline__ void publish_lb(uint64_t* p, uint32_t tag, uint32_t bits, int plain) {
  const uint64_t w = ((uint64_t)tag << 32) | bits;
  if (plain)
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else
    st_dev64(p, w);
}

// This lane's value u of column n (has: valid) of a staged row at dst.  The 8
// lanes of an aligned group hold 8 consecutive columns starting at a multiple of
// 8 (n & 7 == lane & 7).  Every lane of the wave must call this (DPP).
__device__ __forceinline__ void stage_publish(uint64_t* dst, int K, int n, float u, bool has,
                                              uint32_t tag, int plain) {
  const int i8 = otid() & 7;
  const _Float16 h = (_Float16)((i8 & 1) ? u * 0.0625f : u);
  const float hf = (float)h;
  const float uf = (i8 & 1) ? 16.0f * hf : hf;
  const float other = lane_xor4(hf);
  float sh = hf, su = uf;
  sh += dpp<0xB1>(sh);
  su += dpp<0xB1>(su);
  sh += dpp<0x4E>(sh);
  su += dpp<0x4E>(su);
  sh += lane_xor4(sh);
  su += lane_xor4(su);
  if (has) {
    const int w = n >> 3;
    if (i8 < 4)
      publish_lb(dst + 4 * w + i8, tag, __builtin_bit_cast(uint32_t, half2_t{h, (_Float16)other}), plain);
    if (i8 == 0) {
      publish_lb(dst + (K >> 1) + 2 * w, tag, __float_as_uint(sh), plain);
      publish_lb(dst + (K >> 1) + 2 * w + 1, tag, __float_as_uint(su), plain);
    }
  }
}

// Gathers B staged rows of K columns (plus nss sums of squares each) into the
// dot-product LDS layout: pairs into xs, and the per-word sums into sums ([BT][K/4],
// read through ChunkSums) followed by the sums of squares ([BT][nss], read by
// staged_inv).  One barrier: the data is in LDS for every wave on return.  The
// buffers must not be rewritten before a barrier that follows their last reader.
// Returns false, for the whole group, on timeout.
template <int BT, int PT>
__device__ __forceinline__ bool gather_staged(const uint64_t* src, long long stride, int K, int B,
                                              int nss, uint32_t tag, uint4* xs, float* sums, uint32_t lim) {
  const int tid = otid();
  const int CH = K >> 5, K2 = K >> 1, K4 = K >> 2, per = K2 + K4 + nss, total = B * per;
  uint32_t* xs32 = reinterpret_cast<uint32_t*>(xs);
  float* s_sum = sums;             // [B][K/4]
  float* s_ss = sums + BT * K4;    // [B][nss]
  bool ok = true;
  for (int base = 0; base < total && ok; base += kStepThreads * PT) {
    uint64_t v[PT];
    const uint64_t* sp[PT];
    uint32_t* dp[PT];
    bool has[PT];
    // source and LDS destination of every word, worked out before the first poll
#pragma unroll
    for (int q = 0; q < PT; ++q) {
      const int i = base + kStepThreads * q + tid;
      has[q] = i < total;
      int b = 0;
#pragma unroll
      for (int t = 1; t < BT; ++t) b += i >= t * per ? 1 : 0;
      const int k = i - b * per, w8 = k >> 2;
      sp[q] = src + (size_t)b * stride + k;
      dp[q] = k < K2 ? xs32 + ((b * 4 + (w8 & 3)) * CH + (w8 >> 2)) * 4 + (k & 3)
            : k < K2 + K4 ? reinterpret_cast<uint32_t*>(s_sum) + b * K4 + (k - K2)
                          : reinterpret_cast<uint32_t*>(s_ss) + b * nss + (k - K2 - K4);
    }
    uint32_t spins = 0;
    bool fresh;
    do {
#pragma unroll
      for (int q = 0; q < PT; ++q)
        if (has[q]) v[q] = ld_dev64(sp[q]);
      fresh = true;
#pragma unroll
      for (int q = 0; q < PT; ++q)
        if (has[q]) fresh &= (uint32_t)(v[q] >> 32) == tag;
      if (!fresh) {
        if (++spins > lim) { ok = false; break; }
        __builtin_amdgcn_s_sleep(KMR_POLL_SLEEP);
      }
    } while (!fresh);
#pragma unroll
    for (int q = 0; q < PT; ++q)
      if (has[q]) *dp[q] = (uint32_t)v[q];
  }
  return !group_failed(!ok);
}

// 1/sqrt(sum of squares / K + eps) of staged row b from its nss (<= kXSsSlots)
// partial sums in LDS, times kStageUnscale (the row was staged scaled by
// kStageScale); every lane of the calling wave gets it.
__device__ __forceinline__ float staged_inv(const float* s_ss, int b, int nss, int K, float eps) {
  const int lane = otid() & 63;
  float part = 0.f;
  for (int i = lane; i < nss; i += 64) part += s_ss[b * nss + i];
  return rsqrt_f(wave_sum(part) / (float)K + eps) * kStageUnscale;
}

// Lane b < B: staged_inv of row b (the others get 1).  Every lane of the wave must
// call this.
template <int BT>
__device__ __forceinline__ float row_inv(const float* s_ss, int B, int nss, int K, float eps) {
  const int lane = otid() & 63;
  float r = 1.f;
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    if (BT > 1 && b >= B) break;
    const float v = staged_inv(s_ss, b, nss, K, eps);
    if (lane == b) r = v;
  }
  return r;
}

// The norm gain of this thread's column in publish_staged_x, requested early (an
// in-range address, no use here) so that nothing waits on it before it is needed.
__device__ __forceinline__ uint16_t staged_gain(const uint16_t* gain, int H, int RPW, int row0) {
  const int tid = otid();
  const int n = row0 + (tid & (RPW - 1));   // RPW: a power of two
  return gain[n < H ? n : H - 1];
}

// Publishes x rows (element i = tid: row b = i / RPW, column row0 + i % RPW, valid
// if has) of a staged RMSNorm input: u = x * gain * kStageScale (g: this column's
// bf16 gain from staged_gain), and the sum of squares of x of each row from each
// wave that holds part of it, at slot WPR * slot + (wave - first wave of the row),
// WPR = max(1, RPW / 64) (a row starts at a wave boundary or within one wave:
// 64 % RPW == 0 or RPW % 64 == 0, checked on the host).  Every thread of the group
// must call this; it has no barrier.
template <int BT>
__device__ __forceinline__ void publish_staged_x(uint64_t* dst, long long stride, int H, int B,
                                                 int RPW, int row0, float xn, bool has, uint16_t g,
                                                 int slot, uint32_t tag, int plain, uint32_t* status) {
  const int tid = otid(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = tid >> __builtin_ctz((unsigned)RPW), n = row0 + (tid & (RPW - 1));   // RPW: a power of two
  const float u = has ? xn * (bf16_to_f32(g) * kStageScale) : 0.f;
  stage_range_check(u, status);
  stage_publish(dst + (size_t)(has ? b : 0) * stride, H, n, u, has, tag, plain);
  const int WPR = RPW >= 64 ? RPW >> 6 : 1;
#pragma unroll
  for (int bb = 0; bb < BT; ++bb) {
    if (BT > 1 && bb >= B) break;
    const int w0 = (bb * RPW) >> 6, w1 = ((bb + 1) * RPW - 1) >> 6;
    if (wave >= w0 && wave <= w1) {
      const float ss = wave_sum((has && b == bb) ? xn * xn : 0.f);
      if (lane == 0)
        publish_l(dst + (size_t)bb * stride + (H >> 1) + (H >> 2) + WPR * slot + (wave - w0), tag, ss,
                  plain);
    }
  }
}

// Float offset in the attention scratch of the q heads' bf16 splits (16-byte
// aligned), after q/k/v, the wave states and their merge weights.
__host__ __device__ inline int xattn_qb(int D, int QPG) {
  return ((QPG + 2) * D + kStepWaves * QPG * (D + 2) + (kStepWaves + 2) * QPG + 3) & ~3;
}

// ------------------------------------------------------------------ LDS layout
//   xs    uint4 [BT][4][H/32]   staged fp16 input pairs (every GEMV input <= H)
//   cc    float2 [BT][H/32]     per-chunk (C1, C2) of the O input
//   sums  fp32 [BT][H/4], [BT][64]  per-word sums and sums of squares of a
//                               gathered staged vector
//   xin   fp32 scratch          attention q/k/v, wave states and the q heads' bf16
//                               splits, split merge, reduce-scatter partials,
//                               lm_head input
//   xown  fp32 [BT][RPW]        this group's rows of the residual stream
//   cs    float2 [BT][D/2]      RoPE cos/sin of each row
//   red   float [128]
//   wgu   gate/up codes and scale/zero words, [8 waves][6 rows][64] (also the q/k/v
//         rows between the gate/up products, and the q/k/v tile's wave partials)
//   wdn   (batch > 1) the group's down weights: uint4 [3][512] codes, u32 [3][512]
//         scale/zero words
struct StepXLds {
  size_t xs, cc, sums, xin, xown, cs, red, wgu, wdn, total;
};

__host__ __device__ inline StepXLds stepx_lds(int BT, int H, int RPW, int D, int QPG, int GPX) {
  StepXLds s{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += (bytes + 15) & ~(size_t)15; return r; };
  const size_t pw = (size_t)QPG * (D + 2);
  // attention: q/k/v, then the wave states and their merge weights (disjoint)
  size_t xin = (size_t)xattn_qb(D, QPG) * 4 + (size_t)2 * QPG * D * 2;
  const size_t merge = (size_t)BT * GPX * kXMergeChunk * pw * 4 +
                       (size_t)BT * GPX * QPG * (kXMergeChunk + 2) * 4;
  const size_t rs = (size_t)kXcds * BT * RPW * 4;
  const size_t lm = (size_t)BT * H * 4;
  if (xin < merge) xin = merge;
  if (xin < rs) xin = rs;
  if (xin < lm) xin = lm;
  s.xs = take((size_t)BT * 4 * (H / 32) * 16);
  s.cc = take((size_t)BT * (H / 32) * 8);
  s.sums = take((size_t)BT * (H / 4 + kXSsSlots) * 4);
  s.xin = take(xin);
  s.xown = take((size_t)BT * RPW * 4);
  s.cs = take((size_t)BT * (D / 2) * 8);
  s.red = take(128 * 4);
  s.wgu = take((size_t)kStepWaves * kXGuRows * 64 * 20);   // gate/up codes (16 B) + scale/zero (4 B)
  s.wdn = BT > 1 ? take((size_t)kXNarrowCpl * kStepThreads * 20) : 0;
  s.total = o;
  return s;
}

// Streams this wave's gate/up weight rows straight into LDS (no registers held
// while they are in flight): row i of the wave, lane l takes 32-column chunk l
// (16 bytes of codes at codes + (i*64 + l)*16, its scale/zero word at szw + i*64 + l).
// Rows shorter than 64 chunks (K < 2048): the lanes past the row load its chunk 0
// again, so that every address stays inside the row; the dot product skips them.
// The data is in LDS once this wave's vector-memory count has drained.
__device__ __forceinline__ void wrows_to_lds(const uint8_t* packed, const uint32_t* sz, int K, int lgG,
                                             const int* row, uint4* codes, uint32_t* szw) {
  const int lane = otid() & 63, NG = K >> lgG, cl = 32 * lane < K ? lane : 0;
#pragma unroll
  for (int i = 0; i < kXGuRows; ++i) {
    __builtin_amdgcn_global_load_lds(packed + (size_t)row[i] * (K / 2) + 16 * cl, codes + i * 64, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(sz + (size_t)row[i] * NG + ((32 * cl) >> lgG), szw + i * 64, 4, 0, 0);
  }
}

// NR full rows of K <= 64*32 columns into LDS, one 32-column chunk per lane: row i
// of this wave at codes[i * 64 + lane], its scale/zero word at szw[i * 64 + lane]
// (slots of chunks past K, or of rows without ok, keep stale data: the dot products
// skip the chunks, and such rows are never published).
template <int NR>
__device__ __forceinline__ void wrows_dma(const uint8_t* packed, const uint32_t* sz, int K, int lgG,
                                          const int* row, const bool* ok, uint4* codes, uint32_t* szw) {
  const int lane = otid() & 63, NG = K >> lgG;
#pragma unroll
  for (int i = 0; i < NR; ++i)
    if (ok[i] && 32 * lane < K) {
      __builtin_amdgcn_global_load_lds(packed + (size_t)row[i] * (K / 2) + 16 * lane, codes + i * 64, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(sz + (size_t)row[i] * NG + ((32 * lane) >> lgG), szw + i * 64, 4, 0, 0);
    }
}
template <int NR>
__device__ __forceinline__ void wrows_read(WRows<NR, 1>& w, const uint4* codes, const uint32_t* szw) {
  const int lane = otid() & 63;
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    w.raw[i][0] = codes[i * 64 + lane];
    w.sz[i][0] = szw[i * 64 + lane];
  }
}

__device__ __forceinline__ void wrows_from_lds(WRows<kXGuRows, 1>& w, const uint4* codes, const uint32_t* szw) {
  const int lane = otid() & 63;
#pragma unroll
  for (int i = 0; i < kXGuRows; ++i) {
    w.raw[i][0] = codes[i * 64 + lane];
    w.sz[i][0] = szw[i * 64 + lane];
  }
}

// Matrix-core form of the gate/up product, for K = 2048 columns in quantization
// groups of 128 and 24 act rows per group: the group's 48 weight rows (local row r:
// gate of act row r for r < 24, up of act row r - 24 after) form three 16-row tiles,
// and wave w takes all of them over its 256 columns [256 w, 256 w + 256), two
// groups of four 32-column chunks.  The codes stream into LDS a whole 128-byte line
// per row and load: load i, lane l takes local row 8 i + l / 8, chunk
// 8 w + ((l % 8) ^ (l / 8)), into slot i*64 + l (the XOR with the row's low bits puts
// the 8 rows of one chunk that a tile read takes together in distinct LDS banks).
// The scale/zero words of the wave's 96 (row, group) pairs
// follow in two loads: slot p = 2 r + h holds local row r, group 2 w + h.
// The same tile layout serves the group's 16 q/k/v rows (one tile, T = 1).
constexpr int kGuMfmaK = 2048, kGuMfmaRows = 24;
__host__ __device__ constexpr int gu_zloads(int T) { return (32 * T + 63) / 64; }
// (I0, I1: the code loads issued, [I0, I1) of the 2 T; Z0, Z1 likewise of the
// scale/zero loads: a caller may split the stream in parts)
// (sw: the wave whose column slice is loaded, into that wave's slots codes/szw;
// by default the calling wave)
template <int T = 3, int I0 = 0, int I1 = 2 * T, int Z0 = 0, int Z1 = gu_zloads(T)>
__device__ __forceinline__ void gu_tiles_to_lds(const uint8_t* packed, const uint32_t* sz, int lgG,
                                                const int (&row)[2 * T], const int (&zrow)[gu_zloads(T)],
                                                uint4* codes, uint32_t* szw, int sw = -1) {
  const int lane = otid() & 63, wave = sw < 0 ? otid() >> 6 : sw, NG = kGuMfmaK >> lgG;
#pragma unroll
  for (int i = I0; i < I1; ++i)
    __builtin_amdgcn_global_load_lds(packed + (size_t)row[i] * (kGuMfmaK / 2) + 16 * (8 * wave + ((lane & 7) ^ (lane >> 3))),
                                     codes + i * 64, 16, 0, 0);
#pragma unroll
  for (int u = Z0; u < Z1; ++u)
    __builtin_amdgcn_global_load_lds(sz + (size_t)zrow[u] * NG + ((256 * wave + 128 * (lane & 1)) >> lgG),
                                     szw + u * 64, 4, 0, 0);
}

// This wave's part of the 16 T dot products (the 48 gate/up rows, or the 16 q/k/v
// rows) of each staged row b < B, over its 256 columns, into
// part[(wave * BT + b) * 16 T + local row].  Per tile and group the
// four chunk products go through the matrix cores with the staged rows as the first
// operand (row b of it; lanes of higher rows repeat row 0) and the weight tile as
// the second, so lane n < 16 receives every batch row of weight row n.  The group's
// scale and zero point then apply as in wave_dot_c, s (d - C1) + z C2, with the
// staged constants of row b summed over the group's 16 eight-column words.
template <int BT, int T = 3>
__device__ __forceinline__ void gu_mfma_part(const uint4* codes, const uint32_t* szw, const uint4* xs,
                                             const float* sums, int B, float* part) {
  constexpr int CH = kGuMfmaK / 32, K4 = kGuMfmaK / 4;
  const int lane = otid() & 63, wave = otid() >> 6, n = lane & 15, gq = lane >> 4;
  const int bn = (BT > 1 && n < B) ? n : 0;
  // The group constants of every staged row b over this wave's two groups, from one
  // LDS read per lane: lane l takes float l of the row's 64 per-word sums of the
  // wave's 256 columns (group h = l / 32; the word's sum of h if l is even, of the
  // used values if odd), and the 16 lanes of one parity in each 32-lane half are
  // added (lane ^ 2, ^ 4, ^ 8, ^ 16).  Wave-uniform results.
  float C1[BT][2], C2[BT][2];
#pragma unroll
  for (int b = 0; b < BT; ++b) {
    float v = (BT == 1 || b < B) ? sums[b * K4 + 64 * wave + lane] : 0.f;
    v += dpp<0x4E>(v);     // lane ^ 2
    v += lane_xor4(v);     // lane ^ 4
    v += row16_swap8(v);   // lane ^ 8
    float lo, hi;
    lane_pair<16>(v, lo, hi);
    v = lo + hi;           // lane ^ 16
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float sh = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32 * h));
      const float su = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32 * h + 1));
      C1[b][h] = __builtin_fmaf(1024.0f, sh, 8.0f * su);
      C2[b][h] = su;
    }
  }
  float acc[T][BT];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int e = 0; e < BT; ++e) acc[t][e] = 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c0 = 8 * wave + 4 * h;
    // every LDS read of this group first: the staged rows, then the three tiles'
    // codes (local row 16 t + n, chunk c0 + gq: load 2 t + n / 8, lane
    // 8 (n % 8) + ((4 h + gq) ^ (n % 8))) and scale/zero words
    uint4 xv[4], cw[T];
    uint32_t zz[T];
#pragma unroll
    for (int q = 0; q < 4; ++q) xv[q] = xs[(bn * 4 + q) * CH + c0 + gq];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      cw[t] = codes[(2 * t + (n >> 3)) * 64 + 8 * (n & 7) + ((4 * h + gq) ^ (n & 7))];
      zz[t] = szw[2 * (16 * t + n) + h];
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      uint32_t p[16];
      dequant16(cw[t], p);
      f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        d = mfma16x16x32(xv[kt], make_uint4(p[4 * kt], p[4 * kt + 1], p[4 * kt + 2], p[4 * kt + 3]), d);
      // lanes n < 16 hold rows b = e of weight row 16 t + n
      const float sc = bf16_lo(zz[t]), zp = bf16_hi(zz[t]);
#pragma unroll
      for (int e = 0; e < BT; ++e) acc[t][e] += __builtin_fmaf(sc, d[e] - C1[e][h], zp * C2[e][h]);
    }
  }
  if (gq == 0) {
#pragma unroll
    for (int e = 0; e < BT; ++e) {
      if (BT > 1 && e >= B) break;
#pragma unroll
      for (int t = 0; t < T; ++t) part[(wave * BT + e) * (16 * T) + 16 * t + n] = acc[t][e];
    }
  }
}

// XCD-local buffer strides (64-bit words per XCD region, 4 KB aligned), and the
// per-row strides of the staged vectors.
struct StepXSizes {
  long long lx, lqkv, lpart, lact, sx, srow_x, srow_a;
};

__host__ __device__ inline long long xalign(long long words) { return (words + 511) & ~511LL; }

__host__ __device__ inline StepXSizes stepx_sizes(int B, int H, int Hkv, int D, int QPG, int I, int M) {
  const int GPX = Hkv / kXcds, NSX = (M + kXSplit - 1) / kXSplit;
  StepXSizes z{};
  const int IX = I / kXcds;
  z.srow_x = ((long long)(H / 2 + H / 4 + kXSsSlots) + 63) & ~63LL;
  z.srow_a = ((long long)(IX / 2 + IX / 4) + 63) & ~63LL;
  z.lx = xalign((long long)B * H);             // fp32 x after the last layer (lm_head input)
  z.sx = xalign((long long)2 * B * z.srow_x);  // staged x: entering the layer, after O
  z.lqkv = xalign((long long)B * GPX * (QPG + 2) * D);
  z.lpart = xalign((long long)B * GPX * NSX * QPG * (D + 2));
  z.lact = xalign((long long)B * z.srow_a);    // staged SiLU(gate)*up
  return z;
}

// Sizes of the Qwen3-VL-2B text decoder on a 256-group grid: an instantiation with
// FIXED set takes them as constants (the host launches it only when they match),
// so that indices and LDS offsets fold at compile time.
constexpr int kFixH = 2048, kFixHkv = 8, kFixI = 6144, kFixLgG = 7, kFixNwg = 256;

template <int BT, int D, int QPG, bool FIXED = false>
__global__ __launch_bounds__(kStepThreads) void k_stepx(const StepArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int DPL = D / 16, HALF = D / 2, PW = QPG * (D + 2);
  const int tid = otid(), lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwg = FIXED ? kFixNwg : (int)gridDim.x, WPX = nwg / kXcds;
  // The group's XCD is read from the hardware, and its index among that XCD's groups
  // is taken from an arrival counter that wraps at WPX.  The dispatcher deals the
  // groups out over the XCDs in turn, but not always starting at XCD 0, so every XCD
  // receives WPX of them and the indices of one launch are a permutation of
  // 0..WPX-1 on each XCD.
  __shared__ int s_xj;
  if (tid == 0) {
    const uint32_t xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 15u;
    const uint32_t k = atomicInc(a.xarr + xcc % kXcds, (unsigned)(WPX - 1));
    if (xcc >= (uint32_t)kXcds || k >= (uint32_t)WPX) raise_status(a.status, kStatusTopology);
    s_xj = (int)(xcc % kXcds) | (int)(k < (uint32_t)WPX ? k : 0u) << 4;
  }
  __syncthreads();
  const int xj = __builtin_amdgcn_readfirstlane(s_xj);
  const int x = xj & 15, j = xj >> 4;
  const int B = BT == 1 ? 1 : a.B;   // (a batch-1 instantiation runs only at B == 1)
  const int H = FIXED ? kFixH : a.H, Hkv = FIXED ? kFixHkv : a.Hkv, Hq = FIXED ? kFixHkv * QPG : a.Hq;
  const int I = FIXED ? kFixI : a.I, M = a.M, lgG = FIXED ? kFixLgG : a.lgG;
  const int GPX = Hkv / kXcds, QX = GPX * (QPG + 2) * D, OX = GPX * QPG * D, IX = I / kXcds;
  const int RPW = (H + WPX - 1) / WPX, RQ = (QX + WPX - 1) / WPX, RA = (IX + WPX - 1) / WPX;
  const int NSX = (M + kXSplit - 1) / kXSplit;
  const int lgGPX = __builtin_ctz((unsigned)GPX);   // GPX: a power of two (checked on the host)
  const int lgOX = __builtin_ctz((unsigned)OX);     // OX = GPX * 2 * D: a power of two too
  const int NSS = WPX * (RPW >= 64 ? RPW >> 6 : 1);   // sums-of-squares slots of a staged row
  const int plain = a.intra_plain;
  const StepXLds Ld = stepx_lds(BT, H, RPW, D, QPG, GPX);
  group_fail_reset();
  __syncthreads();
  uint4* xs = reinterpret_cast<uint4*>(smem + Ld.xs);
  uint4* wdn_raw = reinterpret_cast<uint4*>(smem + Ld.wdn);
  uint32_t* wdn_sz = reinterpret_cast<uint32_t*>(smem + Ld.wdn + (size_t)kXNarrowCpl * kStepThreads * 16);
  float2* cc = reinterpret_cast<float2*>(smem + Ld.cc);
  float* sums = reinterpret_cast<float*>(smem + Ld.sums);
  float* xin = reinterpret_cast<float*>(smem + Ld.xin);
  float* xown = reinterpret_cast<float*>(smem + Ld.xown);
  float2* cs = reinterpret_cast<float2*>(smem + Ld.cs);
  float* red = reinterpret_cast<float*>(smem + Ld.red);
  uint64_t* lx0 = a.lx + (size_t)x * a.x_lx;          // x after the last layer
  uint64_t* sx0 = a.sx + (size_t)x * a.x_sx;          // staged x entering a layer
  uint64_t* sx1 = sx0 + (size_t)B * a.srow_x;         // staged x after the O projection
  const long long SX = a.srow_x, SA = a.srow_a;
  uint64_t* lqkv = a.lqkv + (size_t)x * a.x_lqkv;
  uint64_t* lpart = a.lpart + (size_t)x * a.x_lpart;
  uint64_t* lact = a.lact + (size_t)x * a.x_lact;
  __shared__ int s_last;
  __shared__ int s_c[16];
  __shared__ int s_ns[16];

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

  // ---- step prologue: cache positions, RoPE tables, embedding
  if (tid < B) {
    const int c = a.cpos[tid];
    s_c[tid] = c;
    s_ns[tid] = (c >= 0 && c < M) ? (c + kXSplit) / kXSplit : 0;
    if (blockIdx.x == 0 && (c < 0 || c >= M)) raise_status(a.status, 1u);
  }
  for (int i = tid; i < B * HALF; i += kStepThreads) {
    const int b = i / HALF, jj = i - b * HALF;
    const int ax = mrope_axis(jj, a.sec0, a.sec1, a.sec2, a.interleaved);
    const double p = (double)a.pos[ax * B + b];
    const double inv_freq = pow(a.theta, -2.0 * (double)jj / (double)D);
    double sn, cn;
    sincos(p * inv_freq, &sn, &cn);
    cs[b * HALF + jj] = make_float2((float)cn, (float)sn);
  }
  {
    // embedding rows of this group (B * RPW <= kStepThreads), published staged
    // for the first layer's input norm
    const int b = tid / RPW, r = tid - b * RPW, n = j * RPW + r;
    const bool has = tid < B * RPW && n < H;
    float v = 0.f;
    if (has) {
      const int id = (a.finished && a.finished[b]) ? a.pad_id : a.ids[b];
      const bool ok = id >= 0 && id < a.V;
      if (!ok && n == 0 && x == 0) raise_status(a.status, 2u);
      v = ok ? bf16_to_f32(a.embed[(size_t)id * H + n]) : 0.f;
      xown[b * RPW + r] = v;
    }
    publish_staged_x<BT>(sx0, SX, H, B, RPW, j * RPW, v, has, staged_gain(a.layers[0].in_norm, H, RPW, j * RPW),
                         j, tag(1), plain, a.status);
  }
  __syncthreads();   // cache positions, split counts and RoPE tables are in LDS
  KMR_TRACE_MARK(0);

  // QKV rows of this group: 2 per wave, of the XCD's kv heads (q heads, k, v)
  constexpr int NRQ = 2;
  auto qkv_rows = [&](int (&row)[NRQ], int (&lr)[NRQ], bool (&ok)[NRQ]) {
    const int wv = __builtin_amdgcn_readfirstlane(otid() >> 6);
#pragma unroll
    for (int i = 0; i < NRQ; ++i) {
      const int rr = wv * NRQ + i;
      lr[i] = j * RQ + rr;
      ok[i] = rr < RQ && lr[i] < QX;
      row[i] = 0;
      if (ok[i]) {
        const int gl = lr[i] / ((QPG + 2) * D), t = lr[i] - gl * (QPG + 2) * D, g = x * GPX + gl;
        row[i] = t < QPG * D ? g * QPG * D + t
               : t < (QPG + 1) * D ? Hq * D + g * D + (t - QPG * D)
                                   : Hq * D + Hkv * D + g * D + (t - (QPG + 1) * D);
      }
    }
  };
  // At batch 1 the QKV and down weight rows are requested one phase early, right
  // after the preceding phase's input has arrived: a poll waits for every load
  // its wave issued before it, so rows requested just ahead of a poll would delay
  // it by a memory latency.  (At larger batches the registers held meanwhile cost
  // more than the latency saved.)
  constexpr bool kAhead = BT == 1;
  WRows<NRQ, 1> wq;
  // The QKV rows go through LDS in the constant-size instantiation (the matrix-core
  // tile) and at larger batches (held in registers they would be spilled): the first
  // rows of each wave's gate/up slots, which are free from the end of one layer's
  // gate/up product to the next layer's O phase.
  // wave w's gate/up (and q/k/v tile) slots in LDS
  auto slot_codes = [&](int w) { return reinterpret_cast<uint4*>(smem + Ld.wgu) + w * kXGuRows * 64; };
  auto slot_sz = [&](int w) {
    return reinterpret_cast<uint32_t*>(smem + Ld.wgu + (size_t)kStepWaves * kXGuRows * 64 * 16) + w * kXGuRows * 64;
  };
  uint4* wq_codes = slot_codes(wave);
  uint32_t* wq_sz = slot_sz(wave);
  // In the constant-size form every wave polls the reduce-scatters (at batch 1 wave
  // w takes XCD w's partials of the group's 64 rows), and a poll returns only after
  // every load its wave issued before it.  At batch 1 wave 0, whose lanes then reduce
  // and publish the rows, requests no weights just ahead of those polls; wave
  // kStepWaves / 2 requests wave 0's instead.  That wave's own next poll, a gather
  // that gives every wave words (K = 2048), returns after them, and the gather's
  // closing barrier orders them before any tile read.  (At batch 4, waves 0-3 with
  // waves 4-7 as their proxies measured slower.)
  const bool xrs_poller = FIXED && BT == 1 && wave == 0;
  const int xrs_proxy = FIXED && BT == 1 && wave == kStepWaves / 2 ? 0 : -1;
  static_assert(NRQ <= kXGuRows, "the QKV rows fit the gate/up slots");
  // The constant-size instantiation takes the group's 16 q/k/v rows as one
  // matrix-core tile, in the gate/up tile layout (every row valid: 32 groups of 16
  // rows cover the XCD's 512); its partial sums go to wave 0's gate/up slots past the
  // tile, which nothing else uses before the O phase.
  static_assert(!FIXED || ((kFixHkv / kXcds) * (QPG + 2) * D == 16 * (kFixNwg / kXcds) && kFixH == kGuMfmaK),
                "the constant-size q/k/v rows form one 16-row tile per group over kGuMfmaK columns");
  auto qkv_row_of = [&](int r) {   // weight row of this group's local q/k/v row r
    const int lr2 = j * RQ + r, gl = lr2 / ((QPG + 2) * D), t = lr2 - gl * (QPG + 2) * D, g = x * GPX + gl;
    return t < QPG * D ? g * QPG * D + t
         : t < (QPG + 1) * D ? Hq * D + g * D + (t - QPG * D)
                             : Hq * D + Hkv * D + g * D + (t - (QPG + 1) * D);
  };
  // part 0: every load; in the matrix-core form part 1 is the first 8 rows and the
  // scale/zero words, part 2 the other 8 rows (the other form requests all with part 2)
  auto qkv_request = [&](const StepLayer& L2, auto part) {
    constexpr int P = decltype(part)::value;
    if constexpr (FIXED) {
      int trow[2], zrow[gu_zloads(1)];
#pragma unroll
      for (int i = 0; i < 2; ++i) trow[i] = qkv_row_of(8 * i + (lane >> 3));
      zrow[0] = qkv_row_of(lane < 32 ? lane >> 1 : 0);   // (row, group) pair lane < 32
      if constexpr (P == 0)
        gu_tiles_to_lds<1>(L2.qkv_p, L2.qkv_s, lgG, trow, zrow, wq_codes, wq_sz);
      else if constexpr (P == 1) {
        // (ahead of the reduce-scatter poll: at batch 1 wave 0's share through wave 4)
        if (!xrs_poller) gu_tiles_to_lds<1, 0, 1, 0, 1>(L2.qkv_p, L2.qkv_s, lgG, trow, zrow, wq_codes, wq_sz);
        if (xrs_proxy >= 0)
          gu_tiles_to_lds<1, 0, 1, 0, 1>(L2.qkv_p, L2.qkv_s, lgG, trow, zrow, slot_codes(xrs_proxy),
                                         slot_sz(xrs_proxy), xrs_proxy);
      }
      else
        gu_tiles_to_lds<1, 1, 2, 0, 0>(L2.qkv_p, L2.qkv_s, lgG, trow, zrow, wq_codes, wq_sz);
    } else if constexpr (P != 1) {
      int row[NRQ], lr[NRQ];
      bool ok[NRQ];
      qkv_rows(row, lr, ok);
      if constexpr (kAhead)
        wrows_load(wq, L2.qkv_p, L2.qkv_s, H, lgG, row, ok);
      else
        wrows_dma<NRQ>(L2.qkv_p, L2.qkv_s, H, lgG, row, ok, wq_codes, wq_sz);
    }
  };
  float* qpart = reinterpret_cast<float*>(reinterpret_cast<uint4*>(smem + Ld.wgu) + 2 * 64);
  qkv_request(a.layers[0], std::integral_constant<int, 0>());

  for (int l = 0; l < a.L && alive; ++l) {
    const StepLayer& Ly = a.layers[l];
    const int ph = 1 + 6 * l;   // tags: ph x (sx0), +1 qkv, +2 partials, +3 O partials,
                                // +4 x after O (sx1), +5 act, +6 down partials and next x
    [[maybe_unused]] const int tev = l < 5 ? 1 + 11 * l : 64;
    uint16_t* kc = a.kc + (size_t)l * a.cacheB * Hkv * M * D;
    uint16_t* vc = a.vc + (size_t)l * a.cacheB * Hkv * M * D;
    int total = 0;
    for (int b = 0; b < B; ++b) total += GPX * s_ns[b];
    uint32_t kr[DPL / 2][4], vr[4][DPL / 2];
    // ================= QKV rows of this XCD's kv heads: RQ rows per group, 2 per wave
    {
      constexpr int NR = NRQ;
      int row[NR], lr[NR];
      bool ok[NR];
      qkv_rows(row, lr, ok);
      if (!gather_staged<BT, 4 * BT>(sx0, SX, H, B, NSS, ctag(ph), xs, sums, lim)) {
        alive = false;
        break;
      }
      // (each lane reads the slots its own wave's DMA wrote, complete once its gather
      // poll has returned; in the matrix-core form the gather's closing barrier makes
      // every wave's slots visible)
      if constexpr (!kAhead && !FIXED) wrows_read<NR>(wq, wq_codes, wq_sz);
      KMR_TRACE_MARK(tev + 0);
      // at batch 1 the K rows of the first attention item are requested now, to be
      // in flight during the QKV rows and their hand-off (the QKV rows, requested a
      // phase ago, are settled first); the V rows follow the q/k/v rows' publish
      // (a wave issues no further instruction until its loads are accepted, so all
      // 64 KB here would hold back the item groups' q/k/v rows, the hand-off's last)
      if constexpr (kAhead) {
        if constexpr (!FIXED) {
#pragma unroll
          for (int i = 0; i < NR; ++i) {
            settle(wq.raw[i][0]);
            settle(wq.sz[i][0]);
          }
        }
        if (j < total) attn_load_kv<DPL, true, false>(kr, vr, kc, vc, j, s_ns, s_c, GPX, x, Hkv, M, D, wave);
      }
      if constexpr (FIXED) {
        // wave partials [8][BT][16], then wave b sums batch row b's 16 rows
        gu_mfma_part<BT, 1>(wq_codes, wq_sz, xs, sums, B, qpart);
        __syncthreads();
        if (wave < B) {
          const float inv = staged_inv(sums + BT * (H / 4), wave, NSS, H, a.eps);
          if (lane < 16) {
            float v = 0.f, pq[kStepWaves];   // (read first, then summed in wave order)
#pragma unroll
            for (int w = 0; w < kStepWaves; ++w) pq[w] = qpart[(w * BT + wave) * 16 + lane];
#pragma unroll
            for (int w = 0; w < kStepWaves; ++w) v += pq[w];
            publish_l(lqkv + (size_t)wave * QX + j * RQ + lane, tag(ph + 1), v * inv, plain);
          }
        }
        if constexpr (BT == 1) {
          // A group without an attention item requests its gate/up tiles now, into
          // slots nothing reads before the gate/up product: the weights then arrive
          // while the items run, when HBM is otherwise idle, and no later poll of
          // this group waits behind them.  The wait first lets the item groups' K/V
          // rows and q/k/v hand-off go ahead of the stream.
          if (j >= total) {
            for (int k = 0; k < kEarlyGuSleeps; ++k) __builtin_amdgcn_s_sleep(8);
            auto grow_e = [&](int r) {   // as grow_of in the gate/up phase
              const int ar = r < kGuMfmaRows ? r : r - kGuMfmaRows;
              return x * IX + j * kGuMfmaRows + ar + (r < kGuMfmaRows ? 0 : I);
            };
            int trow_e[kXGuRows], zrow_e[2];
#pragma unroll
            for (int i = 0; i < kXGuRows; ++i) trow_e[i] = grow_e(8 * i + (lane >> 3));
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int p = 64 * u + lane;
              zrow_e[u] = grow_e(p < 96 ? p >> 1 : 0);
            }
            gu_tiles_to_lds<3>(Ly.gu_p, Ly.gu_s, lgG, trow_e, zrow_e, slot_codes(wave), slot_sz(wave));
          }
        }
      } else {
        float out[NR][BT];
        wave_dot_c<BT, NR, 1>(wq, H, B, xs, ChunkSums{sums, H / 4}, out);
        const float inv = row_inv<BT>(sums + BT * (H / 4), B, NSS, H, a.eps);
        if (lane < B) {
#pragma unroll
          for (int i = 0; i < NR; ++i)
            if (ok[i]) {
              float v = out[i][0];
#pragma unroll
              for (int b = 1; b < BT; ++b) if (lane == b) v = out[i][b];
              publish_l(lqkv + (size_t)lane * QX + lr[i], tag(ph + 1), v * inv, plain);
            }
        }
      }
    }
    // K/V rows (at batch 1 the V rows) of this group's first attention item:
    // requested right after its q/k/v rows are out, so that their latency overlaps
    // the hand-off
    asm volatile("" ::: "memory");   // not ahead of the q/k/v stores
    if constexpr (!kAhead) {
      if (j < total) attn_load_kv<DPL>(kr, vr, kc, vc, j, s_ns, s_c, GPX, x, Hkv, M, D, wave);
    } else {
      if (j < total) attn_load_kv<DPL, false, true>(kr, vr, kc, vc, j, s_ns, s_c, GPX, x, Hkv, M, D, wave);
    }
    KMR_TRACE_MARK(tev + 1);
    // O and down rows of this lane group (at larger batches recomputed where used:
    // held across the attention they would be spilled)
    const int orow_l = j * RPW + wave * 8 + (lane >> 3);
    const bool ook_l = wave * 8 + (lane >> 3) < RPW && orow_l < H;
    auto orow_at = [&]() { return kAhead ? orow_l : j * RPW + wave * 8 + ((otid() & 63) >> 3); };
    auto ook_at = [&](int r) { return kAhead ? ook_l : (r - j * RPW < RPW && r < H); };
    // ================= attention items (row, local kv head, split) of this XCD
    {
      for (int item = j; item < total; item += WPX) {
        if (item != j) attn_load_kv<DPL>(kr, vr, kc, vc, item, s_ns, s_c, GPX, x, Hkv, M, D, wave);
        int b, gl, s;
        xitem(item, s_ns, GPX, b, gl, s);
        const int ns = s_ns[b], g = x * GPX + gl, c = s_c[b];
        const int rr = lane >> 4, li = lane & 15, row = wave * 4 + rr, d0 = li * DPL;
        const size_t head_base = ((size_t)b * Hkv + g) * M;

        // the q/k norm gains of this wave's head, requested ahead of the poll so that
        // they are in registers when the q/k/v rows arrive
        uint16_t gn0 = 0, gn1 = 0;
        if (wave <= QPG && lane < HALF) {
          const uint16_t* gn = wave < QPG ? Ly.q_norm : Ly.k_norm;
          gn0 = gn[lane];
          gn1 = gn[lane + HALF];
        }
        // q heads of kv head g (contiguous), then k, then v: one gather
        float* qv = xin;
        float* s_w = xin + (QPG + 2) * D;                  // [8 waves][QPG][D + 2], after q/k/v
        float* s_e = s_w + kStepWaves * QPG * (D + 2);     // [8][QPG] weights, [QPG] max, [QPG] sum
        uint16_t* qb = reinterpret_cast<uint16_t*>(xin + xattn_qb(D, QPG));   // [2 QPG][D] q splits
        {
          auto addr = [](int i) { return (size_t)i; };
          auto place = [](int i) { return i; };
          if (!gather_tagged<(QPG + 2) * D / kStepThreads + 1>(
                  lqkv + (size_t)b * QX + (size_t)gl * (QPG + 2) * D, (QPG + 2) * D, ctag(ph + 1), qv,
                  addr, place, NoPre(), lim)) {
            alive = false;
            break;
          }
        }
        KMR_TRACE_MARK(tev + 2);
        // per-head RMSNorm + RoPE of the q heads and k, and bf16 rounding of k and
        // v, once per group: wave h takes head h (q heads, then k, then v), lane l
        // the rotate-half pair of dims (l, l + D/2), in place in LDS; q head h also as
        // its bf16 high parts (row 2 h of qb) and low parts (row 2 h + 1)
        if (wave <= QPG + 1) {
          float* hv = qv + wave * D;
          const bool act = lane < HALF;
          float x0 = act ? hv[lane] : 0.f, x1 = act ? hv[lane + HALF] : 0.f;
          if (wave <= QPG) {
            const float ss = wave_sum(x0 * x0 + x1 * x1);
            const float inv = rsqrt_f(ss / (float)D + a.eps);
            if (act) {
              const float y0 = (x0 * inv) * bf16_to_f32(gn0);
              const float y1 = (x1 * inv) * bf16_to_f32(gn1);
              const float2 t = cs[b * HALF + lane];
              x0 = y0 * t.x - y1 * t.y;
              x1 = y1 * t.x + y0 * t.y;
            }
          }
          if (wave >= QPG && act) {
            x0 = round_bf16(x0);
            x1 = round_bf16(x1);
          }
          if (act) {
            hv[lane] = x0;
            hv[lane + HALF] = x1;
          }
          if (wave < QPG && act) {
            uint32_t hi, lo;
            split_bf16x2(x0, x1, hi, lo);
            qb[2 * wave * D + lane] = (uint16_t)hi;
            qb[2 * wave * D + lane + HALF] = (uint16_t)(hi >> 16);
            qb[(2 * wave + 1) * D + lane] = (uint16_t)lo;
            qb[(2 * wave + 1) * D + lane + HALF] = (uint16_t)(lo >> 16);
          }
        }
        __syncthreads();
        // the new slot's k and v: bf16 values held as fp32 in LDS
        const float* nk = qv + QPG * D;
        const float* nv = qv + (QPG + 1) * D;
        auto bf16_pair = [](float lo, float hi) {   // (both already bf16 values)
          return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
        };
        KMR_TRACE_MARK(l == 1 ? 59 : 64);
        if (s == ns - 1 && row == 0) {
          // the new slot's k and v into the cache: nk and nv hold bf16 values as fp32,
          // so each value's bf16 bits are its high half (two vector LDS reads and one
          // store per tensor and lane, DPL dims at d0)
          uint16_t* kd = kc + (head_base + c) * D + d0;
          uint16_t* vd = vc + (head_base + c) * D + d0;
          const float4* nk4 = reinterpret_cast<const float4*>(nk + d0);
          const float4* nv4 = reinterpret_cast<const float4*>(nv + d0);
          if constexpr (DPL == 8) {
            const float4 k0 = nk4[0], k1 = nk4[1], v0 = nv4[0], v1 = nv4[1];
            *reinterpret_cast<uint4*>(kd) = make_uint4(bf16_pair(k0.x, k0.y), bf16_pair(k0.z, k0.w),
                                                       bf16_pair(k1.x, k1.y), bf16_pair(k1.z, k1.w));
            *reinterpret_cast<uint4*>(vd) = make_uint4(bf16_pair(v0.x, v0.y), bf16_pair(v0.z, v0.w),
                                                       bf16_pair(v1.x, v1.y), bf16_pair(v1.z, v1.w));
          } else {
            const float4 k0 = nk4[0], v0 = nv4[0];
            *reinterpret_cast<uint2*>(kd) = make_uint2(bf16_pair(k0.x, k0.y), bf16_pair(k0.z, k0.w));
            *reinterpret_cast<uint2*>(vd) = make_uint2(bf16_pair(v0.x, v0.y), bf16_pair(v0.z, v0.w));
          }
        }
        // The wave's 16 positions p0 + 0..15 on the matrix cores.  Scores S = K Q^T: K rows
        // are the first operand (lane (rr, li) supplies position p0 + li), the second is
        // the columns (q_0 high, q_0 low, q_1 high, q_1 low) of the q heads' bf16 splits
        // (lanes of columns 4..15 repeat them; those columns are never read), and lane
        // (rr, li) receives column li at positions p0 + 4 rr + e.
        const int p0 = s * kXSplit + 16 * wave;
        if (p0 + li == c) {
#pragma unroll
          for (int t = 0; t < DPL / 2; ++t)
#pragma unroll
            for (int w = 0; w < 4; ++w)
              kr[t][w] = bf16_pair(nk[32 * t + 8 * rr + 2 * w], nk[32 * t + 8 * rr + 2 * w + 1]);
        }
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < DPL / 2; ++t) {
          const uint4 bq = *reinterpret_cast<const uint4*>(qb + (li & 3) * D + 32 * t + 8 * rr);
          sacc = mfma16x16x32_bf16(make_uint4(kr[t][0], kr[t][1], kr[t][2], kr[t][3]), bq, sacc);
        }
        // head li / 2 (li < 4): high + low products, in log2 units; -inf past the cache
        // position.  Then the wave's state per head: the max over its 16 positions, the
        // weights relative to it and their sum (rows added (0 + 1) + (2 + 3)).
        float sc[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float t = (sacc[e] + dpp<0xB1>(sacc[e])) * a.scale_log2;
          sc[e] = p0 + 4 * rr + e <= c ? t : -INFINITY;
        }
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        {
          float lo, hi;
          lane_pair<16>(mx, lo, hi);
          mx = fmaxf(lo, hi);
          lane_pair<32>(mx, lo, hi);
          mx = fmaxf(lo, hi);
        }
        float pe[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[e] = sc[e] != -INFINITY ? exp2_fast(sc[e] - mx) : 0.f;
        float ls = (pe[0] + pe[1]) + (pe[2] + pe[3]);
        {
          float lo, hi;
          lane_pair<16>(ls, lo, hi);
          ls = lo + hi;
          lane_pair<32>(ls, lo, hi);
          ls = lo + hi;
        }
        // O = P V: the weights' bf16 splits are the first operand (row 2 h: head h's high
        // parts, row 2 h + 1: the low parts; lane (rr, li) supplies row li at positions
        // p0 + 4 rr + e), V the second (product dt: lane (rr, li) supplies dim DPL li + dt
        // of those positions), and lanes 0..15 receive rows 0..3 at their DPL dims.
        uint32_t wh[2], wl[2];
        split_bf16x2(pe[0], pe[1], wh[0], wl[0]);
        split_bf16x2(pe[2], pe[3], wh[1], wl[1]);
        const uint2 pa = (li & 1) ? make_uint2(wl[0], wl[1]) : make_uint2(wh[0], wh[1]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (p0 + 4 * rr + e == c) {
#pragma unroll
            for (int w = 0; w < DPL / 2; ++w) vr[e][w] = bf16_pair(nv[d0 + 2 * w], nv[d0 + 2 * w + 1]);
          }
        float m[QPG], lsum[QPG], o[QPG][DPL];
#pragma unroll
        for (int dt = 0; dt < DPL; ++dt) {
          const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;   // dim dt of each position pair
          const uint2 bv = make_uint2(__builtin_amdgcn_perm(vr[1][dt >> 1], vr[0][dt >> 1], sel),
                                      __builtin_amdgcn_perm(vr[3][dt >> 1], vr[2][dt >> 1], sel));
          const f32x4_t od = mfma16x16x16_bf16(pa, bv, f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int h = 0; h < QPG; ++h) o[h][dt] = od[2 * h] + od[2 * h + 1];
        }
#pragma unroll
        for (int h = 0; h < QPG; ++h) {
          m[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mx), 2 * h));
          lsum[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ls), 2 * h));
        }
        KMR_TRACE_MARK(l == 1 ? 60 : 64);
        KMR_TRACE_MARK(l == 1 ? 61 : 64);
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
        // Merge the 8 wave states of each head: log-sum-exp weights e = 2^(m - max m),
        // then each output is 8 multiply-adds in wave order and the sum of the weighted
        // sums is taken pairwise (products and sums without contraction, so that both
        // forms below give the same bits).
        uint64_t* pdst = lpart + (((size_t)b * GPX + gl) * NSX + s) * PW;
        if constexpr (BT == 1) {
          // every publishing thread takes the weights of its head's 8 states itself: no
          // one-wave step and no second barrier
          KMR_TRACE_MARK(l == 1 ? 62 : 64);
          for (int i = tid; i < QPG * D; i += kStepThreads) {
            const int h = i / D, d = i - h * D;
            float mw[kStepWaves], lw[kStepWaves], ow[kStepWaves];
#pragma unroll
            for (int wv = 0; wv < kStepWaves; ++wv) {
              const float* st = s_w + (wv * QPG + h) * (D + 2);
              ow[wv] = st[d];
              mw[wv] = st[D];
              lw[wv] = st[D + 1];
            }
            float Mx = mw[0];
#pragma unroll
            for (int wv = 1; wv < kStepWaves; ++wv) Mx = fmaxf(Mx, mw[wv]);
            float e[kStepWaves];
#pragma unroll
            for (int wv = 0; wv < kStepWaves; ++wv) e[wv] = mw[wv] == -INFINITY ? 0.f : exp2_fast(mw[wv] - Mx);
            float Os = 0.f;
#pragma unroll
            for (int wv = 0; wv < kStepWaves; ++wv) Os = __builtin_fmaf(e[wv], ow[wv], Os);
            publish_l(pdst + h * (D + 2) + d, tag(ph + 2), Os, plain);
            if (d == 0) {
#pragma clang fp contract(off)
              float pl[kStepWaves];
#pragma unroll
              for (int wv = 0; wv < kStepWaves; ++wv) pl[wv] = e[wv] * lw[wv];
              const float Ls = ((pl[0] + pl[1]) + (pl[2] + pl[3])) + ((pl[4] + pl[5]) + (pl[6] + pl[7]));
              publish_l(pdst + h * (D + 2) + D, tag(ph + 2), Mx, plain);
              publish_l(pdst + h * (D + 2) + D + 1, tag(ph + 2), Ls, plain);
            }
          }
        } else {
          // the weights once per (wave, head) in one wave, through LDS to every thread
          static_assert(kStepWaves * QPG == 16, "one 16-lane row holds every (wave, head) state");
          if (wave == 0 && lane < 16) {
#pragma clang fp contract(off)
            // lane t = wave * QPG + head: the states of one head sit at lane ^ 2, ^ 4, ^ 8
            const float mw = s_w[lane * (D + 2) + D], lw = s_w[lane * (D + 2) + D + 1];
            float Mx = mw;
            Mx = fmaxf(Mx, dpp<0x4E>(Mx));        // lane ^ 2
            Mx = fmaxf(Mx, lane_xor4(Mx));        // lane ^ 4
            Mx = fmaxf(Mx, row16_swap8(Mx));      // lane ^ 8
            const float e = mw == -INFINITY ? 0.f : exp2_fast(mw - Mx);
            float Ls = e * lw;
            Ls += dpp<0x4E>(Ls);
            Ls += lane_xor4(Ls);
            Ls += row16_swap8(Ls);
            s_e[lane] = e;
            if (lane < QPG) {
              s_e[kStepWaves * QPG + lane] = Mx;
              s_e[(kStepWaves + 1) * QPG + lane] = Ls;
            }
          }
          __syncthreads();
          KMR_TRACE_MARK(l == 1 ? 62 : 64);
          for (int i = tid; i < QPG * D; i += kStepThreads) {
            const int h = i / D, d = i - h * D;
            float Os = 0.f, ow[kStepWaves];
#pragma unroll
            for (int wv = 0; wv < kStepWaves; ++wv) ow[wv] = s_w[(wv * QPG + h) * (D + 2) + d];
#pragma unroll
            for (int wv = 0; wv < kStepWaves; ++wv) Os = __builtin_fmaf(s_e[wv * QPG + h], ow[wv], Os);
            publish_l(pdst + h * (D + 2) + d, tag(ph + 2), Os, plain);
            if (d == 0) {
              publish_l(pdst + h * (D + 2) + D, tag(ph + 2), s_e[kStepWaves * QPG + h], plain);
              publish_l(pdst + h * (D + 2) + D + 1, tag(ph + 2), s_e[(kStepWaves + 1) * QPG + h], plain);
            }
          }
        }
        __syncthreads();
      }
      // (a failed gather leaves the item loop in every thread; the barrier keeps the
      // group's waves together ahead of the merge, which measured faster)
      __syncthreads();
      if (!alive) break;
    }
    KMR_TRACE_MARK(tev + 3);
    // O weights of this group (rows j*RPW + 8 wave + lane/8, the XCD's head columns),
    // in flight while the partials are gathered
    WNarrow wo;
    {
      const int orow = orow_at();
      const bool ook = ook_at(orow);
      wnarrow_load(wo, Ly.o_p, Ly.o_s, Hq * D, lgG, x * OX, OX, ook ? orow : 0, ook);
    }
    // ================= merge every split of the XCD's heads; o -> staged O input
    {
      constexpr int PTM = BT;   // B * OX <= 512 * BT (OX <= 512, checked on the host)
      float mM[PTM], mL[PTM], mO[PTM];
#pragma unroll
      for (int q = 0; q < PTM; ++q) { mM[q] = -INFINITY; mL[q] = 0.f; mO[q] = 0.f; }
      int maxns = 0;
      for (int b = 0; b < B; ++b) maxns = s_ns[b] > maxns ? s_ns[b] : maxns;
      const int CW = kXMergeChunk * PW, words = B * GPX * CW;
      // (at batch 1 the row's split count in a register, read once, not once per
      // poll word)
      const int ns1 = s_ns[0];
      auto ns_of = [&](int bb) { return BT == 1 ? ns1 : s_ns[bb]; };
      for (int t0 = 0; t0 < maxns && alive; t0 += kXMergeChunk) {
        constexpr int PG = 8;
        bool ok = true;
        for (int base = 0; base < words && ok; base += kStepThreads * PG) {
          uint64_t v[PG];
          uint32_t off[PG];
          bool hv[PG];
#pragma unroll
          for (int q = 0; q < PG; ++q) {
            const int i = base + kStepThreads * q + tid;
            const int seg = i / CW, r1 = i - seg * CW, sl = r1 / PW, k = r1 - sl * PW;
            hv[q] = i < words && t0 + sl < ns_of(seg >> lgGPX);
            off[q] = hv[q] ? (uint32_t)((seg * NSX + t0 + sl) * PW + k) : 0u;
          }
          uint32_t spins = 0;
          bool fresh;
          do {
#pragma unroll
            for (int q = 0; q < PG; ++q)
              if (hv[q]) v[q] = ld_dev64(lpart + off[q]);
            fresh = true;
#pragma unroll
            for (int q = 0; q < PG; ++q)
              if (hv[q]) fresh &= (uint32_t)(v[q] >> 32) == ctag(ph + 2);
            if (!fresh) {
              if (++spins > lim) { ok = false; break; }
              __builtin_amdgcn_s_sleep(KMR_POLL_SLEEP);
            }
          } while (!fresh);
#pragma unroll
          for (int q = 0; q < PG; ++q) {
            const int i = base + kStepThreads * q + tid;
            if (hv[q]) xin[i] = __uint_as_float((uint32_t)v[q]);
          }
        }
        if (group_failed(!ok)) { alive = false; break; }
        // log-sum-exp weights of this chunk's splits, once per (row, kv head, q head)
        float* s_wt = xin + words;   // [B*GPX][QPG][kXMergeChunk + 2]: weights, max, sum
        static_assert(kXMergeChunk == 8, "one 8-lane group per (row, kv head, q head)");
        if (wave == 0) {
          // lane = 8 * (seg * QPG + h) + t: split t of the chunk (B * GPX * QPG <= 8, host-checked)
          const int sh = lane >> 3, t = lane & 7, seg = sh / QPG, h = sh - seg * QPG;
          const bool live = seg < B * GPX;
          const int n = live ? (s_ns[seg >> lgGPX] - t0 < kXMergeChunk ? s_ns[seg >> lgGPX] - t0 : kXMergeChunk) : 0;
          const float* pt = xin + ((size_t)seg * kXMergeChunk + t) * PW + h * (D + 2);
          const float mt = t < n ? pt[D] : -INFINITY, lt = t < n ? pt[D + 1] : 0.f;
          float Mc = mt;
          Mc = fmaxf(Mc, dpp<0xB1>(Mc));   // lane ^ 1
          Mc = fmaxf(Mc, dpp<0x4E>(Mc));   // lane ^ 2
          Mc = fmaxf(Mc, lane_xor4(Mc));   // lane ^ 4
          const float e = mt == -INFINITY ? 0.f : exp2_fast(mt - Mc);
          float Lc = e * lt;
          Lc += dpp<0xB1>(Lc);
          Lc += dpp<0x4E>(Lc);
          Lc += lane_xor4(Lc);
          if (live) {
            float* wt = s_wt + sh * (kXMergeChunk + 2);
            wt[t] = e;
            if (t == 0) {
              wt[kXMergeChunk] = Mc;
              wt[kXMergeChunk + 1] = Lc;
            }
          }
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < PTM; ++q) {
          const int idx = kStepThreads * q + tid;
          if (idx >= B * OX) continue;
          const int b = idx >> lgOX, k = idx & (OX - 1), gl = k / (QPG * D), hd = k - gl * QPG * D;
          const int h = hd / D, d = hd - h * D, seg = b * GPX + gl;
          const int n = s_ns[b] - t0 < kXMergeChunk ? s_ns[b] - t0 : kXMergeChunk;
          if (n <= 0) continue;
          const float* wt = s_wt + (seg * QPG + h) * (kXMergeChunk + 2);
          float Oc = 0.f;
          for (int t = 0; t < n; ++t) Oc += wt[t] * xin[((size_t)seg * kXMergeChunk + t) * PW + h * (D + 2) + d];
          lse_merge(mM[q], mL[q], &mO[q], wt[kXMergeChunk], wt[kXMergeChunk + 1], &Oc, 1);
        }
        __syncthreads();   // xin is rewritten by the next chunk, xs by the staging below
      }
      if (!alive) break;
      float e[PTM];
      int eb[PTM], ek[PTM];
      bool has[PTM];
#pragma unroll
      for (int q = 0; q < PTM; ++q) {
        const int idx = kStepThreads * q + tid;
        has[q] = idx < B * OX;
        eb[q] = has[q] ? idx >> lgOX : 0;
        ek[q] = idx - eb[q] * OX;
        e[q] = (has[q] && mL[q] > 0.f) ? mO[q] * (1.0f / mL[q]) : 0.f;
      }
      if (stage_values<PTM>(e, has, eb, ek, OX, xs, cc)) raise_status(a.status, kStatusRange);
      __syncthreads();
    }
    KMR_TRACE_MARK(tev + 4);
    // ================= O split-K partial of this group's rows over the XCD's heads
    {
      float out[BT];
      narrow_dot<BT>(wo, OX, B, xs, ChunkCC{cc, OX >> 5}, out);
      const int sub = lane & 7;
      const int orow = orow_at();
      if (ook_at(orow) && sub < B) {
        float v = out[0];
#pragma unroll
        for (int b = 1; b < BT; ++b) if (sub == b) v = out[b];
        publish(a.pO + ((size_t)x * B + sub) * H + orow, tag(ph + 3), v);
      }
    }
    KMR_TRACE_MARK(tev + 5);
    // gate/up weights of this group (act rows j*RA + 3 wave + i of the XCD's slice)
    constexpr int NP = 3;
    int grow[2 * NP], gla[NP];
    bool gok[2 * NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int la = wave * NP + i;
      gla[i] = j * RA + la;
      gok[i] = gok[NP + i] = la < RA && gla[i] < IX;
      grow[i] = gok[i] ? x * IX + gla[i] : 0;
      grow[NP + i] = gok[i] ? x * IX + gla[i] + I : 0;
    }
    const uint16_t g_post = staged_gain(Ly.post_norm, H, RPW, j * RPW);
    // (K = H = 64 chunks of 32 columns: one chunk per lane, checked on the host)
    uint4* gu_codes = reinterpret_cast<uint4*>(smem + Ld.wgu) + wave * kXGuRows * 64;
    uint32_t* gu_sz = reinterpret_cast<uint32_t*>(smem + Ld.wgu + (size_t)kStepWaves * kXGuRows * 64 * 16) +
                      wave * kXGuRows * 64;
    // matrix-core tiles: local row 16 t + lane % 16 of the group's gate/up rows
    auto grow_of = [&](int r) {   // weight row of local row r (gate rows, then up rows)
      const int ar = r < kGuMfmaRows ? r : r - kGuMfmaRows;
      return x * IX + j * kGuMfmaRows + ar + (r < kGuMfmaRows ? 0 : I);
    };
    int trow[kXGuRows], zrow[2];
    if constexpr (FIXED) {
#pragma unroll
      for (int i = 0; i < kXGuRows; ++i) trow[i] = grow_of(8 * i + (lane >> 3));
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = 64 * u + lane;   // (row, group) pair p < 96; the rest repeat pair 0
        zrow[u] = grow_of(p < 96 ? p >> 1 : 0);
      }
      // (the first half now, the rest once the reduce-scatter poll is in: a poll
      // returns only after every load its wave issued before it; at batch 1 wave 0's
      // through wave 4, and none here for a group that requested them early)
      const bool early = BT == 1 && j >= total;   // (requested after the q/k/v publish)
      if (!xrs_poller && !early) gu_tiles_to_lds<3, 0, 3, 0, 1>(Ly.gu_p, Ly.gu_s, lgG, trow, zrow, gu_codes, gu_sz);
      if (xrs_proxy >= 0 && !early)
        gu_tiles_to_lds<3, 0, 3, 0, 1>(Ly.gu_p, Ly.gu_s, lgG, trow, zrow, slot_codes(xrs_proxy),
                                       slot_sz(xrs_proxy), xrs_proxy);
    } else {
      wrows_to_lds(Ly.gu_p, Ly.gu_s, H, lgG, grow, gu_codes, gu_sz);
    }
    // ================= RS_O: x rows after O, published staged for post_norm
    {
      float xn;
      bool hx;
      if (!reduce_rows<BT>(a.pO, ctag(ph + 3), B, H, RPW, j * RPW, xown, xin, xn, hx, lim)) {
        alive = false;
        break;
      }
      if constexpr (FIXED) {
        if (!(BT == 1 && j >= total))
          gu_tiles_to_lds<3, 3, 6, 1, 2>(Ly.gu_p, Ly.gu_s, lgG, trow, zrow, gu_codes, gu_sz);
      }
      publish_staged_x<BT>(sx1, SX, H, B, RPW, j * RPW, xn, hx, g_post, j, tag(ph + 4), plain, a.status);
    }
    KMR_TRACE_MARK(tev + 6);
    // ================= gate-up + SiLU over the XCD's slice
    WNarrow wd;
    uint16_t g_next;
    {
      if (!gather_staged<BT, 4 * BT>(sx1, SX, H, B, NSS, ctag(ph + 4), xs, sums, lim)) {
        alive = false;
        break;
      }
      KMR_TRACE_MARK(tev + 7);
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's gate/up rows are in LDS
      // the down weights, requested now so that they have arrived before the act
      // gather polls (at larger batches into LDS: held in registers across the
      // gate/up product they would be spilled)
      {
        const int orow = orow_at();
        const bool ook = ook_at(orow);
        if constexpr (kAhead)
          wnarrow_load(wd, Ly.d_p, Ly.d_s, I, lgG, x * IX, IX, ook ? orow : 0, ook);
        else
          wnarrow_to_lds(Ly.d_p, Ly.d_s, I, lgG, x * IX, IX, ook ? orow : 0, ook, wdn_raw, wdn_sz);
        g_next = staged_gain(a.layers[l + 1 < a.L ? l + 1 : l].in_norm, H, RPW, j * RPW);
      }
      if constexpr (FIXED) {
        // wave partials [8][BT][48] in LDS, then wave b sums batch row b's act rows
        float* part = xin;
        gu_mfma_part<BT>(gu_codes, gu_sz, xs, sums, B, part);
        __syncthreads();
        if (wave < B) {
          const float inv = staged_inv(sums + BT * (H / 4), wave, NSS, H, a.eps);
          const bool has = lane < kGuMfmaRows;
          float gt = 0.f, up = 0.f;
          if (has) {
            // (every wave's partials read first, then summed in wave order)
            float pg[kStepWaves], pu[kStepWaves];
#pragma unroll
            for (int w = 0; w < kStepWaves; ++w) {
              pg[w] = part[(w * BT + wave) * 48 + lane];
              pu[w] = part[(w * BT + wave) * 48 + kGuMfmaRows + lane];
            }
#pragma unroll
            for (int w = 0; w < kStepWaves; ++w) {
              gt += pg[w];
              up += pu[w];
            }
          }
          gt *= inv;
          up *= inv;
          // SiLU(gate) * up with the hardware exp and reciprocal (a few ulp)
          // (staged scaled by kStageScale: the down product multiplies back)
          const float act = has ? gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * (up * kStageScale) : 0.f;
          stage_range_check(act, a.status);
          stage_publish(lact + (size_t)wave * SA, IX, j * kGuMfmaRows + lane, act, has, tag(ph + 5), plain);
        }
      } else {
        float out[2 * NP][BT];
        WRows<2 * NP, 1> wgu;
        wrows_from_lds(wgu, gu_codes, gu_sz);
        wave_dot_c<BT, 2 * NP, 1>(wgu, H, B, xs, ChunkSums{sums, H / 4}, out);
        const float inv = row_inv<BT>(sums + BT * (H / 4), B, NSS, H, a.eps);
        // act values of this group into LDS [b][32], then published staged
        float* s_act = xin;
        if (lane < B) {
#pragma unroll
          for (int i = 0; i < NP; ++i) {
            float gt = out[i][0], up = out[NP + i][0];
#pragma unroll
            for (int b = 1; b < BT; ++b) if (lane == b) { gt = out[i][b]; up = out[NP + i][b]; }
            gt *= inv;
            up *= inv;
            // SiLU(gate) * up with the hardware exp and reciprocal (a few ulp), staged
            // scaled by kStageScale (the down product multiplies back)
            if (gok[i])
              s_act[(kAhead ? lane : (otid() & 63)) * 32 + wave * NP + i] =
                  gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * (up * kStageScale);
          }
        }
        __syncthreads();
        {
          const int b = tid >> 5, t = tid & 31;
          const bool has = b < B && t < RA && j * RA + t < IX;
          const float av = has ? s_act[tid] : 0.f;
          stage_range_check(av, a.status);
          stage_publish(lact + (size_t)(has ? b : 0) * SA, IX, j * RA + t, av, has, tag(ph + 5), plain);
        }
      }
      // (s_act in xin is next rewritten by the down reduce-scatter, after the
      // barrier of the act gather)
    }
    KMR_TRACE_MARK(tev + 8);
    // ================= down split-K over the XCD's slice, then RS_D
    {
      if (!gather_staged<BT, 4 * BT>(lact, SA, IX, B, 0, ctag(ph + 5), xs, sums, lim)) {
        alive = false;
        break;
      }
      settle(g_next);
      KMR_TRACE_MARK(tev + 9);
      // (each lane reads the slots its own wave's DMA wrote, complete once its gather
      // poll has returned)
      if constexpr (!kAhead) wnarrow_from_lds(wd, wdn_raw, wdn_sz);
      float out[BT];
      narrow_dot<BT>(wd, IX, B, xs, ChunkSums{sums, IX / 4}, out);
      const int sub = lane & 7;
      const int orow = orow_at();
      if (ook_at(orow) && sub < B) {
        float v = out[0];
#pragma unroll
        for (int b = 1; b < BT; ++b) if (sub == b) v = out[b];
        publish(a.pD + ((size_t)x * B + sub) * H + orow, tag(ph + 6), v * kStageUnscale);
      }
      // half of the next layer's q/k/v rows, ahead of the reduce-scatter poll (the
      // rest follows it)
      if (l + 1 < a.L) qkv_request(a.layers[l + 1], std::integral_constant<int, 1>());
    }
    {
      float xn;
      bool hx;
      if (!reduce_rows<BT>(a.pD, ctag(ph + 6), B, H, RPW, j * RPW, xown, xin, xn, hx, lim)) {
        alive = false;
        break;
      }
      if (l + 1 < a.L) {
        qkv_request(a.layers[l + 1], std::integral_constant<int, 2>());
        publish_staged_x<BT>(sx0, SX, H, B, RPW, j * RPW, xn, hx, g_next, j, tag(ph + 6), plain, a.status);
      } else if (hx) {
        const int b = tid / RPW;
        publish_l(lx0 + (size_t)b * H + j * RPW + (tid - b * RPW), tag(ph + 6), xn, plain);
      }
    }
    KMR_TRACE_MARK(tev + 10);
  }

  if (!alive) {
    step_abandon(a);
    return;
  }
  {
    auto addr = [](int i) { return (size_t)i; };
    auto place = [](int i) { return i; };
    const bool ok = B * H <= kStepThreads * 4
                        ? gather_tagged<4>(lx0, B * H, ctag(1 + 6 * a.L), xin, addr, place, NoPre(), lim)
                        : gather_tagged<16>(lx0, B * H, ctag(1 + 6 * a.L), xin, addr, place, NoPre(), lim);
    if (!ok) {
      step_abandon(a);
      return;
    }
  }
  KMR_TRACE_MARK(56);
  step_tail<BT>(a, xin, red, &s_last, step);
}

}  // namespace kmr
