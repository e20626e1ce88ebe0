// C ABI of the int4 weight-only decode step (declared in include/kmr.h).
//
// Host side: argument checks before any launch, the workspace layout, and the
// launch sequence of one layer / one step on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "kmr.h"
#include "kmr_kernels.h"
#include "kmr_prefill.h"
#include "kmr_step.h"
#include "kmr_stepx.h"

using namespace kmr;

namespace {

thread_local char g_err[512] = "";
#ifdef KMR_TRACE
uint64_t* g_trace = nullptr;   // diagnostic builds: phase timestamps of the step kernels
#endif

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_hip(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(KMR_EHIP, "%s: %s", what, hipGetErrorString(e));
  return KMR_OK;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int check_config(const kmr_config* c) {
  if (!c) return fail(KMR_EINVAL, "config is NULL");
  if (c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 ||
      c->intermediate <= 0 || c->n_layers <= 0 || c->group_size <= 0 || c->vocab < 0)
    return fail(KMR_EINVAL, "config has a non-positive dimension");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(KMR_ESHAPE, "head_dim %d unsupported (64 or 128)", c->head_dim);
  if (c->n_heads % c->n_kv_heads != 0)
    return fail(KMR_ESHAPE, "n_heads %d not a multiple of n_kv_heads %d", c->n_heads, c->n_kv_heads);
  const int qpg = c->n_heads / c->n_kv_heads;
  if (qpg != 1 && qpg != 2 && qpg != 4)
    return fail(KMR_ESHAPE, "n_heads / n_kv_heads = %d unsupported (1, 2 or 4)", qpg);
  if (c->group_size % 32 != 0)
    return fail(KMR_ESHAPE, "group_size %d is not a multiple of 32", c->group_size);
  const int qd = c->n_heads * c->head_dim;
  if (c->hidden % c->group_size || qd % c->group_size || c->intermediate % c->group_size)
    return fail(KMR_ESHAPE, "group_size %d must divide hidden, n_heads*head_dim and intermediate",
                c->group_size);
  if (c->hidden > 4096 || qd > 8192 || c->intermediate > 8192)
    return fail(KMR_ESHAPE, "hidden <= 4096, n_heads*head_dim <= 8192 and intermediate <= 8192 required");
  if (c->mrope_section[0] < 0 || c->mrope_section[1] < 0 || c->mrope_section[2] < 0 ||
      c->mrope_section[0] + c->mrope_section[1] + c->mrope_section[2] != c->head_dim / 2)
    return fail(KMR_ESHAPE, "mrope_section must be non-negative and sum to head_dim/2");
  if (!(c->rms_eps >= 0.0f) || !(c->rope_theta > 0.0))
    return fail(KMR_EINVAL, "rms_eps must be >= 0 and rope_theta > 0");
  return KMR_OK;
}

constexpr int kMaxStepGroups = 1024;   // lm_head partial slots of the persistent kernel
constexpr int kStepBatchMax = 4;       // largest batch of the persistent kernels

// Workspace layout.  Three parts:
//   header       status word, step counter, arrival counters and the placement
//                probe's words, at fixed offsets;
//   exchange     the persistent kernels' tagged buffers, sized for their largest
//                batch, at offsets that depend on the config and max_len only;
//   per-phase    the per-phase kernels' buffers for `batch` rows.
// So a workspace reused with another batch size or call kind (prefill, per-phase
// or persistent decode) keeps its counters, and a word a per-phase call wrote never
// sits where a persistent call polls for a tag.
struct WsLayout {
  size_t status, cs, x, qkv, attn_o, act, part_o, part_ml, lm_part, total;
  size_t step_ctr, lm_cnt, xarr, tx, tqkv, to, tact, tpart, lm_part2;
  size_t lx, sx, lqkv, lpart, lact, pO, pD, probe, pf, kpart;
  int kpart_rows;
  size_t pxs, pc2, pkp;         // prefill GEMM input of B tokens: [B][Kmax/32][4] x 16 B, [B][Kmax/128] x 4 B;
                                // split-K partials [2][B][hidden] x 4 B
  size_t xst, xst_cc, xst_cb;   // staged 16-row GEMV tile: [16][4][Kmax/32] x 16 B, [16][Kmax/32] x 8 B,
                                // [16][Kmax/128] x 8 B
  StepXSizes xz;
  int ns, ns_pp, nblk_lm;   // attention splits: persistent device-wide kernel, per-phase kernels
};

WsLayout ws_layout(const kmr_config* c, int B, int M) {
  WsLayout w{};
  const int D = c->head_dim, Hq = c->n_heads, Hkv = c->n_kv_heads, qpg = Hq / Hkv;
  const int nqkv = (Hq + 2 * Hkv) * D, PB = kStepBatchMax;
  w.ns = (M + kAttnSplit - 1) / kAttnSplit;
  w.ns_pp = (M + kAttnSplitPP - 1) / kAttnSplitPP;
  w.nblk_lm = c->vocab > 0 ? (c->vocab + kLmRowsPerBlock - 1) / kLmRowsPerBlock : 1;
  // header
  w.status = 0;
  w.step_ctr = 64;
  w.lm_cnt = 128;
  w.xarr = 256;   // 8 per-XCD arrival counters
  size_t o = 512;
  w.probe = o; o += align256((size_t)kMaxStepGroups * 4);
  // exchange buffers of the persistent kernels (batch <= PB)
  w.tx = o; o += align256((size_t)PB * c->hidden * 8);
  w.tqkv = o; o += align256((size_t)PB * nqkv * 8);
  w.to = o; o += align256((size_t)PB * Hq * D * 8);
  w.tact = o; o += align256((size_t)PB * c->intermediate * 8);
  w.tpart = o; o += align256((size_t)PB * Hkv * w.ns * qpg * (D + 2) * 8);
  w.lm_part2 = o; o += align256((size_t)PB * kMaxStepGroups * 8);
  o = (o + 4095) & ~(size_t)4095;
  w.xz = stepx_sizes(PB, c->hidden, Hkv, D, qpg, c->intermediate, M);
  w.lx = o; o += (size_t)kXcds * w.xz.lx * 8;
  w.sx = o; o += (size_t)kXcds * w.xz.sx * 8;
  w.lqkv = o; o += (size_t)kXcds * w.xz.lqkv * 8;
  w.lpart = o; o += (size_t)kXcds * w.xz.lpart * 8;
  w.lact = o; o += (size_t)kXcds * w.xz.lact * 8;
  w.pO = o; o += align256((size_t)kXcds * PB * c->hidden * 8);
  w.pD = o; o += align256((size_t)kXcds * PB * c->hidden * 8);
  // per-phase buffers for B rows
  w.cs = o; o += align256((size_t)B * (D / 2) * 8);
  w.x = o; o += align256((size_t)B * c->hidden * 4);
  w.qkv = o; o += align256((size_t)B * nqkv * 4);
  w.attn_o = o; o += align256((size_t)B * Hq * D * 4);
  w.act = o; o += align256((size_t)B * c->intermediate * 4);
  w.part_o = o; o += align256((size_t)B * Hkv * w.ns_pp * qpg * D * 4);
  w.part_ml = o; o += align256((size_t)B * Hkv * w.ns_pp * qpg * 8);
  w.lm_part = o; o += align256((size_t)B * w.nblk_lm * 8);
  {
    int kmax = c->hidden > Hq * D ? c->hidden : Hq * D;
    kmax = kmax > c->intermediate ? kmax : c->intermediate;
    const size_t rows = B > 16 ? (size_t)(B / 16) * 16 : 16;   // the full 16-row tiles, or one tile
    w.xst = o; o += align256(rows * 4 * (kmax / 32) * 16);
    w.xst_cc = o; o += align256(rows * (kmax / 32) * 8);
    w.xst_cb = o; o += align256(rows * (kmax / 128) * 8);
    w.kpart_rows = (int)rows;
    w.kpart = o; o += align256((size_t)2 * rows * c->hidden * 4);   // split-K partials of O and down
    w.pxs = o; o += align256((size_t)B * (kmax / 32) * 4 * 16);
    w.pc2 = o; o += align256((size_t)B * (kmax / 128) * 4);
    w.pkp = o; o += align256((size_t)2 * B * c->hidden * 4);
  }
  w.pf = o; o += align256((size_t)4 * KMR_PREFILL_CHUNK * 4);   // prefill: a chunk's [3][C] positions, [C] cache positions
  w.total = o;
  return w;
}

template <typename T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

int check_qweight(const kmr_qweight& q, int N, int K, const char* name) {
  if (!q.packed || !q.sz) return fail(KMR_EINVAL, "%s: null weight pointer", name);
  if (q.N != N || q.K != K)
    return fail(KMR_ESHAPE, "%s: expected %d x %d, got %d x %d", name, N, K, q.N, q.K);
  return KMR_OK;
}

int check_layer(const kmr_config* c, const kmr_layer* L) {
  if (!L) return fail(KMR_EINVAL, "layer is NULL");
  if (!L->in_norm || !L->q_norm || !L->k_norm || !L->post_norm)
    return fail(KMR_EINVAL, "layer norm gain is NULL");
  const int D = c->head_dim, Hq = c->n_heads, Hkv = c->n_kv_heads;
  int rc;
  if ((rc = check_qweight(L->qkv, (Hq + 2 * Hkv) * D, c->hidden, "qkv"))) return rc;
  if ((rc = check_qweight(L->o, c->hidden, Hq * D, "o"))) return rc;
  if ((rc = check_qweight(L->gate_up, 2 * c->intermediate, c->hidden, "gate_up"))) return rc;
  if ((rc = check_qweight(L->down, c->hidden, c->intermediate, "down"))) return rc;
  return KMR_OK;
}

int check_kv(const kmr_config* c, const kmr_kv* kv, int batch) {
  if (!kv || !kv->k || !kv->v) return fail(KMR_EINVAL, "kv cache is NULL or unbound");
  if (kv->n_kv_heads != c->n_kv_heads || kv->head_dim != c->head_dim)
    return fail(KMR_ESHAPE, "kv cache heads/head_dim do not match the config");
  if (kv->batch < batch) return fail(KMR_ESHAPE, "kv cache has %d rows, batch is %d", kv->batch, batch);
  if (kv->max_len <= 0) return fail(KMR_EINVAL, "kv cache max_len must be positive");
  return KMR_OK;
}

template <typename F>
void allow_lds(F* fn, size_t bytes) {
  if (bytes > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// ---------------------------------------------------------------- GEMV launch
template <int BT, int EPI, int PRO, int CPL>
void launch_gemv_k(const GemvArgs& a, hipStream_t st) {
  const size_t lds = gemv_lds(BT, a.K, PRO == PRO_ATTN).total;
  const int rows_per_block = 4 * kGemvRowsPerWave;
  dim3 grid((a.N + rows_per_block - 1) / rows_per_block);
  allow_lds(k_gemv_int4<BT, EPI, PRO, CPL>, lds);
  hipLaunchKernelGGL((k_gemv_int4<BT, EPI, PRO, CPL>), grid, dim3(256), lds, st, a);
}

template <int BT, int EPI, int PRO>
void launch_gemv_cpl(const GemvArgs& a, hipStream_t st) {
  switch ((a.K + 2047) / 2048) {
    case 1: launch_gemv_k<BT, EPI, PRO, 1>(a, st); break;
    case 2: launch_gemv_k<BT, EPI, PRO, 2>(a, st); break;
    case 3: launch_gemv_k<BT, EPI, PRO, 3>(a, st); break;
    default: launch_gemv_k<BT, EPI, PRO, 4>(a, st); break;
  }
}

// Batch tiles of 9..16 rows go to the matrix cores when the group size and K are
// multiples of 128 (one scale/zero per 128-column block) and K <= 8192 (16 blocks
// per wave).  With a staging buffer (plain or RMSNorm input) the tile's input is
// staged once by k_gemv_stage16 and every group reads it from memory; otherwise each
// group stages it in LDS, where the wave partials must then fit (K >= 256 per
// 16-row weight tile).  The rule depends on the shapes and the tile size only.
// (8-row tiles measured slower there than on the VALU: half of each product is
// padding, and a 16-row block leaves half the CUs idle when N = 2048.)
template <int EPI, int PRO>
inline bool gemv_mfma_shape(const GemvArgs& a) {
  return a.G % 128 == 0 && a.K % 128 == 0 && a.K <= 4 * kMfmaBlocksPerWave * 128;
}
template <int EPI, int PRO>
inline bool gemv_mfma_staged(const GemvArgs& a) {
  return PRO != PRO_ATTN && a.xsg && a.ccg && a.cbg && gemv_mfma_shape<EPI, PRO>(a);
}

// The staged matrix-core product over `tiles` 16-row tiles (a.B rows): one staging
// launch, one product launch.  An accumulating product whose grid would have fewer
// groups than the chip has CUs (one group per 16 weight rows and tile) splits K in
// two halves (the grid's z index) into a.kpart, and k_gemv_kreduce adds them to y.
// (Measured: at 16 rows the O and down products gain; at 64 rows, with 4 tiles, the
// split only adds the partial traffic and a launch.)
constexpr int kSplitBelowGroups = 256;   // MI355X compute units
template <int EPI, int PRO>
void launch_mfma_staged(const GemvArgs& a, int tiles, hipStream_t st, bool inv) {
  hipLaunchKernelGGL((k_gemv_stage16<PRO>), dim3(16 * tiles, (a.K + 2047) / 2048), dim3(64), 0, st, a);
  const size_t lds = (size_t)4 * (EPI == EPI_SILU ? 2 : 1) * 256 * 4;   // wave partials
  const bool split = !inv && EPI == EPI_ADD && a.kpart && a.N <= a.kpart_n && (a.K / 128) % 2 == 0 &&
                     a.kpart_rows >= 16 * tiles && ((a.N + 15) / 16) * tiles < kSplitBelowGroups;
  hipLaunchKernelGGL((k_gemv_int4_mfma<16, EPI, PRO, true>), dim3((a.N + 15) / 16, tiles, split ? 2 : 1),
                     dim3(256), lds, st, a);
  if (split) {
    const int n = a.B * a.N;
    hipLaunchKernelGGL(k_gemv_kreduce, dim3((n + 255) / 256), dim3(256), 0, st, a.y, a.ldy, a.kpart,
                       a.kpart_rows, a.N, a.B);
  }
}

// inv (KMR_BATCH_INVARIANT): one form for every tile whatever its rows -- the staged
// matrix-core product (padded to 16 rows, no split K) when the shapes allow it, else
// the VALU product in its 8-row instantiation -- so a row's bits never depend on
// the batch.  (The merge prologue never runs in this mode: k_attn_combine merges.)
template <int EPI, int PRO>
void launch_gemv_tile(const GemvArgs& a, hipStream_t st, bool inv) {
  if (inv) {
    if constexpr (PRO != PRO_ATTN) {
      if (gemv_mfma_staged<EPI, PRO>(a)) launch_mfma_staged<EPI, PRO>(a, 1, st, true);
      else launch_gemv_cpl<8, EPI, PRO>(a, st);
    }
    return;
  }
  if (a.B >= 9 && gemv_mfma_staged<EPI, PRO>(a)) {
    if constexpr (PRO != PRO_ATTN) launch_mfma_staged<EPI, PRO>(a, 1, st, false);
    return;
  }
  if (a.B >= 9 && gemv_mfma_shape<EPI, PRO>(a) && a.K >= 256 * (EPI == EPI_SILU ? 2 : 1)) {
    const size_t lds = gemv_lds(16, a.K, PRO == PRO_ATTN).total;
    allow_lds(k_gemv_int4_mfma<16, EPI, PRO, false>, lds);
    hipLaunchKernelGGL((k_gemv_int4_mfma<16, EPI, PRO, false>), dim3((a.N + 15) / 16), dim3(256), lds, st, a);
    return;
  }
  switch (a.B) {
    case 1: launch_gemv_cpl<1, EPI, PRO>(a, st); break;
    case 2: launch_gemv_cpl<2, EPI, PRO>(a, st); break;
    case 3: case 4: launch_gemv_cpl<4, EPI, PRO>(a, st); break;
    case 5: case 6: case 7: case 8: launch_gemv_cpl<8, EPI, PRO>(a, st); break;
    default: launch_gemv_cpl<16, EPI, PRO>(a, st); break;
  }
}

// Batch tiles keep the staged input inside the LDS of one CU.  With the input
// staged in memory, all full 16-row tiles run as one launch (the tile is the
// grid's y index): one staging pass and one product launch instead of one each
// per tile, and the tiles stream the same weights at the same time.  Every row's
// result is the same as in a launch of its own tile.
template <int EPI, int PRO>
void launch_gemv(GemvArgs a, hipStream_t st, bool inv = false) {
  int B = a.B;
  if constexpr (PRO != PRO_ATTN) {
    const int full = B / 16;
    if (full >= 2 && gemv_mfma_staged<EPI, PRO>(a)) {
      GemvArgs t = a;
      t.B = 16 * full;
      launch_mfma_staged<EPI, PRO>(t, full, st, inv);
      if (B == 16 * full) return;
      a.x += (size_t)16 * full * a.ldx;   // the remaining rows as before
      a.y += (size_t)16 * full * a.ldy;
      a.b0 += 16 * full;
      a.B = B = B - 16 * full;
    }
  }
  int tile = 16;
  const size_t per_row = (size_t)a.K * 9 / 4 + (PRO == PRO_ATTN ? (size_t)a.K * 4 : 0);
  if (inv) {
    if (!gemv_mfma_staged<EPI, PRO>(a)) tile = 8;
  } else if (!(B >= 9 && gemv_mfma_staged<EPI, PRO>(a))) {   // (staged in memory: no LDS bound)
    while (tile > 1 && tile * per_row + 1024 > 150 * 1024) tile >>= 1;
  }
  for (int b0 = 0; b0 < B; b0 += tile) {
    GemvArgs t = a;
    t.B = B - b0 < tile ? B - b0 : tile;
    t.b0 = a.b0 + b0;
    if (t.x) t.x = a.x + (size_t)b0 * a.ldx;
    t.y = a.y + (size_t)b0 * a.ldy;
    launch_gemv_tile<EPI, PRO>(t, st, inv);
  }
}

void launch_attn(const kmr_config* c, const AttnArgs& a, int B, hipStream_t st) {
  dim3 grid(a.NS, c->n_kv_heads, B);
  const int qpg = c->n_heads / c->n_kv_heads;
#define KMR_ATTN(DD, QQ) hipLaunchKernelGGL((k_attn<DD, QQ>), grid, dim3(256), 0, st, a)
  if (c->head_dim == 128) {
    if (qpg == 1) KMR_ATTN(128, 1); else if (qpg == 2) KMR_ATTN(128, 2); else KMR_ATTN(128, 4);
  } else {
    if (qpg == 1) KMR_ATTN(64, 1); else if (qpg == 2) KMR_ATTN(64, 2); else KMR_ATTN(64, 4);
  }
#undef KMR_ATTN
  if (a.first_split > 0) {   // the shared-prefix splits, once per (split, kv head, row group)
    dim3 pgrid(a.first_split, c->n_kv_heads, (B + kPrefixRows - 1) / kPrefixRows);
#define KMR_ATTNP(DD, QQ) hipLaunchKernelGGL((k_attn_prefix<DD, QQ>), pgrid, dim3(256), 0, st, a)
    if (c->head_dim == 128) {
      if (qpg == 1) KMR_ATTNP(128, 1); else if (qpg == 2) KMR_ATTNP(128, 2); else KMR_ATTNP(128, 4);
    } else {
      if (qpg == 1) KMR_ATTNP(64, 1); else if (qpg == 2) KMR_ATTNP(64, 2); else KMR_ATTNP(64, 4);
    }
#undef KMR_ATTNP
  }
}

template <int BT, int CPL>
void launch_lm_k(const LmArgs& a, hipStream_t st) {
  const size_t lds = (size_t)a.K * 4 * BT;
  allow_lds(k_lmhead<BT, CPL>, lds);
  // at most 4 groups per CU of 256: each normalizes the input once and loops over
  // row blocks (the normalization re-done per 16-row block dominated at B = 16)
  const int grid = a.nblk < 1024 ? a.nblk : 1024;
  hipLaunchKernelGGL((k_lmhead<BT, CPL>), dim3(grid), dim3(256), lds, st, a);
}

template <int BT>
void launch_lm_cpl(const LmArgs& a, hipStream_t st) {
  const int cpl = (a.K + 511) / 512;
  if (cpl <= 1) launch_lm_k<BT, 1>(a, st);
  else if (cpl <= 2) launch_lm_k<BT, 2>(a, st);
  else if (cpl <= 4) launch_lm_k<BT, 4>(a, st);
  else launch_lm_k<BT, 8>(a, st);
}

void launch_lmhead_tile(const LmArgs& a, hipStream_t st) {
  if (a.B == 1) launch_lm_cpl<1>(a, st);
  else if (a.B == 2) launch_lm_cpl<2>(a, st);
  else if (a.B <= 4) launch_lm_cpl<4>(a, st);
  else if (a.B <= 8) launch_lm_cpl<8>(a, st);
  else launch_lm_cpl<16>(a, st);
}

// Tiles of 9..16 rows with hidden 2048 take the matrix-core lm_head: 256 groups
// (one per CU: the staged input fills most of the LDS), each wave at most
// ceil(V / 16 / 1024) vocabulary blocks.
bool lmhead_mfma_fits(const LmArgs& a) { return a.B >= 9 && a.K == 2048 && a.nblk == (a.V + 15) / 16; }

void launch_lmhead_mfma(const LmArgs& a, hipStream_t st) {
  const size_t lds = (size_t)2 * 16 * (2048 + 8) * 2;
  if (a.logits) {
    allow_lds(k_lmhead_mfma<64, true>, lds);
    hipLaunchKernelGGL((k_lmhead_mfma<64, true>), dim3(256), dim3(256), lds, st, a);
  } else {
    allow_lds(k_lmhead_mfma<64, false>, lds);
    hipLaunchKernelGGL((k_lmhead_mfma<64, false>), dim3(256), dim3(256), lds, st, a);
  }
}

// Batch tiles of at most 16 rows (input rows, logits rows and argmax partials offset).
// inv (KMR_BATCH_INVARIANT): the matrix-core lm_head for every tile when hidden is
// 2048, else the VALU lm_head in its 8-row instantiation over tiles of 8 rows.
void launch_lmhead(const LmArgs& a, hipStream_t st, bool inv = false) {
  const bool mfma = a.K == 2048 && a.nblk == (a.V + 15) / 16;
  const int tile = inv && !mfma ? 8 : 16;
  for (int b0 = 0; b0 < a.B; b0 += tile) {
    LmArgs t = a;
    t.B = a.B - b0 < tile ? a.B - b0 : tile;
    t.x = a.x + (size_t)b0 * a.K;
    t.logits = a.logits ? a.logits + (size_t)b0 * a.V : nullptr;
    t.part = a.part + (size_t)b0 * a.nblk;
    if (inv) {
      if (mfma) launch_lmhead_mfma(t, st);
      else launch_lm_cpl<8>(t, st);
    } else if (lmhead_mfma_fits(t)) {
      launch_lmhead_mfma(t, st);
    } else {
      launch_lmhead_tile(t, st);
    }
  }
}

// The O projection merges the attention splits in its own prologue when every
// one of its groups can afford to read all partials (few rows, few splits);
// otherwise a separate merge kernel writes o first.  Both use merge_head, so the
// result is the same bits either way; the choice depends on batch * max_len.
bool fuse_attn_merge(int B, int ns) { return (size_t)B * ns <= 16; }

// One decoder layer on x (fp32 [B][H]) using workspace buffers; the RoPE table
// must already be in ws.cs.
void enqueue_layer(const kmr_config* c, const kmr_layer* L, int layer, const kmr_kv* kv, float* x,
                   const int32_t* cpos, int B, void* ws, const WsLayout& w, hipStream_t st,
                   int prefix_splits = 0, bool inv = false) {
  const int H = c->hidden, D = c->head_dim, Hq = c->n_heads, Hkv = c->n_kv_heads;
  const int nqkv = (Hq + 2 * Hkv) * D, I = c->intermediate, G = c->group_size;
  float* qkv = at<float>(ws, w.qkv);
  float* ao = at<float>(ws, w.attn_o);
  float* act = at<float>(ws, w.act);

  uint4* xsg = at<uint4>(ws, w.xst);
  float2* ccg = at<float2>(ws, w.xst_cc);
  float2* cbg = at<float2>(ws, w.xst_cb);
  float* kpart = at<float>(ws, w.kpart);
  GemvArgs g{};
  g.xsg = xsg; g.ccg = ccg; g.cbg = cbg; g.status = at<uint32_t>(ws, w.status); g.kpart = kpart; g.kpart_rows = w.kpart_rows; g.kpart_n = H;
  g.packed = static_cast<const uint8_t*>(L->qkv.packed);
  g.sz = static_cast<const uint32_t*>(L->qkv.sz);
  g.x = x; g.ldx = H; g.gain = static_cast<const uint16_t*>(L->in_norm); g.eps = c->rms_eps;
  g.y = qkv; g.ldy = nqkv; g.N = nqkv; g.K = H; g.G = G; g.B = B;
  launch_gemv<EPI_STORE, PRO_RMSNORM>(g, st, inv);

  AttnArgs a{};
  const size_t layer_stride = (size_t)kv->batch * Hkv * kv->max_len * D;
  a.qkv = qkv; a.ldqkv = nqkv;
  a.q_norm = static_cast<const uint16_t*>(L->q_norm);
  a.k_norm = static_cast<const uint16_t*>(L->k_norm);
  a.cs = at<float2>(ws, w.cs);
  a.kc = static_cast<uint16_t*>(kv->k) + (size_t)layer * layer_stride;
  a.vc = static_cast<uint16_t*>(kv->v) + (size_t)layer * layer_stride;
  a.cpos = cpos;
  a.part_o = at<float>(ws, w.part_o); a.part_ml = at<float2>(ws, w.part_ml);
  a.status = at<uint32_t>(ws, w.status);
  a.Hq = Hq; a.Hkv = Hkv; a.M = kv->max_len; a.NS = w.ns_pp; a.eps = c->rms_eps;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  a.B = B; a.first_split = prefix_splits; a.prefix_row = 0;
  launch_attn(c, a, B, st);

  AttnPart ap{};
  ap.part_o = a.part_o; ap.part_ml = a.part_ml; ap.cpos = cpos;
  ap.Hkv = Hkv; ap.NS = w.ns_pp; ap.QPG = Hq / Hkv; ap.D = D; ap.M = kv->max_len;

  g = GemvArgs{};
  g.xsg = xsg; g.ccg = ccg; g.cbg = cbg; g.status = at<uint32_t>(ws, w.status); g.kpart = kpart; g.kpart_rows = w.kpart_rows; g.kpart_n = H;
  g.packed = static_cast<const uint8_t*>(L->o.packed);
  g.sz = static_cast<const uint32_t*>(L->o.sz);
  g.y = x; g.ldy = H; g.N = H; g.K = Hq * D; g.G = G; g.B = B;
  if (!inv && fuse_attn_merge(B, w.ns_pp)) {
    g.ap = ap;
    launch_gemv<EPI_ADD, PRO_ATTN>(g, st);
  } else {
    const int threads = 8 * B * Hq * (D / 4);   // 8 lanes per 4 output dims
    hipLaunchKernelGGL(k_attn_combine, dim3((threads + 255) / 256), dim3(256), 0, st, ap, ao, B, Hq);
    g.x = ao; g.ldx = Hq * D;
    launch_gemv<EPI_ADD, PRO_PLAIN>(g, st, inv);
  }

  g = GemvArgs{};
  g.xsg = xsg; g.ccg = ccg; g.cbg = cbg; g.status = at<uint32_t>(ws, w.status); g.kpart = kpart; g.kpart_rows = w.kpart_rows; g.kpart_n = H;
  g.packed = static_cast<const uint8_t*>(L->gate_up.packed);
  g.sz = static_cast<const uint32_t*>(L->gate_up.sz);
  g.x = x; g.ldx = H; g.gain = static_cast<const uint16_t*>(L->post_norm); g.eps = c->rms_eps;
  g.y = act; g.ldy = I; g.N = I; g.K = H; g.G = G; g.B = B;
  launch_gemv<EPI_SILU, PRO_RMSNORM>(g, st, inv);

  g = GemvArgs{};
  g.xsg = xsg; g.ccg = ccg; g.cbg = cbg; g.status = at<uint32_t>(ws, w.status); g.kpart = kpart; g.kpart_rows = w.kpart_rows; g.kpart_n = H;
  g.packed = static_cast<const uint8_t*>(L->down.packed);
  g.sz = static_cast<const uint32_t*>(L->down.sz);
  g.x = act; g.ldx = I; g.gain = nullptr;
  g.y = x; g.ldy = H; g.N = H; g.K = I; g.G = G; g.B = B;
  launch_gemv<EPI_ADD, PRO_PLAIN>(g, st, inv);
}

// ---------------------------------------------------------------- prefill
// The matrix-core GEMM takes a linear when its group size is a multiple of 128 and
// its input width a multiple of 512 (whole 4-block zero-point steps).
bool pf_gemm_fits(const kmr_config* c) {
  return c->group_size % 128 == 0 && c->hidden % 512 == 0 && (c->n_heads * c->head_dim) % 512 == 0 &&
         c->intermediate % 512 == 0;
}

// Staging of a chunk's GEMM input; kp (or null): split-K partials of the projection
// that wrote x, added to x first.
template <int PRO>
void launch_pf_stage(float* x, int ldx, const uint16_t* gain, const float* kp, int K, int M, float eps, void* ws,
                     const WsLayout& w, hipStream_t st) {
  PfStageArgs s{};
  s.x = x; s.ldx = ldx; s.gain = gain; s.kp = kp; s.eps = eps; s.K = K; s.M = M;
  s.xs = at<uint4>(ws, w.pxs); s.c2 = at<float>(ws, w.pc2); s.status = at<uint32_t>(ws, w.status);
  hipLaunchKernelGGL(k_pf_stage<PRO>, dim3(M), dim3(256), 0, st, s);
}

// An EPI_ADD product whose tiles number fewer than 512 splits K in two when each half
// keeps whole 4-block zero-point steps: its partials go to the workspace (w.pkp) and
// the caller's next staging of y adds them.  Returns whether it split.
template <int EPI>
bool launch_pf_gemm(const kmr_qweight& q, float* y, int ldy, int N, int K, int G, int M, void* ws,
                    const WsLayout& w, hipStream_t st) {
  PfGemmArgs g{};
  g.xs = at<const uint4>(ws, w.pxs); g.c2 = at<const float>(ws, w.pc2);
  g.packed = static_cast<const uint8_t*>(q.packed); g.sz = static_cast<const uint32_t*>(q.sz);
  g.y = y; g.ldy = ldy; g.M = M; g.N = N; g.K = K; g.G = G; g.kpart = at<float>(ws, w.pkp);
  const int rows = EPI == EPI_SILU ? kPfTileN / 2 : kPfTileN;
  const dim3 grid((N + rows - 1) / rows, (M + kPfTileM - 1) / kPfTileM);
  const bool split = EPI == EPI_ADD && grid.x * grid.y < 512 && (K / 128) % 8 == 0;
  allow_lds(k_pf_gemm<EPI>, pf_gemm_lds());
  hipLaunchKernelGGL(k_pf_gemm<EPI>, dim3(grid.x, grid.y, split ? 2 : 1), dim3(256), pf_gemm_lds(), st, g);
  return split;
}

// One decoder layer over the M tokens of a prompt chunk (cache row crow, cache
// positions cpos, consecutive).  The linears run as matrix-core GEMMs over the whole
// chunk when pf_gemm_fits (else as the decode path's GEMV tiles); the chunk's q/k/v
// are normalized, rotated and written to the cache first, then every token attends
// causally over slots 0 .. its own.
// `pending`: x still owes the split-K partials of the previous down projection
// (w.pkp); the layer's first staging adds them, and the layer leaves it set when its
// own down projection split.
void enqueue_prefill_layer(const kmr_config* c, const kmr_layer* L, int layer, const kmr_kv* kv, float* x,
                           const int32_t* cpos, int M, int crow, void* ws, const WsLayout& w, hipStream_t st,
                           bool& pending) {
  const int H = c->hidden, D = c->head_dim, Hq = c->n_heads, Hkv = c->n_kv_heads;
  const int nqkv = (Hq + 2 * Hkv) * D, I = c->intermediate, G = c->group_size;
  const bool mm = pf_gemm_fits(c);
  const float* kp = at<const float>(ws, w.pkp);
  float* qkv = at<float>(ws, w.qkv);
  float* ao = at<float>(ws, w.attn_o);
  float* act = at<float>(ws, w.act);
  auto gemv = [&](const kmr_qweight& q, const float* in, int ldx, const uint16_t* gain, float* y, int ldy, int N,
                  int K) {
    GemvArgs g{};
    g.xsg = at<uint4>(ws, w.xst); g.ccg = at<float2>(ws, w.xst_cc); g.cbg = at<float2>(ws, w.xst_cb);
    g.status = at<uint32_t>(ws, w.status); g.kpart = at<float>(ws, w.kpart); g.kpart_rows = w.kpart_rows;
    g.kpart_n = H;
    g.packed = static_cast<const uint8_t*>(q.packed); g.sz = static_cast<const uint32_t*>(q.sz);
    g.x = in; g.ldx = ldx; g.gain = gain; g.eps = c->rms_eps;
    g.y = y; g.ldy = ldy; g.N = N; g.K = K; g.G = G; g.B = M;
    return g;
  };
  // q, k, v
  if (mm) {
    launch_pf_stage<PRO_RMSNORM>(x, H, static_cast<const uint16_t*>(L->in_norm), pending ? kp : nullptr, H, M,
                                 c->rms_eps, ws, w, st);
    pending = false;
    launch_pf_gemm<EPI_STORE>(L->qkv, qkv, nqkv, nqkv, H, G, M, ws, w, st);
  } else {
    launch_gemv<EPI_STORE, PRO_RMSNORM>(gemv(L->qkv, x, H, static_cast<const uint16_t*>(L->in_norm), qkv, nqkv,
                                             nqkv, H), st);
  }
  const size_t layer_stride = (size_t)kv->batch * Hkv * kv->max_len * D;
  uint16_t* kc = static_cast<uint16_t*>(kv->k) + (size_t)layer * layer_stride;
  uint16_t* vc = static_cast<uint16_t*>(kv->v) + (size_t)layer * layer_stride;
  PfQkArgs qa{};
  qa.qkv = qkv; qa.q_norm = static_cast<const uint16_t*>(L->q_norm); qa.k_norm = static_cast<const uint16_t*>(L->k_norm);
  qa.cs = at<float2>(ws, w.cs); qa.kc = kc; qa.vc = vc; qa.cpos = cpos;
  qa.M = M; qa.ldqkv = nqkv; qa.Hq = Hq; qa.Hkv = Hkv; qa.D = D; qa.max_len = kv->max_len; qa.crow = crow;
  qa.eps = c->rms_eps;
  hipLaunchKernelGGL(k_pf_qk, dim3((Hq + 2 * Hkv + 3) / 4, M), dim3(256), 0, st, qa);
  PfAttnArgs aa{};
  aa.q = qkv; aa.ldq = nqkv; aa.kc = kc; aa.vc = vc; aa.cpos = cpos; aa.o = ao; aa.ldo = Hq * D;
  aa.M = M; aa.Hkv = Hkv; aa.max_len = kv->max_len; aa.crow = crow;
  aa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)D));
  const int qpg = Hq / Hkv;
  const dim3 agrid((M + kPfAttnTokens - 1) / kPfAttnTokens, Hkv);
#define KMR_PFATTN(DD, QQ)                                                                            \
  do {                                                                                                \
    allow_lds(k_pf_attn<DD, QQ>, pf_attn_lds(DD, QQ));                                               \
    hipLaunchKernelGGL((k_pf_attn<DD, QQ>), agrid, dim3(64 * QQ * pf_attn_groups(QQ)), pf_attn_lds(DD, QQ), st, aa); \
  } while (0)
  if (D == 128) {
    if (qpg == 1) KMR_PFATTN(128, 1); else if (qpg == 2) KMR_PFATTN(128, 2); else KMR_PFATTN(128, 4);
  } else {
    if (qpg == 1) KMR_PFATTN(64, 1); else if (qpg == 2) KMR_PFATTN(64, 2); else KMR_PFATTN(64, 4);
  }
#undef KMR_PFATTN
  // o projection (+ residual)
  bool o_split = false;
  if (mm) {
    launch_pf_stage<PRO_PLAIN>(ao, Hq * D, nullptr, nullptr, Hq * D, M, c->rms_eps, ws, w, st);
    o_split = launch_pf_gemm<EPI_ADD>(L->o, x, H, H, Hq * D, G, M, ws, w, st);
  } else {
    launch_gemv<EPI_ADD, PRO_PLAIN>(gemv(L->o, ao, Hq * D, nullptr, x, H, H, Hq * D), st);
  }
  // MLP
  if (mm) {
    launch_pf_stage<PRO_RMSNORM>(x, H, static_cast<const uint16_t*>(L->post_norm), o_split ? kp : nullptr, H, M,
                                 c->rms_eps, ws, w, st);
    launch_pf_gemm<EPI_SILU>(L->gate_up, act, I, I, H, G, M, ws, w, st);
    launch_pf_stage<PRO_PLAIN>(act, I, nullptr, nullptr, I, M, c->rms_eps, ws, w, st);
    pending = launch_pf_gemm<EPI_ADD>(L->down, x, H, H, I, G, M, ws, w, st);
  } else {
    launch_gemv<EPI_SILU, PRO_RMSNORM>(gemv(L->gate_up, x, H, static_cast<const uint16_t*>(L->post_norm), act, I,
                                            I, H), st);
    launch_gemv<EPI_ADD, PRO_PLAIN>(gemv(L->down, act, I, nullptr, x, H, H, I), st);
  }
}

// ---------------------------------------------------------------- persistent step
// Shapes the persistent kernel is built for (one 2048-column chunk per lane for
// hidden and n_heads*head_dim, three for intermediate, GQA groups of 2).
bool step_kernel_fits(const kmr_config* c, int B) {
  return B <= 4 && (c->group_size & (c->group_size - 1)) == 0 && c->hidden <= 2048 &&
         c->n_heads * c->head_dim <= 2048 &&
         c->intermediate <= 6144 && c->n_layers <= kMaxStepLayers &&
         c->n_heads == 2 * c->n_kv_heads && c->vocab > 0;
}

// The XCD-local step kernel: shapes its fixed per-group work split covers.
bool stepx_fits(const kmr_config* c, int B, int nwg) {
  if (!step_kernel_fits(c, B) || nwg % kXcds != 0 || c->n_kv_heads % kXcds != 0) return false;
  const int WPX = nwg / kXcds, D = c->head_dim, QPG = c->n_heads / c->n_kv_heads;
  const int GPX = c->n_kv_heads / kXcds, QX = GPX * (QPG + 2) * D, OX = GPX * QPG * D;
  if (c->intermediate % (kXcds * 32) != 0) return false;
  const int IX = c->intermediate / kXcds, H = c->hidden;
  const int RPW = (H + WPX - 1) / WPX, RQ = (QX + WPX - 1) / WPX, RA = (IX + WPX - 1) / WPX;
  if (OX > 512 || OX > H || OX / 32 > 8 * kXNarrowCpl || IX > H || IX / 32 > 8 * kXNarrowCpl) return false;
  if (RPW > 8 * kStepWaves || RQ > 2 * kStepWaves || RA > 3 * kStepWaves) return false;
  // every group owns residual rows and act values (the hand-off order relies on it)
  if (RPW * (WPX - 1) >= H || RA * (WPX - 1) >= IX) return false;
  // staged vectors: 8-column words owned whole, one element per thread, <= 64 producers
  if (RPW % 8 != 0 || RA % 8 != 0 || RA > 32 || 4 * RPW > kStepThreads || WPX > kXMaxPerXcd) return false;
  // a residual row starts at a wave boundary or lies within one wave
  if (RPW <= 64 ? 64 % RPW != 0 : RPW % 64 != 0) return false;
  if (4 * GPX * QPG > 8 || QPG != 2) return false;   // split-merge weights in one wave
  if (GPX & (GPX - 1)) return false;                  // kv heads per XCD: a power of two
  // The weight loaders' chunk assumptions (each loader covers its rows' columns
  // only under these; the address model in tests/test_stepx_loaders.py checks them):
  //  - QKV rows (wrows_load, one chunk per lane) and the gate/up rows (wrows_to_lds,
  //    one chunk per lane, lanes past the row reload chunk 0): hidden <= 64 chunks;
  if (H > 64 * 32 || H % 32 != 0) return false;
  //  - O and down rows (wnarrow_load): the XCD's column slice (OX of n_heads*head_dim,
  //    IX of intermediate) in at most kXNarrowCpl chunks per lane of an 8-lane group,
  //    and 8 XCD slices that tile the row exactly;
  if (OX % 32 != 0 || IX % 32 != 0 || OX / 32 > 8 * kXNarrowCpl || IX / 32 > 8 * kXNarrowCpl ||
      kXcds * OX != c->n_heads * D || kXcds * IX != c->intermediate)
    return false;
  //  - a quantization group never straddles a chunk: G a power of two >= 32.
  if (c->group_size < 32) return false;
  //  - the matrix-core gate/up form (the constant-size instantiation only) takes
  //    kGuMfmaRows act rows per group over exactly kGuMfmaK columns; its shape
  //    match in launch_stepx_k implies IX = WPX * kGuMfmaRows and hidden = kGuMfmaK.
  const size_t lds = stepx_lds(4, H, RPW, D, QPG, GPX).total;
  return lds <= 160 * 1024;
}

static_assert(kFixI / kXcds == (kFixNwg / kXcds) * kGuMfmaRows && kFixH == kGuMfmaK,
              "the constant-size gate/up tiles cover the XCD's act rows and the hidden width exactly");

__global__ void k_xcc_probe(uint32_t* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 15u;
}

// Whether the XCC id register of the current device names 8 XCDs that receive the
// groups of a grid in turn (group g on XCD (s + g) % 8 for some s: the dispatcher's
// starting XCD moves with the groups of earlier dispatches): probed once per device
// (a small kernel on `st`, a synchronous copy of nwg words through `scratch`), then
// cached.  Not probed while `st` is capturing.
std::atomic<int> g_topology[64];   // 0 unknown, 1 verified, 2 other placement

bool xcd_placement_ok(void* scratch, size_t scratch_bytes, int nwg, hipStream_t st) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  const int known = g_topology[dev].load();
  if (known) return known == 1;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return false;
  if (nwg <= 0 || nwg > kMaxStepGroups || scratch_bytes < (size_t)nwg * 4) return false;
  uint32_t ids[kMaxStepGroups];
  hipLaunchKernelGGL(k_xcc_probe, dim3(nwg), dim3(64), 0, st, static_cast<uint32_t*>(scratch));
  if (hipGetLastError() != hipSuccess) return false;
  if (hipMemcpyAsync(ids, scratch, (size_t)nwg * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return false;
  bool ok = nwg % kXcds == 0;
  for (int g = 0; g < nwg && ok; ++g) ok = ids[g] < (uint32_t)kXcds && (int)ids[g] == ((int)ids[0] + g) % kXcds;
  g_topology[dev].store(ok ? 1 : 2);
  return ok;
}

int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return check_hip("hipGetDevice");
  if (hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return check_hip("CU count");
  if (*cus > kMaxStepGroups) *cus = kMaxStepGroups;
  return KMR_OK;
}

// Launches a persistent step kernel: nwg groups that hand work to each other, so all
// of them must be resident at once.  The default is a plain launch after checking that
// the device holds nwg groups of this LDS size at once; on an otherwise idle device
// every group then starts at launch.  Work from other streams or processes can hold
// groups back, which delays the step, and past the bounded hand-off waits (~1 s) ends
// it with KMR_STATUS_TIMEOUT; nothing waits on this kernel, so it cannot deadlock.
// coop asks the runtime for the co-residency guarantee (hipLaunchCooperativeKernel)
// instead, which costs ~20 us more per launch on gfx950.
int launch_persistent(const void* fn, int nwg, size_t lds, StepArgs& a, bool coop, hipStream_t st) {
  if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return check_hip("step kernel LDS attribute");
  void* args[] = {&a};
  if (coop) {
    if (hipLaunchCooperativeKernel(fn, dim3(nwg), dim3(kStepThreads), args, (unsigned)lds, st) != hipSuccess)
      return check_hip("step kernel cooperative launch");
    return KMR_OK;
  }
  int per_cu = 0, cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kStepThreads, lds) != hipSuccess)
    return check_hip("step kernel occupancy");
  if ((long)per_cu * cus < nwg)
    return fail(KMR_EHIP, "step kernel: %d groups do not fit at once (%d per CU, %d CUs)", nwg, per_cu, cus);
  if (hipLaunchKernel(fn, dim3(nwg), dim3(kStepThreads), args, lds, st) != hipSuccess)
    return check_hip("step kernel launch");
  return KMR_OK;
}

template <int BT, int D>
int launch_step_k(const kmr_config* c, StepArgs& a, int nwg, bool coop, hipStream_t st) {
  const int KMAX = std::max(c->hidden, std::max(c->intermediate, c->n_heads * c->head_dim));
  const int RPBX = (c->hidden + nwg - 1) / nwg;
  const size_t lds = step_lds(BT, KMAX, RPBX, c->hidden, D, 2).total;
  return launch_persistent(reinterpret_cast<const void*>(k_step<BT, D, 2>), nwg, lds, a, coop, st);
}

template <int BT, int D>
int launch_stepx_k(const kmr_config* c, StepArgs& a, int nwg, bool coop, hipStream_t st) {
  const int WPX = nwg / kXcds, RPW = (c->hidden + WPX - 1) / WPX;
  const size_t lds = stepx_lds(BT, c->hidden, RPW, D, 2, c->n_kv_heads / kXcds).total;
  // the constant-size instantiation for the shape it was compiled for
  auto fn = k_stepx<BT, D, 2, false>;
  if constexpr (D == 128) {
    if (c->hidden == kFixH && c->n_kv_heads == kFixHkv && c->n_heads == 2 * kFixHkv &&
        c->intermediate == kFixI && c->group_size == (1 << kFixLgG) && nwg == kFixNwg)
      fn = k_stepx<BT, D, 2, true>;
  }
  return launch_persistent(reinterpret_cast<const void*>(fn), nwg, lds, a, coop, st);
}

int launch_stepx(const kmr_config* c, StepArgs& a, int nwg, bool coop, hipStream_t st) {
  const int B = a.B;
  if (c->head_dim == 128)
    return B == 1 ? launch_stepx_k<1, 128>(c, a, nwg, coop, st) : launch_stepx_k<4, 128>(c, a, nwg, coop, st);
  return B == 1 ? launch_stepx_k<1, 64>(c, a, nwg, coop, st) : launch_stepx_k<4, 64>(c, a, nwg, coop, st);
}

// The device-wide kernel runs its 4-row instantiation at every batch of 1..4, so
// that a row's bits do not depend on the batch it is in (its 1-row instantiation
// compiled to different arithmetic for some products).
int launch_step(const kmr_config* c, StepArgs& a, int nwg, bool coop, hipStream_t st) {
  if (c->head_dim == 128) return launch_step_k<4, 128>(c, a, nwg, coop, st);
  return launch_step_k<4, 64>(c, a, nwg, coop, st);
}

void enqueue_prep(const kmr_config* c, const uint16_t* embed, const int32_t* ids,
                  const uint8_t* finished, const int32_t* pos, float* x, int B, void* ws,
                  const WsLayout& w, hipStream_t st) {
  PrepArgs p{};
  p.embed = embed; p.ids = ids; p.finished = finished; p.pos = pos; p.x = x;
  p.cs = at<float2>(ws, w.cs); p.status = at<uint32_t>(ws, w.status);
  p.B = B; p.H = c->hidden; p.V = c->vocab; p.D = c->head_dim; p.pad_id = c->pad_id;
  p.theta = c->rope_theta;
  p.sec0 = c->mrope_section[0]; p.sec1 = c->mrope_section[1]; p.sec2 = c->mrope_section[2];
  p.interleaved = c->mrope_interleaved;
  hipLaunchKernelGGL(k_prep, dim3(B), dim3(256), 0, st, p);
}

void fill_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t words = bytes / 4;
  if (words) {
    size_t blocks = (words + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, st,
                       static_cast<uint32_t*>(p), words);
  }
}

// ---------------------------------------------------------------- static workspace
// The workspace of kmr_decode_step_static: one array per device, held until the
// process ends.  In host code `scratch` is only a stand-in for the symbol; its
// device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) unsigned char scratch[KMR_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices];           // device address of `scratch` on each device
size_t g_static_sig[kMaxDevices][4];       // layout of the last call on each device

// The current device's static workspace for a call whose layout is w: its address
// (set up on the device's first call), and a fill kernel on `st` when the layout
// differs from the previous call's on this device (the first call included), so
// that the header's counters start at zero and no word of another layout can be
// taken for a tag.  Calls with one layout reuse the contents, as a caller-owned
// workspace is reused.
int static_workspace(const kmr_config* c, const WsLayout& w, int M, bool clear, hipStream_t st, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return check_hip("hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(KMR_EINVAL, "device %d outside [0, %d)", dev, kMaxDevices);
  if (w.total > (size_t)KMR_STATIC_WORKSPACE_BYTES)
    return fail(KMR_ENOMEM, "this batch and max_len need a %zu-byte workspace; the static one holds %zu",
                w.total, (size_t)KMR_STATIC_WORKSPACE_BYTES);
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(KMR_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_static_ptr[dev] = p;
  }
  const size_t sig[4] = {w.total, w.lx, (size_t)M,
                         ((size_t)c->hidden << 40) ^ ((size_t)c->intermediate << 20) ^
                             ((size_t)c->n_kv_heads << 8) ^ (size_t)c->head_dim};
  if (clear || memcmp(sig, g_static_sig[dev], sizeof sig) != 0) {
    fill_zero(g_static_ptr[dev], w.total, st);
    memcpy(g_static_sig[dev], sig, sizeof sig);
  }
  *out = g_static_ptr[dev];
  return check_hip("static workspace fill");
}

}  // namespace

extern "C" {

const char* kmr_strerror(int code) {
  switch (code) {
    case KMR_OK: return "ok";
    case KMR_EINVAL: return "invalid argument";
    case KMR_ESHAPE: return "unsupported or mismatched shape";
    case KMR_ENOMEM: return "buffer or workspace too small";
    case KMR_EHIP: return "HIP runtime error";
    default: return "unknown error";
  }
}

const char* kmr_last_error(void) { return g_err; }

#ifdef KMR_TRACE
// Diagnostic builds only: route the step kernel's phase timestamps to `buf`
// (uint64 [groups][64]); NULL turns tracing off.
int kmr_debug_set_trace(void* buf) {
  g_trace = static_cast<uint64_t*>(buf);
  return KMR_OK;
}
#endif

int kmr_kv_alloc(const kmr_config* cfg, int32_t batch, int32_t max_len, void* buf,
                 size_t buf_bytes, int32_t zero_fill, kmr_stream_t stream, kmr_kv* out) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if (!out) return fail(KMR_EINVAL, "out is NULL");
  if (batch <= 0 || batch > KMR_MAX_BATCH || max_len <= 0)
    return fail(KMR_EINVAL, "batch must be in [1, %d] and max_len positive", KMR_MAX_BATCH);
  const size_t half = (size_t)cfg->n_layers * batch * cfg->n_kv_heads * max_len * cfg->head_dim * 2;
  const size_t half_al = align256(half);
  out->bytes = 2 * half_al;
  out->n_layers = cfg->n_layers; out->batch = batch; out->n_kv_heads = cfg->n_kv_heads;
  out->max_len = max_len; out->head_dim = cfg->head_dim;
  out->k = out->v = nullptr;
  if (!buf) return KMR_OK;
  if (buf_bytes < out->bytes)
    return fail(KMR_ENOMEM, "kv buffer has %zu bytes, needs %zu", buf_bytes, out->bytes);
  if (reinterpret_cast<uintptr_t>(buf) % 256) return fail(KMR_EINVAL, "kv buffer not 256-byte aligned");
  out->k = buf;
  out->v = static_cast<char*>(buf) + half_al;
  if (zero_fill) {
    fill_zero(buf, out->bytes, reinterpret_cast<hipStream_t>(stream));
    return check_hip("kv zero fill");
  }
  return KMR_OK;
}

int kmr_quantize_int4(const void* w_bf16, int32_t N, int32_t K, int32_t group, void* packed,
                      void* sz, kmr_stream_t stream) {
  if (!w_bf16 || !packed || !sz) return fail(KMR_EINVAL, "null pointer");
  if (N <= 0 || K <= 0 || group <= 0) return fail(KMR_EINVAL, "N, K and group must be positive");
  if (group % 2 || K % group) return fail(KMR_ESHAPE, "group %d must be even and divide K %d", group, K);
  const long long groups = (long long)N * (K / group);
  const unsigned blocks = (unsigned)((groups + 255) / 256);
  hipLaunchKernelGGL(k_quantize_int4, dim3(blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint16_t*>(w_bf16),
                     N, K, group, static_cast<uint8_t*>(packed), static_cast<uint32_t*>(sz));
  return check_hip("quantize launch");
}

size_t kmr_workspace_bytes(const kmr_config* cfg, int32_t batch, int32_t max_len) {
  if (check_config(cfg) || batch <= 0 || batch > KMR_MAX_BATCH || max_len <= 0) return 0;
  return ws_layout(cfg, batch, max_len).total;
}

int kmr_debug_stepx_fits(const kmr_config* cfg, int32_t batch, int32_t n_groups) {
  if (check_config(cfg) || batch < 1 || n_groups < 1) return -1;
  return stepx_fits(cfg, batch, n_groups) ? 1 : 0;
}

size_t kmr_prefill_workspace_bytes(const kmr_config* cfg, int32_t n_tokens, int32_t max_len) {
  if (check_config(cfg) || n_tokens <= 0 || max_len <= 0) return 0;
  return ws_layout(cfg, n_tokens < KMR_PREFILL_CHUNK ? n_tokens : KMR_PREFILL_CHUNK, max_len).total;
}

int kmr_workspace_init(void* ws, size_t ws_bytes, kmr_stream_t stream) {
  if (!ws || !ws_bytes) return fail(KMR_EINVAL, "workspace is NULL or empty");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  int nwg = 0;
  if (device_cus(&nwg) == KMR_OK) xcd_placement_ok(ws, ws_bytes, nwg, st);
  fill_zero(ws, ws_bytes, st);
  return check_hip("workspace init");
}

int kmr_decode_layer(const kmr_config* cfg, const kmr_layer* layer_w, int32_t layer,
                     const kmr_kv* kv, float* hidden_inout, const int32_t* positions,
                     const int32_t* cache_position, int32_t batch, void* ws, size_t ws_bytes,
                     kmr_stream_t stream) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if ((rc = check_layer(cfg, layer_w))) return rc;
  if (batch <= 0 || batch > KMR_MAX_BATCH) return fail(KMR_EINVAL, "batch %d out of [1, %d]", batch, KMR_MAX_BATCH);
  if ((rc = check_kv(cfg, kv, batch))) return rc;
  if (layer < 0 || layer >= kv->n_layers) return fail(KMR_EINVAL, "layer %d outside the cache", layer);
  if (!hidden_inout || !positions || !cache_position || !ws)
    return fail(KMR_EINVAL, "null hidden/positions/cache_position/workspace");
  const WsLayout w = ws_layout(cfg, batch, kv->max_len);
  if (ws_bytes < w.total) return fail(KMR_ENOMEM, "workspace has %zu bytes, needs %zu", ws_bytes, w.total);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  enqueue_prep(cfg, nullptr, nullptr, nullptr, positions, nullptr, batch, ws, w, st);
  enqueue_layer(cfg, layer_w, layer, kv, hidden_inout, cache_position, batch, ws, w, st);
  return check_hip("decode_layer launch");
}

static int decode_step(const kmr_config* cfg, const kmr_model* model, const kmr_kv* kv,
                       const int32_t* token_ids, int32_t* positions, int32_t* cache_position,
                       uint8_t* finished, int32_t batch, int32_t* next_ids, float* logits,
                       uint32_t flags, void* ws, size_t ws_bytes, kmr_stream_t stream, int prefix_splits) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if (cfg->vocab <= 0) return fail(KMR_EINVAL, "vocab must be positive for a full step");
  if (!model || !model->embed || !model->final_norm || !model->lm_head || !model->layers)
    return fail(KMR_EINVAL, "model pointers are NULL");
  for (int l = 0; l < cfg->n_layers; ++l)
    if ((rc = check_layer(cfg, &model->layers[l]))) return fail(rc, "layer %d: %s", l, g_err);
  if (batch <= 0 || batch > KMR_MAX_BATCH) return fail(KMR_EINVAL, "batch %d out of [1, %d]", batch, KMR_MAX_BATCH);
  if ((rc = check_kv(cfg, kv, batch))) return rc;
  if (kv->n_layers != cfg->n_layers) return fail(KMR_ESHAPE, "kv cache has %d layers, model %d", kv->n_layers, cfg->n_layers);
  if (!token_ids || !positions || !cache_position || !next_ids || !ws)
    return fail(KMR_EINVAL, "null token_ids/positions/cache_position/next_ids/workspace");
  if (flags & ~(KMR_ADVANCE | KMR_MULTI_KERNEL | KMR_DEVICE_WIDE | KMR_COOPERATIVE | KMR_DEVICE_SCOPE_STORES |
                KMR_BATCH_INVARIANT | KMR_TEST_STALL))
    return fail(KMR_EINVAL, "unknown flags 0x%x", flags);
  const WsLayout w = ws_layout(cfg, batch, kv->max_len);
  if (ws_bytes < w.total) return fail(KMR_ENOMEM, "workspace has %zu bytes, needs %zu", ws_bytes, w.total);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bool inv = (flags & KMR_BATCH_INVARIANT) != 0;
  if (!(flags & KMR_MULTI_KERNEL) && !inv && prefix_splits == 0 && step_kernel_fits(cfg, batch)) {
    int nwg = 0;
    if ((rc = device_cus(&nwg))) return rc;
    StepArgs a{};
    a.embed = static_cast<const uint16_t*>(model->embed);
    a.final_norm = static_cast<const uint16_t*>(model->final_norm);
    a.lm_head = static_cast<const uint16_t*>(model->lm_head);
    a.ids = token_ids; a.pos = positions; a.cpos = cache_position; a.finished = finished;
    a.next = next_ids; a.logits = logits;
    a.kc = static_cast<uint16_t*>(kv->k); a.vc = static_cast<uint16_t*>(kv->v);
    a.status = at<uint32_t>(ws, w.status); a.step_ctr = at<uint32_t>(ws, w.step_ctr);
    a.lm_cnt = at<uint32_t>(ws, w.lm_cnt);
    a.xarr = at<uint32_t>(ws, w.xarr);
    a.tx = at<uint64_t>(ws, w.tx); a.tqkv = at<uint64_t>(ws, w.tqkv);
    a.to = at<uint64_t>(ws, w.to); a.tact = at<uint64_t>(ws, w.tact);
    a.tpart = at<uint64_t>(ws, w.tpart);
    a.lm_part = at<float2>(ws, w.lm_part2);
#ifdef KMR_TRACE
    a.trace = g_trace;
#endif
    a.lx = at<uint64_t>(ws, w.lx); a.lqkv = at<uint64_t>(ws, w.lqkv);
    a.lpart = at<uint64_t>(ws, w.lpart); a.lact = at<uint64_t>(ws, w.lact);
    a.pO = at<uint64_t>(ws, w.pO); a.pD = at<uint64_t>(ws, w.pD);
    a.sx = at<uint64_t>(ws, w.sx);
    a.x_lx = w.xz.lx; a.x_lqkv = w.xz.lqkv; a.x_lpart = w.xz.lpart; a.x_lact = w.xz.lact;
    a.x_sx = w.xz.sx; a.srow_x = w.xz.srow_x; a.srow_a = w.xz.srow_a;
    a.B = batch; a.H = cfg->hidden; a.Hq = cfg->n_heads; a.Hkv = cfg->n_kv_heads;
    a.I = cfg->intermediate; a.V = cfg->vocab; a.L = cfg->n_layers; a.G = cfg->group_size;
    a.lgG = 0;
    while ((1 << a.lgG) < a.G) ++a.lgG;
    a.M = kv->max_len; a.cacheB = kv->batch; a.NS = w.ns; a.pad_id = cfg->pad_id;
    a.eos_id = cfg->eos_id; a.flags = flags & KMR_ADVANCE; a.eps = cfg->rms_eps;
    // KMR_TEST_STALL: consumers wait for a phase bit no producer sets (phases stay
    // below 256), and give up after 4096 polls
    a.tag_xor = (flags & KMR_TEST_STALL) ? 0x100u : 0u;
    a.spin_limit = (flags & KMR_TEST_STALL) ? (1u << 12) : kSpinLimit;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)cfg->head_dim));
    a.theta = cfg->rope_theta;
    a.sec0 = cfg->mrope_section[0]; a.sec1 = cfg->mrope_section[1]; a.sec2 = cfg->mrope_section[2];
    a.interleaved = cfg->mrope_interleaved;
    for (int l = 0; l < cfg->n_layers; ++l) {
      const kmr_layer& L = model->layers[l];
      StepLayer& d = a.layers[l];
      d.in_norm = static_cast<const uint16_t*>(L.in_norm);
      d.q_norm = static_cast<const uint16_t*>(L.q_norm);
      d.k_norm = static_cast<const uint16_t*>(L.k_norm);
      d.post_norm = static_cast<const uint16_t*>(L.post_norm);
      d.qkv_p = static_cast<const uint8_t*>(L.qkv.packed); d.qkv_s = static_cast<const uint32_t*>(L.qkv.sz);
      d.o_p = static_cast<const uint8_t*>(L.o.packed); d.o_s = static_cast<const uint32_t*>(L.o.sz);
      d.gu_p = static_cast<const uint8_t*>(L.gate_up.packed); d.gu_s = static_cast<const uint32_t*>(L.gate_up.sz);
      d.d_p = static_cast<const uint8_t*>(L.down.packed); d.d_s = static_cast<const uint32_t*>(L.down.sz);
    }
    if (!(flags & KMR_DEVICE_WIDE) && stepx_fits(cfg, batch, nwg)) {
      a.intra_plain = !(flags & KMR_DEVICE_SCOPE_STORES) &&
                      xcd_placement_ok(at<void>(ws, w.probe), (size_t)kMaxStepGroups * 4, nwg, st);
      return launch_stepx(cfg, a, nwg, (flags & KMR_COOPERATIVE) != 0, st);
    }
    return launch_step(cfg, a, nwg, (flags & KMR_COOPERATIVE) != 0, st);
  }
  float* x = at<float>(ws, w.x);
  enqueue_prep(cfg, static_cast<const uint16_t*>(model->embed), token_ids, finished, positions, x,
               batch, ws, w, st);
  for (int l = 0; l < cfg->n_layers; ++l)
    enqueue_layer(cfg, &model->layers[l], l, kv, x, cache_position, batch, ws, w, st, prefix_splits, inv);
  LmArgs la{};
  la.x = x; la.gain = static_cast<const uint16_t*>(model->final_norm);
  la.W = static_cast<const uint16_t*>(model->lm_head);
  la.logits = logits; la.part = at<float2>(ws, w.lm_part);
  la.V = cfg->vocab; la.K = cfg->hidden; la.B = batch; la.nblk = w.nblk_lm; la.eps = cfg->rms_eps;
  launch_lmhead(la, st, inv);
  LmFinishArgs f{};
  f.part = la.part; f.finished_in = finished; f.finished = finished; f.next = next_ids;
  f.cpos = cache_position; f.pos = positions;
  f.B = batch; f.nblk = w.nblk_lm; f.M = kv->max_len; f.pad_id = cfg->pad_id;
  f.eos_id = cfg->eos_id; f.flags = flags & KMR_ADVANCE;
  hipLaunchKernelGGL(k_lm_finish, dim3(batch), dim3(256), 0, st, f);
  return check_hip("decode_step launch");
}

int kmr_decode_step(const kmr_config* cfg, const kmr_model* model, const kmr_kv* kv,
                    const int32_t* token_ids, int32_t* positions, int32_t* cache_position,
                    uint8_t* finished, int32_t batch, int32_t* next_ids, float* logits,
                    uint32_t flags, void* ws, size_t ws_bytes, kmr_stream_t stream) {
  return decode_step(cfg, model, kv, token_ids, positions, cache_position, finished, batch, next_ids, logits,
                     flags, ws, ws_bytes, stream, 0);
}

int kmr_decode_step_static(const kmr_config* cfg, const kmr_model* model, const kmr_kv* kv,
                           const int32_t* token_ids, int32_t* positions, int32_t* cache_position,
                           uint8_t* finished, int32_t batch, int32_t* next_ids, float* logits,
                           uint32_t flags, kmr_stream_t stream) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if (!kv) return fail(KMR_EINVAL, "kv cache is NULL");
  if (batch <= 0 || batch > KMR_MAX_BATCH) return fail(KMR_EINVAL, "batch %d out of [1, %d]", batch, KMR_MAX_BATCH);
  if (kv->max_len <= 0) return fail(KMR_EINVAL, "kv cache max_len must be positive");
  const WsLayout w = ws_layout(cfg, batch, kv->max_len);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((rc = static_workspace(cfg, w, kv->max_len, (flags & KMR_CLEAR_WORKSPACE) != 0, st, &ws))) return rc;
  return decode_step(cfg, model, kv, token_ids, positions, cache_position, finished, batch, next_ids, logits,
                     flags & ~KMR_CLEAR_WORKSPACE, ws, (size_t)KMR_STATIC_WORKSPACE_BYTES, stream, 0);
}

int kmr_decode_step_prefix(const kmr_config* cfg, const kmr_model* model, const kmr_kv* kv,
                           const int32_t* token_ids, int32_t* positions, int32_t* cache_position,
                           uint8_t* finished, int32_t batch, int32_t* next_ids, float* logits,
                           uint32_t flags, int32_t shared_prefix, void* ws, size_t ws_bytes,
                           kmr_stream_t stream) {
  if (!kv) return fail(KMR_EINVAL, "kv is NULL");
  if (shared_prefix < 0 || shared_prefix > kv->max_len)
    return fail(KMR_EINVAL, "shared_prefix %d outside [0, max_len %d]", shared_prefix, kv->max_len);
  return decode_step(cfg, model, kv, token_ids, positions, cache_position, finished, batch, next_ids, logits,
                     flags | KMR_MULTI_KERNEL, ws, ws_bytes, stream, shared_prefix / kAttnSplitPP);
}

int kmr_prefill(const kmr_config* cfg, const kmr_model* model, const kmr_kv* kv, int32_t row,
                const int32_t* token_ids, const int32_t* positions, int32_t start, int32_t n_tokens,
                int32_t* next_id, float* logits, void* ws, size_t ws_bytes, kmr_stream_t stream) {
  int rc;
  if ((rc = check_config(cfg))) return rc;
  if (cfg->vocab <= 0) return fail(KMR_EINVAL, "vocab must be positive for a prefill");
  if (!kv) return fail(KMR_EINVAL, "kv cache is NULL");
  if (row < 0 || row >= kv->batch) return fail(KMR_EINVAL, "cache row %d out of [0, %d)", row, kv->batch);
  if (n_tokens <= 0 || start < 0 || (long long)start + n_tokens > kv->max_len)
    return fail(KMR_EINVAL, "tokens [%d, %lld) outside the cache [0, %d)", start, (long long)start + n_tokens,
                kv->max_len);
  if ((rc = check_kv(cfg, kv, 1))) return rc;
  if (kv->n_layers != cfg->n_layers) return fail(KMR_ESHAPE, "kv cache has %d layers, model %d", kv->n_layers, cfg->n_layers);
  if (!model || !model->embed || !model->final_norm || !model->lm_head || !model->layers)
    return fail(KMR_EINVAL, "model pointers are NULL");
  for (int l = 0; l < cfg->n_layers; ++l)
    if ((rc = check_layer(cfg, &model->layers[l]))) return fail(rc, "layer %d: %s", l, g_err);
  if (!token_ids || !positions || !next_id || !ws)
    return fail(KMR_EINVAL, "null token_ids/positions/next_id/workspace");
  // chunk: min(n_tokens, KMR_PREFILL_CHUNK) tokens, or the largest of 256, 128, .., 16
  // below that whose layout the workspace holds
  int C = n_tokens < KMR_PREFILL_CHUNK ? n_tokens : KMR_PREFILL_CHUNK;
  const size_t need = ws_layout(cfg, C, kv->max_len).total;
  while (ws_bytes < ws_layout(cfg, C, kv->max_len).total && C > 16) {
    int h = KMR_PREFILL_CHUNK / 2;
    while (h >= C) h /= 2;
    C = h;
  }
  const WsLayout w = ws_layout(cfg, C, kv->max_len);
  if (ws_bytes < w.total) return fail(KMR_ENOMEM, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  float* x = at<float>(ws, w.x);
  int32_t* pos_c = at<int32_t>(ws, w.pf);
  int32_t* cpos_c = pos_c + 3 * KMR_PREFILL_CHUNK;
  int n = 0;
  for (int t0 = 0; t0 < n_tokens; t0 += n) {
    n = n_tokens - t0 < C ? n_tokens - t0 : C;
    hipLaunchKernelGGL(k_prefill_rows, dim3(1), dim3(KMR_PREFILL_CHUNK), 0, st, positions, n_tokens, t0, n, start,
                       pos_c, cpos_c);
    enqueue_prep(cfg, static_cast<const uint16_t*>(model->embed), token_ids + t0, nullptr, pos_c, x, n, ws, w, st);
    bool pending = false;
    for (int l = 0; l < cfg->n_layers; ++l)
      enqueue_prefill_layer(cfg, &model->layers[l], l, kv, x, cpos_c, n, row, ws, w, st, pending);
    // the last layer's split-K partials: only the last token's hidden state is read
    // (by the lm_head after the last chunk); an earlier chunk's are dropped
    if (pending && t0 + n == n_tokens)
      hipLaunchKernelGGL(k_gemv_kreduce, dim3((cfg->hidden + 255) / 256), dim3(256), 0, st,
                         x + (size_t)(n - 1) * cfg->hidden, cfg->hidden,
                         at<const float>(ws, w.pkp) + (size_t)(n - 1) * cfg->hidden, n, cfg->hidden, 1);
  }
  // the next token from the last prompt token only
  LmArgs la{};
  la.x = x + (size_t)(n - 1) * cfg->hidden; la.gain = static_cast<const uint16_t*>(model->final_norm);
  la.W = static_cast<const uint16_t*>(model->lm_head);
  la.logits = logits; la.part = at<float2>(ws, w.lm_part);
  la.V = cfg->vocab; la.K = cfg->hidden; la.B = 1; la.nblk = w.nblk_lm; la.eps = cfg->rms_eps;
  launch_lmhead(la, st);
  LmFinishArgs f{};
  f.part = la.part; f.next = next_id; f.cpos = cpos_c; f.pos = pos_c;
  f.B = 1; f.nblk = w.nblk_lm; f.M = kv->max_len; f.pad_id = cfg->pad_id; f.eos_id = cfg->eos_id; f.flags = 0;
  hipLaunchKernelGGL(k_lm_finish, dim3(1), dim3(256), 0, st, f);
  return check_hip("prefill launch");
}

int kmr_kv_copy_row(const kmr_kv* dst, int32_t dst_row, const kmr_kv* src, int32_t src_row,
                    int32_t n_positions, kmr_stream_t stream) {
  if (!dst || !src || !dst->k || !dst->v || !src->k || !src->v) return fail(KMR_EINVAL, "null cache");
  if (dst->n_layers != src->n_layers || dst->n_kv_heads != src->n_kv_heads || dst->head_dim != src->head_dim)
    return fail(KMR_EINVAL, "caches differ in layers, kv heads or head_dim");
  if (dst->n_layers <= 0 || dst->n_kv_heads <= 0 || dst->head_dim <= 0 || dst->head_dim % 8)
    return fail(KMR_EINVAL, "bad cache dims");
  if (dst_row < 0 || dst_row >= dst->batch || src_row < 0 || src_row >= src->batch)
    return fail(KMR_EINVAL, "row outside its cache (dst %d of %d, src %d of %d)", dst_row, dst->batch,
                src_row, src->batch);
  const int lim = dst->max_len < src->max_len ? dst->max_len : src->max_len;
  if (n_positions < 0 || n_positions > lim)
    return fail(KMR_EINVAL, "n_positions %d outside [0, %d]", n_positions, lim);
  if (dst->k == src->k && dst_row == src_row) return fail(KMR_EINVAL, "row copied onto itself");
  if (n_positions == 0) return KMR_OK;
  KvCopyArgs a{};
  a.sk = static_cast<const uint16_t*>(src->k); a.sv = static_cast<const uint16_t*>(src->v);
  a.dk = static_cast<uint16_t*>(dst->k); a.dv = static_cast<uint16_t*>(dst->v);
  a.Hkv = dst->n_kv_heads; a.D = dst->head_dim; a.n = n_positions;
  a.sB = src->batch; a.sM = src->max_len; a.srow = src_row;
  a.dB = dst->batch; a.dM = dst->max_len; a.drow = dst_row;
  const size_t words = (size_t)n_positions * a.D / 8;
  const unsigned bx = (unsigned)std::min<size_t>((words + 255) / 256, 64);
  hipLaunchKernelGGL(k_kv_copy_row, dim3(bx, 2 * dst->n_layers * dst->n_kv_heads), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), a);
  return check_hip("kv row copy launch");
}

int kmr_slot_admit(int32_t* token_ids, int32_t* positions, int32_t* cache_position,
                   uint8_t* finished, int32_t batch, int32_t row, int32_t token,
                   const int32_t* pos, int32_t cache_pos, kmr_stream_t stream) {
  if (!token_ids || !positions || !cache_position || !finished || !pos) return fail(KMR_EINVAL, "null pointer");
  if (batch <= 0 || batch > KMR_MAX_BATCH || row < 0 || row >= batch)
    return fail(KMR_EINVAL, "row %d outside batch %d (at most %d)", row, batch, KMR_MAX_BATCH);
  if (cache_pos < 0 || pos[0] < 0 || pos[1] < 0 || pos[2] < 0)
    return fail(KMR_EINVAL, "negative cache position or position");
  hipLaunchKernelGGL(k_slot_set, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream), token_ids,
                     positions, cache_position, finished, batch, row, 1, token, pos[0], pos[1], pos[2],
                     cache_pos);
  return check_hip("slot admit launch");
}

int kmr_slot_retire(uint8_t* finished, int32_t batch, int32_t row, kmr_stream_t stream) {
  if (!finished) return fail(KMR_EINVAL, "null pointer");
  if (batch <= 0 || batch > KMR_MAX_BATCH || row < 0 || row >= batch)
    return fail(KMR_EINVAL, "row %d outside batch %d (at most %d)", row, batch, KMR_MAX_BATCH);
  hipLaunchKernelGGL(k_slot_set, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<int32_t*>(nullptr), static_cast<int32_t*>(nullptr),
                     static_cast<int32_t*>(nullptr), finished, batch, row, 0, 0, 0, 0, 0, 0);
  return check_hip("slot retire launch");
}

int kmr_read_probe(const void* buf, size_t bytes, uint32_t* sink, kmr_stream_t stream) {
  if (!buf || !sink) return fail(KMR_EINVAL, "null pointer");
  if (bytes < 16 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16)
    return fail(KMR_EINVAL, "buffer must be 16-byte aligned and a positive multiple of 16 bytes");
  hipLaunchKernelGGL(k_read_probe, dim3(KMR_READ_PROBE_THREADS / 256), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 16, sink);
  return check_hip("read probe launch");
}

int kmr_status(void* ws, kmr_stream_t stream, uint32_t* flags_out) {
  if (!ws || !flags_out) return fail(KMR_EINVAL, "null workspace or flags_out");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint32_t v = 0;
  if (hipMemcpyAsync(&v, ws, 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return check_hip("status read") ? KMR_EHIP : fail(KMR_EHIP, "status read failed");
  // every bit but KMR_STATUS_TIMEOUT is cleared; that one stays until kmr_workspace_init
  hipLaunchKernelGGL(k_status_keep, dim3(1), dim3(1), 0, st, static_cast<uint32_t*>(ws), (uint32_t)KMR_STATUS_TIMEOUT);
  *flags_out = v;
  return check_hip("status clear");
}

}  // extern "C"
