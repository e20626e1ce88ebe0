/*
 * kmr.h -- C ABI of the int4 weight-only decode step for MI355X (gfx950).
 *
 * What the step computes follows the kaminari page ("kaminari - a single-GPU
 * Qwen3-VL inference engine, explained"):
 *   - section 04, "3 . decode": one greedy token per call for every batch row,
 *     from fixed-rank inputs (token ids, 3-axis M-RoPE positions, cache position)
 *     and the full preallocated KV buffers; the argmax token stays on the device;
 *     finished rows keep their batch slot and are fed the pad id;
 *   - section 03 ("State model"): the static KV cache is the one buffer mutated in
 *     place; section 08 (ContinuousBatchScheduler): each row owns a physical cache
 *     row, so cache positions are per row here;
 *   - section 07: only the decoder's attention/MLP linears are int4 weight-only;
 *     embeddings, lm_head and norms stay bf16; int4 is explicit and never falls
 *     back silently;
 *   - attention is softmax(q K^T / sqrt(d)) V ("The Ghost in the Batch", "What
 *     Attention Does (60 Seconds)"); split partials are merged with the
 *     log-sum-exp weights stated there ("The merge math").
 *
 * Conventions for every entry point:
 *   - pointers are DEVICE pointers unless marked "host"; all memory is owned by
 *     the caller; the library never allocates or frees device memory;
 *   - every argument is checked on the host first; an invalid call returns a
 *     negative KMR_E* code and launches nothing (kmr_last_error() says why);
 *   - work is enqueued on the caller's stream, asynchronously; nothing
 *     synchronises except kmr_status();
 *   - bf16 values are stored as 16-bit patterns (uint16_t);
 *   - calls are reentrant given distinct workspaces; calls that share a
 *     workspace must be ordered on one stream.
 */
#ifndef KMR_H
#define KMR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t (a pointer to the runtime's stream object); NULL is
 * the null stream.  Declared here so that the header needs no HIP headers. */
struct ihipStream_t;
typedef struct ihipStream_t* kmr_stream_t;

enum {
  KMR_OK = 0,
  KMR_EINVAL = -1,       /* null pointer, non-positive size, bad index */
  KMR_ESHAPE = -2,       /* dims the kernels do not support (see kmr_config) */
  KMR_ENOMEM = -3,       /* caller buffer or workspace smaller than required */
  KMR_EHIP = -4          /* HIP runtime or launch error */
};

/* Sticky device-side status bits, read (and cleared) by kmr_status(). */
enum {
  KMR_STATUS_CACHE_POS = 1u,  /* a row's cache_position was outside [0, max_len):
                                 that row wrote nothing and its attention is zero */
  KMR_STATUS_TOKEN = 2u,      /* a token id was outside [0, vocab): that row's
                                 embedding was taken as zero */
  KMR_STATUS_TIMEOUT = 4u,    /* a wait inside the persistent step kernel gave up
                                 (no progress for ~1 s): that call wrote -1 to every
                                 next_ids entry and advanced nothing.  The bit is
                                 sticky: kmr_status reports it without clearing it,
                                 and every later persistent step on the workspace
                                 writes -1 again and does nothing else, until
                                 kmr_workspace_init re-initialises the workspace */
  KMR_STATUS_TOPOLOGY = 8u,   /* a work-group of the XCD-local step kernel read an XCD
                                 id above 7 or found more groups on its XCD than the
                                 grid deals to one (diagnostic; such a call may also
                                 time out) */
  KMR_STATUS_RANGE = 16u      /* a GEMV input exceeded the fp16 range in which the int4
                                 products take their activations: the outputs of that
                                 call are invalid.  The XCD-local persistent kernel
                                 stages residual-stream and MLP inputs scaled by 2^-3,
                                 so they reach it past |x * norm gain| or |SiLU(gate) up|
                                 of about 5.2e5; attention outputs, and the per-phase
                                 kernels' MLP activations, are staged unscaled (past
                                 65504); normalised inputs are bounded by sqrt(K)
                                 times the largest norm gain */
};

#define KMR_MAX_BATCH 64
#define KMR_STATIC_WORKSPACE_BYTES (48u << 20)  /* the array kmr_decode_step_static uses */
#define KMR_PREFILL_CHUNK 512   /* largest prompt chunk of kmr_prefill (tokens) */
#define KMR_ADVANCE 1u
#define KMR_MULTI_KERNEL 2u  /* run the step as one kernel per phase instead of the
                                single persistent kernel (diagnostics, cross-checks) */
#define KMR_DEVICE_WIDE 4u   /* persistent kernel with every hand-off device-wide,
                                instead of the XCD-local one (diagnostics, cross-checks) */
#define KMR_COOPERATIVE 8u   /* launch the persistent kernel with hipLaunchCooperativeKernel,
                                whose runtime guarantees that all its work-groups run at
                                once, instead of a plain launch after a host occupancy
                                check (~20 us more per step; for callers that run other
                                long kernels on the device concurrently).  Ignored on the
                                per-phase path. */
#define KMR_BATCH_INVARIANT 16u  /* one arithmetic form for every batch size, so that a
                                row's next id, logits and cache writes are bit for bit the
                                same whatever other rows share its batch ("The Ghost in the
                                Batch", "The Fork in the Code" and "The Fix: Three Options":
                                a kernel choice that depends on the batch changes a row's
                                bits).  The step then runs on the per-phase kernels with the
                                matrix-core int4 GEMV for every 16-row tile (padded; used when
                                group_size and the GEMV K are multiples of 128, else the VALU
                                GEMV in 8-row tiles), the matrix-core lm_head for every tile
                                (hidden 2048; else the VALU lm_head in 8-row tiles), no
                                split-K and the separate split-merge kernel: the form depends
                                on the model shapes only.  Without this flag the default
                                path takes the fastest form for the batch, and a row's
                                results agree across batch sizes within the parity
                                tolerance but not bit for bit (the persistent kernel for
                                batch 1..4, the VALU GEMV tiles for 5..8, the matrix-core
                                tiles from 9). */
#define KMR_DEVICE_SCOPE_STORES 32u  /* XCD-local persistent kernel with every hand-off
                                through device-scope stores, as it runs under stream capture
                                or without a verified placement (cross-checks) */
#define KMR_CLEAR_WORKSPACE 64u  /* kmr_decode_step_static only: clear its static array
                                (a fill kernel) before the step, as kmr_workspace_init clears a
                                workspace; needed after a step that wrote -1 (KMR_EINVAL on the
                                calls that take a workspace) */
#define KMR_TEST_STALL 256u  /* failure-path tests only: the persistent kernel's consumers
                                wait for hand-off tags that no producer writes and give up
                                after 4096 polls, so every work-group exits through its
                                bounded wait and the call ends with KMR_STATUS_TIMEOUT */

/*
 * Model dimensions.  Supported by the kernels: head_dim 64 or 128;
 * n_heads % n_kv_heads == 0 with n_heads / n_kv_heads in {1, 2, 4}; group_size a multiple
 * of 32 dividing hidden, n_heads*head_dim and intermediate;
 * mrope_section[0]+[1]+[2] == head_dim / 2.  Anything else is KMR_ESHAPE.
 */
typedef struct {
  int32_t hidden, n_heads, n_kv_heads, head_dim, intermediate, vocab, n_layers, group_size;
  float rms_eps;             /* RMSNorm epsilon (1e-6 for the Qwen3 family) */
  double rope_theta;         /* RoPE base (5e6 for the Qwen3-VL text decoder) */
  int32_t mrope_section[3];  /* frequency pairs on the t, h, w axes */
  int32_t mrope_interleaved; /* 1: pair j on h if j%3==1 and j<3*s_h, on w if j%3==2 and
                                j<3*s_w, else t; 0: contiguous [t | h | w] blocks */
  int32_t pad_id;            /* token fed to, and emitted by, finished rows */
  int32_t eos_id;            /* token that finishes a row under KMR_ADVANCE; -1: none */
} kmr_config;

/* One int4 matrix of N rows by K columns, as written by kmr_quantize_int4:
 * packed u8 [N][K/2] (byte j of a row holds column 2j in its low nibble and 2j+1
 * in its high nibble) and sz bf16 [N][K/group][2] (scale, zero). */
typedef struct {
  const void* packed;
  const void* sz;
  int32_t N, K;
} kmr_qweight;

/* One decoder layer.  Row order of the fused matrices: qkv = [q heads; k heads;
 * v heads] (N = (n_heads + 2 n_kv_heads) head_dim, K = hidden); o (N = hidden,
 * K = n_heads head_dim); gate_up = [gate; up] (N = 2 intermediate, K = hidden);
 * down (N = hidden, K = intermediate).  Gains are bf16: in_norm/post_norm
 * [hidden], q_norm/k_norm [head_dim]. */
typedef struct {
  const void *in_norm, *q_norm, *k_norm, *post_norm;
  kmr_qweight qkv, o, gate_up, down;
} kmr_layer;

/* The whole decoder: bf16 embed [vocab][hidden], final_norm [hidden], untied
 * lm_head [vocab][hidden]; layers is a HOST array of n_layers entries. */
typedef struct {
  const void *embed, *final_norm, *lm_head;
  const kmr_layer* layers;
} kmr_model;

/* Static KV cache bound to caller memory: k and v are bf16
 * [n_layers][batch][n_kv_heads][max_len][head_dim] each. */
typedef struct {
  void *k, *v;
  int32_t n_layers, batch, n_kv_heads, max_len, head_dim;
  size_t bytes;  /* total bytes of k and v together */
} kmr_kv;

/*
 * kmr_kv_alloc -- size or bind a preallocated static KV cache (kaminari section
 * 03: StaticKVCache, preallocated and slot-addressable).
 * With buf == NULL only out->bytes is filled (a size query).  Otherwise buf (at
 * least out->bytes, 256-byte aligned) is split into k and v; zero_fill != 0 clears
 * it on `stream` with a fill kernel.  Returns KMR_ENOMEM if buf_bytes is short.
 */
int kmr_kv_alloc(const kmr_config* cfg, int32_t batch, int32_t max_len, void* buf,
                 size_t buf_bytes, int32_t zero_fill, kmr_stream_t stream, kmr_kv* out);

/*
 * kmr_quantize_int4 -- group-wise asymmetric int4 quantization of one bf16
 * matrix w [N][K] (kaminari section 07: offline weight-only int4 of the decoder
 * linears; the pages give no formula).  Per row and per group of `group`
 * consecutive columns, in IEEE fp32 in this order, with no fused multiply-add:
 *     s = bf16_rne(max((max - min) / 15, 2^-24)),  z = bf16_rne(min + 8 s),
 *     q = clamp(rne((w - z) / s) + 8, 0, 15),   so that w ~ (q - 8) s + z.
 * Writes packed [N][K/2] and sz [N][K/group][2] in the kmr_qweight layout.
 * group must be even and divide K (KMR_ESHAPE otherwise).
 */
int kmr_quantize_int4(const void* w_bf16, int32_t N, int32_t K, int32_t group, void* packed,
                      void* sz, kmr_stream_t stream);

/* Bytes of workspace the decode calls need for this config, batch and max_len. */
size_t kmr_workspace_bytes(const kmr_config* cfg, int32_t batch, int32_t max_len);
/* The workspace kmr_prefill needs to run a prompt of n_tokens in chunks of
 * min(n_tokens, KMR_PREFILL_CHUNK) tokens; 0 for an invalid config or size.  A
 * workspace sized for fewer tokens makes kmr_prefill take smaller chunks. */
size_t kmr_prefill_workspace_bytes(const kmr_config* cfg, int32_t n_tokens, int32_t max_len);

/* Diagnostic (no device work): 1 if kmr_decode_step would run this config at this
 * batch on the XCD-local persistent kernel with n_groups work-groups (the number of
 * compute units), 0 if not, -1 for an invalid config or size.  Lets a host-side test
 * enumerate the shapes the kernel accepts and check its loaders' addresses. */
int kmr_debug_stepx_fits(const kmr_config* cfg, int32_t batch, int32_t n_groups);

/* Clears a workspace with a fill kernel on `stream`.  Call once after allocating
 * it, and again after a call that returned an error or raised KMR_STATUS_TIMEOUT;
 * the decode and prefill calls otherwise leave it ready for the next call.  One
 * workspace may serve calls of any kind and batch size on the same config and
 * max_len, as long as it is large enough for each: the words that persist between
 * calls (status, step counter, arrival counters) sit in a fixed header, and the
 * persistent kernels' exchange buffers at offsets that do not depend on the batch.
 * The first call on a device also records where the device places the
 * work-groups of a one-group-per-CU grid (a small probe kernel into the workspace
 * and a synchronous copy of one word per CU). */
int kmr_workspace_init(void* ws, size_t ws_bytes, kmr_stream_t stream);

/*
 * kmr_decode_layer -- one decoder layer for `batch` rows (kaminari page, section 03
 * "Architecture overview": the DecoderLayer of model/modules.py, fused-QKV attention
 * with GQA and 3D M-RoPE, then the MLP; section 05 "The native model port"), in place
 * on hidden_inout (fp32 [batch][hidden]):
 *   h = RMSNorm(x; in_norm); [q|k|v] = W_qkv h; per head q, k <- MRoPE(RMSNorm(.; q/k_norm));
 *   K/V of layer `layer`, row b, slot cache_position[b] <- bf16(k), bf16(v);
 *   o = attention of each q head over slots 0..cache_position[b] of its kv head
 *       (q head h reads kv head h / (n_heads / n_kv_heads));
 *   x += W_o o; x += W_down (silu(gate) * up) with [gate|up] = W_gate_up RMSNorm(x; post_norm).
 * positions: int32 [3][batch] (t, h, w); cache_position: int32 [batch].
 * The cache slot cache_position[b] of layer `layer` is the only cache memory
 * written.  A row whose cache_position is out of range sets KMR_STATUS_CACHE_POS.
 */
int kmr_decode_layer(const kmr_config* cfg, const kmr_layer* layer_w, int32_t layer,
                     const kmr_kv* kv, float* hidden_inout, const int32_t* positions,
                     const int32_t* cache_position, int32_t batch, void* ws, size_t ws_bytes,
                     kmr_stream_t stream);

/*
 * kmr_decode_step -- one greedy decode step of the whole decoder for `batch`
 * rows (kaminari section 04, "3 . decode"):
 *   x = embed[id] (id = pad_id for rows with finished[b] != 0), all layers as in
 *   kmr_decode_layer, RMSNorm(x; final_norm), logits = lm_head x (fp32 accumulate),
 *   next_ids[b] = lowest index of the largest logit (pad_id for finished rows).
 * logits: fp32 [batch][vocab] or NULL (written only when given).
 * finished: uint8 [batch] or NULL (no row finished).
 * flags & KMR_ADVANCE: on the device, after the argmax, each unfinished row
 *   whose token is eos_id, or whose cache_position + 1 would reach max_len, is
 *   marked finished (if `finished` is given); every other unfinished row gets
 *   cache_position[b] += 1 and all three positions += 1.  This lets the caller
 *   feed next_ids back as token_ids and replay the step with no host work.
 * Nothing is synchronised: next_ids is valid once `stream` reaches this point,
 * except that a device's first decode call that picks the XCD-local persistent
 * kernel runs the placement probe of kmr_workspace_init (synchronising `stream`
 * once) if no kmr_workspace_init ran on that device; under stream capture the
 * probe is skipped and the kernel keeps every hand-off device-wide.
 * Paths: batch <= 4 with the model shapes the persistent kernels cover runs as one
 * launch of a persistent kernel (XCD-local hand-offs when n_kv_heads is a multiple of
 * 8, else or with KMR_DEVICE_WIDE device-wide ones; its work-groups wait on each other
 * with bounded waits, so other work that holds CUs for longer than ~1 s ends the call
 * with KMR_STATUS_TIMEOUT unless KMR_COOPERATIVE is set); otherwise, or with KMR_MULTI_KERNEL,
 * as one kernel per phase, in batch tiles of at most 16 rows (batch up to
 * KMR_MAX_BATCH).  A tile of 9..16 rows takes the matrix-core int4 GEMV when the
 * group size is a multiple of 128, and the matrix-core lm_head when hidden is
 * 2048; the choice depends on the shapes and the tile size only.  So the
 * arithmetic of a row changes where the batch crosses 4/5 and 8/9 (within the
 * parity tolerance); KMR_BATCH_INVARIANT pins one form for every batch size.
 */
int kmr_decode_step(const kmr_config* cfg, const kmr_model* model, const kmr_kv* kv,
                    const int32_t* token_ids, int32_t* positions, int32_t* cache_position,
                    uint8_t* finished, int32_t batch, int32_t* next_ids, float* logits,
                    uint32_t flags, void* ws, size_t ws_bytes, kmr_stream_t stream);

/*
 * kmr_decode_step_static -- kmr_decode_step without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The workspace is a static array of
 * KMR_STATIC_WORKSPACE_BYTES in the library's device code, one per device, held
 * until the process ends; this call allocates nothing.  Same arguments, kernels
 * and results as kmr_decode_step.  KMR_ENOMEM when kmr_workspace_bytes(cfg, batch,
 * kv->max_len) exceeds the array (48 MiB: every batch up to KMR_MAX_BATCH at
 * max_len 8192 for the Qwen3-VL-2B text decoder).  The array keeps the last call's
 * contents: when the layout (config, max_len or batch-dependent size) differs from
 * the previous call's on the device, the call first clears it with a fill kernel
 * on `stream` (recorded too if the call is captured).  All calls on one device
 * share the array, so calls that overlap in time on one device race and must be
 * ordered by the caller (one stream).  Its status bits are not readable; a step
 * whose waits gave up writes -1 to next_ids, as kmr_decode_step does, and so do
 * later persistent steps until a call with KMR_CLEAR_WORKSPACE (or another layout)
 * clears the array.
 */
int kmr_decode_step_static(const kmr_config* cfg, const kmr_model* model, const kmr_kv* kv,
                           const int32_t* token_ids, int32_t* positions, int32_t* cache_position,
                           uint8_t* finished, int32_t batch, int32_t* next_ids, float* logits,
                           uint32_t flags, kmr_stream_t stream);

/*
 * kmr_decode_step_prefix -- kmr_decode_step with shared-prefix (cascade) attention
 * ("The Ghost in the Batch", cascade attention: a prefix common to many requests
 * is read once for all of them, then merged with each request's own suffix).
 * The caller promises that every row holds the same K/V in cache positions
 * [0, shared_prefix) of every layer (row 0 is the one read).  The step runs on the
 * per-phase kernels; the attention splits of 256 positions that lie wholly inside
 * the prefix are computed once per (split, kv head) for every row whose
 * cache_position is past them, with the same operations as the plain path, so
 * next_ids, logits and the cache are bit for bit those of kmr_decode_step with
 * KMR_MULTI_KERNEL; only the prefix K/V reads shrink.  It is an explicit call:
 * the library never switches to it by itself.  shared_prefix = 0 is the plain
 * per-phase step.  KMR_EINVAL: shared_prefix outside [0, kv->max_len], and every
 * error of kmr_decode_step.
 */
int kmr_decode_step_prefix(const kmr_config* cfg, const kmr_model* model, const kmr_kv* kv,
                           const int32_t* token_ids, int32_t* positions, int32_t* cache_position,
                           uint8_t* finished, int32_t batch, int32_t* next_ids, float* logits,
                           uint32_t flags, int32_t shared_prefix, void* ws, size_t ws_bytes,
                           kmr_stream_t stream);

/*
 * kmr_prefill -- the prompt of one sequence through the decoder (kaminari page,
 * section 04: the prompt's forward fills the static cache, and the first generated
 * token is the argmax of the logits at the last prompt token).
 * token_ids [n_tokens] and positions [3][n_tokens] (t, h, w axis-major, int32) are
 * device arrays; token i takes cache position start + i of cache row `row`, so the
 * call writes that row's K/V slots [start, start + n_tokens) in every layer and
 * reads its slots [0, start) as an earlier part of the same sequence.  Each token
 * attends causally to the slots up to its own.  No other slot or row is touched.
 * next_id [1] receives the argmax at the last token; logits [vocab] fp32 receives
 * that token's logits if not NULL.
 * The tokens run in chunks through the layers: per layer and chunk, the q/k/v,
 * o, gate/up and down projections as matrix-core int4 GEMMs over the whole chunk
 * (group_size a multiple of 128 and hidden, n_heads*head_dim and intermediate
 * multiples of 512; otherwise the decode path's GEMV tiles), the chunk's K/V slots
 * written first and then causal attention over the row's slots 0 .. each token's
 * own.  The chunk is min(n_tokens, KMR_PREFILL_CHUNK) tokens when the workspace
 * holds its layout, else the largest of 256, 128, 64, 32, 16 tokens below that
 * which it holds (KMR_ENOMEM if none).
 * ws must hold kmr_prefill_workspace_bytes(cfg, n_tokens, max_len) bytes (or the
 * bytes of a smaller chunk) and have been initialised once.  Returns KMR_EINVAL for a row outside the
 * cache, n_tokens < 1, or start + n_tokens > max_len, before anything is launched;
 * token ids outside [0, vocab) raise KMR_STATUS_TOKEN as in kmr_decode_step.
 * Nothing is synchronised.
 */
int kmr_prefill(const kmr_config* cfg, const kmr_model* model, const kmr_kv* kv, int32_t row,
                const int32_t* token_ids, const int32_t* positions, int32_t start, int32_t n_tokens,
                int32_t* next_id, float* logits, void* ws, size_t ws_bytes, kmr_stream_t stream);

/*
 * Slot operations of a continuous-batching scheduler (kaminari section 08: the
 * ContinuousBatchScheduler admits requests into free DecodeSlots, each pinned to a
 * physical row of one shared static cache, ticks the active slots one token at a
 * time and finalizes a row the moment it finishes; copy_row_from moves a row's KV
 * state into another row).  All three run on `stream` without a host round trip
 * and allocate nothing.
 *
 * kmr_kv_copy_row -- for every layer and kv head, copies positions
 * [0, n_positions) of row src_row of `src` (K and V) to row dst_row of `dst`,
 * bit for bit; every other position and row of dst is left unchanged.  dst and
 * src may be the same cache (rows must then differ) or two caches with equal
 * n_layers, n_kv_heads and head_dim (batch and max_len may differ).
 * KMR_EINVAL: null pointers, a row outside its cache, n_positions outside
 * [0, min(dst->max_len, src->max_len)], unequal dims, or a row copied onto
 * itself.  n_positions == 0 launches nothing.
 */
int kmr_kv_copy_row(const kmr_kv* dst, int32_t dst_row, const kmr_kv* src, int32_t src_row,
                    int32_t n_positions, kmr_stream_t stream);

/*
 * kmr_slot_admit -- makes row `row` of a batch of `batch` live for the next
 * kmr_decode_step: token_ids[row] = token, positions[a * batch + row] = pos[a] for
 * the t, h, w axes a = 0, 1, 2 (pos is a HOST array of 3), cache_position[row] =
 * cache_pos, finished[row] = 0.  The cache row itself is not touched (fill it
 * with a prefill or kmr_kv_copy_row first).  KMR_EINVAL: null pointers, row
 * outside [0, batch), batch outside [1, KMR_MAX_BATCH], a negative cache_pos or
 * position.  (A cache_pos at or past the cache's max_len is caught by the step,
 * which raises KMR_STATUS_CACHE_POS.)
 */
int kmr_slot_admit(int32_t* token_ids, int32_t* positions, int32_t* cache_position,
                   uint8_t* finished, int32_t batch, int32_t row, int32_t token,
                   const int32_t* pos, int32_t cache_pos, kmr_stream_t stream);

/*
 * kmr_slot_retire -- finished[row] = 1: from the next step on the row is fed the
 * pad id, emits the pad id and keeps its cache position and positions frozen.
 * KMR_EINVAL: null pointer, row outside [0, batch), batch outside [1, KMR_MAX_BATCH].
 */
int kmr_slot_retire(uint8_t* finished, int32_t batch, int32_t row, kmr_stream_t stream);

/* Measurement: reads `bytes` (a positive multiple of 16; buf 16-byte aligned) of
 * device memory with the 16-byte non-temporal loads the int4 GEMVs stream their
 * weights with, on a grid of KMR_READ_PROBE_THREADS threads, each writing one word
 * to sink (uint32 [KMR_READ_PROBE_THREADS]).  Timed over a buffer much larger than
 * the 256 MB Infinity Cache, it gives the device's achievable streaming-read rate,
 * the practical ceiling of the bandwidth-bound decode step. */
#define KMR_READ_PROBE_THREADS (256 * 8 * 256)
int kmr_read_probe(const void* buf, size_t bytes, uint32_t* sink, kmr_stream_t stream);

/* Synchronises `stream`, returns the sticky KMR_STATUS_* bits of `ws` in
 * *flags_out (host pointer) and clears them, except KMR_STATUS_TIMEOUT, which
 * only kmr_workspace_init clears. */
int kmr_status(void* ws, kmr_stream_t stream, uint32_t* flags_out);

/* Message for a KMR_E* code, and the detail of this thread's last failed call. */
const char* kmr_strerror(int code);
const char* kmr_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KMR_H */
