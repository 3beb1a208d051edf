/*
 * gqa_attn.h -- C ABI of the MI355X (gfx950) grouped-query attention forward library.
 *
 * One operation family: scaled-dot-product attention in which Hq query heads share Hkv key/value
 * heads (multi-head when Hkv == Hq, multi-query when Hkv == 1, grouped-query in between).
 *
 * What is computed (sources are the pages this library follows):
 *   - Query head i reads key/value head i / (Hq / Hkv): queries are grouped in contiguous blocks,
 *     never round-robin (GQA lab page "Transformer -- attention by hand: reducing only the
 *     key/value heads", steps 1 and 3; course page "Week 7. Attention", typical errors).
 *   - For every query row: dot with every visible key row of its group's head, multiplied by
 *     `scale` (normally 1/sqrt(d): lab step 4, course step 1), minus the row maximum, exponentiated,
 *     normalised, and used to average the value rows (lab step 4).
 *   - causal != 0: keys after the query's position are removed before the softmax (course step 1).
 *     With Tq < Tkv the queries are the last Tq positions (query t sits at t + Tkv - Tq); a
 *     one-token decode therefore sees the whole cache.
 *   - gqa_fold_kv: position-wise mean of the key/value heads inside each contiguous group (lab
 *     step 2), the head reduction GQA applies to a multi-head checkpoint.
 *
 * Conventions shared by every entry point:
 *   - Tensors are dense, row-major device buffers in the [batch, position, head, head_dim] layout
 *     with head_dim contiguous; all pointers must be 16-byte aligned.
 *   - The caller owns every buffer. The library allocates no device memory at run time (its one
 *     fixed array, the decode scratch of gqa_attn_decode_noalloc, is part of the loaded code
 *     object), keeps no pointer after returning, and never synchronises: all work is enqueued
 *     on `stream` (a HIP stream, NULL for the default stream) and completes asynchronously.
 *   - Arguments are validated before anything is enqueued; on an error status nothing has been
 *     written. Outputs must not overlap inputs. No C++ exception crosses this interface.
 *   - Thread-safe: the only mutable global state is the table of per-GPU addresses of the
 *     decode scratch array (gqa_attn_decode_noalloc), filled once per device under a mutex.
 *   - `scale` multiplies every score. Pass a finite positive value, or GQA_SCALE_DEFAULT (0) for
 *     1/sqrt(d), the factor both the GQA lab page (step 4: scores divided by the square root of
 *     the head dimension) and the course page (step 1) use; the library then computes it as
 *     (float)(1 / sqrt((double)d)). A negative or non-finite scale is GQA_ERR_SHAPE.
 *   - Internal arithmetic is fp32 (bf16 inputs are widened exactly; products accumulate in fp32);
 *     outputs are rounded to nearest-even in the input dtype.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_OK = 0,
  GQA_ERR_NULL_PTR = 1,    /* a required pointer is NULL */
  GQA_ERR_SHAPE = 2,       /* a size is non-positive or inconsistent, or causal with Tq > Tkv */
  GQA_ERR_GROUPING = 3,    /* Hq is not divisible by Hkv (or H by g): heads do not split evenly */
  GQA_ERR_UNSUPPORTED = 4, /* (dtype, d) combination not built, or a pointer not 16-byte aligned */
  GQA_ERR_WORKSPACE = 5,   /* decode workspace missing or smaller than required */
  GQA_ERR_HIP = 6,         /* the HIP runtime reported an error when enqueueing */
  GQA_ERR_ALIAS = 7        /* an output buffer overlaps an input buffer */
} gqa_status_t;

/* `scale` value that selects 1/sqrt(d) (GQA lab page, step 4; course page, step 1). */
#define GQA_SCALE_DEFAULT 0.0f

typedef enum { GQA_DTYPE_F32 = 0, GQA_DTYPE_BF16 = 1 } gqa_dtype_t;

/* Supported head dimensions: bf16 d in {64, 128}; f32 d in {16, 32, 64, 128}. */

/*
 * Prefill (any number of query positions).
 *   q   [B, Tq, Hq, d]     k, v [B, Tkv, Hkv, d]     out [B, Tq, Hq, d]     (all `dtype`)
 * Packed variable-length batch: pass cu_seqlens != NULL, a DEVICE int32 array of B+1 cumulative
 * sequence offsets (cu_seqlens[0] == 0, non-decreasing, cu_seqlens[B] == Tq). Then the tensors
 * are q [1, Tq, Hq, d], k, v [1, Tkv, Hkv, d] with Tq == Tkv == total tokens; each sequence
 * attends only to itself (causal within the sequence when causal != 0), and max_seqlen (host)
 * must be >= the longest sequence: it sizes the launch grid. With cu_seqlens == NULL, max_seqlen
 * is ignored.
 */
gqa_status_t gqa_attn_prefill(const void* q, const void* k, const void* v, void* out, int B,
                              int Tq, int Tkv, int Hq, int Hkv, int d, float scale, int causal,
                              const int32_t* cu_seqlens, int max_seqlen, gqa_dtype_t dtype,
                              hipStream_t stream);

/*
 * Options of the extended entry points (course page "Week 7. Attention", step 3). A NULL
 * options pointer means all defaults (no window, no rotation).
 *   window, n_sink: causal sliding window and sink keys, as for gqa_attn_prefill_window
 *                   (needs causal != 0 in gqa_attn_prefill_ex).
 *   rope_cos, rope_sin: rotary position embedding, DEVICE fp32 tables [rope_rows][d/2], row p
 *                   holding cos / sin of p * theta_i (theta_i = base^(-2i/d) normally; any table
 *                   is accepted). Coordinates (2i, 2i+1) form one pair (a complex number turned
 *                   by p * theta_i). Both NULL: no rotation; exactly one NULL: GQA_ERR_NULL_PTR.
 *                   16-byte aligned. Prefill turns query t at position t + (Tkv - Tq) and key j
 *                   at position j (per sequence in a packed batch), inside the kernel; decode
 *                   turns the query at position cache_lens[b] - 1 and expects the cache to hold
 *                   keys already turned at their positions.
 *   rope_rows:      rows of the tables; must cover every position used (>= Tkv, >= max_seqlen
 *                   for packed batches, >= Tmax for decode), else GQA_ERR_SHAPE.
 *   q_norm_w, k_norm_w, norm_eps: QK-norm (course page, step 3: RMSNorm of q and k before the
 *                   dot product). Every query and key head row x becomes
 *                   x * w / sqrt(mean(x^2) + norm_eps), w the DEVICE fp32 weights [d] (16-byte
 *                   aligned), applied before the rotation. Both NULL: no norm; exactly one
 *                   NULL: GQA_ERR_NULL_PTR; norm_eps must be finite and > 0 (else GQA_ERR_SHAPE).
 *                   Prefill normalises queries at load and keys as they are staged; decode
 *                   normalises the query and expects the cache to hold normalised keys
 *                   (k_norm_w may then be NULL).
 *   keys_prepared:  nonzero: the keys were already normalised and turned (gqa_prepare_keys, or
 *                   a cache written that way); prefill then applies QK-norm and rotation to the
 *                   queries only and k_norm_w may be NULL. Every workgroup stages every key tile
 *                   of its head, so preparing the keys once and passing keys_prepared is faster
 *                   than turning them inside the attention kernel.
 * Windows, rotation and QK-norm are bf16 only (GQA_ERR_UNSUPPORTED for f32).
 */
typedef struct {
  int window;
  int n_sink;
  const float* rope_cos;
  const float* rope_sin;
  int rope_rows;
  float* lse; /* optional OUTPUT (prefill only): DEVICE fp32 [B, Tq, Hq] ([1, total, Hq] when
                 packed), the natural-log log-sum-exp of each row's scaled scores, as
                 gqa_attn_backward needs it; NULL: not written */
  const float* q_norm_w;
  const float* k_norm_w;
  float norm_eps;
  int keys_prepared;
} gqa_attn_options_t;

/* gqa_attn_prefill with options (window, sinks, rotary embedding). */
gqa_status_t gqa_attn_prefill_ex(const void* q, const void* k, const void* v, void* out, int B,
                                 int Tq, int Tkv, int Hq, int Hkv, int d, float scale, int causal,
                                 const int32_t* cu_seqlens, int max_seqlen,
                                 const gqa_attn_options_t* options, gqa_dtype_t dtype,
                                 hipStream_t stream);

/*
 * Prefill with a causal sliding window and attention sinks (course page "Week 7. Attention",
 * step 3: the window bounds what each query sees; the first tokens stay visible as sinks).
 * Same tensors, layout, packing and errors as gqa_attn_prefill with causal = 1; the query at
 * position p (bottom-right aligned, as there) sees key j iff j <= p and (j > p - window or
 * j < n_sink). window = 0 means no window (plain causal attention; n_sink is then irrelevant);
 * window and n_sink must be >= 0 (else GQA_ERR_SHAPE). bf16 only (else GQA_ERR_UNSUPPORTED).
 * Only the sink and window key tiles are read.
 */
gqa_status_t gqa_attn_prefill_window(const void* q, const void* k, const void* v, void* out,
                                     int B, int Tq, int Tkv, int Hq, int Hkv, int d, float scale,
                                     int window, int n_sink, const int32_t* cu_seqlens,
                                     int max_seqlen, gqa_dtype_t dtype, hipStream_t stream);

/*
 * Key preparation (course page "Week 7. Attention", step 3): QK-norm (opt->k_norm_w, norm_eps)
 * and then the rotary turn (opt->rope_cos / rope_sin / rope_rows) of every key row, once, as a
 * model writes its key cache. k, k_out [B, T, Hkv, d] bf16 (packed: [1, T = total, Hkv, d] with
 * B + 1 offsets in cu_seqlens and the longest sequence in max_seqlen); key j of a sequence sits
 * at position pos0 + j (rope_rows must cover pos0 + the longest length). k_out == k (in place)
 * is allowed, any other overlap is GQA_ERR_ALIAS. At least one of the norm and the turn must be
 * requested (else GQA_ERR_SHAPE); the other options fields are ignored. bf16, d in {64, 128}.
 * Feeds gqa_attn_prefill_ex / gqa_attn_decode_ex with opt->keys_prepared set.
 */
gqa_status_t gqa_prepare_keys(const void* k, void* k_out, int B, int T, int Hkv, int d,
                              const int32_t* cu_seqlens, int max_seqlen, int pos0,
                              const gqa_attn_options_t* options, gqa_dtype_t dtype,
                              hipStream_t stream);

/*
 * Grouped value attention, prefill (K3 notes, section 4, GVA: the inverse of grouped-query
 * sharing). H query/key heads serve HV = G*H value heads; value head j is attended with
 * query/key head j / G (contiguous groups: the notes repeat q and k with repeat_interleave)
 * and keeps its own values:
 *   out[b,t,j,:] = softmax_keys(scale * q[b,t,j/G,:] . k[b,:,j/G,:]) v[b,:,j,:]
 *   q [B, Tq, H, d]   k [B, Tkv, H, d]   v [B, Tkv, HV, d]   out [B, Tq, HV, d]
 * (packed batches: [1, total, ., d] with cu_seqlens, as for gqa_attn_prefill.) The scores of a
 * query/key head are computed once for each 128 value columns of its G value heads (G*d a
 * multiple of 128), otherwise once per value head. Options: window, n_sink and lse ([B, Tq, H]:
 * one log-sum-exp per query/key head) as for gqa_attn_prefill_ex; rotary tables are not
 * supported here (GQA_ERR_UNSUPPORTED). bf16 only, d in {64, 128} (else GQA_ERR_UNSUPPORTED).
 * HV not a multiple of H is GQA_ERR_GROUPING; other errors as for gqa_attn_prefill.
 */
gqa_status_t gqa_attn_prefill_gva(const void* q, const void* k, const void* v, void* out, int B,
                                  int Tq, int Tkv, int H, int HV, int d, float scale, int causal,
                                  const int32_t* cu_seqlens, int max_seqlen,
                                  const gqa_attn_options_t* options, gqa_dtype_t dtype,
                                  hipStream_t stream);

/*
 * Decode: one query token per sequence against a key/value cache, split along the cache length.
 *   q [B, 1, Hq, d]     k_cache, v_cache [B, Tkv, Hkv, d]     out [B, 1, Hq, d]
 * Each split writes an fp32 partial result (running max, sum and unnormalised output) to
 * `workspace`, and a second kernel merges the splits. `workspace` is caller-owned device memory
 * of at least gqa_attn_decode_workspace_bytes(B, Tkv, Hq, d) bytes (or the exact figure
 * gqa_attn_decode_workspace_bytes_hkv(B, Tkv, Hq, Hkv, d)), 16-byte aligned; its contents on
 * entry do not matter and are overwritten. Concurrent calls must use distinct workspaces.
 * `causal` is accepted for symmetry with prefill: a single query at the last position sees the
 * whole cache, so it changes nothing. bf16 uses the split-KV kernels; f32 runs the prefill
 * kernel with Tq = 1 and needs no workspace (workspace may then be NULL).
 *
 * gqa_attn_decode_workspace_bytes: an upper bound valid for every Hkv that divides Hq (the
 * split count, and so the fp32 partials [B, Hq, splits, d + 2], depends on Hkv); 0 for
 * non-positive sizes. gqa_attn_decode_workspace_bytes_hkv: the exact requirement for one Hkv
 * (0 for non-positive sizes or Hq not divisible by Hkv); never above the bound.
 */
size_t gqa_attn_decode_workspace_bytes(int B, int Tkv, int Hq, int d);
size_t gqa_attn_decode_workspace_bytes_hkv(int B, int Tkv, int Hq, int Hkv, int d);
gqa_status_t gqa_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                             int B, int Tkv, int Hq, int Hkv, int d, float scale, int causal,
                             void* workspace, size_t workspace_bytes, gqa_dtype_t dtype,
                             hipStream_t stream);

/*
 * Decode that allocates nothing, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation). Same arguments,
 * layout, result and errors as gqa_attn_decode, without the workspace: the split partials go to
 * a fixed scratch array of GQA_DECODE_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends (its address is taken once per device, on the first call there).
 * A call whose partials would not fit (gqa_attn_decode_workspace_bytes_hkv(...) larger than
 * GQA_DECODE_SCRATCH_BYTES) returns GQA_ERR_WORKSPACE and enqueues nothing. Every call on one
 * GPU shares that GPU's scratch: calls that overlap in time on the same GPU (different streams
 * or threads without ordering between them) race and must be serialised by the caller. The
 * scratch needs no clearing between calls. f32 needs no scratch, as for gqa_attn_decode.
 */
#define GQA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)
gqa_status_t gqa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                     void* out, int B, int Tkv, int Hq, int Hkv, int d,
                                     float scale, int causal, gqa_dtype_t dtype,
                                     hipStream_t stream);

/*
 * Decode against a ragged cache, optionally with a sliding window and sinks (course page
 * "Week 7. Attention", step 3).
 *   q [B, 1, Hq, d]     k_cache, v_cache [B, Tmax, Hkv, d] (Tmax = allocated entries per
 *   sequence)     out [B, 1, Hq, d]
 * cache_lens: DEVICE int32[B] (or NULL: every sequence uses all Tmax entries); sequence b uses its
 * entries 0 .. cache_lens[b]-1 and its query sits at position cache_lens[b]-1. A length of 0
 * (an empty cache) gives a zero output row: the query sees no key, and a softmax over an empty
 * set is taken as zero weight everywhere. The lengths live on the device, so the host cannot
 * validate them: a negative length counts as 0 and one above Tmax as Tmax. With window > 0 the
 * query sees only its last `window` entries plus entries 0 .. n_sink-1; window = 0 means the
 * whole (ragged) cache. Only visible entries are read. Workspace as for gqa_attn_decode, sized
 * by gqa_attn_decode_workspace_bytes(B, Tmax, Hq, d). bf16 only (else GQA_ERR_UNSUPPORTED);
 * negative window or n_sink is GQA_ERR_SHAPE.
 */
gqa_status_t gqa_attn_decode_ragged(const void* q, const void* k_cache, const void* v_cache,
                                    void* out, int B, int Tmax, int Hq, int Hkv, int d,
                                    float scale, const int32_t* cache_lens, int window,
                                    int n_sink, void* workspace, size_t workspace_bytes,
                                    gqa_dtype_t dtype, hipStream_t stream);

/* gqa_attn_decode_ragged with options (window, sinks, rotary embedding of the query). */
gqa_status_t gqa_attn_decode_ex(const void* q, const void* k_cache, const void* v_cache,
                                void* out, int B, int Tmax, int Hq, int Hkv, int d, float scale,
                                const int32_t* cache_lens, const gqa_attn_options_t* options,
                                void* workspace, size_t workspace_bytes, gqa_dtype_t dtype,
                                hipStream_t stream);

/*
 * Decode against caches bounded to the sliding window (course page "Week 7. Attention", step 3:
 * the window bounds the cache to its size, and the first tokens, the attention sinks, are never
 * dropped from it). The query sees what gqa_attn_decode_ex with the same window and sinks sees on
 * the whole cache, entries 0 .. n_sink-1 and the last `window` entries, and the cache keeps only
 * those.
 *   q [B, 1, Hq, d]     k_cache, v_cache [B, n_sink + window, Hkv, d]     out [B, 1, Hq, d]
 * Slots: entry e of a sequence (0-based, in the order its tokens arrived) lives in slot e when
 * e < n_sink and in slot n_sink + (e - n_sink) mod window otherwise, so each new entry overwrites
 * the one `window` places before it, which has just left the window.
 * cache_lens: DEVICE int32[B], required (else GQA_ERR_NULL_PTR): the number of entries sequence b
 * has had, which may exceed n_sink + window (a negative count is taken as 0: a zero output row);
 * its query sits at position cache_lens[b]-1.
 * options: required (else GQA_ERR_NULL_PTR) with window >= 1 (else GQA_ERR_SHAPE) and
 * n_sink >= 0; the query's rotary embedding and QK-norm as for gqa_attn_decode_ex (the cache
 * holds turned and normalised keys). The query takes table row min(cache_lens[b], rope_rows) - 1,
 * so the tables must reach the positions decoded (rope_rows >= 1). Workspace as for
 * gqa_attn_decode with Tkv = n_sink + window: gqa_attn_decode_workspace_bytes(B, n_sink + window,
 * Hq, d). Only the visible slots are read. bf16 only (else GQA_ERR_UNSUPPORTED).
 */
gqa_status_t gqa_attn_decode_window_cache(const void* q, const void* k_cache, const void* v_cache,
                                          void* out, int B, int Hq, int Hkv, int d, float scale,
                                          const int32_t* cache_lens,
                                          const gqa_attn_options_t* options, void* workspace,
                                          size_t workspace_bytes, gqa_dtype_t dtype,
                                          hipStream_t stream);

/*
 * Backward of gqa_attn_prefill (dense batches): gradients of sum(out * dout).
 *   q, out, dout [B, Tq, Hq, d]; k, v [B, Tkv, Hkv, d]; lse [B, Tq, Hq] fp32 from the forward
 *   (gqa_attn_options_t.lse of gqa_attn_prefill_ex, same q, k, v, scale, causal);
 *   outputs dq [B, Tq, Hq, d], dk, dv [B, Tkv, Hkv, d] in the input dtype, fully overwritten.
 * The gradient of a key/value head is the SUM of the gradients of the G query heads that read it
 * (K3 notes, section 4, backward: the backward of a replication sums over the copies).
 * workspace: caller-owned device memory of at least gqa_attn_backward_workspace_bytes(B, Tq, Hq)
 * bytes, 16-byte aligned (two per-row float arrays: dout . out and lse log2 e). bf16 only,
 * d in {64, 128}. Outputs must not overlap the inputs,
 * the workspace or each other (GQA_ERR_ALIAS). Errors as for gqa_attn_prefill.
 */
size_t gqa_attn_backward_workspace_bytes(int B, int Tq, int Hq);
gqa_status_t gqa_attn_backward(const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               int B, int Tq, int Tkv, int Hq, int Hkv, int d, float scale,
                               int causal, void* workspace, size_t workspace_bytes,
                               gqa_dtype_t dtype, hipStream_t stream);

/*
 * Backward with the options of the forward (course page "Week 7. Attention", step 3): a causal
 * sliding window with sinks (options->window, n_sink, as for gqa_attn_prefill_ex; NULL options:
 * none) and packed variable-length batches (cu_seqlens / max_seqlen as for gqa_attn_prefill:
 * q, out, dout, dq [1, total, Hq, d], k, v, dk, dv [1, total, Hkv, d], lse [1, total, Hq], each
 * sequence differentiated on its own). The forward must have used the same window, sinks and
 * packing. Rotary tables, QK-norm weights and keys_prepared are GQA_ERR_UNSUPPORTED here (their
 * backward is not built). Workspace: gqa_attn_backward_workspace_bytes(B, Tq, Hq) for a dense
 * batch, gqa_attn_backward_workspace_bytes(1, total, Hq) for a packed one. Other arguments and
 * errors as for gqa_attn_backward.
 */
gqa_status_t gqa_attn_backward_ex(const void* q, const void* k, const void* v, const void* out,
                                  const void* dout, const float* lse, void* dq, void* dk,
                                  void* dv, int B, int Tq, int Tkv, int Hq, int Hkv, int d,
                                  float scale, int causal, const int32_t* cu_seqlens,
                                  int max_seqlen, const gqa_attn_options_t* options,
                                  void* workspace, size_t workspace_bytes, gqa_dtype_t dtype,
                                  hipStream_t stream);

/*
 * Fold key/value heads: src [B, T, H, d] -> dst [B, T, g, d] with
 *   dst[b,t,j,:] = (sum of src[b,t,j*s + i,:] for i < s) / s,   s = H / g,
 * summed in fp32 in head order, divided in fp32, rounded to `dtype`. g == H copies the input.
 * H not divisible by g is GQA_ERR_GROUPING.
 */
gqa_status_t gqa_fold_kv(const void* src, void* dst, int B, int T, int H, int g, int d,
                         gqa_dtype_t dtype, hipStream_t stream);

/* Static, human-readable text for a status code (never NULL). */
const char* gqa_status_string(gqa_status_t s);

/* Interface version of this header: bumped on any incompatible change. */
#define GQA_ATTN_ABI_VERSION 3
int gqa_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
