/*
 * linattn.h -- C ABI of the MI355X (gfx950) segmented linear attention library
 * (liblinattn.so).
 *
 * Citations name the web page "SGLang Lightning Attention 能力矩阵与 seg_la
 * 线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page] and
 * its sections by their headings.
 *
 * The operation ([LA-page] §独立参考实现：逐 token 递推公式, the recurrence):
 * every request b and head h owns a d x d fp32 state S (row = key feature,
 * column = value feature).  For each token t of the request, in order,
 *
 *     S   <- S * exp(-slopes[h]) + outer(k_t, v_t)
 *     o_t  = (q_t @ S) * head_dim^-0.5
 *
 * The state before the first token is read from the request's slot of a state
 * pool and the final state is written back to that slot (prefix states,
 * same section); pool slots no request names are never written ([LA-page]
 * §额外覆盖：mamba 状态跟踪与布局鲁棒性).
 *
 * Layouts (all row-major, contiguous, device memory owned by the caller):
 *   q, out         [T, H, d]  token-major, heads interleaved; identical memory
 *                  to the flattened [T, H*d] output ([LA-page] §生产环境不支持
 *                  item 4).  Element type given by `dtype`; out has the same
 *                  type as q (bf16 outputs are rounded to nearest even).
 *   k, v           [T, Hkv, d], same element type.  Grouped heads: Hkv
 *                  (num_kv_heads) divides H and query head h reads key/value
 *                  head h / (H / Hkv); Hkv == H is plain multi-head.  The
 *                  reference kernel asserts qo_heads == kv_heads ([LA-page]
 *                  §输入与配置覆盖); here state and slope stay per query head
 *                  and only k and v are shared within a group.
 *   state_pool     [pool_slots, H, d, d] float32.
 *   slot_idx       [batch] int32, distinct, in [0, pool_slots); any order.
 *   cu_seqlens     [batch+1] int32, cu_seqlens[0] = 0, non-decreasing,
 *                  cu_seqlens[batch] = total_tokens (packed varlen batch).
 *   slopes         [H] float32 per-head decay rates (see la_alibi_slopes).
 * q, k, v, out, state_pool, state_out and draft_states must be 16-byte aligned
 * (the kernels move them with 16-byte vector accesses; a misaligned pointer is
 * LA_ERR_INVALID_ARG).
 * head_dim (d) is 128 or 64 (the reference's kernels need at least 128 for
 * decode and 64 for prefill, [LA-page] §输入与配置覆盖; both run here on
 * every path).
 *
 * Calls are asynchronous on `stream` (0 = the null stream): the library does
 * no host synchronisation, no device-to-host reads and no allocation, and
 * keeps no state between calls (beyond each device's compute-unit count,
 * read once, and the static scratch of la_prefill_noalloc).  Scratch memory,
 * where a call can use it, is otherwise the caller's: see
 * la_prefill_workspace_bytes.  The inputs must not alias out, state_pool,
 * state_out or the workspace.  Overlapping calls that name the same pool slot
 * or share a workspace race.
 *
 * Errors: every call returns an la_status and never aborts.  Host-visible
 * arguments are validated before anything is launched.  Device-resident
 * metadata (cu_seqlens, slot_idx) is validated on the host only when the
 * environment variable LA_DEBUG=1 is set (that mode synchronises the stream).
 * Without it the kernels still stay in bounds: token ranges are clamped to
 * [0, total_tokens) and a request whose slot index is out of range gets zero
 * output and touches no state.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t *hipStream_t;

typedef enum {
    LA_OK = 0,
    LA_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad metadata (LA_DEBUG) */
    LA_ERR_UNSUPPORTED = -2, /* head_dim not 64/128, unknown dtype, num_draft <= 0 */
    LA_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
    LA_ERR_NO_SCRATCH = -4   /* la_prefill_noalloc: the split needs more than its static scratch */
} la_status;

typedef enum {
    LA_DTYPE_BF16 = 0, /* bfloat16 q, k, v, out */
    LA_DTYPE_F32 = 1   /* float32 q, k, v, out: computed in fp32 end to end */
} la_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char *la_status_string(la_status s);

/*
 * Per-head slopes ([LA-page] §独立参考实现, slope bullet): the ALiBi geometric
 * sequence (Press, Smith & Lewis, ICLR 2022: for n heads a power of two,
 * slope_i = 2^(-8(i+1)/n); otherwise the first 2^floor(log2 n) slopes of that
 * sequence, then every other slope of the sequence for twice as many heads)
 * times the layer factor 1 - layer_id/(num_layers-1) + 1e-5, or 1 + 1e-5 when
 * num_layers == 1.  Computed in double, rounded once to float.
 * slopes_host: caller-owned HOST array of num_heads floats.
 * Errors: LA_ERR_INVALID_ARG for num_heads <= 0, num_layers <= 0,
 * layer_id outside [0, num_layers) or a NULL pointer.
 */
la_status la_alibi_slopes(int num_heads, int layer_id, int num_layers, float *slopes_host);

/*
 * Workspace of a bf16 prefill, in bytes, on the current device: what
 * la_prefill needs to split the requests of a call with these sizes into
 * sequence segments (0 when such a call does not split).
 *
 * A bf16 launch whose (request, head, 32-column block) units fill only part of
 * the GPU's compute units, whose longest request (max_seqlen) has at least
 * 8192 tokens and which takes no snapshots splits every request into up to 8
 * sequence segments of at least 1024 tokens of the longest request, as many
 * as fill the compute units; the segments run side by side from initial
 * states that a state-only pass and a combine step compute first.  The
 * workspace holds their partial states: batch * num_heads * (segments +
 * (segments - 1) * subsegs) * head_dim^2 floats, subsegs = 1..4 state-only
 * workgroups per segment (as many as fill the compute units).  The size
 * depends on the device's compute-unit count, so query it on the device the
 * call will run on.  The environment variable LA_PREFILL_MAX_SEGMENTS (1..8)
 * caps the segment count, in this query and in la_prefill alike.
 * Invalid sizes (negative, head_dim other than 64/128) give 0.
 * fp32 prefills and prefills with track arrays never split and need no
 * workspace, whatever this returns.
 */
size_t la_prefill_workspace_bytes(int batch, int64_t total_tokens, int max_seqlen, int num_heads,
                                  int head_dim);

/*
 * Packed varlen prefill ("extend") over `batch` requests holding
 * `total_tokens` tokens in all ([LA-page] §独立参考实现 and
 * §输入与配置覆盖).  For every request the state is read from
 * state_pool[slot_idx[b]], advanced through the request's tokens, and written
 * back in place; out receives every token's output.  A zero-length request is a
 * no-op.  max_seqlen is an upper bound on any request's length (0 means every
 * request is empty; the call then launches nothing).
 *
 * State tracking ([LA-page] §额外覆盖：mamba 状态跟踪与布局鲁棒性):
 * track_lens and track_slot_idx ([batch] int32 each, device) are both NULL
 * (no tracking) or both given.  Request b with 0 <= track_slot_idx[b] <
 * pool_slots and 0 <= track_lens[b] <= its length also writes its state after
 * its first track_lens[b] tokens (the prefix state itself for 0) to
 * state_pool[track_slot_idx[b]]; a negative track slot means no snapshot.
 * Track slots must be distinct from each other and from every slot_idx entry.
 *
 * bf16 (d = 64 or 128): chunked MFMA kernel (fp32 state, bf16 hi/lo operand
 * splits).  fp32: token-recurrent fp32 kernel, one workgroup per (request,
 * head), the outputs of each group of up to 8 tokens reduced together.
 *
 * workspace, workspace_bytes: device scratch owned by the caller, 16-byte
 * aligned, used only by a call that splits into sequence segments (see
 * la_prefill_workspace_bytes for when and how much).  NULL with 0 bytes runs
 * such a call unsplit (same results to rounding, slower on long requests); a
 * non-NULL workspace smaller than the split needs is LA_ERR_INVALID_ARG.  Its
 * contents before and after the call are of no meaning; the call reads only
 * what it writes there first, in stream order.  The library never allocates.
 *
 * Errors: LA_ERR_INVALID_ARG for NULL or misaligned pointers (q/k/v/out may be
 * NULL only when total_tokens == 0), negative sizes, num_kv_heads not dividing
 * num_heads, only one of the two track arrays, batch > pool_slots, a NULL
 * workspace with nonzero workspace_bytes, a workspace too small for the
 * split, or, with LA_DEBUG=1, inconsistent cu_seqlens/slot_idx/track arrays;
 * LA_ERR_UNSUPPORTED for a head_dim other than 64/128 or an unknown dtype;
 * LA_ERR_HIP on a launch failure.
 */
la_status la_prefill(const void *q, const void *k, const void *v, la_dtype dtype,
                     const int32_t *cu_seqlens, int batch, int64_t total_tokens, int max_seqlen,
                     int num_heads, int num_kv_heads, int head_dim,
                     float *state_pool, int64_t pool_slots, const int32_t *slot_idx,
                     const int32_t *track_lens, const int32_t *track_slot_idx,
                     const float *slopes, void *out, void *workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * la_prefill for callers that cannot allocate or own device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, semantics and errors as la_prefill without the workspace:
 * a call that splits into sequence segments takes its scratch from a static
 * device array of LA_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * every GPU it runs on until the process ends.  No allocation, no host
 * synchronisation.  A split that needs more scratch than that (never on a
 * 256-CU MI355X, whose largest split needs 18 MiB) returns
 * LA_ERR_NO_SCRATCH before anything is launched.
 * All calls on one GPU share its array: calls that overlap on one GPU (on
 * different streams, or concurrently from several host threads) race.  Each
 * call writes every part of the array it later reads, so nothing needs
 * clearing between calls.
 */
#define LA_NOALLOC_SCRATCH_BYTES (32u << 20)
la_status la_prefill_noalloc(const void *q, const void *k, const void *v, la_dtype dtype,
                             const int32_t *cu_seqlens, int batch, int64_t total_tokens, int max_seqlen,
                             int num_heads, int num_kv_heads, int head_dim,
                             float *state_pool, int64_t pool_slots, const int32_t *slot_idx,
                             const int32_t *track_lens, const int32_t *track_slot_idx,
                             const float *slopes, void *out, hipStream_t stream);

/*
 * Decode: one token per request (q, out are [batch, H, d]; k, v [batch, Hkv, d]).
 * Each request's state is read, advanced by one step of the recurrence and
 * written back in place ([LA-page] §输入与配置覆盖, the decode kernel's role).
 * Errors as for la_prefill (no cu_seqlens or track arrays).
 */
la_status la_decode(const void *q, const void *k, const void *v, la_dtype dtype,
                    int batch, int num_heads, int num_kv_heads, int head_dim,
                    float *state_pool, int64_t pool_slots, const int32_t *slot_idx,
                    const float *slopes, void *out, hipStream_t stream);

/*
 * Chain verify: request b owns the num_draft draft tokens
 * b*num_draft .. b*num_draft+num_draft-1 of q, k, v, out and processes them as
 * one chain from its pool state ([LA-page] §生产环境不支持 item 3: drafts are
 * verified as a chain, topk = 1).  Outputs are written for every draft token.
 * The final state goes to state_out[b] ([batch, H, d, d] float32) and the pool
 * is left untouched; with state_out == NULL the final state is written back to
 * the pool slot instead.
 * Errors as for la_decode, plus LA_ERR_UNSUPPORTED for num_draft <= 0.
 */
la_status la_verify(const void *q, const void *k, const void *v, la_dtype dtype,
                    int batch, int num_draft, int num_heads, int num_kv_heads, int head_dim,
                    float *state_pool, int64_t pool_slots, const int32_t *slot_idx,
                    const float *slopes, void *out, float *state_out, hipStream_t stream);

/*
 * Tree verify with per-position states ([LA-page] §生产环境不支持 item 3 and
 * Next Work item 2: each draft token forks from its parent's saved state
 * instead of continuing the chain).  Request b owns draft tokens
 * b*num_draft .. b*num_draft+num_draft-1 of q, k, v, out.  parent_idx
 * [batch, num_draft] int32 (device): parent_idx[b][j] is -1 (the request's
 * pool state) or an earlier draft p < j.  Draft j's state is
 *     S_j = exp(-slopes[h]) * S_parent + outer(k_j, v_j),   o_j = (q_j @ S_j) * d^-0.5.
 * Parents (-1, 0, 1, ..., num_draft-2) are the chain of la_verify.
 * draft_states [batch, num_draft, H, d, d] float32 receives every S_j (NULL:
 * outputs only).  The pool is never written.
 * A request whose slot or any parent is out of range gets zero outputs and no
 * state written (with LA_DEBUG=1 the call returns LA_ERR_INVALID_ARG instead).
 * Errors as for la_verify.
 */
la_status la_verify_tree(const void *q, const void *k, const void *v, la_dtype dtype,
                         int batch, int num_draft, int num_heads, int num_kv_heads, int head_dim,
                         const float *state_pool, int64_t pool_slots, const int32_t *slot_idx,
                         const int32_t *parent_idx, const float *slopes, void *out,
                         float *draft_states, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
