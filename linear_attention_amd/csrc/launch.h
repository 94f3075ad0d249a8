// Kernel launchers behind the C ABI.  Arguments are already validated on the
// host; the kernels still clamp token ranges and check slot indices.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// Token-recurrent path: one workgroup per (request, head), state in registers.
// Request b covers tokens [cu_seqlens[b], cu_seqlens[b+1]) when cu_seqlens is
// non-null, else [b*tokens_per_req, (b+1)*tokens_per_req).  The final state
// goes to state_out[b] when state_out is non-null, else back to the pool slot.
// track_lens / track_slot_idx (both null or both set): state snapshots.
struct RecurrentArgs {
    const void *q, *k, *v;
    const int32_t *cu_seqlens;
    int tokens_per_req;
    int num_heads, num_kv_heads;
    int64_t total_tokens;
    float *pool;
    int64_t pool_slots;
    const int32_t *slot_idx;
    const int32_t *track_lens, *track_slot_idx;
    const float *slopes;
    void *out;
    float *state_out;
};
hipError_t launch_recurrent(const RecurrentArgs &a, bool bf16, int head_dim, int batch,
                            hipStream_t stream);

// Tree verify: one workgroup per (request, head); num_draft drafts per request,
// parent_idx [batch, num_draft]; draft_states may be null.
struct TreeArgs {
    const void *q, *k, *v;
    int num_draft;
    int num_heads, num_kv_heads;
    const float *pool;
    int64_t pool_slots;
    const int32_t *slot_idx;
    const int32_t *parent_idx;
    const float *slopes;
    void *out;
    float *draft_states;
};
hipError_t launch_tree(const TreeArgs &a, bool bf16, int head_dim, int batch, hipStream_t stream);

// Chunked bf16 MFMA prefill (head_dim 128 or 64): one workgroup per (request,
// head, 32-column block of the state), chunks of 64 tokens.  With segments > 1
// every request is split into that many sequence segments, using the caller's
// workspace seg_ws (size and layout: plan_segments in host_logic.h).
struct PrefillArgs {
    const uint16_t *q, *k, *v;
    const int32_t *cu_seqlens;
    int num_heads, num_kv_heads, pairs;
    int64_t total_tokens;
    float *pool;
    int64_t pool_slots;
    const int32_t *slot_idx;
    const int32_t *track_lens, *track_slot_idx;
    const float *slopes;
    uint16_t *out;
    int segments;   // sequence segments per request (1: no split)
    int subsegs;    // sub-segments per segment in the state-only pass
    float *seg_ws;  // their workspace (device memory, owned by the caller)
};
hipError_t launch_prefill_chunked(const PrefillArgs &a, int batch, int head_dim, hipStream_t stream);

}  // namespace la
