// C ABI of liblinattn.so: argument validation and dispatch.  The operation,
// layouts and error behaviour are specified in include/linattn.h.
//
// Citations name the web page "SGLang Lightning Attention 能力矩阵与 seg_la
// 线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page].
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "host_logic.h"
#include "launch.h"
#include "linattn.h"

using la::aligned16;
using la::common_checks;

// Scratch of la_prefill_noalloc: a file-scope device array, one copy per GPU.
// In host code `scratch` only names the symbol; the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is handed to kernels.
static_assert(LA_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");
static __device__ __align__(256) float scratch[LA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

bool debug_mode() {
    const char *s = std::getenv("LA_DEBUG");
    return s && s[0] == '1';
}

template <typename T>
bool copy_to_host(std::vector<T> &dst, const T *src, size_t n) {
    dst.resize(n > 0 ? n : 1);
    return n == 0 || hipMemcpy(dst.data(), src, sizeof(T) * n, hipMemcpyDeviceToHost) == hipSuccess;
}

// Debug mode: copy the device metadata to the host (synchronising `stream`)
// and check it there.
la_status debug_check(const int32_t *cu_seqlens, int batch, int64_t total_tokens, int max_seqlen,
                      int fixed_len, const int32_t *slot_idx, int64_t pool_slots,
                      const int32_t *track_lens, const int32_t *track_slot_idx,
                      const int32_t *parents, hipStream_t stream) {
    std::vector<int32_t> slots, cu, tl, ts, par;
    if (hipStreamSynchronize(stream) != hipSuccess) return LA_ERR_HIP;
    if (!copy_to_host(slots, slot_idx, batch)) return LA_ERR_HIP;
    if (cu_seqlens && !copy_to_host(cu, cu_seqlens, batch + 1)) return LA_ERR_HIP;
    if (track_lens && (!copy_to_host(tl, track_lens, batch) || !copy_to_host(ts, track_slot_idx, batch)))
        return LA_ERR_HIP;
    if (parents && !copy_to_host(par, parents, static_cast<size_t>(batch) * fixed_len)) return LA_ERR_HIP;
    return la::check_metadata(cu_seqlens ? cu.data() : nullptr, batch, total_tokens, max_seqlen, fixed_len,
                              slots.data(), pool_slots, track_lens ? tl.data() : nullptr,
                              track_lens ? ts.data() : nullptr, parents ? par.data() : nullptr);
}

la_status from_hip(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_HIP; }

// Compute units of the current device (cached per device).
int cu_count() {
    static std::atomic<int> count[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = count[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        count[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// The most sequence segments a prefill may use: kMaxSegments, lowered by the
// environment variable LA_PREFILL_MAX_SEGMENTS (1 turns the split off).
int segment_cap() {
    int cap = la::kMaxSegments;
    if (const char *env = std::getenv("LA_PREFILL_MAX_SEGMENTS")) cap = std::atoi(env);
    return cap < 1 ? 1 : (cap > la::kMaxSegments ? la::kMaxSegments : cap);
}

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_addr[kMaxDevices];

// The current device's copy of `scratch`, or null if its address cannot be had.
void *scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_addr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        scratch_addr[dev] = ptr;
    }
    return scratch_addr[dev];
}

}  // namespace

extern "C" {

const char *la_status_string(la_status s) {
    switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG: invalid argument";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: unsupported configuration";
    case LA_ERR_HIP: return "LA_ERR_HIP: HIP runtime error";
    case LA_ERR_NO_SCRATCH:
        return "LA_ERR_NO_SCRATCH: the prefill split needs more than the static scratch (LA_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown la_status";
}

la_status la_alibi_slopes(int num_heads, int layer_id, int num_layers, float *slopes_host) {
    return la::alibi_slopes(num_heads, layer_id, num_layers, slopes_host);
}

size_t la_prefill_workspace_bytes(int batch, int64_t total_tokens, int max_seqlen, int num_heads,
                                  int head_dim) {
    if (total_tokens < 0 || max_seqlen < 0) return 0;
    return la::plan_segments(cu_count(), batch, num_heads, head_dim, max_seqlen, false, segment_cap())
        .workspace_bytes;
}

la_status la_prefill(const void *q, const void *k, const void *v, la_dtype dtype,
                     const int32_t *cu_seqlens, int batch, int64_t total_tokens, int max_seqlen,
                     int num_heads, int num_kv_heads, int head_dim, float *state_pool,
                     int64_t pool_slots, const int32_t *slot_idx, const int32_t *track_lens,
                     const int32_t *track_slot_idx, const float *slopes, void *out,
                     void *workspace, size_t workspace_bytes, hipStream_t stream) {
    la_status st = common_checks(q, k, v, dtype, total_tokens, batch, num_heads, num_kv_heads,
                                 head_dim, state_pool, pool_slots, slot_idx, slopes, out);
    if (st != LA_OK) return st;
    if (max_seqlen < 0 || (batch > 0 && !cu_seqlens)) return LA_ERR_INVALID_ARG;
    if (!track_lens != !track_slot_idx) return LA_ERR_INVALID_ARG;
    if ((!workspace && workspace_bytes != 0) || !aligned16(workspace)) return LA_ERR_INVALID_ARG;
    la::SegmentPlan plan;
    if (dtype == LA_DTYPE_BF16 && batch > 0 && !track_lens && max_seqlen >= la::kMinSplitTokens) {
        plan = la::plan_segments(cu_count(), batch, num_heads, head_dim, max_seqlen, track_lens != nullptr,
                                 segment_cap());
        if (plan.segments > 1) {
            if (!workspace) plan = la::SegmentPlan{};  // no workspace: run unsplit
            else if (workspace_bytes < plan.workspace_bytes) return LA_ERR_INVALID_ARG;
        }
    }
    if (debug_mode()) {
        st = debug_check(cu_seqlens, batch, total_tokens, max_seqlen, 0, slot_idx, pool_slots,
                         track_lens, track_slot_idx, nullptr, stream);
        if (st != LA_OK) return st;
    }
    // with every request empty there is nothing to compute, but a snapshot
    // after 0 tokens still copies the prefix state
    if (batch == 0 || ((max_seqlen == 0 || total_tokens == 0) && !track_lens)) return LA_OK;
    if (dtype == LA_DTYPE_BF16) {
        la::PrefillArgs a{};
        a.q = static_cast<const uint16_t *>(q);
        a.k = static_cast<const uint16_t *>(k);
        a.v = static_cast<const uint16_t *>(v);
        a.cu_seqlens = cu_seqlens;
        a.num_heads = num_heads;
        a.num_kv_heads = num_kv_heads;
        a.total_tokens = total_tokens;
        a.pool = state_pool;
        a.pool_slots = pool_slots;
        a.slot_idx = slot_idx;
        a.track_lens = track_lens;
        a.track_slot_idx = track_slot_idx;
        a.slopes = slopes;
        a.out = static_cast<uint16_t *>(out);
        a.segments = plan.segments;
        a.subsegs = plan.subsegs;
        a.seg_ws = plan.segments > 1 ? static_cast<float *>(workspace) : nullptr;
        return from_hip(la::launch_prefill_chunked(a, batch, head_dim, stream));
    }
    la::RecurrentArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.cu_seqlens = cu_seqlens;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.total_tokens = total_tokens;
    a.pool = state_pool;
    a.pool_slots = pool_slots;
    a.slot_idx = slot_idx;
    a.track_lens = track_lens;
    a.track_slot_idx = track_slot_idx;
    a.slopes = slopes;
    a.out = out;
    return from_hip(la::launch_recurrent(a, dtype == LA_DTYPE_BF16, head_dim, batch, stream));
}

la_status la_prefill_noalloc(const void *q, const void *k, const void *v, la_dtype dtype,
                             const int32_t *cu_seqlens, int batch, int64_t total_tokens, int max_seqlen,
                             int num_heads, int num_kv_heads, int head_dim, float *state_pool,
                             int64_t pool_slots, const int32_t *slot_idx, const int32_t *track_lens,
                             const int32_t *track_slot_idx, const float *slopes, void *out,
                             hipStream_t stream) {
    la_status st = common_checks(q, k, v, dtype, total_tokens, batch, num_heads, num_kv_heads,
                                 head_dim, state_pool, pool_slots, slot_idx, slopes, out);
    if (st != LA_OK) return st;
    if (max_seqlen < 0 || (batch > 0 && !cu_seqlens)) return LA_ERR_INVALID_ARG;
    void *ws = scratch_on_current_device();
    if (!ws) return LA_ERR_HIP;
    if (dtype == LA_DTYPE_BF16 && batch > 0 && !track_lens && max_seqlen >= la::kMinSplitTokens &&
        la::plan_segments(cu_count(), batch, num_heads, head_dim, max_seqlen, false, segment_cap())
                .workspace_bytes > LA_NOALLOC_SCRATCH_BYTES)
        return LA_ERR_NO_SCRATCH;
    return la_prefill(q, k, v, dtype, cu_seqlens, batch, total_tokens, max_seqlen, num_heads, num_kv_heads,
                      head_dim, state_pool, pool_slots, slot_idx, track_lens, track_slot_idx, slopes, out, ws,
                      LA_NOALLOC_SCRATCH_BYTES, stream);
}

la_status la_decode(const void *q, const void *k, const void *v, la_dtype dtype, int batch,
                    int num_heads, int num_kv_heads, int head_dim, float *state_pool,
                    int64_t pool_slots, const int32_t *slot_idx, const float *slopes, void *out,
                    hipStream_t stream) {
    return la_verify(q, k, v, dtype, batch, 1, num_heads, num_kv_heads, head_dim, state_pool,
                     pool_slots, slot_idx, slopes, out, nullptr, stream);
}

la_status la_verify(const void *q, const void *k, const void *v, la_dtype dtype, int batch,
                    int num_draft, int num_heads, int num_kv_heads, int head_dim,
                    float *state_pool, int64_t pool_slots, const int32_t *slot_idx,
                    const float *slopes, void *out, float *state_out, hipStream_t stream) {
    if (num_draft <= 0) return batch < 0 ? LA_ERR_INVALID_ARG : LA_ERR_UNSUPPORTED;
    const int64_t tokens = static_cast<int64_t>(batch) * num_draft;
    la_status st = common_checks(q, k, v, dtype, tokens, batch, num_heads, num_kv_heads, head_dim,
                                 state_pool, pool_slots, slot_idx, slopes, out);
    if (st != LA_OK) return st;
    if (!aligned16(state_out)) return LA_ERR_INVALID_ARG;
    if (debug_mode()) {
        st = debug_check(nullptr, batch, tokens, num_draft, num_draft, slot_idx, pool_slots,
                         nullptr, nullptr, nullptr, stream);
        if (st != LA_OK) return st;
    }
    la::RecurrentArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.tokens_per_req = num_draft;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.total_tokens = tokens;
    a.pool = state_pool;
    a.pool_slots = pool_slots;
    a.slot_idx = slot_idx;
    a.slopes = slopes;
    a.out = out;
    a.state_out = state_out;
    return from_hip(la::launch_recurrent(a, dtype == LA_DTYPE_BF16, head_dim, batch, stream));
}

la_status la_verify_tree(const void *q, const void *k, const void *v, la_dtype dtype, int batch,
                         int num_draft, int num_heads, int num_kv_heads, int head_dim,
                         const float *state_pool, int64_t pool_slots, const int32_t *slot_idx,
                         const int32_t *parent_idx, const float *slopes, void *out,
                         float *draft_states, hipStream_t stream) {
    if (num_draft <= 0) return batch < 0 ? LA_ERR_INVALID_ARG : LA_ERR_UNSUPPORTED;
    const int64_t tokens = static_cast<int64_t>(batch) * num_draft;
    la_status st = common_checks(q, k, v, dtype, tokens, batch, num_heads, num_kv_heads, head_dim,
                                 state_pool, pool_slots, slot_idx, slopes, out);
    if (st != LA_OK) return st;
    if (batch > 0 && !parent_idx) return LA_ERR_INVALID_ARG;
    if (!aligned16(draft_states)) return LA_ERR_INVALID_ARG;
    if (debug_mode()) {
        st = debug_check(nullptr, batch, tokens, num_draft, num_draft, slot_idx, pool_slots,
                         nullptr, nullptr, parent_idx, stream);
        if (st != LA_OK) return st;
    }
    la::TreeArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.num_draft = num_draft;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.pool = state_pool;
    a.pool_slots = pool_slots;
    a.slot_idx = slot_idx;
    a.parent_idx = parent_idx;
    a.slopes = slopes;
    a.out = out;
    a.draft_states = draft_states;
    return from_hip(la::launch_tree(a, dtype == LA_DTYPE_BF16, head_dim, batch, stream));
}

}  // extern "C"
