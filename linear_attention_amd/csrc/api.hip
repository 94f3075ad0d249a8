// C ABI of liblinattn.so: argument validation and dispatch.  The operation,
// layouts and error behaviour are specified in include/linattn.h.
//
// Citations name the web page "SGLang Lightning Attention 能力矩阵与 seg_la
// 线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page].
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "common.h"
#include "launch.h"
#include "linattn.h"

namespace {

constexpr int64_t kMaxGrid = 0x7fffffff;

bool debug_mode() {
    const char *s = std::getenv("LA_DEBUG");
    return s && s[0] == '1';
}

template <typename T>
bool copy_to_host(std::vector<T> &dst, const T *src, size_t n) {
    dst.resize(n > 0 ? n : 1);
    return n == 0 || hipMemcpy(dst.data(), src, sizeof(T) * n, hipMemcpyDeviceToHost) == hipSuccess;
}

// Debug-mode validation of device-resident metadata ([LA-page] §生产环境不支持
// item 1: unsupported inputs are rejected before the kernel runs).  Synchronises
// `stream`.  cu_seqlens may be null (fixed-length requests of `fixed_len`
// tokens); track arrays and parents may be null.
la_status debug_check(const int32_t *cu_seqlens, int batch, int64_t total_tokens, int max_seqlen,
                      int fixed_len, const int32_t *slot_idx, int64_t pool_slots,
                      const int32_t *track_lens, const int32_t *track_slot_idx,
                      const int32_t *parents, hipStream_t stream) {
    std::vector<int32_t> slots, cu, tl, ts, par;
    if (hipStreamSynchronize(stream) != hipSuccess) return LA_ERR_HIP;
    if (!copy_to_host(slots, slot_idx, batch)) return LA_ERR_HIP;
    std::vector<int64_t> lens(batch > 0 ? batch : 1, fixed_len);
    if (cu_seqlens) {
        if (!copy_to_host(cu, cu_seqlens, batch + 1)) return LA_ERR_HIP;
        if (cu[0] != 0 || cu[batch] != total_tokens) return LA_ERR_INVALID_ARG;
        for (int b = 0; b < batch; ++b) {
            lens[b] = static_cast<int64_t>(cu[b + 1]) - cu[b];
            if (lens[b] < 0 || lens[b] > max_seqlen) return LA_ERR_INVALID_ARG;
        }
    }
    std::vector<char> seen(static_cast<size_t>(pool_slots), 0);
    for (int b = 0; b < batch; ++b) {
        const int32_t s = slots[b];
        if (s < 0 || s >= pool_slots || seen[s]) return LA_ERR_INVALID_ARG;
        seen[s] = 1;
    }
    if (track_lens) {
        if (!copy_to_host(tl, track_lens, batch) || !copy_to_host(ts, track_slot_idx, batch))
            return LA_ERR_HIP;
        for (int b = 0; b < batch; ++b) {
            if (ts[b] < 0) continue;  // no snapshot for this request
            if (ts[b] >= pool_slots || seen[ts[b]] || tl[b] < 0 || tl[b] > lens[b])
                return LA_ERR_INVALID_ARG;
            seen[ts[b]] = 1;
        }
    }
    if (parents) {
        if (!copy_to_host(par, parents, static_cast<size_t>(batch) * fixed_len)) return LA_ERR_HIP;
        for (size_t i = 0; i < static_cast<size_t>(batch) * fixed_len; ++i) {
            const int j = static_cast<int>(i % fixed_len);
            if (par[i] < -1 || par[i] >= j) return LA_ERR_INVALID_ARG;
        }
    }
    return LA_OK;
}

// The kernels move q, k, v, out and states with 16-byte vector accesses.
bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

la_status common_checks(const void *q, const void *k, const void *v, la_dtype dtype,
                        int64_t total_tokens, int batch, int num_heads, int num_kv_heads,
                        int head_dim, const float *state_pool, int64_t pool_slots,
                        const int32_t *slot_idx, const float *slopes, const void *out) {
    if (batch < 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || pool_slots <= 0 ||
        total_tokens < 0)
        return LA_ERR_INVALID_ARG;
    if (num_heads % num_kv_heads != 0) return LA_ERR_INVALID_ARG;
    if (dtype != LA_DTYPE_BF16 && dtype != LA_DTYPE_F32) return LA_ERR_UNSUPPORTED;
    if (head_dim != 128 && head_dim != 64) return LA_ERR_UNSUPPORTED;
    if (batch > pool_slots) return LA_ERR_INVALID_ARG;  // slots must be distinct
    if (!state_pool || !slopes || (batch > 0 && !slot_idx)) return LA_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !k || !v || !out)) return LA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(state_pool))
        return LA_ERR_INVALID_ARG;
    if (static_cast<int64_t>(batch) * num_heads * 4 > kMaxGrid) return LA_ERR_INVALID_ARG;
    if (total_tokens > kMaxGrid) return LA_ERR_INVALID_ARG;  // int32 cu_seqlens
    return LA_OK;
}

la_status from_hip(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_HIP; }

}  // namespace

extern "C" {

const char *la_status_string(la_status s) {
    switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID_ARG: return "LA_ERR_INVALID_ARG: invalid argument";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: unsupported configuration";
    case LA_ERR_HIP: return "LA_ERR_HIP: HIP runtime error";
    }
    return "unknown la_status";
}

la_status la_alibi_slopes(int num_heads, int layer_id, int num_layers, float *slopes_host) {
    if (num_heads <= 0 || num_layers <= 0 || layer_id < 0 || layer_id >= num_layers || !slopes_host)
        return LA_ERR_INVALID_ARG;
    int pow2 = 1;  // largest power of two <= num_heads
    while (pow2 <= num_heads / 2) pow2 <<= 1;
    const double layer = num_layers == 1
                             ? 1.0 + 1e-5
                             : 1.0 - static_cast<double>(layer_id) / static_cast<double>(num_layers - 1) + 1e-5;
    for (int h = 0; h < num_heads; ++h) {
        // geometric sequence 2^(-8(h+1)/pow2); the heads past pow2 take the odd
        // positions of the 2*pow2 sequence, 2^(-4(2j+1)/pow2)
        const double e = h < pow2 ? -8.0 * (h + 1) / pow2 : -4.0 * (2 * (h - pow2) + 1) / pow2;
        slopes_host[h] = static_cast<float>(std::exp2(e) * layer);
    }
    return LA_OK;
}

la_status la_prefill(const void *q, const void *k, const void *v, la_dtype dtype,
                     const int32_t *cu_seqlens, int batch, int64_t total_tokens, int max_seqlen,
                     int num_heads, int num_kv_heads, int head_dim, float *state_pool,
                     int64_t pool_slots, const int32_t *slot_idx, const int32_t *track_lens,
                     const int32_t *track_slot_idx, const float *slopes, void *out,
                     hipStream_t stream) {
    la_status st = common_checks(q, k, v, dtype, total_tokens, batch, num_heads, num_kv_heads,
                                 head_dim, state_pool, pool_slots, slot_idx, slopes, out);
    if (st != LA_OK) return st;
    if (max_seqlen < 0 || (batch > 0 && !cu_seqlens)) return LA_ERR_INVALID_ARG;
    if (!track_lens != !track_slot_idx) return LA_ERR_INVALID_ARG;
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
        return from_hip(la::launch_prefill_chunked(a, batch, head_dim, max_seqlen, stream));
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
