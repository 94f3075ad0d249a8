// Host-side logic of the C ABI that needs no device: argument checks, the
// ALiBi slopes, the sequence-segment plan of a bf16 prefill launch with its
// workspace size, and the checks of device metadata once it is on the host.
// Plain C++ (no HIP), so the same code also builds with g++ under the
// address and undefined-behaviour sanitizers.
//
// Citations name the web page "SGLang Lightning Attention 能力矩阵与 seg_la
// 线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page].
#pragma once
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <vector>

#include "linattn.h"

namespace la {

// Chunked prefill geometry shared by the launcher and the host plan.
constexpr int kChunk = 64;              // tokens per chunk
constexpr int kColBlock = 32;           // state columns per prefill workgroup
constexpr int kMaxSegments = 8;         // sequence segments per request, at most
constexpr int kMaxSubsegs = 4;          // state-only workgroups per segment, at most
constexpr int kMinSegmentTokens = 1024; // tokens of the longest request per segment, at least
// A split call pays a fixed cost (two more launches and the idle gaps between
// short kernels), so only launches whose longest request has this many
// tokens are split: measured at 8 heads, a 4096-token request gains nothing,
// 8192 tokens go from 152 to 93 us.
constexpr int kMinSplitTokens = 8192;

// The grid and token counts the kernels index with 32-bit values.
constexpr int64_t kMaxGrid = 0x7fffffff;

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every entry point, on host-visible arguments only.
inline la_status common_checks(const void *q, const void *k, const void *v, la_dtype dtype,
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
    // (batch * num_heads < 2^62 here, so the product cannot overflow)
    if (static_cast<int64_t>(batch) * num_heads > kMaxGrid / 4) return LA_ERR_INVALID_ARG;
    if (total_tokens > kMaxGrid) return LA_ERR_INVALID_ARG;  // int32 cu_seqlens
    return LA_OK;
}

// Per-head slopes ([LA-page] §独立参考实现, slope bullet): the ALiBi geometric
// sequence (Press, Smith & Lewis, ICLR 2022) times the layer factor, in
// double, rounded once to float.
inline la_status alibi_slopes(int num_heads, int layer_id, int num_layers, float *slopes_host) {
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

// How a bf16 prefill launch runs.  A launch whose (request, head, column
// block) units fill only part of the GPU's compute units splits every request
// into `segments` sequence segments, run side by side from initial states
// that a state-only pass (`subsegs` workgroups per non-final segment) and a
// combine step compute first.  Those need a workspace of `workspace_bytes`:
// the contributions of the sub-segments, [pair][segments - 1][subsegs][d][d],
// then the initial states, [pair][segments][d][d], fp32.
struct SegmentPlan {
    int segments = 1;
    int subsegs = 0;
    size_t workspace_bytes = 0;
};

// cap: the most segments allowed (kMaxSegments, or less to restrict the split;
// 1 turns it off).  Requests with state tracking are never split.
inline SegmentPlan plan_segments(int cu_count, int batch, int num_heads, int head_dim, int max_seqlen,
                                 bool track, int cap) {
    SegmentPlan p;
    if (batch <= 0 || num_heads <= 0 || (head_dim != 64 && head_dim != 128) || cu_count <= 0) return p;
    const int64_t pairs = static_cast<int64_t>(batch) * num_heads;  // < 2^62
    if (track || max_seqlen < kMinSplitTokens || pairs >= cu_count) return p;
    const int64_t units = pairs * (head_dim / kColBlock);
    if (units >= cu_count) return p;
    int ns = static_cast<int>(cu_count / units);
    cap = cap < 1 ? 1 : (cap > kMaxSegments ? kMaxSegments : cap);
    if (ns > cap) ns = cap;
    if (ns > max_seqlen / kMinSegmentTokens) ns = max_seqlen / kMinSegmentTokens;
    if (ns <= 1) return p;
    const int64_t per = pairs * (ns - 1);  // state-only sub-segment groups
    int64_t sub = cu_count / per;
    sub = sub < 1 ? 1 : (sub > kMaxSubsegs ? kMaxSubsegs : sub);
    const int64_t slices = per * sub + pairs * ns;
    p.segments = ns;
    p.subsegs = static_cast<int>(sub);
    p.workspace_bytes = static_cast<size_t>(slices) * head_dim * head_dim * sizeof(float);
    return p;
}

// Checks of the device metadata after a copy to the host (debug mode,
// [LA-page] §生产环境不支持 item 1: unsupported inputs are rejected before
// anything runs).  cu may be null (fixed-length requests of fixed_len tokens);
// track arrays and parents may be null.
inline la_status check_metadata(const int32_t *cu, int batch, int64_t total_tokens, int max_seqlen,
                                int fixed_len, const int32_t *slots, int64_t pool_slots,
                                const int32_t *track_lens, const int32_t *track_slots,
                                const int32_t *parents) {
    if (batch < 0 || pool_slots <= 0 || (parents && fixed_len <= 0)) return LA_ERR_INVALID_ARG;
    std::vector<int64_t> lens(static_cast<size_t>(batch), fixed_len);
    if (cu) {
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
        for (int b = 0; b < batch; ++b) {
            const int32_t ts = track_slots[b];
            if (ts < 0) continue;  // no snapshot for this request
            if (ts >= pool_slots || seen[ts] || track_lens[b] < 0 || track_lens[b] > lens[b])
                return LA_ERR_INVALID_ARG;
            seen[ts] = 1;
        }
    }
    if (parents) {
        for (size_t i = 0; i < static_cast<size_t>(batch) * fixed_len; ++i) {
            const int j = static_cast<int>(i % fixed_len);
            if (parents[i] < -1 || parents[i] >= j) return LA_ERR_INVALID_ARG;
        }
    }
    return LA_OK;
}

}  // namespace la
