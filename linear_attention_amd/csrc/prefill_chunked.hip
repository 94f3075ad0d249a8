// Chunked bf16 MFMA prefill for seg_la on gfx950.
//
// Citations name the web page "SGLang Lightning Attention 能力矩阵与 seg_la
// 线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page].
//
// The recurrence of [LA-page] §独立参考实现 (S <- e^{-l} S + k v^T,
// o = q S / sqrt(d)) is re-associated over chunks of C = 64 tokens.  With
// S_prev the state before a chunk of c tokens and i, j local token indices:
//   o_i    = scale * [ sum_{j<=i} e^{-l(i-j)} (q_i.k_j) v_j  +  e^{-l(i+1)} q_i S_prev ]
//   S_next = e^{-l c} S_prev + sum_j k_j (e^{-l(c-1-j)} v_j)^T
// which is exact up to rounding order.  The four products run on MFMA
// (v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   A  = Q K^T          (causal 16x16 tiles only)
//   Oi = P V            P = A * e^{-l(i-j)} masked to j <= i, split hi+lo
//   Oq = Q S_prev       S_prev split hi+lo (bf16 copies of the fp32 state)
//   S  = e^{-l c} S + K^T Vd,   Vd = decayed V split hi+lo
// The hi+lo split (x = hi + lo, both bf16) keeps every operand that is not an
// exact bf16 input to ~2^-17 relative error; without it the bf16 rounding of
// P, S_prev and the decayed V each add errors of the order of 1e-2 to outputs
// of small-slope heads.
//
// Parallelism: one workgroup (4 waves) per (request, head, 32-column block of
// S).  Each block re-reads the head's Q and K; the block id is mapped so the
// four column blocks of one head land on the same XCD (blocks are dispatched
// round-robin over the 8 XCDs) and share its L2.  The master state block
// (128 x 32 fp32) stays in MFMA accumulators for the whole request; chunk
// inputs are prefetched into registers while the previous chunk computes.
#include "common.h"
#include "launch.h"

namespace la {
namespace {

constexpr int D = kHeadDim;  // 128
constexpr int C = 64;        // chunk length
constexpr int VB = 32;       // state columns per workgroup
constexpr int NVB = D / VB;  // column blocks per head
constexpr int NT = 256;      // threads per workgroup
constexpr int LDQ = D + 8;   // row stride (elements) of feature-contiguous tiles
constexpr int LDT = C + 8;   // row stride (elements) of token-contiguous tiles

struct Smem {
    uint16_t q[C][LDQ];      // Q chunk, token-major
    uint16_t k[C][LDQ];      // K chunk, token-major
    uint16_t kt[D][LDT];     // K chunk, feature-major
    uint16_t vt[VB][LDT];    // V column block, feature-major
    uint16_t vd_hi[VB][LDT]; // decayed V column block, feature-major, hi/lo
    uint16_t vd_lo[VB][LDT];
    uint16_t p_hi[C][LDT];   // masked decayed scores, hi/lo
    uint16_t p_lo[C][LDT];
    uint16_t st_hi[VB][LDQ]; // S_prev column block, value-column-major, hi/lo
    uint16_t st_lo[VB][LDQ];
};

__device__ __forceinline__ f32x4 mma(u16x8 a, u16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u16x8 lds8(const uint16_t *p) { return *reinterpret_cast<const u16x8 *>(p); }

__device__ __forceinline__ void split(float x, uint16_t &hi, uint16_t &lo) {
    hi = f32_to_bf16(x);
    lo = f32_to_bf16(x - bf16_to_f32(hi));
}

// Workgroup id -> (pair = request*H + head, column block).  Ids are dealt to
// XCDs round-robin (id % 8), so groups of 8 pairs are laid out with the pair
// in the low 3 bits: the NVB blocks of one pair share id % 8.
__device__ __forceinline__ void map_block(int id, int pairs, int &pair, int &vb) {
    const int full = (pairs / 8) * 8 * NVB;
    if (id < full) {
        const int x = id & 7, y = id >> 3;
        vb = y % NVB;
        pair = (y / NVB) * 8 + x;
    } else {
        const int r = id - full;
        pair = (pairs / 8) * 8 + r / NVB;
        vb = r % NVB;
    }
}

__global__ __launch_bounds__(NT) void prefill_chunked_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const int32_t *__restrict__ cu_seqlens, int num_heads, int pairs, int64_t total_tokens,
    float *__restrict__ pool, int64_t pool_slots, const int32_t *__restrict__ slot_idx,
    const float *__restrict__ slopes, uint16_t *__restrict__ out) {
    __shared__ Smem sm;

    int pair, vb;
    map_block(blockIdx.x, pairs, pair, vb);
    const int b = pair / num_heads;
    const int h = pair - b * num_heads;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g = lane >> 4;

    int64_t t0 = cu_seqlens[b], t1 = cu_seqlens[b + 1];
    t0 = t0 < 0 ? 0 : (t0 > total_tokens ? total_tokens : t0);
    t1 = t1 < t0 ? t0 : (t1 > total_tokens ? total_tokens : t1);
    const int64_t len = t1 - t0;
    if (len <= 0) return;  // empty request: no-op

    const size_t row = static_cast<size_t>(num_heads) * D;
    const size_t hcol = static_cast<size_t>(h) * D;
    const int col0 = vb * VB;
    const int slot = slot_idx[b];
    if (slot < 0 || slot >= pool_slots) {
        // out-of-range slot: zero output for this column block, no state touched
        for (int64_t idx = tid; idx < len * (VB / 8); idx += NT) {
            const int64_t t = t0 + idx / (VB / 8);
            *reinterpret_cast<u16x8 *>(out + t * row + hcol + col0 + 8 * (idx % (VB / 8))) =
                u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        return;
    }
    float *state = pool + (static_cast<size_t>(slot) * num_heads + h) * (D * D);

    const float lam = slopes[h];
    const float scale = 0.08838834764831845f;  // 128^-1/2

    // per-lane decay constants for full chunks: score tile (jt, r) holds
    // (i, j) = (16w + 4g + r, 16jt + l16); query decay for row i is e^{-l(i+1)}
    float mdec[4][4], qdec[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = 16 * w + 4 * g + r;
        qdec[r] = expf(-lam * static_cast<float>(i + 1));
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            const int j = 16 * jt + l16;
            mdec[jt][r] = (j <= i) ? expf(-lam * static_cast<float>(i - j)) : 0.f;
        }
    }

    // master state block: wave w owns key rows 32w..32w+31; tile (mt, nt) lane
    // element r is S[32w + 16mt + 4g + r][col0 + 16nt + l16]
    f32x4 S[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mt][nt][r] = state[(32 * w + 16 * mt + 4 * g + r) * D + col0 + 16 * nt + l16];

    // staging registers: Q/K 16-byte pieces p = tid + 256u (row p/16, piece p%16),
    // V piece row tid/4, 8 columns at col0 + 8*(tid%4)
    u16x8 pq[4], pk[4], pv;
    const u16x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    auto fetch = [&](int64_t t, int c) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = tid + NT * u;
            const int r = p >> 4, pc = p & 15;
            if (r < c) {
                const size_t off = (t + r) * row + hcol + 8 * pc;
                pq[u] = *reinterpret_cast<const u16x8 *>(q + off);
                pk[u] = *reinterpret_cast<const u16x8 *>(k + off);
            } else {
                pq[u] = zero8;
                pk[u] = zero8;
            }
        }
        const int r = tid >> 2;
        pv = (r < c) ? *reinterpret_cast<const u16x8 *>(v + (t + r) * row + hcol + col0 + 8 * (tid & 3))
                     : zero8;
    };

    const int nchunks = static_cast<int>((len + C - 1) / C);
    fetch(t0, static_cast<int>(len < C ? len : C));

    for (int ci = 0; ci < nchunks; ++ci) {
        const int64_t t = t0 + static_cast<int64_t>(ci) * C;
        const int c = static_cast<int>((len - static_cast<int64_t>(ci) * C) < C ? (len - static_cast<int64_t>(ci) * C) : C);

        __syncthreads();  // previous chunk's LDS reads are done
        // stage the chunk
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = tid + NT * u;
            const int r = p >> 4, pc = p & 15;
            *reinterpret_cast<u16x8 *>(&sm.q[r][8 * pc]) = pq[u];
            *reinterpret_cast<u16x8 *>(&sm.k[r][8 * pc]) = pk[u];
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.kt[8 * pc + e][r] = pk[u][e];
        }
        {
            const int r = tid >> 2, pc = tid & 3;
            const float vdec = (r < c) ? expf(-lam * static_cast<float>(c - 1 - r)) : 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                sm.vt[8 * pc + e][r] = pv[e];
                uint16_t hi, lo;
                split(bf16_to_f32(pv[e]) * vdec, hi, lo);
                sm.vd_hi[8 * pc + e][r] = hi;
                sm.vd_lo[8 * pc + e][r] = lo;
            }
        }
        // S_prev as bf16 hi/lo, value-column-major
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                u16x4 hi, lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint16_t a, bb;
                    split(S[mt][nt][r], a, bb);
                    hi[r] = a;
                    lo[r] = bb;
                }
                const int n = 16 * nt + l16, kk = 32 * w + 16 * mt + 4 * g;
                *reinterpret_cast<u16x4 *>(&sm.st_hi[n][kk]) = hi;
                *reinterpret_cast<u16x4 *>(&sm.st_lo[n][kk]) = lo;
            }
        __syncthreads();

        if (ci + 1 < nchunks) {
            const int64_t rem = len - static_cast<int64_t>(ci + 1) * C;
            fetch(t + C, static_cast<int>(rem < C ? rem : C));
        }

        // ---- scores for rows 16w..16w+15 (causal tiles jt <= w)
        u16x8 qa[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) qa[s] = lds8(&sm.q[16 * w + l16][32 * s + 8 * g]);
        f32x4 sc[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            sc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (jt <= w) {
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    sc[jt] = mma(qa[s], lds8(&sm.k[16 * jt + l16][32 * s + 8 * g]), sc[jt]);
            }
        }
        // mask + decay, split, to LDS (only this wave reads these rows); tiles
        // up to the 32-token contraction extent PV uses are written
        const int jlim = 2 * (w / 2 + 1);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            if (jt < jlim) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint16_t hi, lo;
                    split(sc[jt][r] * mdec[jt][r], hi, lo);
                    sm.p_hi[16 * w + 4 * g + r][16 * jt + l16] = hi;
                    sm.p_lo[16 * w + 4 * g + r][16 * jt + l16] = lo;
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // ---- intra-chunk P V and inter-chunk Q S_prev
        f32x4 oi[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        f32x4 oq[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            if (s2 <= w / 2) {
                const u16x8 ah = lds8(&sm.p_hi[16 * w + l16][32 * s2 + 8 * g]);
                const u16x8 al = lds8(&sm.p_lo[16 * w + l16][32 * s2 + 8 * g]);
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const u16x8 bv = lds8(&sm.vt[16 * nt + l16][32 * s2 + 8 * g]);
                    oi[nt] = mma(ah, bv, oi[nt]);
                    oi[nt] = mma(al, bv, oi[nt]);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                oq[nt] = mma(qa[s], lds8(&sm.st_hi[16 * nt + l16][32 * s + 8 * g]), oq[nt]);
                oq[nt] = mma(qa[s], lds8(&sm.st_lo[16 * nt + l16][32 * s + 8 * g]), oq[nt]);
            }
        // ---- outputs: row i = 16w + 4g + r, column col0 + 16nt + l16
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * w + 4 * g + r;
            if (i < c) {
                uint16_t *orow = out + (t + i) * row + hcol + col0 + l16;
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    orow[16 * nt] = f32_to_bf16(scale * (oi[nt][r] + qdec[r] * oq[nt][r]));
            }
        }

        // ---- state update: S = e^{-l c} S + K^T Vd
        const float dc = expf(-lam * static_cast<float>(c));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                S[mt][nt] *= dc;
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const u16x8 a = lds8(&sm.kt[32 * w + 16 * mt + l16][32 * s2 + 8 * g]);
                    S[mt][nt] = mma(a, lds8(&sm.vd_hi[16 * nt + l16][32 * s2 + 8 * g]), S[mt][nt]);
                    S[mt][nt] = mma(a, lds8(&sm.vd_lo[16 * nt + l16][32 * s2 + 8 * g]), S[mt][nt]);
                }
            }
    }

#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                state[(32 * w + 16 * mt + 4 * g + r) * D + col0 + 16 * nt + l16] = S[mt][nt][r];
}

}  // namespace

hipError_t launch_prefill_chunked(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                  const int32_t *cu_seqlens, int batch, int num_heads,
                                  int64_t total_tokens, float *pool, int64_t pool_slots,
                                  const int32_t *slot_idx, const float *slopes, uint16_t *out,
                                  hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    int pairs = batch * num_heads;
    void *args[] = {&q, &k, &v, &cu_seqlens, &num_heads, &pairs, &total_tokens,
                    &pool, &pool_slots, &slot_idx, &slopes, &out};
    return hipLaunchKernel(reinterpret_cast<const void *>(&prefill_chunked_kernel),
                           dim3(static_cast<unsigned>(pairs) * NVB), dim3(NT), args, 0, stream);
}

}  // namespace la
