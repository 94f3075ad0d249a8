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
// which is exact up to rounding order.  Everything runs on
// v_mfma_f32_16x16x32_bf16 with fp32 accumulation, computing the transposed
// output O^T (value column x token):
//   scores   A^T = K Q^T                     16x16 causal tiles (j <= i)
//   intra    O^T += V^T P^T,   P = A * e^{-l(i-j)}, split hi + lo
//   inter    O^T += S_prev^T Q^T             S_prev split hi + lo, scaled by e^{-l(i+1)}
//   update   S = e^{-l c} S + K^T Vd,  Vd = decayed V split hi + lo
// The hi + lo split (x = hi + lo, both bf16) keeps every operand that is not
// an exact bf16 input to ~2^-17 relative error; without it the bf16 rounding
// of P, S_prev and Vd each add output errors of order 1e-2 on small-slope heads.
//
// Work split.  One workgroup of 4 waves per (request, head, 32-column block of
// S); the block id is mapped so the 4 column blocks of a head share an XCD
// (ids are dealt to the 8 XCDs round-robin) and its L2 serves their repeated
// Q/K reads.  Wave w keeps the fp32 state rows 32w..32w+31 of the block in
// MFMA accumulators for the whole request.  Per chunk every wave computes
//   * the inter term restricted to its own 32 state rows, for all 64 tokens,
//     straight from its accumulators (no state exchange),
//   * a balanced share of the 10 causal score tiles and their P V products,
//   * the update of its own state rows,
// and the four partial O^T tiles of each 16-token row block are summed through
// LDS by the wave that stores them.  Operands that the MFMA needs with tokens
// along the contraction (K^T, V^T, Vd) are read from token-major LDS tiles
// with ds_read_b64_tr_b16, whose 16-lane groups return the columns of a
// 4-row block.  The next chunk's global loads are issued before the current
// chunk's MFMAs.
#include "common.h"
#include "launch.h"

namespace la {
namespace {

constexpr int D = kHeadDim;  // 128
constexpr int C = 64;        // chunk length
constexpr int VB = 32;       // state columns per workgroup
constexpr int NVB = D / VB;  // column blocks per head
constexpr int NT = 256;      // threads per workgroup
constexpr int QLD = D + 8;   // row stride (elements) of the Q and K tiles
constexpr int VLD = VB + 16; // row stride (elements) of the V tiles

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct Smem {
    uint16_t q[C][QLD];
    uint16_t k[C][QLD];
    uint16_t v[C][VLD];
    uint16_t vd_hi[C][VLD];
    uint16_t vd_lo[C][VLD];
    f32x4 part[4][4][2][64];  // [source wave][row block][column tile][lane]
};

__device__ __forceinline__ f32x4 mma(u16x8 a, u16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u16x8 lds8(const uint16_t *p) { return *reinterpret_cast<const u16x8 *>(p); }
__device__ __forceinline__ u16x4 lds4(const uint16_t *p) { return *reinterpret_cast<const u16x4 *>(p); }

// Transposed 4x16 read: the 16-lane group g addresses rows row0 + 4g .. +3 and
// columns col0 .. col0+15 of a row-major bf16 tile with row stride ld; lane
// (g, i) receives column col0 + i of those four rows.
__device__ __forceinline__ u16x4 ldtr(const uint16_t *tile, int ld, int row0, int col0, int g, int l16) {
    const uint16_t *p = tile + (row0 + 4 * g + (l16 >> 2)) * ld + col0 + 4 * (l16 & 3);
    bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
    return __builtin_bit_cast(u16x4, r);
}

__device__ __forceinline__ u16x8 cat(u16x4 a, u16x4 b) {
    return u16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// float pair -> bf16 pair (hardware round to nearest even)
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

__device__ __forceinline__ float lo16f(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float hi16f(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// x -> (hi, lo) bf16 quads with x = hi + lo up to ~2^-17 relative
__device__ __forceinline__ void split4(f32x4 x, u16x4 &hi, u16x4 &lo) {
    const uint32_t h01 = cvt2(x[0], x[1]), h23 = cvt2(x[2], x[3]);
    const uint32_t l01 = cvt2(x[0] - lo16f(h01), x[1] - hi16f(h01));
    const uint32_t l23 = cvt2(x[2] - lo16f(h23), x[3] - hi16f(h23));
    hi = __builtin_bit_cast(u16x4, (uint64_t)h01 | ((uint64_t)h23 << 32));
    lo = __builtin_bit_cast(u16x4, (uint64_t)l01 | ((uint64_t)l23 << 32));
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

// Score tiles (j-tile, i-tile), j <= i, dealt to the waves 3/3/2/2; each
// wave's P V products group its tiles by i-tile (at most two j-tiles, which
// together fill one 32-token contraction).
template <int W> struct Tiles;
template <> struct Tiles<0> { static constexpr int n = 3, jt[3] = {0, 0, 1}, it[3] = {0, 1, 1};
                              static constexpr int ng = 2, git[2] = {0, 1}, ga[2] = {0, 1}, gb[2] = {-1, 2}; };
template <> struct Tiles<1> { static constexpr int n = 3, jt[3] = {2, 2, 3}, it[3] = {2, 3, 3};
                              static constexpr int ng = 2, git[2] = {2, 3}, ga[2] = {0, 1}, gb[2] = {-1, 2}; };
template <> struct Tiles<2> { static constexpr int n = 2, jt[3] = {0, 0, 0}, it[3] = {2, 3, 0};
                              static constexpr int ng = 2, git[2] = {2, 3}, ga[2] = {0, 1}, gb[2] = {-1, -1}; };
template <> struct Tiles<3> { static constexpr int n = 2, jt[3] = {1, 1, 0}, it[3] = {2, 3, 0};
                              static constexpr int ng = 2, git[2] = {2, 3}, ga[2] = {0, 1}, gb[2] = {-1, -1}; };

// One chunk for wave W: accumulate the partial O^T tiles part[it][nt] and
// advance this wave's state rows S[mt][nt].
// mdec[4t + r]: causal decay of score tile t element r; qdec[it]:
// e^{-l(i+1)} for i = 16 it + l16; dc: e^{-l c}
template <int W>
__device__ __forceinline__ void chunk_compute(Smem &sm, const float (&mdec)[12], const float (&qdec)[4],
                                              float dc, int g, int l16, f32x4 (&S)[2][2],
                                              f32x4 (&part)[4][2]) {
    using T = Tiles<W>;

    // inter term over this wave's 32 state rows: O^T[v][i] = sum_k S^T[v][k] Q^T[k][i].
    // A operand (v x k) comes from the accumulators: lane (g, l16) holds
    // rows k = 32W + 4g + r (mt 0) and 32W + 16 + 4g + r (mt 1) of column v = l16.
    u16x8 sa_hi[2], sa_lo[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
        u16x4 h0, l0, h1, l1;
        split4(S[0][nt], h0, l0);
        split4(S[1][nt], h1, l1);
        sa_hi[nt] = cat(h0, h1);
        sa_lo[nt] = cat(l0, l1);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const uint16_t *qrow = &sm.q[16 * it + l16][32 * W + 4 * g];
        const u16x8 qb = cat(lds4(qrow), lds4(qrow + 16));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            acc = mma(sa_hi[nt], qb, acc);
            acc = mma(sa_lo[nt], qb, acc);
            part[it][nt] += acc * qdec[it];
        }
    }

    // causal score tiles A^T[j][i] = k_j . q_i, masked and decayed, split hi/lo
    u16x4 p_hi[3], p_lo[3];
#pragma unroll
    for (int t = 0; t < T::n; ++t) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = mma(lds8(&sm.k[16 * T::jt[t] + l16][32 * s + 8 * g]),
                      lds8(&sm.q[16 * T::it[t] + l16][32 * s + 8 * g]), acc);
        f32x4 p;
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = acc[r] * mdec[4 * t + r];
        split4(p, p_hi[t], p_lo[t]);
    }
    // intra term O^T[v][i] += sum_j V[j][v] P[i][j]; B operand slots 0..3 hold
    // j-tile ga's rows 4g..4g+3, slots 4..7 j-tile gb's (or zero)
    const u16x4 z4 = {0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < T::ng; ++q) {
        const int ta = T::ga[q], tb = T::gb[q];
        const int it = T::git[q];
        const u16x8 bh = cat(p_hi[ta], tb >= 0 ? p_hi[tb] : z4);
        const u16x8 bl = cat(p_lo[ta], tb >= 0 ? p_lo[tb] : z4);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const u16x4 va = ldtr(&sm.v[0][0], VLD, 16 * T::jt[ta], 16 * nt, g, l16);
            const u16x4 vb = tb >= 0 ? ldtr(&sm.v[0][0], VLD, 16 * T::jt[tb], 16 * nt, g, l16) : z4;
            const u16x8 av = cat(va, vb);
            part[it][nt] = mma(av, bh, part[it][nt]);
            part[it][nt] = mma(av, bl, part[it][nt]);
        }
    }

    // state update of rows 32W..32W+31: S[k][v] = e^{-l c} S + sum_j K[j][k] Vd[j][v]
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) S[mt][nt] *= dc;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        u16x8 ka[2], vh[2], vl[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
            ka[mt] = cat(ldtr(&sm.k[0][0], QLD, 32 * s2, 32 * W + 16 * mt, g, l16),
                         ldtr(&sm.k[0][0], QLD, 32 * s2 + 16, 32 * W + 16 * mt, g, l16));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            vh[nt] = cat(ldtr(&sm.vd_hi[0][0], VLD, 32 * s2, 16 * nt, g, l16),
                         ldtr(&sm.vd_hi[0][0], VLD, 32 * s2 + 16, 16 * nt, g, l16));
            vl[nt] = cat(ldtr(&sm.vd_lo[0][0], VLD, 32 * s2, 16 * nt, g, l16),
                         ldtr(&sm.vd_lo[0][0], VLD, 32 * s2 + 16, 16 * nt, g, l16));
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                S[mt][nt] = mma(ka[mt], vh[nt], S[mt][nt]);
                S[mt][nt] = mma(ka[mt], vl[nt], S[mt][nt]);
            }
    }
}

// per-lane causal decay of wave W's score tiles: element (t, r) is
// (j, i) = (16 jt + 4g + r, 16 it + l16)
template <int W>
__device__ __forceinline__ void score_decay(float lam, int g, int l16, float (&mdec)[12]) {
    using T = Tiles<W>;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * T::jt[t] + 4 * g + r, i = 16 * T::it[t] + l16;
            mdec[4 * t + r] = (t < T::n && j <= i) ? expf(-lam * static_cast<float>(i - j)) : 0.f;
        }
}

struct Job {
    const uint16_t *q, *k, *v;
    uint16_t *out;
    float *state;   // this (request, head)'s pool slot
    int64_t t0, len;
    size_t row, hcol;
    int col0;
    float lam;
};

// Whole request for wave W of the workgroup.
template <int W>
__device__ __forceinline__ void run_wave(Smem &sm, const Job &jb) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const float lam = jb.lam;
    const float scale = 0.08838834764831845f;  // 128^-1/2
    const size_t row = jb.row, hcol = jb.hcol;
    const int col0 = jb.col0;

    float mdec[12], qdec[4];
    score_decay<W>(lam, g, l16, mdec);
#pragma unroll
    for (int it = 0; it < 4; ++it) qdec[it] = expf(-lam * static_cast<float>(16 * it + l16 + 1));

    // state rows 32W..32W+31 of the block: tile (mt, nt), element r is
    // S[32W + 16mt + 4g + r][col0 + 16nt + l16]
    f32x4 S[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mt][nt][r] = jb.state[(32 * W + 16 * mt + 4 * g + r) * D + col0 + 16 * nt + l16];

    // staging registers: Q/K 16-byte pieces p = tid + 256u (row p/16, piece
    // p%16); V piece row tid/4, columns col0 + 8*(tid%4) .. +7
    u16x8 pq[4], pk[4], pv;
    const u16x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    auto fetch = [&](int64_t t, int c) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = tid + NT * u;
            const int r = p >> 4, pc = p & 15;
            if (r < c) {
                const size_t off = (t + r) * row + hcol + 8 * pc;
                pq[u] = *reinterpret_cast<const u16x8 *>(jb.q + off);
                pk[u] = *reinterpret_cast<const u16x8 *>(jb.k + off);
            } else {
                pq[u] = zero8;
                pk[u] = zero8;
            }
        }
        const int r = tid >> 2;
        pv = (r < c) ? *reinterpret_cast<const u16x8 *>(jb.v + (t + r) * row + hcol + col0 + 8 * (tid & 3))
                     : zero8;
    };

    const int64_t len = jb.len;
    const int nchunks = static_cast<int>((len + C - 1) / C);
    fetch(jb.t0, static_cast<int>(len < C ? len : C));

    for (int ci = 0; ci < nchunks; ++ci) {
        const int64_t t = jb.t0 + static_cast<int64_t>(ci) * C;
        const int64_t rem = len - static_cast<int64_t>(ci) * C;
        const int c = static_cast<int>(rem < C ? rem : C);

        // stage the chunk (every wave is past the previous chunk's reads of
        // these tiles: it waited at the partial-sum barrier below)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = tid + NT * u;
            const int r = p >> 4, pc = p & 15;
            *reinterpret_cast<u16x8 *>(&sm.q[r][8 * pc]) = pq[u];
            *reinterpret_cast<u16x8 *>(&sm.k[r][8 * pc]) = pk[u];
        }
        {
            const int r = tid >> 2, pc = tid & 3;
            const float vdec = (r < c) ? expf(-lam * static_cast<float>(c - 1 - r)) : 0.f;
            *reinterpret_cast<u16x8 *>(&sm.v[r][8 * pc]) = pv;
            f32x4 x0, x1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x0[e] = bf16_to_f32(pv[e]) * vdec;
                x1[e] = bf16_to_f32(pv[4 + e]) * vdec;
            }
            u16x4 h0, l0, h1, l1;
            split4(x0, h0, l0);
            split4(x1, h1, l1);
            *reinterpret_cast<u16x8 *>(&sm.vd_hi[r][8 * pc]) = cat(h0, h1);
            *reinterpret_cast<u16x8 *>(&sm.vd_lo[r][8 * pc]) = cat(l0, l1);
        }
        __syncthreads();

        if (ci + 1 < nchunks) {
            const int64_t rem1 = rem - C;
            fetch(t + C, static_cast<int>(rem1 < C ? rem1 : C));
        }

        f32x4 part[4][2];
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) part[it][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        chunk_compute<W>(sm, mdec, qdec, expf(-lam * static_cast<float>(c)), g, l16, S, part);

        // hand the partial O^T tiles of the other row blocks to their owners
#pragma unroll
        for (int it = 0; it < 4; ++it)
            if (it != W)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) sm.part[W][it][nt][lane] = part[it][nt];
        __syncthreads();

        // row block W: sum the four partials and store o = scale * O.
        // O^T tile nt, element r: value column col0 + 16nt + 4g + r, token 16W + l16
        const int i = 16 * W + l16;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x4 o = part[W][nt];
#pragma unroll
            for (int src = 0; src < 4; ++src)
                if (src != W) o += sm.part[src][W][nt][lane];
            if (i < c) {
                o *= scale;
                const uint64_t packed = (uint64_t)cvt2(o[0], o[1]) | ((uint64_t)cvt2(o[2], o[3]) << 32);
                *reinterpret_cast<uint64_t *>(jb.out + (t + i) * row + hcol + col0 + 16 * nt + 4 * g) = packed;
            }
        }
    }

#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                jb.state[(32 * W + 16 * mt + 4 * g + r) * D + col0 + 16 * nt + l16] = S[mt][nt][r];
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
    Job jb{q, k, v, out, pool + (static_cast<size_t>(slot) * num_heads + h) * (D * D), t0, len,
           row, hcol, col0, slopes[h]};
    switch (__builtin_amdgcn_readfirstlane(tid >> 6)) {
    case 0: run_wave<0>(sm, jb); break;
    case 1: run_wave<1>(sm, jb); break;
    case 2: run_wave<2>(sm, jb); break;
    default: run_wave<3>(sm, jb); break;
    }
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
