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
constexpr int VLD = VB + 16; // row stride (elements) of the V tiles (conflict-free for the
                             // 4-row transposed reads: rows land 24 banks apart)

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Q and K tiles: 64 rows of 128 elements (256 B, one pass over the 64 LDS
// banks) with the 16-byte units of row r permuted by u -> u ^ swz(r).  swz takes
// 16 distinct values over any 16 consecutive rows (16-byte reads of one column
// unit from 16 rows hit distinct banks) and maps the unit pair {2m, 2m+1} of 4
// consecutive rows to 4 distinct pairs (the 4x16 transposed reads hit
// distinct banks).
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int qk_off(int r, int col) {
    return r * D + ((((col >> 3) ^ swz(r)) << 3) | (col & 7));
}

struct Smem {
    uint16_t q[C * D];
    uint16_t k[C * D];
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
__device__ __forceinline__ u16x4 tr_at(const uint16_t *p) {
    bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
    return __builtin_bit_cast(u16x4, r);
}
__device__ __forceinline__ u16x4 ldtr(const uint16_t *tile, int ld, int row0, int col0, int g, int l16) {
    return tr_at(tile + (row0 + 4 * g + (l16 >> 2)) * ld + col0 + 4 * (l16 & 3));
}
// the same read from a swizzled Q/K tile (col0 a multiple of 16)
__device__ __forceinline__ u16x4 ldtr_qk(const uint16_t *tile, int row0, int col0, int g, int l16) {
    return tr_at(tile + qk_off(row0 + 4 * g + (l16 >> 2), col0 + 4 * (l16 & 3)));
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

// Decay handling.  With kF ("factored", used for 0 <= l <= 2) the state is
// kept in the scaled frame S_m = e^{-32 l} S, the score tiles are weighted by
// e^{l (j - 31)} and the sum of all partials is multiplied once by
// e^{-l (i - 31)}: that is the same o_i, because
//   e^{-l(i-j)} = e^{-l(i-31)} e^{l(j-31)}  and  e^{-l(i+1)} S = e^{-l(i-31)} S_m,
// and every factor stays inside the fp32/bf16 exponent range for l <= 2.
// Without kF the weights e^{-l(i-j)} and e^{-l(i+1)} are applied directly.

// One chunk for wave W: produce the partial O^T tiles part[it][nt] and
// advance this wave's state rows S[mt][nt].  mdec[4t + r]: weight of score
// tile t element r; qdec[it]: weight of the inter term for i = 16 it + l16
// (only used without kF); dc: e^{-l c}.
template <int W, bool kF>
__device__ __forceinline__ void chunk_compute(Smem &sm, const float (&mdec)[12], const float (&qdec)[4],
                                              float dc, int g, int l16, f32x4 (&S)[2][2],
                                              f32x4 (&part)[4][2]) {
    using T = Tiles<W>;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};

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
        const int qr = 16 * it + l16;
        const u16x8 qb = cat(lds4(&sm.q[qk_off(qr, 32 * W + 4 * g)]),
                             lds4(&sm.q[qk_off(qr, 32 * W + 16 + 4 * g)]));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x4 acc = mma(sa_hi[nt], qb, z);
            acc = mma(sa_lo[nt], qb, acc);
            part[it][nt] = kF ? acc : acc * qdec[it];
        }
    }

    // causal score tiles A^T[j][i] = k_j . q_i, weighted and masked, split hi/lo
    u16x4 p_hi[3], p_lo[3];
#pragma unroll
    for (int t = 0; t < T::n; ++t) {
        f32x4 acc = z;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = mma(lds8(&sm.k[qk_off(16 * T::jt[t] + l16, 32 * s + 8 * g)]),
                      lds8(&sm.q[qk_off(16 * T::it[t] + l16, 32 * s + 8 * g)]), acc);
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
            ka[mt] = cat(ldtr_qk(sm.k, 32 * s2, 32 * W + 16 * mt, g, l16),
                         ldtr_qk(sm.k, 32 * s2 + 16, 32 * W + 16 * mt, g, l16));
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

// per-lane weights of wave W's score tiles: element (t, r) is
// (j, i) = (16 jt + 4g + r, 16 it + l16), zero above the diagonal
template <int W, bool kF>
__device__ __forceinline__ void score_decay(float lam, int g, int l16, float (&mdec)[12]) {
    using T = Tiles<W>;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * T::jt[t] + 4 * g + r, i = 16 * T::it[t] + l16;
            const float e = kF ? static_cast<float>(j - 31) : -static_cast<float>(i - j);
            mdec[4 * t + r] = (t < T::n && j <= i) ? expf(lam * e) : 0.f;
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
template <int W, bool kF>
__device__ __forceinline__ void run_wave(Smem &sm, const Job &jb) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const float lam = jb.lam;
    const float scale = 0.08838834764831845f;  // 128^-1/2
    const uint32_t row = static_cast<uint32_t>(jb.row);
    const int col0 = jb.col0;

    float mdec[12], qdec[4];
    score_decay<W, kF>(lam, g, l16, mdec);
#pragma unroll
    for (int it = 0; it < 4; ++it) qdec[it] = expf(-lam * static_cast<float>(16 * it + l16 + 1));
    // output factor of row block W (token i = 16W + l16)
    const float fin = kF ? scale * expf(-lam * static_cast<float>(16 * W + l16 - 31)) : scale;
    // state frame: S_m = sigma * S
    const float sigma = kF ? expf(-32.f * lam) : 1.f;
    const float vshift = kF ? 32.f : 0.f;

    // state rows 32W..32W+31 of the block: tile (mt, nt), element r is
    // S[32W + 16mt + 4g + r][col0 + 16nt + l16]
    f32x4 S[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mt][nt][r] = sigma * jb.state[(32 * W + 16 * mt + 4 * g + r) * D + col0 + 16 * nt + l16];

    // staging: Q/K 16-byte pieces p = tid + 256u (row p/16, piece p%16); V
    // piece row tid/4, columns col0 + 8*(tid%4) .. +7.  Per-lane offsets are
    // fixed; each chunk only moves the uniform base.
    uint32_t offqk[4];  // byte offsets
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int p = tid + NT * u;
        offqk[u] = 2u * (static_cast<uint32_t>(p >> 4) * row + 8 * (p & 15));
    }
    const int vr = tid >> 2;
    const uint32_t offv = 2u * (static_cast<uint32_t>(vr) * row + 8 * (tid & 3));
    const uint32_t offo = 2u * (static_cast<uint32_t>(16 * W + l16) * row + 4 * g);

    const int64_t len = jb.len;
    const int nchunks = static_cast<int>((len + C - 1) / C);
    const int c_last = static_cast<int>(len - static_cast<int64_t>(nchunks - 1) * C);
    // weight of V row vr and the state decay in a full chunk and in the last one
    const float vdec_full = expf(-lam * (static_cast<float>(C - 1 - vr) + vshift));
    const float vdec_last = vr < c_last ? expf(-lam * (static_cast<float>(c_last - 1 - vr) + vshift)) : 0.f;
    const float dc_full = expf(-lam * static_cast<float>(C));
    const float dc_last = expf(-lam * static_cast<float>(c_last));

    u16x8 pq[4], pk[4], pv;
    const u16x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
    auto ld16 = [](const char *base, uint32_t off) {
        return *reinterpret_cast<const u16x8 *>(base + off);
    };
    auto fetch = [&](int64_t t, int c) {
        const char *qb = reinterpret_cast<const char *>(jb.q + t * jb.row + jb.hcol);
        const char *kb = reinterpret_cast<const char *>(jb.k + t * jb.row + jb.hcol);
        const char *vb = reinterpret_cast<const char *>(jb.v + t * jb.row + jb.hcol + col0);
        if (c == C) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                pq[u] = ld16(qb, offqk[u]);
                pk[u] = ld16(kb, offqk[u]);
            }
            pv = ld16(vb, offv);
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool ok = ((tid + NT * u) >> 4) < c;
                pq[u] = ok ? ld16(qb, offqk[u]) : zero8;
                pk[u] = ok ? ld16(kb, offqk[u]) : zero8;
            }
            pv = vr < c ? ld16(vb, offv) : zero8;
        }
    };

    fetch(jb.t0, static_cast<int>(len < C ? len : C));

    for (int ci = 0; ci < nchunks; ++ci) {
        const int64_t t = jb.t0 + static_cast<int64_t>(ci) * C;
        const int64_t rem = len - static_cast<int64_t>(ci) * C;
        const int c = static_cast<int>(rem < C ? rem : C);
        const bool full = c == C;

        // stage the chunk (every wave is past the previous chunk's reads of
        // these tiles: it waited at the partial-sum barrier below)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int p = tid + NT * u;
            const int r = p >> 4, pc = p & 15;
            *reinterpret_cast<u16x8 *>(&sm.q[qk_off(r, 8 * pc)]) = pq[u];
            *reinterpret_cast<u16x8 *>(&sm.k[qk_off(r, 8 * pc)]) = pk[u];
        }
        {
            const int pc = tid & 3;
            const float vdec = full ? vdec_full : vdec_last;
            *reinterpret_cast<u16x8 *>(&sm.v[vr][8 * pc]) = pv;
            f32x4 x0, x1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x0[e] = bf16_to_f32(pv[e]) * vdec;
                x1[e] = bf16_to_f32(pv[4 + e]) * vdec;
            }
            u16x4 h0, l0, h1, l1;
            split4(x0, h0, l0);
            split4(x1, h1, l1);
            *reinterpret_cast<u16x8 *>(&sm.vd_hi[vr][8 * pc]) = cat(h0, h1);
            *reinterpret_cast<u16x8 *>(&sm.vd_lo[vr][8 * pc]) = cat(l0, l1);
        }
        __syncthreads();

        if (ci + 1 < nchunks) {
            const int64_t rem1 = rem - C;
            fetch(t + C, static_cast<int>(rem1 < C ? rem1 : C));
        }

        f32x4 part[4][2];
        chunk_compute<W, kF>(sm, mdec, qdec, full ? dc_full : dc_last, g, l16, S, part);

        // hand the partial O^T tiles of the other row blocks to their owners
#pragma unroll
        for (int it = 0; it < 4; ++it)
            if (it != W)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) sm.part[W][it][nt][lane] = part[it][nt];
        __syncthreads();

        // row block W: sum the four partials and store o.
        // O^T tile nt, element r: value column col0 + 16nt + 4g + r, token 16W + l16
        char *ob = reinterpret_cast<char *>(jb.out + t * jb.row + jb.hcol + col0);
        const bool store = full || (16 * W + l16) < c;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x4 o = part[W][nt];
#pragma unroll
            for (int src = 0; src < 4; ++src)
                if (src != W) o += sm.part[src][W][nt][lane];
            if (store) {
                o *= fin;
                const uint64_t packed = (uint64_t)cvt2(o[0], o[1]) | ((uint64_t)cvt2(o[2], o[3]) << 32);
                *reinterpret_cast<uint64_t *>(ob + offo + 32 * nt) = packed;
            }
        }
    }

    const float unscale = kF ? expf(32.f * lam) : 1.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                jb.state[(32 * W + 16 * mt + 4 * g + r) * D + col0 + 16 * nt + l16] = S[mt][nt][r] * unscale;
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
    // slopes in [0, 2] take the factored decay path (the largest ALiBi slope
    // is below 1); anything else the explicit one
    const bool factored = jb.lam >= 0.f && jb.lam <= 2.f;
    switch (__builtin_amdgcn_readfirstlane(tid >> 6) + (factored ? 0 : 4)) {
    case 0: run_wave<0, true>(sm, jb); break;
    case 1: run_wave<1, true>(sm, jb); break;
    case 2: run_wave<2, true>(sm, jb); break;
    case 3: run_wave<3, true>(sm, jb); break;
    case 4: run_wave<0, false>(sm, jb); break;
    case 5: run_wave<1, false>(sm, jb); break;
    case 6: run_wave<2, false>(sm, jb); break;
    default: run_wave<3, false>(sm, jb); break;
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
