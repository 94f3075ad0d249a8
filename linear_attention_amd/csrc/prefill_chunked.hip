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
//   inter    O^T += S_prev^T Q^T             S_prev split hi + lo, times e^{-l(i+1)}
//   update   S = e^{-l c} S + K^T Vd,  Vd = decayed V split hi + lo
// The hi + lo split (x = hi + lo, both bf16) keeps every operand that is not
// an exact bf16 input to ~2^-17 relative error; without it the bf16 rounding
// of P, S_prev and Vd each add output errors of order 1e-2 on small-slope heads.
//
// Work split.  One workgroup of 12 waves (three per SIMD) per (request, head,
// 32-column block of S); the block id is mapped so the column blocks of a
// head share an XCD (ids are dealt to the 8 XCDs round-robin) and its L2
// serves their repeated Q/K reads.  The waves take three roles, so that each
// fits in a third of a SIMD's registers and a SIMD can overlap one wave's
// MFMAs with the others' vector, LDS and memory work:
//   * state wave (rh, ch) keeps the fp32 state rows rh*D/2 .. rh*D/2 + D/2 - 1
//     of column tile ch (16 columns) in MFMA accumulators for the whole
//     request; per chunk it computes the inter term of all 64 tokens
//     restricted to its rows and tile (no state exchange) and the update of
//     its rows, and it sums and stores the output of the 16-token row blocks
//     2rh and 2rh + 1 of its tile, for which the wave with the other row half
//     hands it the missing half of the inter term;
//   * score wave w (4 of them) computes a balanced share of the 10 causal
//     score tiles and their P V products;
//   * staging waves (4 of them, two groups of two) move the tiles from global
//     memory to LDS and decay the next chunk's V, so that neither compute role
//     waits on a load: in each chunk one group stages and the other decays.
// The partial O^T tiles meet in LDS.  Each chunk takes one barrier: the
// partials of chunk i are summed and stored while chunk i + 1 is computed, so
// they, the decayed V and the Q/K tiles are double-buffered by chunk parity,
// and V, which is decayed one chunk before it is used, has a 3-slot ring.
//
// Data movement.  Global loads take about two microseconds under this load,
// so the tiles of two chunks are kept in flight.  The staging waves work in
// two groups of two: unit n (Q and K of chunk n, V of chunk n + 1) is staged
// by group n % 2.  While chunk i is computed, the group that holds unit i + 1
// in registers writes it to LDS, where the next barrier publishes it, and then
// loads unit i + 3 into the same registers, two chunk times before they are
// written.  Each wave has at most one unit of loads in flight, so vmcnt(0)
// before the write waits for exactly that unit; the first chunk's V and unit 0
// are loaded together behind one wait.  (Copying global memory straight into
// LDS was slower once made safe: those copies do not complete in issue order,
// and copies left in flight across a barrier gave stale tiles under load.)
// Operands that
// the MFMA needs with tokens along the contraction (K^T, V^T, Vd) are read
// from the token-major tiles with ds_read_b64_tr_b16, whose 16-lane groups
// return the columns of a 4-row block.  Tile rows are XOR-swizzled in
// 16-byte units so that every read pattern here is free of bank conflicts.
// Rows past the end of a short last chunk are loaded from the chunk's last
// row (always in bounds) and given zero weight.
//
// Launches with fewer (request, head, column block) units than CUs split
// their requests into sequence segments that run side by side (see "Sequence
// segments" below): a full-width state-only pass and a combine step give each
// segment its initial state first.
//
// State tracking ([LA-page] §额外覆盖): a request that snapshots its state
// after tl tokens runs as two consecutive passes, over [0, tl) and [tl, len);
// the first pass stores its final state to the track slot and the second
// starts from it.  Grouped heads read k and v at the query head's group
// (head h / (H / Hkv)) with their own token stride.
#include <cstdlib>

#include "common.h"
#include "host_logic.h"
#include "launch.h"

namespace la {
namespace {

constexpr int C = kChunk;      // chunk length
constexpr int VB = kColBlock;  // state columns per workgroup

// Geometry for head dimension D (128 or 64).  State wave (rh, ch) keeps the
// state rows rh*HR .. rh*HR + HR - 1 of column tile ch (16 columns) of the
// block and stores the 16-token row blocks 2rh and 2rh + 1 of that tile; four
// score waves share the score tiles.
template <int D> struct Geo {
    static constexpr int NVB = D / VB;       // column blocks per head
    static constexpr int KS = D / 32;        // 32-wide contraction steps of a score tile
    static constexpr int HR = D / 2;         // state rows per state wave
    static constexpr int HKS = HR / 32;      // 32-row contraction steps over them
    static constexpr int HMT = HR / 16;      // 16-row tiles of them
    static constexpr int UPR = D / 8;        // 16-byte units per Q/K row
    static constexpr int RPB = 512 / D;      // Q/K rows per 1 KB block
    static constexpr int QBLK = C * D / 512; // 1 KB blocks per Q/K tile
};
constexpr int NT = 768;  // threads per workgroup: 4 state, 4 score and 4 staging waves
// D^-1/2
template <int D> constexpr float kScale = D == 128 ? 0.08838834764831845f : 0.125f;

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Q and K tiles: 64 rows of D elements; the 16-byte units of row r are
// permuted by u -> u ^ m(r), with a mask per tile chosen for the reads that
// tile serves.  For D = 128 (a row is one 256-byte pass over the 64 LDS banks)
// each mask was measured free of bank conflicts on gfx950 (LDS conflict
// counters on a microbenchmark of every access pattern):
//   Q: 16-byte score-fragment reads and 8-byte inter-term reads -> m(r) = r
//   K: 16-byte score-fragment reads and 4x16 transposed reads
//      -> m(r) = ((r & 7) << 1) | (r & 1)
// (No single mask serves both tiles: the 16-byte reads want rows r and r + 8
// to share a mask, the 8-byte reads want them apart, and the transposed reads
// want bits 1..3 of the mask to differ within every 8 rows.)
// For D = 64 two rows share a pass, so a row pair p = r >> 1 plays the part
// of a row: Q takes m(r) = p & 7, K m(r) = ((p & 3) << 1) | ((p >> 2) & 1),
// which keeps the eight row pairs of 16 rows apart and, for the transposed
// reads, bits 1..2 apart within every 4 pairs.
template <int D> __device__ __forceinline__ int swz_q(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D> __device__ __forceinline__ int swz_k(int r) {
    return D == 128 ? (((r & 7) << 1) | (r & 1)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
}
template <int D> __device__ __forceinline__ int q_off(int r, int col) {
    return r * D + ((((col >> 3) ^ swz_q<D>(r)) << 3) | (col & 7));
}
template <int D> __device__ __forceinline__ int k_off(int r, int col) {
    return r * D + ((((col >> 3) ^ swz_k<D>(r)) << 3) | (col & 7));
}
// V tiles: 64 rows of 32 elements (64 B); units permuted by u -> u ^ swv(r),
// which moves rows 4..7 of every 8 to the other half of the banks.
__device__ __forceinline__ int swv(int r) { return ((r >> 2) & 1) << 1; }
__device__ __forceinline__ int v_off(int r, int col) {
    return r * VB + ((((col >> 3) ^ swv(r)) << 3) | (col & 7));
}

template <int D> struct Smem {
    uint16_t q[2][C * D];        // Q/K ring: the chunk being computed and the next
    uint16_t k[2][C * D];
    uint16_t v[3][C * VB];       // V ring, one chunk further ahead
    uint16_t vd_hi[2][C * VB];   // decayed V of the chunk being computed and the next
    uint16_t vd_lo[2][C * VB];
    f32x4 inter[2][4][2][64];    // [chunk parity][state wave][partner's row block][lane]
    f32x4 intra[2][4][2][2][64]; // [chunk parity][score wave][tile group][column tile][lane]
};

__device__ __forceinline__ f32x4 mma(u16x8 a, u16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ u16x8 lds8(const uint16_t *p) { return *reinterpret_cast<const u16x8 *>(p); }
// An 8-byte read that the compiler may not pair with another into a
// ds_read2_b64: the two halves of such a pair go to the same 8-byte half of a
// 16-byte unit in every lane, which is a 2-way bank conflict under any row
// swizzle (measured: all of the kernel's conflict cycles came from the paired
// Q^T reads of the inter term).
typedef __attribute__((address_space(3))) const volatile u16x4 lds_u16x4_cv;
__device__ __forceinline__ u16x4 lds4_single(const uint16_t *p) {
    return *reinterpret_cast<lds_u16x4_cv *>((const lds_void *)p);
}

// Transposed 4x16 read: the 16-lane group g addresses rows row0 + 4g .. +3 and
// columns col0 .. col0+15 (col0 a multiple of 16); lane (g, i) receives
// column col0 + i of those four rows.
//
// The read is issued as inline assembly, so the compiler does not track when
// its result arrives.  The caller waits with lds_wait() (a wait on the LDS
// counter) and then pin()s each value, an empty asm that orders every
// consumer after the wait.  (LDS operations complete in order, so the extra
// outstanding reads only make the compiler's own LDS waits more conservative.)
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_void *)p));
}
__device__ __forceinline__ u16x4 tr_at(const uint16_t *p) {
    uint64_t r;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
    return __builtin_bit_cast(u16x4, r);
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void pin(u16x8 &x) { asm volatile("" : "+v"(x)); }
template <int D>
__device__ __forceinline__ u16x4 ldtr_k(const uint16_t *tile, int row0, int col0, int g, int l16) {
    return tr_at(tile + k_off<D>(row0 + 4 * g + (l16 >> 2), col0 + 4 * (l16 & 3)));
}
__device__ __forceinline__ u16x4 ldtr_v(const uint16_t *tile, int row0, int col0, int g, int l16) {
    return tr_at(tile + v_off(row0 + 4 * g + (l16 >> 2), col0 + 4 * (l16 & 3)));
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

// Workgroup id -> (pair = request*H + head, column block; "request" is the
// request's rank in length order for batches that are sorted, see
// request_of_rank).  Ids are dealt to XCDs round-robin (id % 8), so groups of
// 8 pairs are laid out with the pair in the low 3 bits: the NVB blocks of one
// pair share id % 8.
template <int NVB> __device__ __forceinline__ void map_block(int id, int pairs, int &pair, int &vb) {
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

// Score tiles (j-tile, i-tile), j <= i, dealt to the waves 3/3/2/2: wave 0
// takes the causal block of i-tiles 0-1, wave 1 that of i-tiles 2-3, and
// waves 2 and 3 the full rows j-tiles 0-1 of i-tiles 2 and 3.  Each wave loads
// the K fragments of its distinct j-tiles (jl) and the Q fragments of its
// distinct i-tiles (il) once; tile t uses jl[tj[t]] and il[ti[t]].  The P V
// products group a wave's tiles by i-tile (at most two j-tiles, which together
// fill one 32-token contraction): group q covers i-tile git[q] with tiles
// ga[q] and gb[q] (-1: none).  So an output row block gets at most two intra
// partials (row blocks 2 and 3: one from wave 1, one from wave 2 or 3).
template <int W> struct Tiles;
template <> struct Tiles<0> {
    static constexpr int n = 3, tj[3] = {0, 0, 1}, ti[3] = {0, 1, 1};
    static constexpr int nj = 2, jl[2] = {0, 1}, ni = 2, il[2] = {0, 1};
    static constexpr int ng = 2, git[2] = {0, 1}, ga[2] = {0, 1}, gb[2] = {-1, 2};
};
template <> struct Tiles<1> {
    static constexpr int n = 3, tj[3] = {0, 0, 1}, ti[3] = {0, 1, 1};
    static constexpr int nj = 2, jl[2] = {2, 3}, ni = 2, il[2] = {2, 3};
    static constexpr int ng = 2, git[2] = {2, 3}, ga[2] = {0, 1}, gb[2] = {-1, 2};
};
template <> struct Tiles<2> {
    static constexpr int n = 2, tj[3] = {0, 1, 0}, ti[3] = {0, 0, 0};
    static constexpr int nj = 2, jl[2] = {0, 1}, ni = 1, il[2] = {2, 2};
    static constexpr int ng = 1, git[2] = {2, -1}, ga[2] = {0, -1}, gb[2] = {1, -1};
};
template <> struct Tiles<3> {
    static constexpr int n = 2, tj[3] = {0, 1, 0}, ti[3] = {0, 0, 0};
    static constexpr int nj = 2, jl[2] = {0, 1}, ni = 1, il[2] = {3, 3};
    static constexpr int ng = 1, git[2] = {3, -1}, ga[2] = {0, -1}, gb[2] = {1, -1};
};

// Decay handling.  With kF ("factored", used for 0 <= l <= 2) the state is
// kept in the scaled frame S_m = e^{-32 l} S, the score tiles are weighted by
// e^{l (j - 31)} and the sum of all partials is multiplied once by
// e^{-l (i - 31)}: that is the same o_i, because
//   e^{-l(i-j)} = e^{-l(i-31)} e^{l(j-31)}  and  e^{-l(i+1)} S = e^{-l(i-31)} S_m,
// and every factor stays inside the fp32/bf16 exponent range for l <= 2.
// Without kF the weights e^{-l(i-j)} and e^{-l(i+1)} are applied directly.

// One chunk for state wave (RH, CH): the inter term of all 64 tokens
// restricted to its state rows R0..R0+HR-1 (R0 = RH HR) and column tile CH,
// part[it], and the update of those rows, S[k][v] = e^{-l c} S + sum_j K[j][k]
// Vd[j][v].  qdec[it]: weight of the inter term for token i = 16 it + l16
// (only without kF); dcm1: e^{-l c} - 1 (the decay is applied as S + dcm1 S, which
// keeps the decay rate exact to float rounding of dcm1 even for tiny l).
template <int D, int RH, int CH, bool kF>
__device__ __forceinline__ void state_chunk(const uint16_t *sq, const uint16_t *sk, const uint16_t *svh,
                                            const uint16_t *svl, const float (&qdec)[4], float dcm1, int g,
                                            int l16, f32x4 (&S)[Geo<D>::HMT], f32x4 (&part)[4]) {
    using G = Geo<D>;
    constexpr int R0 = RH * G::HR;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};

    // Q^T restricted to the wave's rows (B operand of contraction step ks:
    // lane (g, l16) holds token 16 it + l16 and features R0 + 32ks + 4g + r,
    // R0 + 32ks + 16 + 4g + r, the order in which the state rows sit in the A
    // operand below)
    u16x8 qb[4][G::HKS];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int ks = 0; ks < G::HKS; ++ks) {
            const int qr = 16 * it + l16;
            qb[it][ks] = cat(lds4_single(&sq[q_off<D>(qr, R0 + 32 * ks + 4 * g)]),
                             lds4_single(&sq[q_off<D>(qr, R0 + 32 * ks + 16 + 4 * g)]));
        }
    // the state as bf16 hi/lo A operand (v x k): for step ks lane (g, l16) holds
    // rows R0 + 32ks + 4g + r (tile 2ks) and R0 + 32ks + 16 + 4g + r (tile
    // 2ks + 1) of column v = 16 CH + l16
    u16x8 sa_hi[G::HKS], sa_lo[G::HKS];
#pragma unroll
    for (int ks = 0; ks < G::HKS; ++ks) {
        u16x4 h0, l0, h1, l1;
        split4(S[2 * ks], h0, l0);
        split4(S[2 * ks + 1], h1, l1);
        sa_hi[ks] = cat(h0, h1);
        sa_lo[ks] = cat(l0, l1);
    }
    __builtin_amdgcn_sched_barrier(0);

    // inter term O^T[v][i] = sum_k S^T[v][k] Q^T[k][i] over the wave's rows
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        f32x4 acc = z;
#pragma unroll
        for (int ks = 0; ks < G::HKS; ++ks) {
            acc = mma(sa_hi[ks], qb[it][ks], acc);
            acc = mma(sa_lo[ks], qb[it][ks], acc);
        }
        part[it] = kF ? acc : acc * qdec[it];
    }
    // fragments of the update: K^T rows of the wave and its column tile of the
    // decayed V, with tokens along the contraction
    u16x8 ka[2][G::HMT], vh[2], vl[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int mt = 0; mt < G::HMT; ++mt)
            ka[s2][mt] = cat(ldtr_k<D>(sk, 32 * s2, R0 + 16 * mt, g, l16),
                             ldtr_k<D>(sk, 32 * s2 + 16, R0 + 16 * mt, g, l16));
        vh[s2] = cat(ldtr_v(svh, 32 * s2, 16 * CH, g, l16), ldtr_v(svh, 32 * s2 + 16, 16 * CH, g, l16));
        vl[s2] = cat(ldtr_v(svl, 32 * s2, 16 * CH, g, l16), ldtr_v(svl, 32 * s2 + 16, 16 * CH, g, l16));
    }
#pragma unroll
    for (int mt = 0; mt < G::HMT; ++mt) S[mt] += dcm1 * S[mt];
    __builtin_amdgcn_sched_barrier(0);
    lds_wait();
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int mt = 0; mt < G::HMT; ++mt) pin(ka[s2][mt]);
        pin(vh[s2]);
        pin(vl[s2]);
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int mt = 0; mt < G::HMT; ++mt) {
            S[mt] = mma(ka[s2][mt], vh[s2], S[mt]);
            S[mt] = mma(ka[s2][mt], vl[s2], S[mt]);
        }
}

// One chunk for score wave W: its score tiles (A^T[j][i] = k_j . q_i), weighted
// and masked by mdec and split hi + lo, times V^T: ipart[q][nt] is the intra
// term of i-tile Tiles<W>::git[q], column tile nt.  B operand slots 0..3 hold
// j-tile ga's rows 4g..4g+3, slots 4..7 j-tile gb's (or zero).
template <int D, int W, bool kF>
__device__ __forceinline__ void score_chunk(const uint16_t *sq, const uint16_t *sk, const uint16_t *sv,
                                            const float (&mdec)[12], int g, int l16, f32x4 (&ipart)[2][2]) {
    using T = Tiles<W>;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const u16x4 z4 = {0, 0, 0, 0};

    constexpr int KS = Geo<D>::KS;
    u16x8 kf[2][KS], qf[2][KS];
#pragma unroll
    for (int a = 0; a < T::nj; ++a)
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[a][s] = lds8(&sk[k_off<D>(16 * T::jl[a] + l16, 32 * s + 8 * g)]);
#pragma unroll
    for (int b = 0; b < T::ni; ++b)
#pragma unroll
        for (int s = 0; s < KS; ++s) qf[b][s] = lds8(&sq[q_off<D>(16 * T::il[b] + l16, 32 * s + 8 * g)]);
    u16x8 av[2][2];
#pragma unroll
    for (int q = 0; q < T::ng; ++q) {
        const int ta = T::ga[q], tb = T::gb[q];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            av[q][nt] = cat(ldtr_v(sv, 16 * T::jl[T::tj[ta]], 16 * nt, g, l16),
                            tb >= 0 ? ldtr_v(sv, 16 * T::jl[T::tj[tb]], 16 * nt, g, l16) : z4);
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sc[3];
#pragma unroll
    for (int t = 0; t < T::n; ++t) sc[t] = z;
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
        for (int t = 0; t < T::n; ++t) sc[t] = mma(kf[T::tj[t]][s], qf[T::ti[t]][s], sc[t]);
    u16x4 p_hi[3], p_lo[3];
#pragma unroll
    for (int t = 0; t < T::n; ++t) {
        f32x4 p;
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = sc[t][r] * mdec[4 * t + r];
        split4(p, p_hi[t], p_lo[t]);
    }
    __builtin_amdgcn_sched_barrier(0);
    lds_wait();
#pragma unroll
    for (int q = 0; q < T::ng; ++q)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) pin(av[q][nt]);
#pragma unroll
    for (int q = 0; q < T::ng; ++q) {
        const int ta = T::ga[q], tb = T::gb[q];
        const u16x8 bh = cat(p_hi[ta], tb >= 0 ? p_hi[tb] : z4);
        const u16x8 bl = cat(p_lo[ta], tb >= 0 ? p_lo[tb] : z4);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            ipart[q][nt] = mma(av[q][nt], bh, z);
            ipart[q][nt] = mma(av[q][nt], bl, ipart[q][nt]);
        }
    }
}

// Score-wave partials of row block B and column tile nt in the partial
// buffer par, added to o (B is a constant once the caller's loops are unrolled).
template <int W, int D>
__device__ __forceinline__ void add_intra(const Smem<D> &sm, int par, int B, int nt, int lane, f32x4 &o) {
    using T = Tiles<W>;
#pragma unroll
    for (int q = 0; q < T::ng; ++q)
        if (T::git[q] == B) o += sm.intra[par][W][q][nt][lane];
}

// per-lane weights of wave W's score tiles: element (t, r) is
// (j, i) = (16 jt + 4g + r, 16 it + l16), zero above the diagonal and for
// key rows j >= c (past the end of a short chunk)
template <int W, bool kF>
__device__ __forceinline__ void score_weights(float lam, int g, int l16, int c, float (&mdec)[12]) {
    using T = Tiles<W>;
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = 16 * T::jl[T::tj[t]] + 4 * g + r, i = 16 * T::il[T::ti[t]] + l16;
            const float e = kF ? static_cast<float>(j - 31) : -static_cast<float>(i - j);
            mdec[4 * t + r] = (t < T::n && j <= i && j < c) ? expf(lam * e) : 0.f;
        }
}

// Workgroup barrier for LDS data only.  __syncthreads() would also make every
// wave wait for its outstanding global loads (it is a release fence), which
// would drain the staging waves' loads of the chunk after next.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

struct Job {
    const uint16_t *q, *k, *v;
    uint16_t *out;
    const float *state_in;  // state before the pass (not read by a state-only pass: zero)
    float *state_out;       // state after the pass
    int64_t t0, len;        // tokens [t0, t0 + len), len >= 1
    size_t row, hcol;       // q/out token stride and head column
    size_t kvrow, kvcol;    // k/v token stride and head column
    int col0;
    float lam;
};

// One pass over a request for wave W of the workgroup (0..3 state waves, 4..7
// score waves, 8..11 staging waves).  Chunk ci is computed between barrier ci
// and barrier ci + 1, one barrier per chunk:
//   * state waves first finish chunk ci - 1 (sum its partials, store o), then
//     compute chunk ci and hand the partner its inter partials;
//   * score waves compute the intra partials of chunk ci;
//   * the staging group of unit ci + 1 (Q and K of chunk ci + 1, V of chunk
//     ci + 2) writes it to LDS and loads unit ci + 3, and the other group
//     decays the V of chunk ci + 1.
// Partials, decayed V and the Q/K tiles are double-buffered by chunk parity,
// V is a 3-slot ring, so nothing written in one interval is read in it.
template <int D, int W, bool kF>
__device__ __forceinline__ void run_wave(Smem<D> &sm, const Job &jb) {
    using G = Geo<D>;
    constexpr bool kState = W < 4;
    constexpr bool kScore = W >= 4 && W < 8;
    constexpr bool kHelper = W >= 8;        // staging and V decay
    constexpr int R = W & 3;                // index within the role
    constexpr int HG = R >> 1, HI = R & 1;  // staging wave: group (unit parity), index in the group
    constexpr int RH = R >> 1, CH = R & 1;  // state wave: row half, column tile
    constexpr int PARTNER = (1 - RH) * 2 + CH;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int l16 = lane & 15, g = lane >> 4;
    const float lam = jb.lam;
    const float scale = kScale<D>;
    const uint32_t row = static_cast<uint32_t>(jb.row);
    const int col0 = jb.col0;

    const int64_t len = jb.len;
    const int nchunks = static_cast<int>((len + C - 1) / C);
    const int c_last = static_cast<int>(len - static_cast<int64_t>(nchunks - 1) * C);
    // state frame: S_m = sigma * S
    const float sigma = kF ? expf(-32.f * lam) : 1.f;
    const float vshift = kF ? 32.f : 0.f;

    // ---- state role: tile mt element r is S[RH HR + 16mt + 4g + r][col0 + 16CH + l16];
    // the wave stores row blocks 2RH and 2RH + 1 of column tile CH
    f32x4 S[G::HMT];
    float qdec[4];
    float fin[2];
    f32x4 keep[2];  // the wave's own inter partials of those row blocks, until stored
    const float dc_full = expm1f(-lam * static_cast<float>(C));  // e^{-l c} - 1
    const float dc_last = expm1f(-lam * static_cast<float>(c_last));
    if constexpr (kState) {
#pragma unroll
        for (int mt = 0; mt < G::HMT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[mt][r] = sigma * jb.state_in[(RH * G::HR + 16 * mt + 4 * g + r) * D + col0 + 16 * CH + l16];
#pragma unroll
        for (int it = 0; it < 4; ++it) qdec[it] = expf(-lam * static_cast<float>(16 * it + l16 + 1));
        // output factor of the stored row blocks (token i = 16B + l16)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int B = 2 * RH + m;
            fin[m] = kF ? scale * expf(-lam * static_cast<float>(16 * B + l16 - 31)) : scale;
        }
    }

    // ---- score role
    float mdec[12];
    if constexpr (kScore) score_weights<R, kF>(lam, g, l16, nchunks == 1 ? c_last : C, mdec);

    // Staging.  Unit n is Q and K of chunk n and V of chunk n + 1.  Wave HI of
    // a staging group moves Q/K blocks HI*QPW..+QPW-1 (1 KB each: rows RPB b ..
    // RPB b + RPB - 1) and V rows 32HI..32HI+31: lane L holds unit L of each 1
    // KB block, so it loads the logical unit that the swizzle places there.
    // Rows past the end of a short chunk repeat its last row.
    constexpr int QPW = G::QBLK / 2;
    int qk_row[QPW], q_unit[QPW], k_unit[QPW];
#pragma unroll
    for (int u = 0; u < QPW; ++u) {
        qk_row[u] = G::RPB * (HI * QPW + u) + lane / G::UPR;
        q_unit[u] = (lane % G::UPR) ^ swz_q<D>(qk_row[u]);
        k_unit[u] = (lane % G::UPR) ^ swz_k<D>(qk_row[u]);
    }
    int v_row[2], v_unit[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        v_row[u] = 16 * (2 * HI + u) + (lane >> 2);
        v_unit[u] = (lane & 3) ^ swv(v_row[u]);
    }
    const uint32_t kvrow = static_cast<uint32_t>(jb.kvrow);
    auto chunk_t = [&](int n) { return jb.t0 + static_cast<int64_t>(n) * C; };
    auto chunk_c = [&](int n) { return n + 1 == nchunks ? c_last : C; };
    u16x8 rq[QPW], rk[QPW], rv[2];  // the unit in flight
    auto load_v = [&](int n) {
        const int c = chunk_c(n);
        const uint16_t *vb = jb.v + chunk_t(n) * jb.kvrow + jb.kvcol + col0;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t r = static_cast<uint32_t>(v_row[u] < c ? v_row[u] : c - 1);
            rv[u] = *reinterpret_cast<const u16x8 *>(vb + (r * kvrow + 8 * v_unit[u]));
        }
    };
    auto store_v = [&](int n) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
            *reinterpret_cast<u16x8 *>(&sm.v[n % 3][512 * (2 * HI + u) + 8 * lane]) = rv[u];
    };
    auto load_unit = [&](int n) {
        const int c = chunk_c(n);
        const uint16_t *qb = jb.q + chunk_t(n) * jb.row + jb.hcol;
        const uint16_t *kb = jb.k + chunk_t(n) * jb.kvrow + jb.kvcol;
#pragma unroll
        for (int u = 0; u < QPW; ++u) {
            const uint32_t r = static_cast<uint32_t>(qk_row[u] < c ? qk_row[u] : c - 1);
            rq[u] = *reinterpret_cast<const u16x8 *>(qb + (r * row + 8 * q_unit[u]));
            rk[u] = *reinterpret_cast<const u16x8 *>(kb + (r * kvrow + 8 * k_unit[u]));
        }
        if (n + 1 < nchunks) load_v(n + 1);
    };
    auto store_unit = [&](int n) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the loads of the unit landed
        const int buf = n & 1;
#pragma unroll
        for (int u = 0; u < QPW; ++u) {
            const int dst = 512 * (HI * QPW + u) + 8 * lane;
            *reinterpret_cast<u16x8 *>(&sm.q[buf][dst]) = rq[u];
            *reinterpret_cast<u16x8 *>(&sm.k[buf][dst]) = rk[u];
        }
        if (n + 1 < nchunks) store_v(n + 1);
    };

    // Decayed V: thread u (0..127) of the decaying staging group converts V
    // rows u/4 and u/4 + 32, logical unit u%4 (8 values each), into hi/lo at
    // the same (swizzled) position.
    const int du = ((W - 8) & 1) * 64 + lane;
    float vdec_full[2], vdec_last[2];
    int dv_pos[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int dv_row = (du >> 2) + 32 * e;
        dv_pos[e] = v_off(dv_row, 8 * (du & 3));
        vdec_full[e] = expf(-lam * (static_cast<float>(C - 1 - dv_row) + vshift));
        vdec_last[e] = dv_row < c_last ? expf(-lam * (static_cast<float>(c_last - 1 - dv_row) + vshift)) : 0.f;
    }
    auto decay_v = [&](int n) {  // V of chunk n, into slot n & 1
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float vdec = n + 1 == nchunks ? vdec_last[e] : vdec_full[e];
            const u16x8 pv = lds8(&sm.v[n % 3][dv_pos[e]]);
            f32x4 x0, x1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x0[k] = bf16_to_f32(pv[k]) * vdec;
                x1[k] = bf16_to_f32(pv[4 + k]) * vdec;
            }
            u16x4 h0, l0, h1, l1;
            split4(x0, h0, l0);
            split4(x1, h1, l1);
            *reinterpret_cast<u16x8 *>(&sm.vd_hi[n & 1][dv_pos[e]]) = cat(h0, h1);
            *reinterpret_cast<u16x8 *>(&sm.vd_lo[n & 1][dv_pos[e]]) = cat(l0, l1);
        }
    };

    // Sum the partials of chunk p for the wave's row blocks and store o.
    // O^T tile CH, element r: value column col0 + 16CH + 4g + r, token 16B + l16
    auto finalize = [&](int p) {
        const int par = p & 1;
        const bool last = p + 1 == nchunks;
        const int c = last ? c_last : C;
        char *ob = reinterpret_cast<char *>(jb.out + chunk_t(p) * jb.row + jb.hcol + col0);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int B = 2 * RH + m;
            f32x4 o = keep[m] + sm.inter[par][PARTNER][m][lane];
            add_intra<0>(sm, par, B, CH, lane, o);
            add_intra<1>(sm, par, B, CH, lane, o);
            add_intra<2>(sm, par, B, CH, lane, o);
            add_intra<3>(sm, par, B, CH, lane, o);
            if (!last || 16 * B + l16 < c) {
                o *= fin[m];
                const uint32_t offo = 2u * (static_cast<uint32_t>(16 * B + l16) * row + 4 * g);
                const uint64_t packed = (uint64_t)cvt2(o[0], o[1]) | ((uint64_t)cvt2(o[2], o[3]) << 32);
                *reinterpret_cast<uint64_t *>(ob + offo + 32 * CH) = packed;
            }
        }
    };

    // unit n is staged by staging group n % 2
    auto stages = [](int n) { return kHelper && (n & 1) == HG; };

    // prologue: V of chunk 0 (also decayed) and unit 0 in LDS, units 1 and 2
    // in flight.  Group 0 loads V of chunk 0 and unit 0 together and decays
    // its own V rows in registers: the staging layout of a V tile is the
    // swizzled layout v_off that the decay writes, so each lane's decayed
    // unit lands where it holds the raw one.
    if (stages(0)) {
        u16x8 v0[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const uint32_t r = static_cast<uint32_t>(v_row[u] < chunk_c(0) ? v_row[u] : chunk_c(0) - 1);
            v0[u] = *reinterpret_cast<const u16x8 *>(jb.v + chunk_t(0) * jb.kvrow + jb.kvcol + col0 +
                                                     (r * kvrow + 8 * v_unit[u]));
        }
        load_unit(0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pos = 512 * (2 * HI + u) + 8 * lane;
            const float vdec =
                nchunks == 1
                    ? (v_row[u] < c_last ? expf(-lam * (static_cast<float>(c_last - 1 - v_row[u]) + vshift)) : 0.f)
                    : expf(-lam * (static_cast<float>(C - 1 - v_row[u]) + vshift));
            f32x4 x0, x1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x0[k] = bf16_to_f32(v0[u][k]) * vdec;
                x1[k] = bf16_to_f32(v0[u][4 + k]) * vdec;
            }
            u16x4 h0, l0, h1, l1;
            split4(x0, h0, l0);
            split4(x1, h1, l1);
            *reinterpret_cast<u16x8 *>(&sm.v[0][pos]) = v0[u];
            *reinterpret_cast<u16x8 *>(&sm.vd_hi[0][pos]) = cat(h0, h1);
            *reinterpret_cast<u16x8 *>(&sm.vd_lo[0][pos]) = cat(l0, l1);
        }
        store_unit(0);
    }
    for (int n = 1; n <= 2; ++n)
        if (n < nchunks && stages(n)) load_unit(n);
    __syncthreads();

    for (int ci = 0; ci < nchunks; ++ci) {
        const bool last = ci + 1 == nchunks;
        lds_barrier();  // unit ci, decayed V of chunk ci and the partials of chunk ci - 1 are in LDS
        // unit ci+1 from registers to LDS (published at the next barrier), then
        // unit ci+3 from global memory to the same registers
        if constexpr (kHelper) {
            if (ci + 1 < nchunks && stages(ci + 1)) {
                store_unit(ci + 1);
                if (ci + 3 < nchunks) load_unit(ci + 3);
            }
            // the group that does not stage this chunk decays the next V
            if (!last && HG == (ci & 1)) decay_v(ci + 1);
        }
        const int buf = ci & 1;
        if constexpr (kState) {
            if (ci > 0) finalize(ci - 1);
            f32x4 part[4];
            state_chunk<D, RH, CH, kF>(sm.q[buf], sm.k[buf], sm.vd_hi[buf], sm.vd_lo[buf], qdec,
                                       last ? dc_last : dc_full, g, l16, S, part);
            // row blocks of the partner to the partner, the own ones kept
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                sm.inter[buf][R][m][lane] = part[2 * (1 - RH) + m];
                keep[m] = part[2 * RH + m];
            }
        }
        if constexpr (kScore) {
            if (last && c_last != C && nchunks > 1) score_weights<R, kF>(lam, g, l16, c_last, mdec);
            f32x4 ipart[2][2];
            score_chunk<D, R, kF>(sm.q[buf], sm.k[buf], sm.v[ci % 3], mdec, g, l16, ipart);
#pragma unroll
            for (int q = 0; q < Tiles<R>::ng; ++q)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) sm.intra[buf][R][q][nt][lane] = ipart[q][nt];
        }
    }
    lds_barrier();  // the partials of the last chunk are in LDS
    if constexpr (kState) {
        finalize(nchunks - 1);
        const float unscale = kF ? expf(32.f * lam) : 1.f;
#pragma unroll
        for (int mt = 0; mt < G::HMT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                jb.state_out[(RH * G::HR + 16 * mt + 4 * g + r) * D + col0 + 16 * CH + l16] = S[mt][r] * unscale;
    }
}

// The passes of wave W over a request: one over [0, len), or with a snapshot
// inside the request [0, tl) into the track slot and then [tl, len) from it.
template <int D, int W, bool kF>
__device__ __forceinline__ void run_passes(Smem<D> &sm, const Job &base, float *track, int64_t tl) {
    if (!track) {
        run_wave<D, W, kF>(sm, base);
        return;
    }
    for (int i = 0; i < 2; ++i) {
        Job jb = base;
        jb.t0 = i == 0 ? base.t0 : base.t0 + tl;
        jb.len = i == 0 ? tl : base.len - tl;
        jb.state_in = i == 0 ? base.state_in : track;
        jb.state_out = i == 0 ? track : base.state_out;
        run_wave<D, W, kF>(sm, jb);
    }
}

// The wave's role and decay path for one pass: wave index and, for slopes
// outside [0, 2], the explicit (not factored) decay.  Slopes in [0, 2] take
// the factored path (the largest ALiBi slope is below 1).
template <int D>
__device__ __forceinline__ void dispatch(Smem<D> &sm, const Job &base, float *split, int64_t tl) {
    const bool factored = base.lam >= 0.f && base.lam <= 2.f;
    switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) + (factored ? 0 : 12)) {
    case 0: run_passes<D, 0, true>(sm, base, split, tl); break;
    case 1: run_passes<D, 1, true>(sm, base, split, tl); break;
    case 2: run_passes<D, 2, true>(sm, base, split, tl); break;
    case 3: run_passes<D, 3, true>(sm, base, split, tl); break;
    case 4: run_passes<D, 4, true>(sm, base, split, tl); break;
    case 5: run_passes<D, 5, true>(sm, base, split, tl); break;
    case 6: run_passes<D, 6, true>(sm, base, split, tl); break;
    case 7: run_passes<D, 7, true>(sm, base, split, tl); break;
    case 8: run_passes<D, 8, true>(sm, base, split, tl); break;
    case 9: run_passes<D, 9, true>(sm, base, split, tl); break;
    case 10: run_passes<D, 10, true>(sm, base, split, tl); break;
    case 11: run_passes<D, 11, true>(sm, base, split, tl); break;
    case 12: run_passes<D, 0, false>(sm, base, split, tl); break;
    case 13: run_passes<D, 1, false>(sm, base, split, tl); break;
    case 14: run_passes<D, 2, false>(sm, base, split, tl); break;
    case 15: run_passes<D, 3, false>(sm, base, split, tl); break;
    case 16: run_passes<D, 4, false>(sm, base, split, tl); break;
    case 17: run_passes<D, 5, false>(sm, base, split, tl); break;
    case 18: run_passes<D, 6, false>(sm, base, split, tl); break;
    case 19: run_passes<D, 7, false>(sm, base, split, tl); break;
    case 20: run_passes<D, 8, false>(sm, base, split, tl); break;
    case 21: run_passes<D, 9, false>(sm, base, split, tl); break;
    case 22: run_passes<D, 10, false>(sm, base, split, tl); break;
    default: run_passes<D, 11, false>(sm, base, split, tl); break;
    }
}

// Request b's token range [t0, t1): cu_seqlens clamped to [0, total_tokens]
// and made non-decreasing, so that a malformed entry gives an empty request.
__device__ __forceinline__ void request_range(const PrefillArgs &a, int b, int64_t &t0, int64_t &t1) {
    t0 = a.cu_seqlens[b];
    t1 = a.cu_seqlens[b + 1];
    t0 = t0 < 0 ? 0 : (t0 > a.total_tokens ? a.total_tokens : t0);
    t1 = t1 < t0 ? t0 : (t1 > a.total_tokens ? a.total_tokens : t1);
}

// Longest request first.  A batch of up to kSortMax requests is taken in
// order of decreasing length (ties by index): rank r of that order is the
// request that workgroups with pair index r*H .. r*H + H - 1 serve.  When the
// grid is larger than the GPU holds at once, the long requests then start in
// the first round of workgroups and the short ones fill in behind them, so
// the launch ends with the longest request instead of a long request that
// was dispatched late.  Every workgroup ranks the (at most kSortMax) lengths
// itself; the results do not depend on the order.
constexpr int kSortMax = 256;
struct Ranked {
    int64_t t0[kSortMax];   // each request's range and slot, kept from the ranking
    int64_t len[kSortMax];  // pass so that the picked one needs no second read
    int slot[kSortMax];
    int pick;
};
__device__ __forceinline__ int64_t uniform64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(x) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ int request_of_rank(const PrefillArgs &a, int batch, int r, Ranked &rk) {
    const int tid = threadIdx.x;
    for (int i = tid; i < batch; i += NT) {
        int64_t t0, t1;
        request_range(a, i, t0, t1);
        rk.t0[i] = t0;
        rk.len[i] = t1 - t0;
        rk.slot[i] = a.slot_idx[i];
    }
    __syncthreads();
    if (tid < batch) {
        const int64_t li = rk.len[tid];
        int rank = 0;
        for (int j = 0; j < batch; ++j) {
            const int64_t lj = rk.len[j];
            rank += (lj > li || (lj == li && j < tid)) ? 1 : 0;
        }
        if (rank == r) rk.pick = tid;
    }
    __syncthreads();
    return rk.pick;
}

// Sequence segments.  A launch whose (request, head, column block) units
// fill only part of the GPU splits every request into up to a.segments
// segments of whole chunks, cps chunks each, and runs them side by side:
//   1. prefill_delta_full_kernel: the state contribution of every segment but
//      the last, in sub-segments of whole chunks: dS_{s,q} = sum over the
//      tokens t of sub-segment q of e^{-l(end_q - 1 - t)} k_t v_t^T (the
//      recurrence from a zero state, no outputs);
//   2. prefill_combine_kernel: the state before each segment, by the same
//      recurrence at sub-segment granularity from the pool state S_0;
//   3. prefill_chunked_kernel: every segment from its own initial state, as a
//      request of its own; the last segment stores the final state.
// All three use the caller's workspace a.seg_ws in stream order; the pool slot
// is read by step 2 only and written by step 3 only.
struct SegGeom {
    int nchunks;  // chunks of the request
    int cps;      // chunks per segment
    int ne;       // non-empty segments
};
__device__ __forceinline__ SegGeom seg_geom(int64_t len, int segments) {
    SegGeom g;
    g.nchunks = static_cast<int>((len + C - 1) / C);
    g.cps = (g.nchunks + segments - 1) / segments;
    g.ne = g.cps > 0 ? (g.nchunks + g.cps - 1) / g.cps : 0;
    return g;
}
// Workspace a.seg_ws: the contributions dS_{s,q} of sub-segment q of segment s,
// [pair][segments - 1][subsegs][D][D], then the initial states S_s,
// [pair][segments][D][D], fp32.
template <int D> __device__ __forceinline__ float *ds_slice(const PrefillArgs &a, int pair, int s, int q) {
    return a.seg_ws + ((static_cast<size_t>(pair) * (a.segments - 1) + s) * a.subsegs + q) * (D * D);
}
template <int D> __device__ __forceinline__ float *seg_slice(const PrefillArgs &a, int pair, int s) {
    return a.seg_ws + (static_cast<size_t>(a.pairs) * (a.segments - 1) * a.subsegs +
                       static_cast<size_t>(pair) * a.segments + s) * (D * D);
}
// Sub-segment q of a segment of cps chunks: chunks [c0, c0 + n) of it.
__device__ __forceinline__ void subseg_range(int cps, int subsegs, int q, int &c0, int &n) {
    const int spc = (cps + subsegs - 1) / subsegs;
    c0 = q * spc;
    n = c0 >= cps ? 0 : (cps - c0 < spc ? cps - c0 : spc);
}

template <int D> __global__ __launch_bounds__(NT) void prefill_chunked_kernel(PrefillArgs a) {
    using G = Geo<D>;
    __shared__ Smem<D> sm;
    __shared__ Ranked ranked;

    const int H = a.num_heads;
    const int units = a.pairs * G::NVB;
    const int seg = static_cast<int>(blockIdx.x) / units;  // 0 without segments
    int pair, vb;
    map_block<G::NVB>(static_cast<int>(blockIdx.x) - seg * units, a.pairs, pair, vb);
    const int batch = a.pairs / H;
    int b = pair / H;
    const int h = pair - b * H;
    const int tid = threadIdx.x;
    int64_t t0, len;
    int slot;
    if (batch > 1 && batch <= kSortMax) {
        // the picked request is the same for the whole workgroup: keep it scalar
        b = __builtin_amdgcn_readfirstlane(request_of_rank(a, batch, b, ranked));
        t0 = uniform64(ranked.t0[b]);
        len = uniform64(ranked.len[b]);
        slot = __builtin_amdgcn_readfirstlane(ranked.slot[b]);
    } else {
        int64_t t1;
        request_range(a, b, t0, t1);
        len = t1 - t0;
        slot = a.slot_idx[b];
    }
    const bool segmented = a.segments > 1;
    int nseg = 1;
    if (segmented) {
        const SegGeom sg = seg_geom(len, a.segments);
        if (seg >= sg.ne) return;  // past the end of the request (or an empty one)
        const int64_t s0 = static_cast<int64_t>(seg) * sg.cps * C;
        t0 += s0;
        len = len - s0 < static_cast<int64_t>(sg.cps) * C ? len - s0 : static_cast<int64_t>(sg.cps) * C;
        nseg = sg.ne;
    }

    const size_t row = static_cast<size_t>(H) * D;
    const size_t hcol = static_cast<size_t>(h) * D;
    const int col0 = vb * VB;
    if (slot < 0 || slot >= a.pool_slots) {
        // out-of-range slot: zero output for this column block, no state touched
        for (int64_t idx = tid; idx < len * (VB / 8); idx += NT) {
            const int64_t t = t0 + idx / (VB / 8);
            *reinterpret_cast<u16x8 *>(a.out + t * row + hcol + col0 + 8 * (idx % (VB / 8))) =
                u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        }
        return;
    }
    float *state = a.pool + (static_cast<size_t>(slot) * H + h) * (D * D);
    float *track = nullptr;
    int64_t tl = len;
    if (a.track_lens) {  // (never with segments)
        const int ts = a.track_slot_idx[b];
        const int64_t n = a.track_lens[b];
        if (ts >= 0 && ts < a.pool_slots && n >= 0 && n <= len) {
            track = a.pool + (static_cast<size_t>(ts) * H + h) * (D * D);
            tl = n;
        }
    }
    if (track && (tl == 0 || len == 0)) {
        // snapshot after 0 tokens: a copy of this block's prefix state
        for (int e = tid; e < D * VB; e += NT) {
            const int r = e / VB, c = col0 + e % VB;
            track[r * D + c] = state[r * D + c];
        }
    }
    if (len <= 0) return;  // empty request: no-op
    const int hk = h / (H / a.num_kv_heads);
    // with segments: initial state from the workspace; only the last segment
    // stores the final state in the pool, the others over their own (already
    // read) initial state
    float *s_in = segmented ? seg_slice<D>(a, b * H + h, seg) : state;
    float *s_out = !segmented || seg == nseg - 1 ? state : s_in;
    const Job base{a.q, a.k, a.v, a.out, s_in, s_out, t0, len, row, hcol,
                   static_cast<size_t>(a.num_kv_heads) * D, static_cast<size_t>(hk) * D, col0, a.slopes[h]};
    // a snapshot strictly inside the request splits it into two passes
    float *split = track && tl > 0 && tl < len ? track : nullptr;
    dispatch<D>(sm, base, split, tl);
    if (track && tl == len) {
        // snapshot after the whole request: the final state, as stored above
        __syncthreads();
        for (int e = tid; e < D * VB; e += NT) {
            const int r = e / VB, c = col0 + e % VB;
            track[r * D + c] = state[r * D + c];
        }
    }
}

// Step 1, full width: workgroup (pair, segment s, sub-segment q) keeps the
// whole D x D contribution of its sub-segment, so each chunk's K is loaded
// once and not once per column block.  All chunks of a non-final segment are
// full.  Eight waves: update wave W (0..3) holds value columns
// W*D/4 .. W*D/4 + D/4 - 1 of all D rows in MFMA accumulators; staging wave R
// (4..7) moves token rows 16(R-4) .. 16(R-4) + 15 of every chunk, two chunks
// ahead, and writes K and the decayed V (e^{-l(C - 1 - j)} v_j, split hi + lo)
// to LDS, double-buffered by chunk parity, one barrier per chunk.
constexpr int kDeltaWaves = 8;
template <int D> struct DeltaSmem {
    uint16_t k[2][C * D];   // K, token-major, K-tile swizzle
    uint16_t vh[2][C * D];  // decayed V, hi and lo, same layout
    uint16_t vl[2][C * D];
};

template <int D, int W>
__device__ __forceinline__ void delta_wave(DeltaSmem<D> &sm, const uint16_t *kb, const uint16_t *vb, size_t kvrow,
                                           int nchunks, float lam, float *out) {
    using G = Geo<D>;
    constexpr bool kStage = W >= 4;
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, g = lane >> 4;

    // ---- update waves
    constexpr int MT = D / 16;   // row tiles
    constexpr int NTW = D / 64;  // column tiles per wave
    f32x4 acc[MT][NTW];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int n = 0; n < NTW; ++n) acc[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float dcm1 = expm1f(-lam * static_cast<float>(C));  // e^{-l C} - 1
    auto update = [&](int buf) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int n = 0; n < NTW; ++n) acc[mt][n] += dcm1 * acc[mt][n];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            u16x8 ka[MT], bh[NTW], bl[NTW];
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                const int c0 = 16 * ((W & 3) * NTW + n);
                bh[n] = cat(ldtr_k<D>(sm.vh[buf], 32 * s2, c0, g, l16), ldtr_k<D>(sm.vh[buf], 32 * s2 + 16, c0, g, l16));
                bl[n] = cat(ldtr_k<D>(sm.vl[buf], 32 * s2, c0, g, l16), ldtr_k<D>(sm.vl[buf], 32 * s2 + 16, c0, g, l16));
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                ka[mt] = cat(ldtr_k<D>(sm.k[buf], 32 * s2, 16 * mt, g, l16),
                             ldtr_k<D>(sm.k[buf], 32 * s2 + 16, 16 * mt, g, l16));
            lds_wait();
#pragma unroll
            for (int n = 0; n < NTW; ++n) {
                pin(bh[n]);
                pin(bl[n]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) pin(ka[mt]);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int n = 0; n < NTW; ++n) {
                    acc[mt][n] = mma(ka[mt], bh[n], acc[mt][n]);
                    acc[mt][n] = mma(ka[mt], bl[n], acc[mt][n]);
                }
        }
    };

    // ---- staging waves: 16 token rows of K and of V per chunk, KB blocks of 1 KB each
    constexpr int KB = D / 32;
    const int R = (W & 3);
    int row[KB], unit[KB];
    float wv[KB];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
        row[b] = 16 * R + G::RPB * b + lane / G::UPR;
        unit[b] = (lane % G::UPR) ^ swz_k<D>(row[b]);
        wv[b] = expf(-lam * static_cast<float>(C - 1 - row[b]));
    }
    u16x8 rk[2][KB], rv[2][KB];
    auto load = [&](int n0, int set) {  // chunks past the end reload the last one
        const int n = n0 < nchunks ? n0 : nchunks - 1;
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const size_t off = (static_cast<size_t>(n) * C + row[b]) * kvrow + 8 * unit[b];
            rk[set][b] = *reinterpret_cast<const u16x8 *>(kb + off);
            rv[set][b] = *reinterpret_cast<const u16x8 *>(vb + off);
        }
    };
    auto store = [&](int n, int set) {
        const int buf = n & 1;
#pragma unroll
        for (int b = 0; b < KB; ++b) {
            const int dst = 512 * (R * KB + b) + 8 * lane;
            *reinterpret_cast<u16x8 *>(&sm.k[buf][dst]) = rk[set][b];
            f32x4 x0, x1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x0[e] = bf16_to_f32(rv[set][b][e]) * wv[b];
                x1[e] = bf16_to_f32(rv[set][b][4 + e]) * wv[b];
            }
            u16x4 h0, l0, h1, l1;
            split4(x0, h0, l0);
            split4(x1, h1, l1);
            *reinterpret_cast<u16x8 *>(&sm.vh[buf][dst]) = cat(h0, h1);
            *reinterpret_cast<u16x8 *>(&sm.vl[buf][dst]) = cat(l0, l1);
        }
    };

    if constexpr (kStage) {
        load(0, 0);
        store(0, 0);
        load(1, 1);
        load(2, 0);
    }
    __syncthreads();
    // chunk ci: the staging waves write chunk ci + 1 (register set (ci + 1) % 2)
    // and load chunk ci + 3 into the same set; the loop runs two chunks per
    // iteration so that the set is a constant and every path issues the same
    // loads (exact wait counts)
    auto step = [&](int ci, int set) {
        lds_barrier();
        if constexpr (kStage) {
            if (ci + 1 < nchunks) store(ci + 1, set);
            load(ci + 3, set);
        } else {
            update(ci & 1);
        }
    };
    int ci = 0;
    for (; ci + 1 < nchunks; ci += 2) {
        step(ci, 1);
        step(ci + 1, 0);
    }
    if (ci < nchunks) step(ci, 1);
    if constexpr (kStage) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the loads past the end
    } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    out[(16 * mt + 4 * g + r) * D + 16 * ((W & 3) * NTW + n) + l16] = acc[mt][n][r];
    }
}

template <int D> __global__ __launch_bounds__(64 * kDeltaWaves) void prefill_delta_full_kernel(PrefillArgs a) {
    __shared__ DeltaSmem<D> sm;
    const int H = a.num_heads;
    const int per_pair = (a.segments - 1) * a.subsegs;
    const int pair = static_cast<int>(blockIdx.x) / per_pair;
    const int rest = static_cast<int>(blockIdx.x) - pair * per_pair;
    const int seg = rest / a.subsegs, q = rest - seg * a.subsegs;
    const int b = pair / H;
    const int h = pair - b * H;
    int64_t t0, t1;
    request_range(a, b, t0, t1);
    const SegGeom sg = seg_geom(t1 - t0, a.segments);
    const int slot = a.slot_idx[b];
    if (slot < 0 || slot >= a.pool_slots || seg >= sg.ne - 1) return;
    int c0, nch;
    subseg_range(sg.cps, a.subsegs, q, c0, nch);
    if (nch == 0) return;
    const int hk = h / (H / a.num_kv_heads);
    const size_t kvrow = static_cast<size_t>(a.num_kv_heads) * D;
    const int64_t tstart = t0 + (static_cast<int64_t>(seg) * sg.cps + c0) * C;
    const size_t base = static_cast<size_t>(tstart) * kvrow + static_cast<size_t>(hk) * D;
    float *out = ds_slice<D>(a, pair, seg, q);
    const float lam = a.slopes[h];
    switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: delta_wave<D, 0>(sm, a.k + base, a.v + base, kvrow, nch, lam, out); break;
    case 1: delta_wave<D, 1>(sm, a.k + base, a.v + base, kvrow, nch, lam, out); break;
    case 2: delta_wave<D, 2>(sm, a.k + base, a.v + base, kvrow, nch, lam, out); break;
    case 3: delta_wave<D, 3>(sm, a.k + base, a.v + base, kvrow, nch, lam, out); break;
    case 4: delta_wave<D, 4>(sm, a.k + base, a.v + base, kvrow, nch, lam, out); break;
    case 5: delta_wave<D, 5>(sm, a.k + base, a.v + base, kvrow, nch, lam, out); break;
    case 6: delta_wave<D, 6>(sm, a.k + base, a.v + base, kvrow, nch, lam, out); break;
    default: delta_wave<D, 7>(sm, a.k + base, a.v + base, kvrow, nch, lam, out); break;
    }
}

// Step 2: the kCombineParts workgroups of a column block turn the pool state
// and the sub-segment contributions of a quarter of its rows each into the
// initial states S_0 .. S_{ne-1}: S_{s+1} is S_s carried through the
// sub-segments q of segment s, S <- e^{-l n_q C} S + dS_{s,q}.  Each thread
// owns 4 consecutive columns of some rows and loads every dS it needs before
// it runs the chain.  (Workgroup x = part * units + unit.)
constexpr int kCombineThreads = 256;
constexpr int kCombineParts = 4;
template <int D> __global__ __launch_bounds__(kCombineThreads) void prefill_combine_kernel(PrefillArgs a) {
    using G = Geo<D>;
    const int H = a.num_heads;
    const int units = a.pairs * G::NVB;
    const int part = static_cast<int>(blockIdx.x) / units;
    int pair, vb;
    map_block<G::NVB>(static_cast<int>(blockIdx.x) - part * units, a.pairs, pair, vb);
    const int b = pair / H;
    const int h = pair - b * H;
    int64_t t0, t1;
    request_range(a, b, t0, t1);
    const SegGeom sg = seg_geom(t1 - t0, a.segments);
    const int slot = a.slot_idx[b];
    if (slot < 0 || slot >= a.pool_slots || sg.ne == 0) return;
    const float *state = a.pool + (static_cast<size_t>(slot) * H + h) * (D * D);
    const float lam = a.slopes[h];
    float dq[kMaxSubsegs];  // decay over each sub-segment minus 1 (0: empty)
    int nq[kMaxSubsegs];
#pragma unroll
    for (int q = 0; q < kMaxSubsegs; ++q) {
        int c0 = 0, n = 0;
        if (q < a.subsegs) subseg_range(sg.cps, a.subsegs, q, c0, n);
        nq[q] = n;
        dq[q] = expm1f(-lam * static_cast<float>(n * C));
    }
    constexpr int kQuads = D * VB / 4;  // 4-column groups of the block
    static_assert(kQuads % kCombineParts == 0, "rows split evenly");
    constexpr int kPartQuads = kQuads / kCombineParts;
    for (int e = part * kPartQuads + threadIdx.x; e < (part + 1) * kPartQuads; e += kCombineThreads) {
        const int idx = (e / (VB / 4)) * D + vb * VB + 4 * (e % (VB / 4));
        f32x4 ds[kMaxSegments - 1][kMaxSubsegs];
#pragma unroll
        for (int s = 0; s < kMaxSegments - 1; ++s)
#pragma unroll
            for (int q = 0; q < kMaxSubsegs; ++q)
                if (s + 1 < sg.ne && nq[q] > 0)
                    ds[s][q] = *reinterpret_cast<const f32x4 *>(ds_slice<D>(a, pair, s, q) + idx);
        f32x4 cur = *reinterpret_cast<const f32x4 *>(state + idx);
#pragma unroll
        for (int s = 0; s < kMaxSegments; ++s) {
            if (s < sg.ne) {
                *reinterpret_cast<f32x4 *>(seg_slice<D>(a, pair, s) + idx) = cur;
                if (s + 1 < sg.ne) {
#pragma unroll
                    for (int q = 0; q < kMaxSubsegs; ++q)
                        if (nq[q] > 0) cur += dq[q] * cur + ds[s][q];
                }
            }
        }
    }
}

// Launches on `stream`: the chunked kernel alone, or (a.segments > 1, with the
// caller's workspace in a.seg_ws) the state-only pass, the combine step and
// the chunked kernel over every segment.
template <int D> hipError_t launch(const PrefillArgs &a, int batch, hipStream_t stream) {
    PrefillArgs copy = a;
    copy.pairs = batch * a.num_heads;
    const unsigned units = static_cast<unsigned>(copy.pairs) * Geo<D>::NVB;
    void *args[] = {&copy};
    if (copy.segments <= 1) {
        copy.segments = 1;
        return hipLaunchKernel(reinterpret_cast<const void *>(&prefill_chunked_kernel<D>), dim3(units), dim3(NT),
                               args, 0, stream);
    }
    const int per = copy.pairs * (copy.segments - 1);
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&prefill_delta_full_kernel<D>),
                                   dim3(static_cast<unsigned>(per * copy.subsegs)), dim3(64 * kDeltaWaves), args,
                                   0, stream);
    if (e == hipSuccess)
        e = hipLaunchKernel(reinterpret_cast<const void *>(&prefill_combine_kernel<D>),
                            dim3(units * kCombineParts), dim3(kCombineThreads), args, 0, stream);
    if (e == hipSuccess)
        e = hipLaunchKernel(reinterpret_cast<const void *>(&prefill_chunked_kernel<D>),
                            dim3(units * copy.segments), dim3(NT), args, 0, stream);
    return e;
}

}  // namespace

hipError_t launch_prefill_chunked(const PrefillArgs &a, int batch, int head_dim, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    if (head_dim == 128) return launch<128>(a, batch, stream);
    if (head_dim == 64) return launch<64>(a, batch, stream);
    return hipErrorInvalidValue;
}

}  // namespace la
