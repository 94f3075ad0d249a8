// Token-recurrent seg_la kernels: decode (one token), chain verify (k tokens),
// tree verify (each draft forks from its parent's state), and the prefill path
// for fp32 inputs and for head_dim 64.
//
// Citations name the web page "SGLang Lightning Attention 能力矩阵与 seg_la
// 线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page].
//
// Per (request, head) the recurrence of [LA-page] §独立参考实现 is advanced
// one token at a time with the d x d fp32 state held in registers:
//     S <- exp(-slope) * S + k v^T ;  o = (q @ S) / sqrt(d)
// This path is bound by HBM traffic: per (request, head) it streams the state
// in and out once, so each of the 256 threads owns RPT rows x 4 columns of S
// and moves it with coalesced 128-bit loads and stores (nontemporal: the state
// is touched once per call).  The q.S column sums are reduced across the row
// groups of a wave with cross-lane shuffles and across the 4 waves in LDS.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int kGroup = 8;  // tokens per decay group of the token-recurrent kernel

// Thread layout for head_dim D: column group cg = tid % CG owns value columns
// 4cg..4cg+3, row group rg = tid / CG owns key rows RPT*rg .. RPT*rg+RPT-1.
// A wave holds 64/CG row groups, so each 128-bit state load reads 64/CG full
// rows.
template <int D> struct Layout {
    static constexpr int CG = D / 4;
    static constexpr int RG = kThreads / CG;
    static constexpr int RPT = D / RG;
    static constexpr float kScale = D == 128 ? 0.08838834764831845f : 0.125f;  // D^-1/2
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
};

// N consecutive elements starting at p (8-byte aligned for bf16, 16 for fp32)
template <int N> __device__ __forceinline__ void load_n(const uint16_t *p, float (&x)[N]) {
    if constexpr (N % 8 == 0) {
#pragma unroll
        for (int i = 0; i < N / 8; ++i) {
            const u16x8 a = *reinterpret_cast<const u16x8 *>(p + 8 * i);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[8 * i + e] = bf16_to_f32(a[e]);
        }
    } else {
        static_assert(N == 4, "4 or a multiple of 8 elements");
        const u16x4 a = *reinterpret_cast<const u16x4 *>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = bf16_to_f32(a[e]);
    }
}

template <int N> __device__ __forceinline__ void load_n(const float *p, float (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p + 4 * i);
        x[4 * i + 0] = a.x;
        x[4 * i + 1] = a.y;
        x[4 * i + 2] = a.z;
        x[4 * i + 3] = a.w;
    }
}

// N consecutive elements kept as loaded (bf16 stays packed, two per register)
// and converted where they are used.
template <typename T, int N> struct Row;
template <int N> struct Row<uint16_t, N> {
    static_assert(N == 4 || N % 8 == 0, "4 or a multiple of 8 elements");
    static constexpr int W = N == 4 ? 4 : 8;  // elements per load
    typedef uint16_t vec __attribute__((ext_vector_type(W)));
    vec x[N / W];
    __device__ void load(const uint16_t *p) {
#pragma unroll
        for (int i = 0; i < N / W; ++i) x[i] = *reinterpret_cast<const vec *>(p + W * i);
    }
    __device__ float operator[](int r) const { return bf16_to_f32(x[r / W][r % W]); }
};
template <int N> struct Row<float, N> {
    f32x4 x[N / 4];
    __device__ void load(const float *p) {
#pragma unroll
        for (int i = 0; i < N / 4; ++i) x[i] = *reinterpret_cast<const f32x4 *>(p + 4 * i);
    }
    __device__ float operator[](int r) const { return x[r / 4][r % 4]; }
};

__device__ __forceinline__ f32x4 load4(const uint16_t *p) {
    u16x4 a = *reinterpret_cast<const u16x4 *>(p);
    return f32x4{bf16_to_f32(a[0]), bf16_to_f32(a[1]), bf16_to_f32(a[2]), bf16_to_f32(a[3])};
}

__device__ __forceinline__ f32x4 load4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

__device__ __forceinline__ void store4(uint16_t *p, f32x4 x) {
    u16x4 r = {f32_to_bf16(x.x), f32_to_bf16(x.y), f32_to_bf16(x.z), f32_to_bf16(x.w)};
    *reinterpret_cast<u16x4 *>(p) = r;
}

__device__ __forceinline__ void store4(float *p, f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }

template <int D, int RPT>
__device__ __forceinline__ void load_state(const float *s, int soff, f32x4 (&S)[RPT]) {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        S[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(s + soff + r * D));
}

template <int D, int RPT>
__device__ __forceinline__ void store_state(float *s, int soff, const f32x4 (&S)[RPT]) {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
        __builtin_nontemporal_store(S[r], reinterpret_cast<f32x4 *>(s + soff + r * D));
}

// o = oscale * q @ S for this thread's columns, summed over all row groups and
// stored by wave 0.  red is double-buffered by `parity`, so one barrier per
// token suffices: a buffer is rewritten only after the next barrier.
template <int D, typename T>
__device__ __forceinline__ void reduce_store(f32x4 o, f32x4 (&red)[2][4][Layout<D>::CG], int &parity,
                                             T *dst, float oscale = Layout<D>::kScale) {
    using L = Layout<D>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, cg = tid % L::CG;
#pragma unroll
    for (int m = L::CG; m < 64; m <<= 1) {
        o.x += __shfl_xor(o.x, m);
        o.y += __shfl_xor(o.y, m);
        o.z += __shfl_xor(o.z, m);
        o.w += __shfl_xor(o.w, m);
    }
    if (lane < L::CG) red[parity][wave][cg] = o;
    __syncthreads();
    if (wave == 0 && lane < L::CG) {
        const f32x4 s = red[parity][0][lane] + red[parity][1][lane] + red[parity][2][lane] +
                        red[parity][3][lane];
        store4(dst + 4 * lane, s * oscale);
    }
    parity ^= 1;
}

template <typename T, int D>
__device__ __forceinline__ void zero_rows(T *out, int64_t t0, int64_t t1, size_t row, int h) {
    const int tid = threadIdx.x;
    if (tid < D / 4)
        for (int64_t t = t0; t < t1; ++t)
            store4(out + t * row + static_cast<size_t>(h) * D + 4 * tid, f32x4{0, 0, 0, 0});
}

// x <- dhi x + t, one rounding, written in place: as plain code the compiler
// emits the accumulate form, whose result lands in t's register, and the
// loop-carried state then costs a copy and extra registers every step.
__device__ __forceinline__ void decay_step(f32x4 &x, float dhi, f32x4 t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) asm("v_fma_f32 %0, %1, %0, %2" : "+v"(x[i]) : "v"(dhi), "v"(t[i]));
}

// kTrack: the prefill variant that may take a state-tracking snapshot.
// kMulti: requests of more than one token (without it every token is a group
// of its own: decode, whose one-token body then needs fewer registers).
template <typename T, int D, bool kTrack, bool kMulti, bool kBatched>
__global__ __launch_bounds__(kThreads) void recurrent_kernel(RecurrentArgs a) {
    using L = Layout<D>;
    constexpr int RPT = L::RPT;
    const T *__restrict__ q = static_cast<const T *>(a.q);
    const T *__restrict__ k = static_cast<const T *>(a.k);
    const T *__restrict__ v = static_cast<const T *>(a.v);
    T *__restrict__ out = static_cast<T *>(a.out);
    const int H = a.num_heads;
    const int b = blockIdx.x / H;
    const int h = blockIdx.x - b * H;
    const int hk = h / (H / a.num_kv_heads);
    const int tid = threadIdx.x;
    const int cg = tid % L::CG, rg = tid / L::CG;

    int64_t t0, t1;
    if (a.cu_seqlens) {
        t0 = a.cu_seqlens[b];
        t1 = a.cu_seqlens[b + 1];
    } else {
        t0 = static_cast<int64_t>(b) * a.tokens_per_req;
        t1 = t0 + a.tokens_per_req;
    }
    t0 = t0 < 0 ? 0 : (t0 > a.total_tokens ? a.total_tokens : t0);
    t1 = t1 < t0 ? t0 : (t1 > a.total_tokens ? a.total_tokens : t1);

    const size_t row = static_cast<size_t>(H) * D;                // q/out token stride
    const size_t kvrow = static_cast<size_t>(a.num_kv_heads) * D;  // k/v token stride
    const int slot = a.slot_idx[b];
    if (slot < 0 || slot >= a.pool_slots) {
        zero_rows<T, D>(out, t0, t1, row, h);  // out-of-range slot: no state touched
        return;
    }
    const size_t sdd = static_cast<size_t>(D) * D;
    float *s_in = a.pool + (static_cast<size_t>(slot) * H + h) * sdd;
    float *s_out = a.state_out ? a.state_out + (static_cast<size_t>(b) * H + h) * sdd : s_in;
    // state-tracking snapshot after the first `tl` tokens ([LA-page] §额外覆盖)
    float *snap = nullptr;
    int64_t tl = -1;
    if (kTrack && a.track_lens) {
        const int ts = a.track_slot_idx[b];
        tl = a.track_lens[b];
        if (ts >= 0 && ts < a.pool_slots && tl >= 0 && tl <= t1 - t0)
            snap = a.pool + (static_cast<size_t>(ts) * H + h) * sdd;
    }
    const int soff = (RPT * rg) * D + 4 * cg;

    f32x4 S[RPT];
    load_state<D>(s_in, soff, S);
    // Decay arithmetic.  Multiplying the state by fl(e^{-l}) at every token
    // compounds the factor's rounding over a request and over successive
    // calls: the decay rate is off by up to 2^-25 / l relative (1.53x at
    // l = 3.9e-8, the slope of a last layer).  Here the tokens go in groups
    // of up to kGroup; with e the group's last token, the group runs in the
    // frame Y_s = e^{-l(e-s)} S_s:
    //   first token t:  Y <- round(whi S + (wlo S + w_t k_t v_t^T))
    //   later tokens:   Y <- Y + w_s k_s v_s^T,   w_s = e^{-l(e-s)} <= 1
    //   outputs:        o_s = scale e^{l(e-s)} q_s Y_s
    // and Y_e = S_e.  The group's decay e^{-l G} is the float pair whi + wlo
    // (wlo = expm1(-l G) - (whi - 1), whi - 1 exact), applied in the same
    // rounding as the first update, so the state decays at the exact rate
    // wherever the updates randomize the rounding, and each token costs two
    // operations per state element instead of three.  (Where they do not --
    // |S| < 256 |k v| for bf16 inputs, whose products lie on a grid no finer
    // than the state's ulp -- a sub-ulp decay per group rounds to a whole
    // number of ulps, and no round-to-nearest update is exact.)  The output
    // factor e^{l(e-s)} is kept below e^32 by the group length.
    const float lam = a.slopes[h];
    const float alam = fabsf(lam);
    int gmax = kMulti ? kGroup : 1;
    if (kMulti && !(alam * (kGroup - 1) <= 32.f)) gmax = alam <= 32.f ? 1 + static_cast<int>(32.f / alam) : 1;

    __shared__ f32x4 red[2][4][L::CG];
    int parity = 0;
    // the next token's k, q and v rows (fp32 several-token requests)
    Row<T, RPT> kk_next, qq_next;
    f32x4 vv_next;
    auto fetch = [&](int64_t s) {
        const size_t kvoff = s * kvrow + static_cast<size_t>(hk) * D;
        kk_next.load(k + kvoff + RPT * rg);
        qq_next.load(q + s * row + static_cast<size_t>(h) * D + RPT * rg);
        vv_next = load4(v + kvoff + 4 * cg);
    };
    if constexpr (kBatched)
        if (t0 < t1) fetch(t0);
    // one token; kFirst: the first of its group, which also applies the decay
    auto token = [&](int64_t s, int64_t e, float whi, float wlo, auto first) {
        constexpr bool kFirst = decltype(first)::value;
        const float w = expf(-lam * static_cast<float>(e - s));
        const size_t off = s * row + static_cast<size_t>(h) * D;
        const size_t kvoff = s * kvrow + static_cast<size_t>(hk) * D;
        Row<T, RPT> kk, qq;
        kk.load(k + kvoff + RPT * rg);
        qq.load(q + off + RPT * rg);
        const f32x4 vv = load4(v + kvoff + 4 * cg);
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RPT; ++r) {
            if constexpr (kFirst)
                decay_step(S[r], whi, wlo * S[r] + (w * kk[r]) * vv);
            else
                S[r] += (w * kk[r]) * vv;
            o += qq[r] * S[r];
        }
        reduce_store<D>(o, red, parity, out + off, L::kScale * expf(lam * static_cast<float>(e - s)));
    };
    // One group of G <= kGroup tokens from t (fp32 several-token requests).
    // weights e^{-l d} and output factors e^{l d} of a full group (d = 0..7),
    // computed once per call (a partial group computes its own)
    float wfull[kGroup], ofull[kGroup];
    if constexpr (kBatched) {
#pragma unroll
        for (int d = 0; d < kGroup; ++d) {
            wfull[d] = expf(-lam * static_cast<float>(d));
            ofull[d] = L::kScale * expf(lam * static_cast<float>(d));
        }
    }
    auto group = [&](int64_t t, int G, float whi, float wlo) {
        if constexpr (kBatched) {
            __shared__ f32x4 redg[2][4][kGroup][L::CG];
            const bool full = G == kGroup;
            static_assert(sizeof(redg) <= 32768, "group reduction buffer");
            f32x4 po[kGroup];
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                if (i < G) {
                    const int64_t s = t + i;
                    const float w = full ? wfull[kGroup - 1 - i] : expf(-lam * static_cast<float>(G - 1 - i));
                    const Row<T, RPT> kk = kk_next, qq = qq_next;
                    const f32x4 vv = vv_next;
                    if (s + 1 < t1) fetch(s + 1);
                    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int r = 0; r < RPT; ++r) {
                        if (i == 0)
                            decay_step(S[r], whi, wlo * S[r] + (w * kk[r]) * vv);
                        else
                            S[r] += (w * kk[r]) * vv;
                        o += qq[r] * S[r];
                    }
                    po[i] = o;
                }
            }
            const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
            for (int i = 0; i < kGroup; ++i) {
                if (i < G) {
#pragma unroll
                    for (int m = L::CG; m < 64; m <<= 1) {
                        po[i].x += __shfl_xor(po[i].x, m);
                        po[i].y += __shfl_xor(po[i].y, m);
                        po[i].z += __shfl_xor(po[i].z, m);
                        po[i].w += __shfl_xor(po[i].w, m);
                    }
                    if (lane < L::CG) redg[parity][wave][i][cg] = po[i];
                }
            }
            __syncthreads();
            if (wave == 0 && lane < L::CG) {
#pragma unroll
                for (int i = 0; i < kGroup; ++i) {
                    if (i < G) {
                        const f32x4 sum = redg[parity][0][i][lane] + redg[parity][1][i][lane] +
                                          redg[parity][2][i][lane] + redg[parity][3][i][lane];
                        const size_t off = (t + i) * row + static_cast<size_t>(h) * D;
                        const float oscale =
                            full ? ofull[kGroup - 1 - i] : L::kScale * expf(lam * static_cast<float>(G - 1 - i));
                        store4(out + off + 4 * lane, sum * oscale);
                    }
                }
            }
            parity ^= 1;
        }
    };
    // kBatched (fp32 prefill): the partial outputs of a group's tokens are
    // reduced across the row groups together, one barrier per group instead
    // of one per token, and each token's inputs are fetched while the one
    // before is computed.  Same arithmetic, in the same order, as the
    // token-at-a-time body above, which chain verify keeps: its requests are
    // a few tokens each, and the extra registers and LDS would cost it
    // occupancy (fp32 verify measured 4% slower with it).
    static_assert(!kBatched || (kMulti && std::is_same<T, float>::value), "batched groups: fp32, several tokens");
    for (int64_t t = t0; t < t1;) {
        int64_t G = t1 - t < gmax ? t1 - t : gmax;
        if (kTrack && snap) {
            // groups end at the snapshot point, where the frame is the state
            if (t - t0 == tl) store_state<D>(snap, soff, S);
            if (t - t0 < tl && tl - (t - t0) < G) G = tl - (t - t0);
        }
        const int64_t e = t + G - 1;
        const float whi = expf(-lam * static_cast<float>(G));
        const float wlo = whi >= 0.5f ? expm1f(-lam * static_cast<float>(G)) - (whi - 1.f) : 0.f;
        if constexpr (kBatched) {
            group(t, static_cast<int>(G), whi, wlo);
        } else {
            token(t, e, whi, wlo, std::true_type{});
            if constexpr (kMulti)
                for (int64_t s = t + 1; s <= e; ++s) token(s, e, whi, wlo, std::false_type{});
        }
        t = e + 1;
    }
    if (kTrack && snap && tl == t1 - t0) store_state<D>(snap, soff, S);
    store_state<D>(s_out, soff, S);
}

// Tree verify ([LA-page] §生产环境不支持 item 3, Next Work item 2).  Draft j
// of request b forks from its parent's state:
//     S_j = e^{-l} S_parent + k_j v_j^T
// With A the state of draft j-1 in registers and R the request's pool state
// (read where it is needed with cached loads: this call never writes the pool,
// and the repeat reads mostly hit in cache; a copy kept in registers or LDS
// measured slower):
//   parent j-1:  A <- e^{-l} A + k_j v_j^T       (the chain case)
//   parent -1:   A <- e^{-l} R + k_j v_j^T
//   otherwise:   unroll S_j up the parent chain a_1 = parent, a_2, ...:
//                A <- k_j v_j^T + sum_m e^{-l m} k_{a_m} v_{a_m}^T + e^{-l depth} R
// Parents are checked first (each in [-1, j)), so the walk strictly descends
// and ends.  A request with a bad slot or parent gets zero output.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void tree_kernel(TreeArgs a) {
    using L = Layout<D>;
    constexpr int RPT = L::RPT;
    const T *__restrict__ q = static_cast<const T *>(a.q);
    const T *__restrict__ k = static_cast<const T *>(a.k);
    const T *__restrict__ v = static_cast<const T *>(a.v);
    T *__restrict__ out = static_cast<T *>(a.out);
    const int H = a.num_heads, n = a.num_draft;
    const int b = blockIdx.x / H;
    const int h = blockIdx.x - b * H;
    const int hk = h / (H / a.num_kv_heads);
    const int tid = threadIdx.x;
    const int cg = tid % L::CG, rg = tid / L::CG;
    const size_t row = static_cast<size_t>(H) * D;
    const size_t kvrow = static_cast<size_t>(a.num_kv_heads) * D;
    const int64_t t0 = static_cast<int64_t>(b) * n;
    const int32_t *par = a.parent_idx + t0;

    const int slot = a.slot_idx[b];
    bool ok = slot >= 0 && slot < a.pool_slots;
    for (int j = 0; j < n && ok; ++j) ok = par[j] >= -1 && par[j] < j;
    if (!ok) {
        zero_rows<T, D>(out, t0, t0 + n, row, h);
        return;
    }
    const size_t sdd = static_cast<size_t>(D) * D;
    const int soff = (RPT * rg) * D + 4 * cg;
    const float *R = a.pool + (static_cast<size_t>(slot) * H + h) * sdd + soff;
    f32x4 A[RPT];
    // Decay as a float pair dhi + dlo (see recurrent_kernel): every draft
    // state may become the request's next state.
    const float lam = a.slopes[h];
    const float dhi = expf(-lam);
    const float dlo = dhi >= 0.5f ? (1.f - dhi) + expm1f(-lam) : 0.f;

    auto kv = [&](int j, float (&kk)[RPT], f32x4 &vv) {
        const size_t kvoff = (t0 + j) * kvrow + static_cast<size_t>(hk) * D;
        load_n<RPT>(k + kvoff + RPT * rg, kk);
        vv = load4(v + kvoff + 4 * cg);
    };

    __shared__ f32x4 red[2][4][L::CG];
    int parity = 0;
    for (int j = 0; j < n; ++j) {
        float kk[RPT], qq[RPT];
        f32x4 vv;
        kv(j, kk, vv);
        const size_t off = (t0 + j) * row + static_cast<size_t>(h) * D;
        load_n<RPT>(q + off + RPT * rg, qq);
        const int p = par[j];
        if (p >= 0 && p == j - 1) {
#pragma unroll
            for (int r = 0; r < RPT; ++r) decay_step(A[r], dhi, dlo * A[r] + kk[r] * vv);
        } else if (p < 0) {
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const f32x4 root = *reinterpret_cast<const f32x4 *>(R + r * D);
                A[r] = dhi * root + (dlo * root + kk[r] * vv);
            }
        } else {
#pragma unroll
            for (int r = 0; r < RPT; ++r) A[r] = kk[r] * vv;
            // the weight of an ancestor m steps up is dhi^m (m <= num_draft, so
            // the factor's rounding stays below m 2^-25, once per call); the
            // root's weight e^{-l depth} is a pair whi + wlo, as for one step
            float w = dhi;
            int depth = 1;
            for (int x = p; x >= 0; x = par[x]) {
                float ka[RPT];
                f32x4 va;
                kv(x, ka, va);
#pragma unroll
                for (int r = 0; r < RPT; ++r) A[r] += (w * ka[r]) * va;
                w *= dhi;
                ++depth;
            }
            // e^{-l depth} - w = expm1(-l depth) - (w - 1), with w - 1 exact for
            // w >= 1/2 (below that the rate error of w alone is negligible)
            const float wlo = dlo == 0.f || w < 0.5f ? 0.f : expm1f(-lam * static_cast<float>(depth)) - (w - 1.f);
#pragma unroll
            for (int r = 0; r < RPT; ++r) {
                const f32x4 root = *reinterpret_cast<const f32x4 *>(R + r * D);
                A[r] += w * root + wlo * root;
            }
        }
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < RPT; ++r) o += qq[r] * A[r];
        reduce_store<D>(o, red, parity, out + off);
        if (a.draft_states)
            store_state<D>(a.draft_states + ((t0 + j) * H + h) * sdd, soff, A);
    }
}

template <typename T, int D>
hipError_t launch_rec(const RecurrentArgs &a, int batch, hipStream_t stream) {
    RecurrentArgs copy = a;
    void *args[] = {&copy};
    const bool one = !a.cu_seqlens && a.tokens_per_req == 1;  // decode
    const void *fn = a.track_lens ? reinterpret_cast<const void *>(&recurrent_kernel<T, D, true, true, false>)
                     : one        ? reinterpret_cast<const void *>(&recurrent_kernel<T, D, false, false, false>)
                                  : reinterpret_cast<const void *>(&recurrent_kernel<T, D, false, true, false>);
    if constexpr (std::is_same<T, float>::value) {
        if (a.cu_seqlens)  // fp32 prefill (with or without a snapshot): groups reduced together
            fn = a.track_lens ? reinterpret_cast<const void *>(&recurrent_kernel<T, D, true, true, true>)
                              : reinterpret_cast<const void *>(&recurrent_kernel<T, D, false, true, true>);
    }
    return hipLaunchKernel(fn,
                           dim3(static_cast<unsigned>(batch) * a.num_heads), dim3(kThreads), args,
                           0, stream);
}

template <typename T, int D>
hipError_t launch_tree_t(const TreeArgs &a, int batch, hipStream_t stream) {
    TreeArgs copy = a;
    void *args[] = {&copy};
    return hipLaunchKernel(reinterpret_cast<const void *>(&tree_kernel<T, D>),
                           dim3(static_cast<unsigned>(batch) * a.num_heads), dim3(kThreads), args,
                           0, stream);
}

}  // namespace

hipError_t launch_recurrent(const RecurrentArgs &a, bool bf16, int head_dim, int batch,
                            hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    if (head_dim == 128)
        return bf16 ? launch_rec<uint16_t, 128>(a, batch, stream) : launch_rec<float, 128>(a, batch, stream);
    return bf16 ? launch_rec<uint16_t, 64>(a, batch, stream) : launch_rec<float, 64>(a, batch, stream);
}

hipError_t launch_tree(const TreeArgs &a, bool bf16, int head_dim, int batch, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    if (head_dim == 128)
        return bf16 ? launch_tree_t<uint16_t, 128>(a, batch, stream)
                    : launch_tree_t<float, 128>(a, batch, stream);
    return bf16 ? launch_tree_t<uint16_t, 64>(a, batch, stream) : launch_tree_t<float, 64>(a, batch, stream);
}

}  // namespace la
