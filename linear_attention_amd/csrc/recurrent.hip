// Token-recurrent seg_la kernel: decode (one token), chain verify (k tokens)
// and the fp32 prefill path.
//
// Citations name the web page "SGLang Lightning Attention 能力矩阵与 seg_la
// 线性注意力测试覆盖深度解析" (www.2kiu.com/news/4599301) as [LA-page].
//
// Per (request, head) the recurrence of [LA-page] §独立参考实现 is advanced
// one token at a time with the 128x128 fp32 state held in registers:
//     S <- exp(-slope) * S + k v^T ;  o = (q @ S) / sqrt(128)
// This path is bound by HBM traffic: per (request, head) it streams the 64 KiB
// state in and out once, so each thread owns 16 rows x 4 columns of S and
// moves it with 16 coalesced 128-bit loads and stores (nontemporal: the state
// is touched once per call).  The q.S column sums are reduced across the 8
// row groups with one cross-half-wave shuffle and a 4-wave LDS pass.
#include "common.h"
#include "launch.h"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int kStateElems = kHeadDim * kHeadDim;

// 16 consecutive elements starting at p (16-byte aligned), as floats
__device__ __forceinline__ void load16(const uint16_t *p, float (&x)[16]) {
    u16x8 a = *reinterpret_cast<const u16x8 *>(p);
    u16x8 b = *reinterpret_cast<const u16x8 *>(p + 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        x[e] = bf16_to_f32(a[e]);
        x[8 + e] = bf16_to_f32(b[e]);
    }
}

__device__ __forceinline__ void load16(const float *p, float (&x)[16]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f32x4 a = *reinterpret_cast<const f32x4 *>(p + 4 * e);
        x[4 * e + 0] = a.x;
        x[4 * e + 1] = a.y;
        x[4 * e + 2] = a.z;
        x[4 * e + 3] = a.w;
    }
}

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

// Thread layout: column group cg = tid % 32 owns value columns 4cg..4cg+3,
// row group rg = tid / 32 owns key rows 16rg..16rg+15.  A wave covers two row
// groups, so each 128-bit load instruction reads two full 512-byte rows.
template <typename T>
__global__ __launch_bounds__(kThreads) void recurrent_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const int32_t *__restrict__ cu_seqlens, int tokens_per_req, int num_heads,
    int64_t total_tokens, float *__restrict__ pool, int64_t pool_slots,
    const int32_t *__restrict__ slot_idx, const float *__restrict__ slopes, T *__restrict__ out,
    float *__restrict__ state_out) {
    const int b = blockIdx.x / num_heads;
    const int h = blockIdx.x - b * num_heads;
    const int tid = threadIdx.x;
    const int cg = tid & 31, rg = tid >> 5, lane = tid & 63, wave = tid >> 6;

    int64_t t0, t1;
    if (cu_seqlens) {
        t0 = cu_seqlens[b];
        t1 = cu_seqlens[b + 1];
    } else {
        t0 = static_cast<int64_t>(b) * tokens_per_req;
        t1 = t0 + tokens_per_req;
    }
    t0 = t0 < 0 ? 0 : (t0 > total_tokens ? total_tokens : t0);
    t1 = t1 < t0 ? t0 : (t1 > total_tokens ? total_tokens : t1);

    const size_t row = static_cast<size_t>(num_heads) * kHeadDim;  // token stride
    const int slot = slot_idx[b];
    if (slot < 0 || slot >= pool_slots) {
        // out-of-range slot: zero output, no state touched
        if (wave == 0 && lane < 32)
            for (int64_t t = t0; t < t1; ++t)
                store4(out + t * row + static_cast<size_t>(h) * kHeadDim + 4 * lane, f32x4{0, 0, 0, 0});
        return;
    }

    float *s_in = pool + (static_cast<size_t>(slot) * num_heads + h) * kStateElems;
    float *s_out = state_out ? state_out + (static_cast<size_t>(b) * num_heads + h) * kStateElems : s_in;
    const int soff = (16 * rg) * kHeadDim + 4 * cg;

    f32x4 S[16];
#pragma unroll
    for (int r = 0; r < 16; ++r)
        S[r] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(s_in + soff + r * kHeadDim));

    const float decay = expf(-slopes[h]);
    const float scale = 0.08838834764831845f;  // 128^-1/2

    __shared__ f32x4 red[2][4][32];
    int parity = 0;
    for (int64_t t = t0; t < t1; ++t) {
        const size_t off = t * row + static_cast<size_t>(h) * kHeadDim;
        float kk[16], qq[16];
        load16(k + off + 16 * rg, kk);
        load16(q + off + 16 * rg, qq);
        const f32x4 vv = load4(v + off + 4 * cg);
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            S[r] = decay * S[r] + kk[r] * vv;
            o += qq[r] * S[r];
        }
        o.x += __shfl_xor(o.x, 32);
        o.y += __shfl_xor(o.y, 32);
        o.z += __shfl_xor(o.z, 32);
        o.w += __shfl_xor(o.w, 32);
        if (lane < 32) red[parity][wave][cg] = o;
        __syncthreads();
        if (wave == 0 && lane < 32) {
            f32x4 s = red[parity][0][lane] + red[parity][1][lane] + red[parity][2][lane] +
                      red[parity][3][lane];
            store4(out + off + 4 * lane, s * scale);
        }
        parity ^= 1;
    }

#pragma unroll
    for (int r = 0; r < 16; ++r)
        __builtin_nontemporal_store(S[r], reinterpret_cast<f32x4 *>(s_out + soff + r * kHeadDim));
}

template <typename T>
hipError_t launch(const void *q, const void *k, const void *v, const int32_t *cu_seqlens,
                  int tokens_per_req, int batch, int num_heads, int64_t total_tokens, float *pool,
                  int64_t pool_slots, const int32_t *slot_idx, const float *slopes, void *out,
                  float *state_out, hipStream_t stream) {
    const T *qp = static_cast<const T *>(q), *kp = static_cast<const T *>(k),
            *vp = static_cast<const T *>(v);
    T *op = static_cast<T *>(out);
    void *args[] = {&qp, &kp, &vp, &cu_seqlens, &tokens_per_req, &num_heads, &total_tokens,
                    &pool, &pool_slots, &slot_idx, &slopes, &op, &state_out};
    return hipLaunchKernel(reinterpret_cast<const void *>(&recurrent_kernel<T>),
                           dim3(static_cast<unsigned>(batch) * num_heads), dim3(kThreads), args, 0,
                           stream);
}

}  // namespace

hipError_t launch_recurrent(bool bf16, const void *q, const void *k, const void *v,
                            const int32_t *cu_seqlens, int tokens_per_req, int batch,
                            int num_heads, int64_t total_tokens, float *pool,
                            int64_t pool_slots, const int32_t *slot_idx, const float *slopes,
                            void *out, float *state_out, hipStream_t stream) {
    if (batch == 0) return hipSuccess;
    if (bf16)
        return launch<uint16_t>(q, k, v, cu_seqlens, tokens_per_req, batch, num_heads,
                                total_tokens, pool, pool_slots, slot_idx, slopes, out, state_out,
                                stream);
    return launch<float>(q, k, v, cu_seqlens, tokens_per_req, batch, num_heads, total_tokens,
                         pool, pool_slots, slot_idx, slopes, out, state_out, stream);
}

}  // namespace la
