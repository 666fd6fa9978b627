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

// With `slots` (an indexed state table, for batches that come and go while
// their states stay in a pool): row b's state is pool entry slots[b]; rows
// whose slot is negative or not below `nslots` are padding: their o is
// zero and no state is touched (so a batch can be padded to a fixed size).
// With ROPE the first rope_dims dims of q and k are rotated at the row's
// position positions[b] (pair i: dims i and i + rope_dims / 2, angle
// positions[b] * base^(-2i / rope_dims)).
template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(kDecThreads) void k_decode(const T *__restrict__ q, const T *__restrict__ k,
                                                      const T *__restrict__ v, float *__restrict__ state,
                                                      T *__restrict__ o, const int32_t *__restrict__ slots,
                                                      int heads, int nslots, int rope_dims, double rope_base,
                                                      const int32_t *__restrict__ positions) {
    constexpr int CT = D / 4;                 // threads across one row (4 columns each)
    constexpr int RG = kDecThreads / CT;      // row groups
    constexpr int RPT = D / RG;               // rows per thread
    __shared__ float sq[D], sk[D];
    __shared__ f32x4_t red[RG][CT];

    // Workgroups are dealt to the 8 XCDs round-robin; give each XCD a
    // contiguous range of units (measured ~1.5% faster than unit = blockIdx.x
    // on MI355X; pseudo-random orders were slower).
    const int64_t nb = gridDim.x;
    const int64_t unit = (nb % 8 == 0) ? (int64_t)(blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8 : blockIdx.x;
    const int t = threadIdx.x;
    const T *qu = q + unit * D, *ku = k + unit * D, *vu = v + unit * D;
    int64_t su = unit;                        // state entry of this (row, head)
    if (slots != nullptr) {
        const int64_t b = unit / heads, h = unit - b * heads;
        const int slot = slots[b];
        if (slot < 0 || slot >= nslots) {     // padding row
            if (t < D) from_f32(0.f, o + unit * D + t);
            return;
        }
        su = (int64_t)slot * heads + h;
    }
    float *S = state + su * (int64_t)D * D;
    if (t < D) {
        float qx = to_f32(qu[t]), kx = to_f32(ku[t]);
        if (ROPE && t < rope_dims) {
            const int half = rope_dims / 2;
            const bool first = t < half;
            const int i = first ? t : t - half, pt = first ? t + half : t - half;
            const float qp = to_f32(qu[pt]), kp = to_f32(ku[pt]);
            const double f = (0.5 / 3.14159265358979323846) * exp2(-2.0 * i / rope_dims * log2(rope_base));
            float c, sn;
            rope_cs((double)positions[unit / heads], f, c, sn);
            if (first) sn = -sn;
            qx = qx * c + qp * sn;
            kx = kx * c + kp * sn;
        }
        sq[t] = qx;
        sk[t] = kx;
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

template <typename T, bool ROPE>
static void launch_dec_t(const void *q, const void *k, const void *v, float *state, void *o, int heads,
                         int head_dim, dim3 grid, hipStream_t st, const int32_t *slots, int nslots,
                         int rope_dims, double rope_base, const int32_t *positions) {
    auto *qq = reinterpret_cast<const T *>(q);
    auto *kk = reinterpret_cast<const T *>(k);
    auto *vv = reinterpret_cast<const T *>(v);
    auto *oo = reinterpret_cast<T *>(o);
    if (head_dim == 64)
        hipLaunchKernelGGL((k_decode<T, 64, ROPE>), grid, dim3(kDecThreads), 0, st, qq, kk, vv, state, oo,
                           slots, heads, nslots, rope_dims, rope_base, positions);
    else
        hipLaunchKernelGGL((k_decode<T, 128, ROPE>), grid, dim3(kDecThreads), 0, st, qq, kk, vv, state, oo,
                           slots, heads, nslots, rope_dims, rope_base, positions);
}

int launch_decode(const void *q, const void *k, const void *v, float *state, void *o, int batch,
                  int heads, int head_dim, int dtype, void *stream, const int32_t *slots, int nslots,
                  int rope_dims, double rope_base, const int32_t *positions) {
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)((int64_t)batch * heads));
    const bool rope = rope_dims > 0;
    if (dtype == 0) {
        if (rope) launch_dec_t<bf16_t, true>(q, k, v, state, o, heads, head_dim, grid, st, slots, nslots, rope_dims, rope_base, positions);
        else launch_dec_t<bf16_t, false>(q, k, v, state, o, heads, head_dim, grid, st, slots, nslots, 0, 0.0, nullptr);
    } else {
        if (rope) launch_dec_t<float, true>(q, k, v, state, o, heads, head_dim, grid, st, slots, nslots, rope_dims, rope_base, positions);
        else launch_dec_t<float, false>(q, k, v, state, o, heads, head_dim, grid, st, slots, nslots, 0, 0.0, nullptr);
    }
    return (int)hipGetLastError();
}

}  // namespace la
