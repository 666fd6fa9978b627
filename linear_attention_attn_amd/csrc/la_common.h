// la_common.h -- device-side building blocks shared by the Lightning Attention
// kernels for gfx950 (CDNA4): element types, 8-element MFMA operand
// fragments, the 16x16 matrix-core step, swizzled LDS addressing and bf16
// packing.
//
// MFMA conventions used everywhere (64-lane wavefront, 16x16 output tile):
//   lane l, g = l / 16, c = l % 16
//   A operand (M x K): lane holds row c, eight K values ("k-slots") of group g
//   B operand (K x N): lane holds column c, the same eight k-slots of group g
//   C/D (M x N, fp32): lane holds column c, rows 4g + r for r = 0..3
// The reduction order inside a 32-wide K step is free, so every product below
// picks the k-slot -> index mapping that lets both operands be read with
// contiguous LDS loads (or be taken straight from an earlier accumulator).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- element traits -----------------------------------------------------

struct bf16_t { uint16_t bits; };

template <typename T> struct Elem;
template <> struct Elem<bf16_t> { static constexpr int kBytes = 2; };
template <> struct Elem<float>  { static constexpr int kBytes = 4; };

// Eight operand values for one 32-wide K step.
//   bf16: 4 dwords (one v_mfma_f32_16x16x32_bf16)
//   fp32: 8 floats (eight v_mfma_f32_16x16x4_f32, slot m in step m)
template <typename T> struct Frag;
template <> struct Frag<bf16_t> { u32x4_t u; };
template <> struct Frag<float>  { float f[8]; };

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// acc += A x B over one 32-wide K step.
__device__ __forceinline__ void mma(f32x4_t &acc, const Frag<bf16_t> &a, const Frag<bf16_t> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a.u),
                                                  __builtin_bit_cast(bf16x8_t, b.u), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4_t &acc, const Frag<float> &a, const Frag<float> &b) {
#pragma unroll
    for (int m = 0; m < 8; ++m) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[m], b.f[m], acc, 0, 0, 0);
}

// ---- fp32 -> bf16, round to nearest even (NaN kept quiet) ---------------

__device__ __forceinline__ uint32_t bf16_bits_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return bf16_bits_rne(lo) | (bf16_bits_rne(hi) << 16);
}

// Build an operand fragment from eight fp32 values (used for the masked
// score tile that feeds the P V product).
__device__ __forceinline__ Frag<bf16_t> frag_from_f32(const f32x4_t &x0, const f32x4_t &x1, bf16_t) {
    Frag<bf16_t> r;
    r.u[0] = pack_bf16x2(x0[0], x0[1]);
    r.u[1] = pack_bf16x2(x0[2], x0[3]);
    r.u[2] = pack_bf16x2(x1[0], x1[1]);
    r.u[3] = pack_bf16x2(x1[2], x1[3]);
    return r;
}
__device__ __forceinline__ Frag<float> frag_from_f32(const f32x4_t &x0, const f32x4_t &x1, float) {
    Frag<float> r;
#pragma unroll
    for (int m = 0; m < 4; ++m) { r.f[m] = x0[m]; r.f[4 + m] = x1[m]; }
    return r;
}

// ---- swizzled LDS rows --------------------------------------------------
// Rows of `kRowBytes` bytes, addressed in 16-byte chunks; the chunk index is
// XOR-ed with a function of the row so that 16 consecutive rows read at the
// same logical column land on distinct banks.
template <int kRowBytes>
struct LdsRows {
    static_assert(kRowBytes == 128 || kRowBytes == 256 || kRowBytes == 512, "row size");
    __device__ __forceinline__ static uint32_t swz(uint32_t row) {
        return kRowBytes >= 256 ? (row & 15u) : ((row >> 1) & 7u);
    }
    // byte offset of byte `b` of the logical row
    __device__ __forceinline__ static uint32_t off(uint32_t row, uint32_t b) {
        return row * kRowBytes + ((((b >> 4) ^ swz(row)) << 4) | (b & 15u));
    }
};

// 8 consecutive elements starting at element e0 (e0 multiple of 8) of a row.
template <typename T, int kRowBytes>
__device__ __forceinline__ Frag<T> lds_read8(const char *base, uint32_t row, uint32_t e0) {
    using R = LdsRows<kRowBytes>;
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        f.u = *reinterpret_cast<const u32x4_t *>(base + R::off(row, e0 * 2));
    } else {
        f32x4_t a = *reinterpret_cast<const f32x4_t *>(base + R::off(row, e0 * 4));
        f32x4_t b = *reinterpret_cast<const f32x4_t *>(base + R::off(row, e0 * 4 + 16));
#pragma unroll
        for (int m = 0; m < 4; ++m) { f.f[m] = a[m]; f.f[4 + m] = b[m]; }
    }
    return f;
}

// Two runs of 4 elements, at e0 and e1 (each a multiple of 4): slots 0..3
// from e0, slots 4..7 from e1.
template <typename T, int kRowBytes>
__device__ __forceinline__ Frag<T> lds_read4x2(const char *base, uint32_t row, uint32_t e0, uint32_t e1) {
    using R = LdsRows<kRowBytes>;
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        u32x2_t a = *reinterpret_cast<const u32x2_t *>(base + R::off(row, e0 * 2));
        u32x2_t b = *reinterpret_cast<const u32x2_t *>(base + R::off(row, e1 * 2));
        f.u = u32x4_t{a[0], a[1], b[0], b[1]};
    } else {
        f32x4_t a = *reinterpret_cast<const f32x4_t *>(base + R::off(row, e0 * 4));
        f32x4_t b = *reinterpret_cast<const f32x4_t *>(base + R::off(row, e1 * 4));
#pragma unroll
        for (int m = 0; m < 4; ++m) { f.f[m] = a[m]; f.f[4 + m] = b[m]; }
    }
    return f;
}

// 8 consecutive elements from global memory (16 or 32 bytes, aligned), or
// zeros when !valid.
template <typename T>
__device__ __forceinline__ Frag<T> gload8(const T *p, bool valid) {
    Frag<T> f;
    if constexpr (sizeof(T) == 2) {
        f.u = valid ? *reinterpret_cast<const u32x4_t *>(p) : u32x4_t{0u, 0u, 0u, 0u};
    } else {
        f32x4_t a = valid ? *reinterpret_cast<const f32x4_t *>(p) : zero4();
        f32x4_t b = valid ? *reinterpret_cast<const f32x4_t *>(p + 4) : zero4();
#pragma unroll
        for (int m = 0; m < 4; ++m) { f.f[m] = a[m]; f.f[4 + m] = b[m]; }
    }
    return f;
}

// Store four fp32 values as 4 consecutive elements of T.
__device__ __forceinline__ void store4(bf16_t *p, const f32x4_t &x) {
    *reinterpret_cast<u32x2_t *>(p) = u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
}
__device__ __forceinline__ void store4(float *p, const f32x4_t &x) {
    *reinterpret_cast<f32x4_t *>(p) = x;
}

// Write four fp32 values as 4 consecutive elements of T into an LDS row.
template <typename T, int kRowBytes>
__device__ __forceinline__ void lds_write4(char *base, uint32_t row, uint32_t e0, const f32x4_t &x) {
    using R = LdsRows<kRowBytes>;
    if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<u32x2_t *>(base + R::off(row, e0 * 2)) =
            u32x2_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    } else {
        *reinterpret_cast<f32x4_t *>(base + R::off(row, e0 * 4)) = x;
    }
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }
__device__ __forceinline__ uint32_t wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace la
