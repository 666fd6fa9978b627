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

// ---- fp32 -> bf16, round to nearest even --------------------------------
// gfx950 converts two floats to packed bf16 in one instruction
// (v_cvt_pk_bf16_f32, rounding to nearest even in the default mode).

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) { return pack_bf16x2(x, 0.f) & 0xffffu; }

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

// ---- LDS transpose reads and global -> LDS DMA (gfx950) ------------------

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// ds_read_b64_tr_b16: within each 16-lane group, lanes 4r..4r+3 each name a
// run of four 16-bit elements; together they form row r of a 4 x 16 matrix
// X.  Lane i of the group receives column i: X[0][i], X[1][i], X[2][i],
// X[3][i].  With lane 4r+q pointing at element 4q of row r of a 16-column
// window, lane i gets the window's column i from four rows: a token-strided
// MFMA operand read from a token-major (row-major) tile.
__device__ __forceinline__ u32x2_t lds_read_tr16(const char *p) {
    v4i16_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(p));
    return __builtin_bit_cast(u32x2_t, r);
}

// Raw buffer resource over `bytes` bytes at `base` (stride 0): loads past the
// end return zeros and stores past the end are dropped, by the hardware's
// range check (offset = voffset + soffset + instruction offset).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer load of 16 bytes per lane straight into LDS (lane l's bytes at
// lds + 16 l), visible to the compiler: it tracks the LDS destination and
// waits for this load before an LDS access that may read it.
__device__ __forceinline__ void dma_lds16(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
}

// 16-byte buffer store from inline asm, so that the compiler's vmcnt
// bookkeeping holds loads only (it treats a counter with loads and stores
// pending as unordered and then waits for everything).  The s_nop keeps the
// data registers unchanged for the wait state a store of more than 8 bytes
// needs before they are written again.
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t voff, u32x4_t v) {
    asm volatile("buffer_store_dwordx4 %0, %1, %2, 0 offen\n\ts_nop 1"
                 :
                 : "v"(v), "v"(voff), "s"(r)
                 : "memory");
}

// 8-byte LDS write from inline asm.  Used for LDS that the compiler would
// otherwise order behind pending LDS DMA (with a full vmcnt wait) although
// the DMA writes elsewhere; the caller's lgkmcnt wait and barrier publish it.
__device__ __forceinline__ void lds_store8(char *p, u32x2_t v) {
    const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)p;
    asm volatile("ds_write_b64 %0, %1" : : "v"(a), "v"(v) : "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 left at its maximum, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// Runtime count (wave-uniform) mapped onto the immediate forms.
__device__ __forceinline__ void wait_vm_lgkm0(int n) {
    switch (n) {
#define LA_WAIT_CASE(k) case k: wait_vm_lgkm0<k>(); break;
        LA_WAIT_CASE(0) LA_WAIT_CASE(1) LA_WAIT_CASE(2) LA_WAIT_CASE(3) LA_WAIT_CASE(4)
        LA_WAIT_CASE(5) LA_WAIT_CASE(6) LA_WAIT_CASE(7) LA_WAIT_CASE(8) LA_WAIT_CASE(9)
        LA_WAIT_CASE(10) LA_WAIT_CASE(11) LA_WAIT_CASE(12) LA_WAIT_CASE(13) LA_WAIT_CASE(14)
        LA_WAIT_CASE(15) LA_WAIT_CASE(16) LA_WAIT_CASE(17) LA_WAIT_CASE(18) LA_WAIT_CASE(19)
        LA_WAIT_CASE(20) LA_WAIT_CASE(21) LA_WAIT_CASE(22) LA_WAIT_CASE(23) LA_WAIT_CASE(24)
        LA_WAIT_CASE(25) LA_WAIT_CASE(26) LA_WAIT_CASE(27) LA_WAIT_CASE(28) LA_WAIT_CASE(29)
        LA_WAIT_CASE(30) LA_WAIT_CASE(31) LA_WAIT_CASE(32) LA_WAIT_CASE(33) LA_WAIT_CASE(34)
        LA_WAIT_CASE(35) LA_WAIT_CASE(36) LA_WAIT_CASE(37) LA_WAIT_CASE(38) LA_WAIT_CASE(39)
        LA_WAIT_CASE(40) LA_WAIT_CASE(41) LA_WAIT_CASE(42) LA_WAIT_CASE(43) LA_WAIT_CASE(44)
        LA_WAIT_CASE(45) LA_WAIT_CASE(46) LA_WAIT_CASE(47) LA_WAIT_CASE(48) LA_WAIT_CASE(49)
        LA_WAIT_CASE(50) LA_WAIT_CASE(51) LA_WAIT_CASE(52) LA_WAIT_CASE(53) LA_WAIT_CASE(54)
        LA_WAIT_CASE(55) LA_WAIT_CASE(56) LA_WAIT_CASE(57) LA_WAIT_CASE(58) LA_WAIT_CASE(59)
        LA_WAIT_CASE(60) LA_WAIT_CASE(61) LA_WAIT_CASE(62) LA_WAIT_CASE(63)
#undef LA_WAIT_CASE
        default: wait_vm_lgkm0<0>(); break;
    }
}

// Workgroup barrier with no implied memory wait: the caller has already
// waited for exactly what the next phase reads.  The empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Makes the fragments' registers live (and their loads complete) at this
// point, so a batch of LDS reads is issued back to back and waited for once
// instead of being interleaved one by one with the products that use them.
template <int N, typename F>
__device__ __forceinline__ void hold(const F (&f)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : : "v"(f[i].u));
}

// Keeps the compiler from hoisting memory accesses across this point (used to
// bound how many operand fragments are live at once).
__device__ __forceinline__ void sched_fence() { asm volatile("" ::: "memory"); }

// ---- rotary position embedding (bf16 operands) ---------------------------
// Pair i of a token at position pos turns by the angle pos * theta_i with
// theta_i = base^(-2i / r) (r rotated dims; pair i is dims i and i + r/2).
// The angle is kept in turns: t = frac(pos * f_i) with f_i = theta_i / (2 pi).
// Positions reach millions, so the product and its fractional part are taken
// in fp64; the sine and cosine of the turn fraction come from the hardware's
// v_sin_f32 / v_cos_f32, which take their argument in turns.  Consecutive
// pairs' frequencies differ by the factor rho = base^(-2/r).

// rho = base^(-2/r), the ratio f_{i+1} / f_i.
__device__ __forceinline__ double rope_rho(double base, int r) { return exp2(-2.0 / r * log2(base)); }

// A kernel-uniform double held in scalar registers.
__device__ __forceinline__ double uniform_f64(double x) {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Frequencies in turns of the first pair of each group of eight:
// fj = f_{8j} = rho^{8j} / (2 pi), j < 4 (kernel-uniform, scalar registers;
// separate members, not an array, so that a lane's pick is a register select).
struct RopeFreqs {
    double f0, f1, f2, f3;
    double rho;
};

__device__ __forceinline__ RopeFreqs rope_freqs(double base, int r) {
    RopeFreqs q;
    q.rho = uniform_f64(rope_rho(base, r));
    const double r8 = q.rho * q.rho * q.rho * q.rho * q.rho * q.rho * q.rho * q.rho;
    const double f0 = 0.5 / 3.14159265358979323846;
    q.f0 = uniform_f64(f0);
    q.f1 = uniform_f64(f0 * r8);
    q.f2 = uniform_f64(f0 * r8 * r8);
    q.f3 = uniform_f64(f0 * r8 * r8 * r8);
    return q;
}

// f_{8 grp} for a lane's pair group grp (0..3), picked with bit masks (a
// plain select of the members can be turned into an indexed load from a
// stack copy of the struct).
__device__ __forceinline__ double rope_f(int grp, const RopeFreqs &q) {
    const uint64_t m1 = 0ull - (uint64_t)(grp & 1), m2 = 0ull - (uint64_t)((grp >> 1) & 1);
    const uint64_t f0 = __builtin_bit_cast(uint64_t, q.f0), f1 = __builtin_bit_cast(uint64_t, q.f1);
    const uint64_t f2 = __builtin_bit_cast(uint64_t, q.f2), f3 = __builtin_bit_cast(uint64_t, q.f3);
    const uint64_t lo = (f0 & ~m1) | (f1 & m1), hi = (f2 & ~m1) | (f3 & m1);
    return __builtin_bit_cast(double, (lo & ~m2) | (hi & m2));
}

__device__ __forceinline__ void rope_cs(double pos, double f, float &c, float &s) {
    const float tf = (float)__builtin_amdgcn_fract(pos * f);   // in [0, 1)
    s = __builtin_amdgcn_sinf(tf);
    c = __builtin_amdgcn_cosf(tf);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Rotate the eight pairs (x[e], y[e]), e = 0..7, of pairs i0 + e (f = f_{i0})
// at position pos; x holds the first dims of the pairs, y their partners.
__device__ __forceinline__ void rope_rot8(u32x4_t &x, u32x4_t &y, double pos, double f, double rho) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        float c0, s0, c1, s1;
        rope_cs(pos, f, c0, s0);
        f *= rho;
        rope_cs(pos, f, c1, s1);
        f *= rho;
        const float x0 = bf16_lo(x[d]), x1 = bf16_hi(x[d]), y0 = bf16_lo(y[d]), y1 = bf16_hi(y[d]);
        x[d] = pack_bf16x2(x0 * c0 - y0 * s0, x1 * c1 - y1 * s1);
        y[d] = pack_bf16x2(x0 * s0 + y0 * c0, x1 * s1 + y1 * c1);
    }
}

// One side of eight pairs whose two halves sit in different lanes: `mine`
// becomes its rotated self, given the partner's values `other`; `first` says
// whether `mine` holds the pairs' first dims.
__device__ __forceinline__ u32x4_t rope_rot8_half(const u32x4_t &mine, const u32x4_t &other, bool first,
                                                  double pos, double f, double rho) {
    u32x4_t r;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        float c0, s0, c1, s1;
        rope_cs(pos, f, c0, s0);
        f *= rho;
        rope_cs(pos, f, c1, s1);
        f *= rho;
        if (first) { s0 = -s0; s1 = -s1; }
        r[d] = pack_bf16x2(bf16_lo(mine[d]) * c0 + bf16_lo(other[d]) * s0,
                           bf16_hi(mine[d]) * c1 + bf16_hi(other[d]) * s1);
    }
    return r;
}

__device__ __forceinline__ uint32_t lane_id() { return threadIdx.x & 63u; }
// The lane id produced afresh at each call (opaque to the optimiser): values
// derived from it are recomputed where they are used instead of being held in
// registers across a loop.
__device__ __forceinline__ uint32_t lane_id_fresh() {
    uint32_t l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}
__device__ __forceinline__ uint32_t wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

}  // namespace la
