// Device helpers shared by the register-resident kernels (gfx950 matrix
// cores, packed-f16 complex arithmetic, lane maps of the 32 x 32 engine).
#pragma once

#include "fftconv_internal.h"

namespace fftconv {

typedef _Float16 rhalf8 __attribute__((ext_vector_type(8)));
typedef __bf16 rbf8 __attribute__((ext_vector_type(8)));
typedef float rfloat4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t pk_f16(float a, float b) {
    _Float16 h[2] = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, h);
}

template <int IO>
__device__ __forceinline__ uint32_t pk_io(float a, float b) {
    if (IO == IO_BF16) {
        __bf16 h[2] = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(uint32_t, h);
    }
    return pk_f16(a, b);
}

__device__ __forceinline__ rfloat4 mma_f16(uint4 a, uint4 b, rfloat4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(rhalf8, a), __builtin_bit_cast(rhalf8, b), c, 0, 0, 0);
}
__device__ __forceinline__ rfloat4 mma_bf16(uint4 a, uint4 b, rfloat4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(rbf8, a), __builtin_bit_cast(rbf8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float2 cmul2(float2 a, float2 b) {
    return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}

// a*z + b*conj(p)
__device__ __forceinline__ float2 pair2(float4 ab, float2 z, float2 p) {
    return make_float2(ab.x * z.x - ab.y * z.y + ab.z * p.x + ab.w * p.y,
                       ab.x * z.y + ab.y * z.x + ab.w * p.x - ab.z * p.y);
}

__device__ __forceinline__ int rmid_perm(int slot, int n) {
    return slot < (n >> 1) ? slot : (3 * n / 2 - 1 - slot);
}
__device__ __forceinline__ int kmap32(int kt, int x) {
    return kt == 0 ? x : (x == 0 ? 16 : 32 - x);
}
// n_b held by row y of tile t.  For NB = 32 the n_b digit uses the same
// mirror map as k_a, which makes the forward and inverse twiddle positions
// of every lane coincide (one register table, conjugated for the inverse).
template <int NB>
__device__ __forceinline__ int nbmap(int t, int y) {
    return NB == 32 ? kmap32(t, y) : 16 * t + y;
}

typedef _Float16 rhalf2 __attribute__((ext_vector_type(2)));
typedef __bf16 rbf2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk2(float a, float b) {
    rhalf2 v;
    v.x = (_Float16)a;
    v.y = (_Float16)b;
    uint32_t r = __builtin_bit_cast(uint32_t, v);
    // opaque to the optimiser: keeps the single packed conversion instead of
    // two scalar ones feeding half-selects of the following packed ops
    asm("" : "+v"(r));
    return r;
}
template <int IO>
__device__ __forceinline__ uint32_t pk2io(float a, float b) {
    if (IO == IO_BF16) {
        rbf2 v;
        v.x = (__bf16)a;
        v.y = (__bf16)b;
        return __builtin_bit_cast(uint32_t, v);
    }
    return pk2(a, b);
}

// Packed-f16 complex arithmetic (re in the low half, im in the high half).
// The operands of the next matrix product are f16 anyway; doing the twiddle
// and spectrum products in packed f16 halves their vector-ALU cost.
__device__ __forceinline__ rhalf2 as_h2(uint32_t v) { return __builtin_bit_cast(rhalf2, v); }
__device__ __forceinline__ uint32_t as_u32(rhalf2 v) { return __builtin_bit_cast(uint32_t, v); }
// d * t.  The swizzle is taken on the data, never on t: t is usually a
// loop-invariant twiddle, and a swizzled copy of it would be hoisted out of
// the loop into extra registers.
__device__ __forceinline__ rhalf2 hmul(rhalf2 d, rhalf2 t) {
    const rhalf2 txx = {t.x, t.x}, tyy = {t.y, t.y};
    const rhalf2 dn = {-d.y, d.x};
    return __builtin_elementwise_fma(dn, tyy, d * txx);
}
// d * conj(t)
__device__ __forceinline__ rhalf2 hmulc(rhalf2 d, rhalf2 t) {
    const rhalf2 txx = {t.x, t.x}, tyy = {t.y, t.y};
    const rhalf2 dn = {d.y, -d.x};
    return __builtin_elementwise_fma(dn, tyy, d * txx);
}
// a*z + b*conj(p); the swizzles are taken on the data (z, p), whose
// negated/swapped halves fold into the packed FMA's operand modifiers
__device__ __forceinline__ rhalf2 hpair(rhalf2 a, rhalf2 z, rhalf2 b, rhalf2 p) {
    const rhalf2 axx = {a.x, a.x}, ayy = {a.y, a.y};
    const rhalf2 bxx = {b.x, b.x}, byy = {b.y, b.y};
    const rhalf2 zn = {-z.y, z.x};   // i z
    const rhalf2 pc = {p.x, -p.y};   // conj(p)
    const rhalf2 pn = {p.y, p.x};    // i conj(p)
    rhalf2 r = __builtin_elementwise_fma(ayy, zn, axx * z);
    r = __builtin_elementwise_fma(bxx, pc, r);
    return __builtin_elementwise_fma(byy, pn, r);
}

// Gates (element-wise products with a second tensor of the I/O layout).
// u (.) w of two packed 16-bit I/O pairs, as packed f16: each product is
// exact in fp32 (or formed by the correctly rounded packed f16 multiply)
// and rounded once.
template <int IO>
__device__ __forceinline__ uint32_t gate_in(uint32_t u, uint32_t w) {
    if constexpr (IO == IO_BF16) {
        return pk2(__uint_as_float(u << 16) * __uint_as_float(w << 16),
                   __uint_as_float(u & 0xffff0000u) * __uint_as_float(w & 0xffff0000u));
    } else {
        return as_u32(as_h2(u) * as_h2(w));
    }
}
// the low and high values of a packed 16-bit I/O pair in fp32
template <int IO>
__device__ __forceinline__ float io_lo(uint32_t v) {
    if constexpr (IO == IO_BF16) return __uint_as_float(v << 16);
    else return (float)as_h2(v).x;
}
template <int IO>
__device__ __forceinline__ float io_hi(uint32_t v) {
    if constexpr (IO == IO_BF16) return __uint_as_float(v & 0xffff0000u);
    else return (float)as_h2(v).y;
}

// Exchange between 16-lane rows: the odd rows of a trade places with the
// even rows of c (rows 1 <-> 0 and 3 <-> 2).
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& c) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, c, false, false);
    a = r[0];
    c = r[1];
}

}  // namespace fftconv
