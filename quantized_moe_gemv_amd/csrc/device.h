// Device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace mq {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: branches on it are scalar branches, not exec-masked ones, so a
// load under such a branch never shares its destination registers with a
// masked write that would have to wait for it.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16, round to nearest even (finite values).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// c + a.lo*b.lo + a.hi*b.hi with bf16 pairs, fp32 accumulation.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                           false);
}

// (a & m) | c in one v_and_or_b32.  With constant m and c the compiler uses
// a VOP2 AND and a VOP2 OR with literals (gfx9 VOP3 takes no literal); OR-ed
// plus a zero it cannot see through, the constants live in vector registers
// (set once per kernel) and the compiler forms the VOP3.  The zero is the
// work-item's y index: every launch of this library is one-dimensional.
// (Inline assembly that writes a vector register is avoided on purpose: the
// compiler may give it a register that a matrix-core operation still in
// flight is about to write.)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
    const uint32_t z = __builtin_amdgcn_workitem_id_y();
    return (a & (m + z)) | (c + z);
}

// Pair m (m = 0..3) of a DEV_V1 4-bit word as two bf16 values 128 + q:
// the nibbles of columns 2m and 2m+1 sit at bits 4m and 16 + 4m, and OR-ing
// them under the exponent of 128.0 (0x4300) gives 128 + q exactly.
__device__ __forceinline__ uint32_t q4_pair(uint32_t w, int m) {
    return and_or(m ? w >> (4 * m) : w, 0x000F000Fu, 0x43004300u);
}

// The eight codes of a DEV_V1 4-bit word as eight bf16 operands 128 + q, in
// column order (pair m holds columns 2m and 2m + 1).
__device__ __forceinline__ bf16x8_t codes8_bf16(uint32_t w) {
    u32x4_t v;
#pragma unroll
    for (int m = 0; m < 4; ++m) v[m] = q4_pair(w, m);
    return __builtin_bit_cast(bf16x8_t, v);
}

// Partial dots of one lane over one 4-bit DEV_V1 block: rows 16*ms + lane%16
// (ms = 0..3), over the lane's 16 columns 32*ks + 8*(lane/16) + 0..7.
// xa, xb: the lane's x values for ks = 0 and 1 as bf16 pairs.
// Adds sum((128 + q) * x) of row ms to d[ms].
__device__ __forceinline__ void q4_block_dot(const uint4& c0, const uint4& c1, const uint4& xa, const uint4& xb,
                                             float d[4]) {
    const uint32_t w[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const uint32_t xk[2][4] = {{xa.x, xa.y, xa.z, xa.w}, {xb.x, xb.y, xb.z, xb.w}};
#pragma unroll
    for (int a = 0; a < 8; ++a) {
#pragma unroll
        for (int m = 0; m < 4; ++m) d[a >> 1] = dot2_bf16(q4_pair(w[a], m), xk[a & 1][m], d[a >> 1]);
    }
}

// True when an fp16 value is inf or NaN (all exponent bits set): the
// conversion of an activation overflowed fp16's range (|v| >= 65520) or the
// value was already NaN.
__device__ __forceinline__ bool f16_bad(_Float16 h) {
    return (__builtin_bit_cast(uint16_t, h) & 0x7C00u) == 0x7C00u;
}

// Records kErrRange-type errors in the sticky error word (rare path only).
__device__ __forceinline__ void flag_error(uint32_t* err, bool bad, uint32_t bit) {
    if (__builtin_expect(bad, 0)) atomicOr(err, bit);
}

// Cross-lane sums without the LDS crossbar.  A ds_bpermute (what a shuffle
// compiles to) is an LDS round trip; these take VALU data-parallel
// primitives (DPP) and gfx950's permlane swaps instead.  Each step pairs
// the same lanes as the xor butterfly it replaces, and lane i and its
// partner add the same two values (IEEE addition commutes), so every sum
// keeps the bits of the butterfly:
//   xor 1, xor 2: quad_perm [1,0,3,2] and [2,3,0,1];
//   xor 8 within a 16-lane row: row_ror:8;
//   xor 4: row_ror:4 once the values already agree across xor 8 (lane i
//     then reads lane i+4 mod 16, which holds the value of lane i^4), or
//     row_half_mirror once they agree within each quad (quad 0 <-> 1);
//   xor 16, xor 32: v_permlane16_swap / v_permlane32_swap of the value with
//     itself, which hands back the two halves of each pair.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128, kDppHalfMirror = 0x141,
              kDppShl1 = 0x101;

// v + v[lane ^ 16]
__device__ __forceinline__ float add_xor16(float v) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// v + v[lane ^ 32]
__device__ __forceinline__ float add_xor32(float v) {
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Sum over the 64 lanes of a wave (butterfly xor 32, 16, 8, 4, 2, 1).
__device__ __forceinline__ float wave_sum(float v) {
    v = add_xor32(v);
    v = add_xor16(v);
    v += dpp_f<kDppRor8>(v);
    v += dpp_f<kDppRor4>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppXor1>(v);
    return v;
}

// Sum over the 16 lanes lane / 16 * 16 + 0..15 of a wave (xor 1, 2, 4, 8).
__device__ __forceinline__ float sum16(float v) {
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppRor8>(v);
    return v;
}

// Sum over the four lanes lane%16 + 16*kb (kb = 0..3) of a wave (xor 16, 32).
__device__ __forceinline__ float sum_kb(float v) {
    v = add_xor16(v);
    v = add_xor32(v);
    return v;
}
// The same sum through the LDS crossbar (ds_bpermute), for kernels that
// measured faster with it; the bits are the same.
__device__ __forceinline__ float sum_kb_bpermute(float v) {
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

// Integer sum over the 4 (or, with EIGHT, 8) lanes of each aligned group.
template <bool EIGHT>
__device__ __forceinline__ int group_sum_i(int v) {
    v += dpp_i<kDppXor1>(v);
    v += dpp_i<kDppXor2>(v);
    if constexpr (EIGHT) v += dpp_i<kDppHalfMirror>(v);
    return v;
}

// v of lane + 1 within the lane's 16-lane row (lane 15 of a row reads 0).
__device__ __forceinline__ uint32_t next_lane_in_row(uint32_t v) {
    return (uint32_t)dpp_i<kDppShl1>((int)v);
}

__device__ __forceinline__ float gelu_tanh(float z) {
    const float k = 0.7978845608028654f;   // sqrt(2/pi)
    return 0.5f * z * (1.0f + tanhf(k * (z + 0.044715f * z * z * z)));
}

// The eight codes of a DEV_V1 4-bit word as eight fp16 operands, with four
// AND-ORs under the fp16 exponent of 1024.0 (0x6400): columns c = 0, 1, 4, 5
// of the eight come out as 1024 + q (the code in the low mantissa bits),
// columns 2, 3, 6, 7 as 1024 + 16 q (the code four bits higher).  An
// activation operand that holds the columns with (c & 2) != 0 divided by 16
// (an exact power-of-two step) then gives, over a group of 64 columns with
// a_c the stored activations,
//     sum_c code_c a_c = sum_c q_c x_c + 1024 sum_c a_c.
__device__ __forceinline__ half8_t codes8(uint32_t w) {
    const uint32_t t = w >> 8, e = 0x64006400u;
    u32x4_t v;
    v[0] = and_or(w, 0x000F000Fu, e);
    v[1] = and_or(w, 0x00F000F0u, e);
    v[2] = and_or(t, 0x000F000Fu, e);
    v[3] = and_or(t, 0x00F000F0u, e);
    return __builtin_bit_cast(half8_t, v);
}

// 16-byte streaming load (non-temporal: the weights are read once per call).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

}  // namespace mq
