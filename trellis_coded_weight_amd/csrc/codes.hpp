// codes.hpp -- device-side computed codes and small shared helpers for the gfx950
// kernels.
//
// Computed codes follow QTIP blog, "The codebook is computed": an LCG of the L-bit
// state, then either the byte sum of the LCG output (1MAD) or an fp16 bit trick with
// one fp16 add (3INST; XOR-Trellis explainer, "The sign at each junction has to be
// cheap").  The final rescale is a binary64 division rounded once to binary32, so every
// code value is a fixed bit pattern.  The device multiplies by the binary64 reciprocal
// of the divisor instead of dividing: over the whole input domain of each code (byte
// sums 0..1020; every finite fp16 value) the product rounds to the same binary32 value
// as the quotient -- checked exhaustively on the host -- and it costs one fp64 multiply
// instead of an IEEE division sequence.  v_sad_u8 forms the byte sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qtcq {

enum : int { kCode1Mad = 0, kCode3Inst = 1 };

__device__ __forceinline__ uint32_t lcg_step(uint32_t x)
{
    return x * 34038481u + 76625530u;   // modulo 2^32
}

// Sum of the four bytes of u: v_sad_u8 accumulates |byte_i(u) - byte_i(0)|.
__device__ __forceinline__ uint32_t byte_sum(uint32_t u)
{
    return __builtin_amdgcn_sad_u8(u, 0u, 0u);
}

// 1MAD for a byte sum S in [0, 1020]: (S - 510) / 147.8 in binary64, then binary32.
__device__ __forceinline__ float mad_value_from_bytesum(uint32_t S)
{
    constexpr double kInv = 1.0 / 147.8;   // binary64 reciprocal of the binary64 divisor
    double q = (double)((int)S - 510) * kInv;
    return (float)q;
}

__device__ __forceinline__ float code_1mad(uint32_t x)
{
    return mad_value_from_bytesum(byte_sum(lcg_step(x)));
}

// 3INST raw value: the two fp16 halves of (u & 0x8FFF8FFF) ^ 0x3B603B60 added in fp16.
__device__ __forceinline__ _Float16 code_3inst_raw(uint32_t x)
{
    uint32_t v = (lcg_step(x) & 0x8FFF8FFFu) ^ 0x3B603B60u;
    _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
    _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
    return hi + lo;   // one fp16 add, round to nearest even
}

__device__ __forceinline__ float code_3inst(uint32_t x)
{
    constexpr double kInv = 1.0 / 1.244;
    double q = (double)(float)code_3inst_raw(x) * kInv;
    return (float)q;
}

template <int CODE>
__device__ __forceinline__ float code_value(uint32_t x)
{
    if constexpr (CODE == kCode1Mad)
        return code_1mad(x);
    else
        return code_3inst(x);
}

// Step error of the path cost: fl(fl(c - s)^2), optionally fl(w * that).  The build
// disables floating-point contraction, so these stay three separately rounded ops.
template <bool WEIGHTED>
__device__ __forceinline__ float step_err(float c, float s, float w)
{
    float d = c - s;
    float e = d * d;
    if constexpr (WEIGHTED) e = w * e;
    return e;
}

}  // namespace qtcq
