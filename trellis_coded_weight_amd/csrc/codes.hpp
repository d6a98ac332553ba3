// codes.hpp -- device-side computed codes and small shared helpers for the gfx950
// kernels.
//
// Computed codes follow QTIP blog, "The codebook is computed": an LCG of the L-bit
// state, then either the byte sum of the LCG output (1MAD) or an fp16 bit trick with
// one fp16 add (3INST; XOR-Trellis explainer, "The sign at each junction has to be
// cheap").  The final rescale is a binary64 division rounded once to binary32, so every
// code value is a fixed bit pattern.  The device gets the same bits with binary32 work
// only: v * (1/D) is split as v * r_hi + v * r_lo, where r_hi (13 significant bits)
// makes v * r_hi exact and one FMA adds v * r_lo with a single rounding.  Over the whole
// input domain of each code (byte sums 0..1020; every finite fp16 value below 4 in
// magnitude) this rounds to the same binary32 value as the binary64 quotient -- checked
// exhaustively on the host with exact rational arithmetic.  The LCG product uses a 24-bit
// multiply-add and a shift-add (states have at most 24 bits), and v_sad_u8 forms the
// byte sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qtcq {

enum : int { kCode1Mad = 0, kCode3Inst = 1 };

// LCG of a state x < 2^24: (34038481 x + 76625530) mod 2^32.  The multiplier is
// 2^25 + 484049, so one 24-bit multiply-add forms 484049 x + 76625530 and one shift-add
// adds x << 25; both are exact modulo 2^32.  Both constants are VGPR operands (an SGPR
// operand halves a VALU op's issue rate here).
// (Written as instructions: the compiler would fold the two back into one 32-bit
// v_mul_lo_u32, a multi-pass instruction.)
__device__ __forceinline__ uint32_t lcg_step(uint32_t x)
{
    uint32_t lo, u;
    asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(lo) : "v"(x), "v"(484049u), "v"(76625530u));
    asm("v_lshl_add_u32 %0, %1, 25, %2" : "=v"(u) : "v"(x), "v"(lo));
    return u;
}

// Binary32 split of 1/147.8 and 1/1.244 (the binary64 divisors): r_hi has 13 significant
// bits, r_lo = fl32(1/D - r_hi).
constexpr float k1MadRhi = 0x1.bb7p-8f;        // 0x3BDDB800
constexpr float k1MadRlo = -0x1.c2569ap-22f;    // 0xB4E12B4D
constexpr float k3InstRhi = 0x1.9b9p-1f;        // 0x3F4DC800
constexpr float k3InstRlo = 0x1.ac09ep-16f;     // 0x37D604F0

// fl32(v / D) for the code's domain: v * r_hi is exact, the FMA rounds once.
__device__ __forceinline__ float rescale(float v, float rhi, float rlo)
{
    return __builtin_fmaf(v, rlo, v * rhi);
}

// 1MAD before the rescale: S - 510 (exact) for the byte sum S of u.  v_sad_u8 adds the
// byte sum to an accumulator whose bits are those of the float 2^23 + 514, so the sum
// reads as the float 2^23 + 514 + S exactly, and one exact subtraction gives S - 510.
__device__ __forceinline__ float code_1mad_raw(uint32_t x)
{
    constexpr uint32_t kBias = 0x4B000000u + 514u;   // float 8389122.0
    const uint32_t t = __builtin_amdgcn_sad_u8(lcg_step(x), 0u, kBias);
    return __builtin_bit_cast(float, t) - 8389632.0f;   // 2^23 + 1024
}

// 1MAD: (S - 510) / 147.8
__device__ __forceinline__ float code_1mad(uint32_t x)
{
    return rescale(code_1mad_raw(x), k1MadRhi, k1MadRlo);
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
    return rescale((float)code_3inst_raw(x), k3InstRhi, k3InstRlo);
}

// The same values in the form the search kernels compute once per workgroup: the
// 32-bit LCG product and the rescale by the binary64 reciprocal of the divisor (which
// rounds to the same binary32 value as the binary64 quotient on the same domains, also
// checked exhaustively on the host).  Their cost does not matter there, and with this
// form the step loops keep their register allocation (no spills).
template <int CODE>
__device__ __forceinline__ float code_value_prologue(uint32_t x)
{
    const uint32_t u = x * 34038481u + 76625530u;
    if constexpr (CODE == kCode1Mad) {
        const int n = (int)__builtin_amdgcn_sad_u8(u, 0u, 0u) - 510;
        return (float)((double)n * (1.0 / 147.8));
    } else {
        const uint32_t v = (u & 0x8FFF8FFFu) ^ 0x3B603B60u;
        const _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
        const _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
        const _Float16 h = hi + lo;   // one fp16 add, round to nearest even
        return (float)((double)(float)h * (1.0 / 1.244));
    }
}

// The code before its rescale (exact in binary32), and the rescale itself:
// code_value(x) = code_rescale(code_raw(x)) bit for bit.
template <int CODE>
__device__ __forceinline__ float code_raw(uint32_t x)
{
    if constexpr (CODE == kCode1Mad)
        return code_1mad_raw(x);
    else
        return (float)code_3inst_raw(x);
}

template <int CODE>
__device__ __forceinline__ float code_rescale(float v)
{
    if constexpr (CODE == kCode1Mad)
        return rescale(v, k1MadRhi, k1MadRlo);
    else
        return rescale(v, k3InstRhi, k3InstRlo);
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
