// codes.hpp -- device-side computed codes and small shared helpers for the gfx950
// kernels.
//
// Computed codes follow QTIP blog, "The codebook is computed": an LCG of the L-bit
// state, then either the byte sum of the LCG output (1MAD) or an fp16 bit trick with
// one fp16 add (3INST; XOR-Trellis explainer, "The sign at each junction has to be
// cheap").  The XOR-Trellis palette code (same explainer and section) reads four masked
// parities of the state's history bits: two pick one of four printed FP4 palettes, two
// permute which branch takes which entry (see code_xor).  The final rescale of 1MAD and
// 3INST is a binary64 division rounded once to binary32, so every code value is a fixed
// bit pattern.  The device gets the same bits with binary32 work
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

enum : int { kCode1Mad = 0, kCode3Inst = 1, kCodeXor = 2 };

// Run-time parameters of a code, passed by value to every kernel: the four parity masks
// of the XOR-Trellis palette code (unused by 1MAD and 3INST).
struct CodeArg {
    uint32_t m[4];
};

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

// The same LCG in three instructions, the multiplier split as 519 * 2^16 + 25297 (two
// 24-bit multiplies with SGPR constants, then a shift-add); the same values.  The fp32
// VALU product of the 1MAD code at eight batch rows, whose loop is mostly FMAs, runs
// faster with this form (measured on MI355X); elsewhere the two-instruction form is.
__device__ __forceinline__ uint32_t lcg_step_split(uint32_t x)
{
    uint32_t lo, hi;
    asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(lo) : "v"(x), "s"(25297u), "v"(76625530u));
    asm("v_mul_u32_u24 %0, %1, %2" : "=v"(hi) : "s"(519u), "v"(x));
    return lo + (hi << 16);
}

template <bool SPLIT>
__device__ __forceinline__ uint32_t lcg(uint32_t x)
{
    if constexpr (SPLIT)
        return lcg_step_split(x);
    else
        return lcg_step(x);
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
template <bool SPLIT = false>
__device__ __forceinline__ float code_1mad_raw(uint32_t x)
{
    constexpr uint32_t kBias = 0x4B000000u + 514u;   // float 8389122.0
    const uint32_t t = __builtin_amdgcn_sad_u8(lcg<SPLIT>(x), 0u, kBias);
    return __builtin_bit_cast(float, t) - 8389632.0f;   // 2^23 + 1024
}

// 1MAD: (S - 510) / 147.8
__device__ __forceinline__ float code_1mad(uint32_t x)
{
    return rescale(code_1mad_raw(x), k1MadRhi, k1MadRlo);
}

// 3INST raw value: the two fp16 halves of (u & 0x8FFF8FFF) ^ 0x3B603B60 added in fp16.
template <bool SPLIT = false>
__device__ __forceinline__ _Float16 code_3inst_raw(uint32_t x)
{
    uint32_t v = (lcg<SPLIT>(x) & 0x8FFF8FFFu) ^ 0x3B603B60u;
    _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
    _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu));
    return hi + lo;   // one fp16 add, round to nearest even
}

__device__ __forceinline__ float code_3inst(uint32_t x)
{
    return rescale((float)code_3inst_raw(x), k3InstRhi, k3InstRlo);
}

// XOR-Trellis palette code of an L-bit state x (L <= 16): the newest k = 2 bits are the
// branch b = x & 3 and the L - 2 bits above them the branch history h = x >> 2.  Four
// parities p_i = parity(h & m_i) of masked history bits give the palette index
// 2 p_0 + p_1 and the shuffle 2 p_2 + p_3, which is XORed into the branch to pick the
// entry.  The four successors of a state share its low history bits, hence the palette
// and the shuffle, so their values are the four distinct entries of one palette.  The
// palettes hold the FP4 values [-6, -1.5, 0, 2], [-4, -1, 0.5, 3], [-3, -0.5, 1, 4] and
// [-2, 0, 1.5, 6], used as they are (exact in fp16 and binary32; a per-group scale of
// the weights lies outside the trellis).  Here each value is stored doubled as a signed
// byte, palette p in the four bytes of one 32-bit constant, entry e in byte e.
constexpr uint32_t kXorPaletteTwice[4] = {
    0x0400FDF4u,   // 2 x [-6, -1.5, 0, 2]
    0x0601FEF8u,   // 2 x [-4, -1, 0.5, 3]
    0x0802FFFAu,   // 2 x [-3, -0.5, 1, 4]
    0x0C0300FCu,   // 2 x [-2, 0, 1.5, 6]
};

__device__ __forceinline__ float code_xor(uint32_t x, const CodeArg& ca)
{
    const uint32_t h = x >> 2;
    const uint32_t p = ((__builtin_popcount(h & ca.m[0]) & 1u) << 1) | (__builtin_popcount(h & ca.m[1]) & 1u);
    const uint32_t sh = ((__builtin_popcount(h & ca.m[2]) & 1u) << 1) | (__builtin_popcount(h & ca.m[3]) & 1u);
    const uint32_t e = (x & 3u) ^ sh;
    const uint32_t d01 = (p & 1u) ? kXorPaletteTwice[1] : kXorPaletteTwice[0];
    const uint32_t d23 = (p & 1u) ? kXorPaletteTwice[3] : kXorPaletteTwice[2];
    const uint32_t d = (p & 2u) ? d23 : d01;
    const int twice = (int)(d << (24u - 8u * e)) >> 24;          // byte e, sign-extended
    return (float)twice * 0.5f;
}

// fp16 bits of twice / 2 for a small integer twice (the palette values: exact in fp16)
constexpr uint32_t f16_of_half(int twice)
{
    if (twice == 0) return 0u;
    const uint32_t sign = twice < 0 ? 0x8000u : 0u;
    const uint32_t a = (uint32_t)(twice < 0 ? -twice : twice);
    int e = 0;
    while ((a >> (e + 1)) != 0u) ++e;                 // a in [2^e, 2^(e+1))
    return sign | ((uint32_t)(e - 1 + 15) << 10) | ((a - (1u << e)) << (10 - e));
}
// entries 2 w and 2 w + 1 of XOR palette p as an fp16 pair (entry 2 w in the low half)
constexpr uint32_t xor_pal_pair_f16(int p, int w)
{
    const uint32_t d = kXorPaletteTwice[p];
    const int e0 = (int)(int8_t)(uint8_t)(d >> (16 * w)), e1 = (int)(int8_t)(uint8_t)(d >> (16 * w + 8));
    return f16_of_half(e0) | (f16_of_half(e1) << 16);
}
static_assert(xor_pal_pair_f16(0, 0) == 0xBE00C600u && xor_pal_pair_f16(3, 1) == 0x46003E00u,
              "fp16 palette pairs");

// The XOR palette code of every L-bit state as fp16 (the palette values themselves) in
// table[0 .. 2^(L-1)) words, state x in half x, written by threads tid = 0 .. nthreads - 1
// together.  Per history h, the four states 4 h + b at once: palette 2 p0 + p1 as two
// fp16 pairs, entry b taking palette entry b XOR (2 s0 + s1) -- s1 swaps the halves of
// each pair, s0 swaps the pairs -- stored as 8 bytes.  The same values as code_xor.
template <int L>
__device__ __forceinline__ void xor_table_f16(uint32_t* table, const CodeArg& ca, int tid, int nthreads)
{
    for (int h = tid; h < (1 << (L - 2)); h += nthreads) {
        const uint32_t hh = (uint32_t)h;
        const bool p0 = __builtin_popcount(hh & ca.m[0]) & 1, p1 = __builtin_popcount(hh & ca.m[1]) & 1;
        const bool s0 = __builtin_popcount(hh & ca.m[2]) & 1, s1 = __builtin_popcount(hh & ca.m[3]) & 1;
        const uint32_t lo = p0 ? (p1 ? xor_pal_pair_f16(3, 0) : xor_pal_pair_f16(2, 0))
                               : (p1 ? xor_pal_pair_f16(1, 0) : xor_pal_pair_f16(0, 0));
        const uint32_t hi = p0 ? (p1 ? xor_pal_pair_f16(3, 1) : xor_pal_pair_f16(2, 1))
                               : (p1 ? xor_pal_pair_f16(1, 1) : xor_pal_pair_f16(0, 1));
        const uint32_t lo1 = s1 ? __builtin_amdgcn_alignbit(lo, lo, 16) : lo;
        const uint32_t hi1 = s1 ? __builtin_amdgcn_alignbit(hi, hi, 16) : hi;
        *reinterpret_cast<uint2*>(&table[2 * h]) = make_uint2(s0 ? hi1 : lo1, s0 ? lo1 : hi1);
    }
}

// Fourth word of a raw (unstructured, stride 0) buffer descriptor on gfx9-family chips:
// DATA_FORMAT = 32 bits, no swizzle, no index, so the range check compares each byte
// offset against the descriptor's size and an access past it returns zero.
constexpr int kRawBufferWord3 = 0x00020000;

// A value the compiler must keep as computed: it may not recompute it later from its
// inputs (which, for the cheap palette code, it would otherwise do inside the step loops,
// at the cost of the registers of the inputs and constants).
template <typename V>
__device__ __forceinline__ V keep(V v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// The same values in the form the search kernels compute once per workgroup: the
// 32-bit LCG product and the rescale by the binary64 reciprocal of the divisor (which
// rounds to the same binary32 value as the binary64 quotient on the same domains, also
// checked exhaustively on the host).  Their cost does not matter there, and with this
// form the step loops keep their register allocation (no spills).
template <int CODE>
__device__ __forceinline__ float code_value_prologue(uint32_t x, const CodeArg& ca)
{
    const uint32_t u = x * 34038481u + 76625530u;
    if constexpr (CODE == kCodeXor) {
        return code_xor(x, ca);
    } else if constexpr (CODE == kCode1Mad) {
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

// The code before its rescale (exact in binary32 and fp16), and the rescale itself:
// code_value(x) = code_rescale(code_raw(x)) bit for bit.  The palette values need no
// rescale.
// SPLIT: the LCG in its three-instruction form (lcg_step_split); the same values
template <int CODE, bool SPLIT = false>
__device__ __forceinline__ float code_raw(uint32_t x, const CodeArg& ca)
{
    if constexpr (CODE == kCode1Mad)
        return code_1mad_raw<SPLIT>(x);
    else if constexpr (CODE == kCode3Inst)
        return (float)code_3inst_raw<SPLIT>(x);
    else
        return code_xor(x, ca);
}

template <int CODE>
__device__ __forceinline__ float code_rescale(float v)
{
    if constexpr (CODE == kCode1Mad)
        return rescale(v, k1MadRhi, k1MadRlo);
    else if constexpr (CODE == kCode3Inst)
        return rescale(v, k3InstRhi, k3InstRlo);
    else
        return v;
}

template <int CODE>
__device__ __forceinline__ float code_value(uint32_t x, const CodeArg& ca)
{
    if constexpr (CODE == kCode1Mad)
        return code_1mad(x);
    else if constexpr (CODE == kCode3Inst)
        return code_3inst(x);
    else
        return code_xor(x, ca);
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
