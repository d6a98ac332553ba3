// bcjr.hpp -- BCJR soft relaxation on the bitshift trellis, gfx950.
//
// BCJR-QAT abstract: replace the Viterbi argmax by the forward-backward sum-product
// recursion at temperature tau; the soft codeword is the Boltzmann expectation of the
// reconstructed value over trellis walks, weight exp(-E / tau) with E the search's path
// cost.  Start state uniform (plain trellis), so the recursion is the Viterbi one with
// (min, +) replaced by (log-sum-exp, +).
//
// Log2 domain, kappa = log2(e) / tau.  Forward messages per group (a group m = j >> 2
// shares its predecessors, as in the search):
//     A_t[(c, x)] = LSE2_a( A_{t-1}[(a, c)] - kappa e_{t-1}((a, c, x)) ),   A_0 = 0,
// backward messages per low-(L-2)-bit group:
//     B_{t-1}[(a, c)] = LSE2_x( B_t[(c, x)] - kappa e_t((a, c, x)) ),       B_{T-1} = 0.
// The same 16 states (a, c, x) and code values serve both directions, so the thread
// mapping and the LDS chunk swizzle are the search kernel's (viterbi.hpp).
//
// Precision.  A message accumulates one rounding per step; in fp32 at tau = 0.01 the
// per-step increments (kappa e ~ 10 log2 units) make those roundings ~1e-6 each, which
// over ~250 steps shifts competing walks' weights by ~1e-5.  So messages are stored and
// combined in fp64: each state's energy term is formed in fp64 from the binary32 inputs
// (shifted by a per-step constant that cancels, StepEnergy), each LSE's four inputs stay
// in fp64 (the candidate that wins once its energy term is added can sit far below the
// largest input, so a reduced-precision difference from that input would carry its
// rounding into the winner), the LSE's max and differences are fp64, and only exp2 /
// log2 of small arguments run in fp32.
// Messages live in one fp64 LDS buffer (128 KiB at L = 16): each step reads all its
// inputs, barrier, writes all outputs, barrier.
// Normalisation: stored X_t = A_t - G_{t-1}; the next step subtracts g_t = max X_t
// (from per-wave maxima) and G accumulates the g's, likewise h/H for the backward.
// Stash: while step t + 1 reads X_t it also writes Xn_t = X_t - g_t = A_t - G_t (every
// value <= 0, the maximum just below 0) to HBM in 32 bits (to_fix): fixed point with a
// uniform 2.4e-7 log2 resolution down to -1024, binary32 of the distance below -1024
// further down.  Plain fp32 would lose precision on the moderately negative values that
// still matter once the backward message is added.
// Posterior at t: gamma_t(j) = 2^( la_t(j) + lb_t(j) - log2 Z ), computed in the backward
// sweep from the stashed Xn_t[(a, c)], the normalised backward input Yn_t[(c, x)] =
// Y_t - h_t and the step energy, with the exact offset O_t = log2 Z - G_t - H_t.  The
// four states (a, c, x), x = 0..3, are the inputs of one backward LSE, so their
// posteriors reuse its exponentials: one more exp2 per group instead of four.
// soft_t = sum gamma C / sum gamma: per-wave partial sums per step go to the
// workspace, a small kernel divides.
// VJP mode (for the gradient kernel, bcjr_vjp.hpp) also stashes Yn_t in the same
// fixed point and O_t in binary64.
#pragma once

#include "codes.hpp"
#include "viterbi.hpp"


namespace qtcq {

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// fp64 maximum of two values that are never NaN (plain v_max_f64, without the
// canonicalising moves the compiler adds for IEEE maxnum on loaded values)
__device__ __forceinline__ double max64(double a, double b)
{
    double r;
    asm("v_max_f64 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// log2(2^v0 + 2^v1 + 2^v2 + 2^v3) with the max and the differences in fp64.
__device__ __forceinline__ double lse2_4(double v0, double v1, double v2, double v3)
{
    const double m = max64(max64(v0, v1), max64(v2, v3));
    const float s = (fast_exp2((float)(v0 - m)) + fast_exp2((float)(v1 - m))) +
                    (fast_exp2((float)(v2 - m)) + fast_exp2((float)(v3 - m)));
    return m + (double)fast_log2(s);
}

// Reductions over the first WIDTH lanes of a wave (WIDTH = min(threads, 64)).
template <int WIDTH>
__device__ __forceinline__ float wave_max(float x)
{
#pragma unroll
    for (int off = WIDTH / 2; off >= 1; off >>= 1) x = __builtin_fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

template <int WIDTH>
__device__ __forceinline__ double wave_max64(double x)
{
#pragma unroll
    for (int off = WIDTH / 2; off >= 1; off >>= 1) x = max64(x, __shfl_xor(x, off, 64));
    return x;
}

template <int WIDTH>
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = WIDTH / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// The smallest binary32 value above x (x itself for +inf and NaN).  The per-step
// normalisers are binary32 maxima of fp64 messages; rounding each wave's maximum up once
// makes the normaliser an upper bound of every message of its step, so a normalised
// message X - g is <= 0 exactly (fp64 subtraction keeps the sign), however large |X| is.
__host__ __device__ __forceinline__ float next_up(float x)
{
    if (!(x < __builtin_inff())) return x;
    if (x == 0.0f) return __builtin_bit_cast(float, 1u);
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    return __builtin_bit_cast(float, x > 0.0f ? b + 1u : b - 1u);
}

// Stash values (normalised messages, <= 0 since the normaliser rounds up) in 32 bits:
//   v >= -1024: 2^31 + rint(v 2^21) -- units of 2^-21 log2, codes 0 .. 2^31: a uniform
//               2.4e-7 resolution near the step's maximum, where a posterior term depends
//               on it;
//   v <  -1024: the binary32 bit pattern of v + 1024, a negative float (codes above
//               2^31) -- an absolute precision of 2^-24 (-1024 - v), continuous with the
//               fixed point at the boundary and fp32's relative precision far below it.
// Far below the maximum a state can still matter at low temperature: its backward
// message can lift it back, so the tail keeps finite, smoothly degrading values rather
// than a clamp.  Decoding gives v + kStashShift with a single conversion in either range
// (from_fix_shifted); every caller folds the constant into an offset it subtracts anyway
// or into a log-sum-exp, which a common shift leaves unchanged -- an explicit add here
// costs the backward loops their register allocation.
constexpr double kFixScale = 2097152.0;
constexpr double kStashShift = 1024.0;
// Encoded without a branch.  For v in [-1024, 0] the sum t = v + (1.5 2^31 + 2^10) lies in
// [1.5 2^31, 1.5 2^31 + 2^10], where a binary64 unit in the last place is 2^-21, and the
// constant is a multiple of 2^-21: the single rounding of the sum is the constant plus
// rint(v 2^21) 2^-21 (ties to even, the constant's last place being even).  The low word
// of t is then 2^31 + rint(v 2^21) (its mantissa is 2^51 + 2^31 + rint(v 2^21)).  Both
// codes are formed and one is selected.
__host__ __device__ __forceinline__ int to_fix(double v)
{
    const double t = v + (0x1.8p31 + 0x1p10);
    const uint32_t fixed = (uint32_t)__builtin_bit_cast(uint64_t, t);
    const uint32_t tail = __builtin_bit_cast(uint32_t, (float)(v + kStashShift));
    return (int)(v >= -1024.0 ? fixed : tail);
}
__host__ __device__ __forceinline__ double from_fix_shifted(int q)
{
    const uint32_t u = (uint32_t)q;
    if (u <= 0x80000000u) return (double)u * (1.0 / kFixScale);
    return (double)__builtin_bit_cast(float, u);
}
// the code of 0 (= to_fix(0.0))
constexpr int kFixZero = (int)0x80000000u;
// the value itself (reference form; the kernels use from_fix_shifted)
__host__ __device__ __forceinline__ double from_fix(int q) { return from_fix_shifted(q) - kStashShift; }

// The wide stash of gradient mode at low temperature keeps the fp64 values themselves:
// there a state whose forward message is thousands of log2 units below the step's
// maximum can be lifted back by its backward message, where the 32-bit form keeps only
// fp32 resolution.  StashVal<WIDE> is the stored type and its value.
template <bool WIDE> struct StashVal;
// The soft pass itself always reads the 32-bit form (so the soft codeword of a gradient
// call is the soft pass's bit for bit at every temperature); the wide copy is written
// alongside it for the gradient sweep.
// get() returns the value plus kShift (the 32-bit form's decode, from_fix_shifted).
template <> struct StashVal<false> {
    using T = int;
    static constexpr int kZero = kFixZero;   // the stored form of 0
    static constexpr double kShift = kStashShift;
    __device__ static double get(int q) { return from_fix_shifted(q); }
};
template <> struct StashVal<true> {
    using T = double;
    static constexpr double kZero = 0.0;
    static constexpr double kShift = 0.0;
    __device__ static double get(double v) { return v; }
};

// Forward stash Xn_t[(a, 4 tid + r)], t = 1..T-1, at step index i = t - 1.  The soft pass
// keeps [i][a][tid] int4 (r = 0..3); in VJP mode the layout is [i][a][h][tid] int2
// (r = 2h, 2h + 1) so that the gradient kernel, which works on one half of a thread's
// butterflies at a time, reads it lane-contiguously.
template <int NT, bool VJP>
__device__ __forceinline__ void xn_store(int* st, size_t i, int a, int tid, int4 v)
{
    if constexpr (VJP) {
        int2* p = reinterpret_cast<int2*>(st);
        p[((i * 4 + a) * 2 + 0) * NT + tid] = make_int2(v.x, v.y);
        p[((i * 4 + a) * 2 + 1) * NT + tid] = make_int2(v.z, v.w);
    } else {
        reinterpret_cast<int4*>(st)[(i * 4 + a) * NT + tid] = v;
    }
}

// the wide stash: [i][a][h][tid] double2 (r = 2h, 2h + 1)
template <int NT>
__device__ __forceinline__ void xn_store_wide(char* st, size_t i, int a, int tid, const double (&v)[4])
{
    double2* p = reinterpret_cast<double2*>(st);
    p[((i * 4 + a) * 2 + 0) * NT + tid] = make_double2(v[0], v[1]);
    p[((i * 4 + a) * 2 + 1) * NT + tid] = make_double2(v[2], v[3]);
}

template <int NT, bool VJP>
__device__ __forceinline__ int4 xn_load(const int* st, size_t i, int a, int tid)
{
    if constexpr (VJP) {
        const int2* p = reinterpret_cast<const int2*>(st);
        const int2 lo = p[((i * 4 + a) * 2 + 0) * NT + tid];
        const int2 hi = p[((i * 4 + a) * 2 + 1) * NT + tid];
        return make_int4(lo.x, lo.y, hi.x, hi.y);
    } else {
        return reinterpret_cast<const int4*>(st)[(i * 4 + a) * NT + tid];
    }
}

// Longest sequence the BCJR kernels take (the entry points reject longer ones): per-step
// scalars (the forward normalisers, the soft codeword) are staged in LDS.
constexpr int kBcjrMaxT = 4096;

template <int L>
struct BcjrLayout {
    using Tr = Trellis<L>;
    static constexpr int kWaves = (Tr::kThreads + 63) / 64;
    // Per-sequence workspace, each part 256-byte aligned:
    //   log2 Z (double) | posterior partial sums [T][kWaves][2]
    //   | stash Xn_1..Xn_{T-1} (groups (a, 4 tau + r): see xn_store)
    // and in VJP mode, after those:
    //   | the same Xn in fp64 (the wide stash of low temperatures: xn_store_wide; unused
    //     otherwise)
    //   | Yn_0..Yn_{T-1} ([T][4][kThreads] int4: groups (4 tau + r, x), x = 0..3, at
    //     [r][tau]; wide: [T][4][2][kThreads] double2, x = 2 hh, 2 hh + 1 at [r][hh][tau])
    //     | O_0..O_{T-1} (double) | Phi_0..Phi_{T-1} ([T][4][2][kThreads] float2: groups
    //     (a, 4 tau + 2h + i), i = 0, 1, at [a][h][tau]) | gradient partial sums
    //     [T][kWaves][4] (float)
    __host__ __device__ static size_t up(size_t b) { return (b + 255) / 256 * 256; }
    __host__ __device__ static size_t off_part(int) { return 256; }
    __host__ __device__ static size_t off_stash(int T) { return off_part(T) + up((size_t)T * kWaves * 8); }
    __host__ __device__ static size_t bytes_per_seq(int T) { return off_stash(T) + up((size_t)(T - 1) * Tr::kGroups * 4); }
    __host__ __device__ static size_t off_xwide(int T) { return bytes_per_seq(T); }
    __host__ __device__ static size_t off_ystash(int T) { return off_xwide(T) + up((size_t)(T - 1) * Tr::kGroups * 8); }
    __host__ __device__ static size_t off_ofs(int T) { return off_ystash(T) + up((size_t)T * Tr::kGroups * 8); }
    __host__ __device__ static size_t off_phi(int T) { return off_ofs(T) + up((size_t)T * 8); }
    __host__ __device__ static size_t off_vpart(int T) { return off_phi(T) + up((size_t)T * Tr::kGroups * 4); }
    __host__ __device__ static size_t bytes_per_seq_vjp(int T) { return off_vpart(T) + up((size_t)T * kWaves * 16); }
};

// fp64 message buffer: a chunk = 4 consecutive groups = 32 bytes, stored as two 16-byte
// halves in separate planes so that a wave's 16-byte accesses stay lane-contiguous.
// Planes are P bytes apart inside blocks of 2P bytes, P <= 32 KiB, so the second half
// is reached through the DS instruction's immediate offset.
template <int L>
struct BcjrLds {
    static constexpr int NB = Trellis<L>::kButterflies;   // chunks per message vector
    static constexpr int kPerBlock = NB < 2048 ? NB : 2048;
    static constexpr int P = kPerBlock * 16;
    static constexpr int kBytes = NB * 32;
    __device__ static int addr(int g)   // g = swizzled chunk index
    {
        return (g / kPerBlock) * 2 * P + (g % kPerBlock) * 16;
    }
};

// A wave-uniform double kept in two SGPRs (the running normalisation sums would
// otherwise occupy VGPR pairs for the whole sweep).
__device__ __forceinline__ double uniform64(double x)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// float -> double, emitted at every use: keeps the compiler from hoisting sixteen
// widened copies (32 registers) out of the inner loops.
__device__ __forceinline__ double widen(float f)
{
    double d;
    asm volatile("v_cvt_f64_f32 %0, %1" : "=v"(d) : "v"(f));
    return d;
}

// The log2-domain energy term of a state at one step, shifted by the state-independent
// kappa w s^2:
//     -kappa w (C - s)^2 + kappa w s^2 = C (2 kappa w s - kappa w C),
// two fp64 FMAs on the exactly widened code value (instead of the exact binary64 square
// and one FMA with kappa: one operation fewer per state).  All states of a step get the
// same shift, so it cancels in every LSE and in every posterior and gradient weight
// (normalised within a step, or formed with log2 Z computed from the same shifted
// energies); only log Z itself is corrected, by the sum of the shifts.
struct StepEnergy {
    double kw;   // kappa * w_t
    double a2;   // 2 kappa w_t s_t
    // (2 s is formed first: a loop-invariant 2 kappa would be kept in, and spilled from,
    // a VGPR pair)
    __device__ __forceinline__ StepEnergy(double kappa, float s, float w)
        : kw(kappa * (double)w), a2(kappa * (double)w * (2.0 * (double)s)) {}
    // x + shifted energy term of code value c
    __device__ __forceinline__ double add_to(float c, double x) const
    {
        const double cd = widen(c);
        return __builtin_fma(cd, __builtin_fma(-kw, cd, a2), x);
    }
    // the shift kappa w s^2 itself
    __device__ __forceinline__ double shift(float s) const { return kw * (double)s * (double)s; }
};

__device__ __forceinline__ void lds_read4(const char* base, int addr, int P, double (&v)[4])
{
    const double2 lo = *reinterpret_cast<const double2*>(base + addr);
    const double2 hi = *reinterpret_cast<const double2*>(base + addr + P);
    v[0] = lo.x; v[1] = lo.y; v[2] = hi.x; v[3] = hi.y;
}

__device__ __forceinline__ void lds_write4(char* base, int addr, int P, double v0, double v1,
                                           double v2, double v3)
{
    *reinterpret_cast<double2*>(base + addr) = make_double2(v0, v1);
    *reinterpret_cast<double2*>(base + addr + P) = make_double2(v2, v3);
}

// The code values of a thread's 64 states (a, c = 4 tid + r, x) held as their raw values
// (1MAD: S - 510, an integer of magnitude below 2^10; 3INST: the fp16 sum; the XOR
// palette values -- all exact in fp16), two per register, and rescaled at each use (code_rescale: the same bits as
// code_value).  The widening is written as an instruction so that it stays at its use:
// hoisted out of a step loop, the 64 decoded values would need 64 registers again.
template <int L, int CODE>
struct PackedCodes {
    uint32_t w[4][4][2];   // [a][r][x >> 1], x even in the low half

    // OPAQUE: the raw code of a state is the same function here as in the forward
    // prologue; an opaque index keeps the compiler from carrying the prologue's values
    // across the forward loop (spilled) instead of recomputing them.  Needed for the cheap
    // palette code, and wherever the forward loop holds more registers.
    template <bool OPAQUE = (CODE == kCodeXor)>
    __device__ __forceinline__ void init(int tid, const CodeArg& ca)
    {
        constexpr int M = Trellis<L>::kGroups;
        if constexpr (OPAQUE) tid = keep(tid);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int hx = 0; hx < 2; ++hx) {
                    const uint32_t j = (uint32_t)(a * M + 16 * tid + 4 * r + 2 * hx);
                    const float lo = code_raw<CODE>(j, ca), hi = code_raw<CODE>(j + 1, ca);
                    w[a][r][hx] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
                    if constexpr (CODE == kCodeXor) w[a][r][hx] = keep(w[a][r][hx]);
                    __builtin_amdgcn_sched_barrier(0);
                }
    }

    __device__ __forceinline__ float at(int a, int r, int x) const
    {
        float f;
        if (x & 1)
            asm volatile("v_cvt_f32_f16_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1"
                         : "=v"(f) : "v"(w[a][r][x >> 1]));
        else
            asm volatile("v_cvt_f32_f16 %0, %1" : "=v"(f) : "v"(w[a][r][x >> 1]));
        return code_rescale<CODE>(f);
    }
};

inline size_t bcjr_bytes_per_seq(int T, int L, bool vjp = false)
{
    switch (L) {
    case 6: return vjp ? BcjrLayout<6>::bytes_per_seq_vjp(T) : BcjrLayout<6>::bytes_per_seq(T);
    case 8: return vjp ? BcjrLayout<8>::bytes_per_seq_vjp(T) : BcjrLayout<8>::bytes_per_seq(T);
    case 10: return vjp ? BcjrLayout<10>::bytes_per_seq_vjp(T) : BcjrLayout<10>::bytes_per_seq(T);
    case 12: return vjp ? BcjrLayout<12>::bytes_per_seq_vjp(T) : BcjrLayout<12>::bytes_per_seq(T);
    case 14: return vjp ? BcjrLayout<14>::bytes_per_seq_vjp(T) : BcjrLayout<14>::bytes_per_seq(T);
    default: return vjp ? BcjrLayout<16>::bytes_per_seq_vjp(T) : BcjrLayout<16>::bytes_per_seq(T);
    }
}

// grid.x = sequences in the chunk; block = Trellis<L>::kThreads.  ws points at the
// chunk's workspace, bytes_per_seq(T) (VJP: bytes_per_seq_vjp(T)) per sequence.
// kappa = log2(e) / tau.
// WIDE (VJP only): the stashes hold fp64 values (StashVal).
template <int L, int CODE, bool WEIGHTED, bool VJP = false, bool WIDE = false>
__global__ void __launch_bounds__(Trellis<L>::kThreads)
bcjr_sweep(const float* __restrict__ seq, const float* __restrict__ wts, int T, int64_t b0,
           double kappa, char* __restrict__ ws, CodeArg ca)
{
    static_assert(VJP || !WIDE, "the wide stash is a gradient-mode layout");
    using Tr = Trellis<L>;
    using Ly = BcjrLayout<L>;
    using Ld = BcjrLds<L>;
    constexpr int NT = Tr::kThreads;
    constexpr int M = Tr::kGroups;
    constexpr int kWaves = Ly::kWaves;
    constexpr int WID = NT < 64 ? NT : 64;
    constexpr int P = Ld::P;
    __shared__ __align__(16) char buf[Ld::kBytes];
    __shared__ float wmax[2][kWaves];
    __shared__ double redm[kWaves];
    __shared__ float reds[kWaves];
    __shared__ float gsh[kBcjrMaxT];   // the forward normalisers g_0 .. g_{T-1}

    const int tid = threadIdx.x;
    // the wave index in an SGPR: kept in a VGPR across the step loops it would be spilled
    // and reloaded (an exposed scratch read) at every per-wave store
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int64_t row = b0 + blockIdx.x;
    const float* s = seq + row * T;
    const float* w = WEIGHTED ? wts + row * T : nullptr;
    char* base = ws + (size_t)blockIdx.x * (VJP ? Ly::bytes_per_seq_vjp(T) : Ly::bytes_per_seq(T));
    double* l2z = reinterpret_cast<double*>(base);
    float* part = reinterpret_cast<float*>(base + Ly::off_part(T));
    int* stash = reinterpret_cast<int*>(base + Ly::off_stash(T));
    char* stash_w = base + Ly::off_xwide(T);                               // WIDE only
    int4* ystash = reinterpret_cast<int4*>(base + Ly::off_ystash(T));     // VJP only
    double* ofs = reinterpret_cast<double*>(base + Ly::off_ofs(T));        // VJP only

    float Cv[4][4][4];   // code value of state (a, c = 4 tid + r, x), one at a time
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                Cv[a][r][x] = code_value_prologue<CODE>((uint32_t)(a * M + 16 * tid + 4 * r + x), ca);
                if constexpr (CODE == kCodeXor) Cv[a][r][x] = keep(Cv[a][r][x]);
                __builtin_amdgcn_sched_barrier(0);
            }

    // byte addresses of the chunks (a, 4tid..4tid+3) and (4tid+r, 0..3).  With at least
    // 64 threads (L >= 12) the chunk swizzle leaves a * NT alone, so chunk (a, 4tid + ..)
    // is at rb + addr(a * NT), a compile-time offset, and chunk (4tid + r, ..) at wb XOR 16 r
    // (r flips the two low chunk bits, which are bits 4 and 5 of the byte address).  The two
    // bases are derived once per step from an opaque copy of the thread index (derive),
    // so they are never live across steps and the compiler cannot hoist eight
    // loop-invariant addresses out of the step loops (they would be spilled).  Without
    // the split (smaller workgroups, or instantiations whose registers are full) each
    // address is recomputed at its use from an opaque copy of the thread index.
    // (The split costs registers across a step: the weighted gradient-mode forward would
    // spill with it, and so would every weighted or gradient-mode backward with the write
    // base, which stays live over the step; the backward's read base is used at once.)
    constexpr bool kSplitFwd = NT >= 64 && !(WEIGHTED && VJP);
    constexpr bool kSplitBwdRd = NT >= 64;
    constexpr bool kSplitBwd = NT >= 64 && !WEIGHTED && !VJP;
    auto opaque_tid = [&]() {
        int v = tid;
        asm volatile("v_mov_b32 %0, %0" : "+v"(v));
        return v;
    };
    using FwdSplit = std::integral_constant<bool, kSplitFwd>;
    using BwdSplit = std::integral_constant<bool, kSplitBwd>;
    using BwdRdSplit = std::integral_constant<bool, kSplitBwdRd>;
    int rb = 0, wb = 0;
    // derive(split): only where the phase uses the bases (no dead opaque copy otherwise)
    auto derive = [&](auto split) {
        if constexpr (decltype(split)::value) {
            const int t = opaque_tid();
            rb = Ld::addr(lds_chunk(t));
            wb = Ld::addr(lds_chunk(4 * t));
        }
    };
    auto rd_at = [&](int a, auto split) {
        if constexpr (decltype(split)::value) return rb + Ld::addr(a * NT);
        else return Ld::addr(lds_chunk(a * NT + opaque_tid()));
    };
    auto wr_at = [&](int r, auto split) {
        if constexpr (decltype(split)::value) return wb ^ (16 * r);
        else return Ld::addr(lds_chunk(4 * opaque_tid() + r));
    };
    auto rd = [&](int a) { return rd_at(a, FwdSplit{}); };
    auto wr = [&](int r) { return wr_at(r, FwdSplit{}); };
    auto rdb = [&](int a) { return rd_at(a, BwdSplit{}); };
    auto wrb_rd = [&](int r) { return wr_at(r, BwdRdSplit{}); };   // the backward's reads
    auto wrb = [&](int r) { return wr_at(r, BwdSplit{}); };

    auto step_energy = [&](int t) { return StepEnergy(kappa, s[t], WEIGHTED ? w[t] : 1.0f); };

    // ---------------- forward ----------------
    derive(FwdSplit{});
#pragma unroll
    for (int r = 0; r < 4; ++r) lds_write4(buf, wr(r), P, 0.0, 0.0, 0.0, 0.0);
    if (tid < kWaves) wmax[0][tid] = 0.f;
    __syncthreads();

    double G = 0.0;    // sum of g_0 .. g_{t-1}
    double Sh = 0.0;   // sum of the energy shifts kappa w s^2 of the steps so far
    int par = 0;
    for (int t = 1; t < T; ++t) {
        derive(FwdSplit{});
        float g = wmax[par][0];
#pragma unroll
        for (int q = 1; q < kWaves; ++q) g = __builtin_fmaxf(g, wmax[par][q]);
        const double g64 = (double)g;
        // Inputs of butterfly 4 tid + r, normalised: X_{t-1}[(a, 4 tid + r)] - g, a = 0..3,
        // held in fp64.  The candidate that wins an LSE once its energy term is added can be
        // any of the four (at low temperature or large energies, often one far below the
        // others), so every input keeps full precision.
        double xn[4][4];    // [a][r]
        {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                lds_read4(buf, rd(a), P, xn[a]);
#pragma unroll
                for (int r = 0; r < 4; ++r) xn[a][r] -= g64;
                // Xn_{t-1}[(a, 4 tid + r)] (Xn_0 = 0 is not stored)
                if (t >= 2) {
                    xn_store<NT, VJP>(stash, (size_t)(t - 2), a, tid,
                                      make_int4(to_fix(xn[a][0]), to_fix(xn[a][1]),
                                                to_fix(xn[a][2]), to_fix(xn[a][3])));
                    if constexpr (WIDE) xn_store_wide<NT>(stash_w, (size_t)(t - 2), a, tid, xn[a]);
                }
            }
        }
        __syncthreads();   // every input read before any output overwrites it
        G = uniform64(G + g64);
        if (tid == 0) gsh[t - 1] = g;
        const StepEnergy se = step_energy(t - 1);
        Sh = uniform64(Sh + se.shift(s[t - 1]));
        float lmax = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {        // output pairs x = 2h, 2h + 1
                double o[2];
#pragma unroll
                for (int xx = 0; xx < 2; ++xx) {
                    const int x = 2 * h + xx;
                    double v[4];
#pragma unroll
                    for (int a = 0; a < 4; ++a)
                        v[a] = se.add_to(Cv[a][r][x], xn[a][r]);
                    o[xx] = lse2_4(v[0], v[1], v[2], v[3]);
                    lmax = __builtin_fmaxf(lmax, (float)o[xx]);
                }
                *reinterpret_cast<double2*>(buf + wr(r) + h * P) = make_double2(o[0], o[1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        lmax = wave_max<WID>(lmax);
        if (lane == 0) wmax[par ^ 1][wave] = next_up(lmax);
        par ^= 1;
        __syncthreads();
    }

    // log2 Z = G_{T-1} + LSE2_j( X_{T-1}[j >> 2] - g_{T-1} - kappa e_{T-1}(j) ), in two
    // passes (maximum, then the sum of powers) to keep registers low
    float gl = wmax[par][0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) gl = __builtin_fmaxf(gl, wmax[par][q]);
    G = uniform64(G + (double)gl);
    if (tid == 0) gsh[T - 1] = gl;
    double log2z;
    {
        derive(FwdSplit{});
        const StepEnergy se = step_energy(T - 1);
        Sh = uniform64(Sh + se.shift(s[T - 1]));
        const double gl64 = (double)gl;
        double m = -__builtin_inf();
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            double xa[4];
            lds_read4(buf, rd(a), P, xa);
            if (T >= 2) {   // Xn_{T-1}
                const double xw[4] = {xa[0] - gl64, xa[1] - gl64, xa[2] - gl64, xa[3] - gl64};
                xn_store<NT, VJP>(stash, (size_t)(T - 2), a, tid,
                                  make_int4(to_fix(xw[0]), to_fix(xw[1]), to_fix(xw[2]), to_fix(xw[3])));
                if constexpr (WIDE) xn_store_wide<NT>(stash_w, (size_t)(T - 2), a, tid, xw);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    m = max64(m, se.add_to(Cv[a][r][x], xa[r] - gl64));
        }
        // the exact fp64 maximum (once per sequence): a binary32-rounded one can sit
        // hundreds of log2 units below the largest term once the messages reach ~1e10,
        // and its power of two would overflow
        const double wm = wave_max64<WID>(m);
        if (lane == 0) redm[wave] = wm;
        __syncthreads();
        double bm64 = redm[0];
#pragma unroll
        for (int qq = 1; qq < kWaves; ++qq) bm64 = max64(bm64, redm[qq]);
        float sum = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            double xa[4];
            lds_read4(buf, rd(a), P, xa);
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int x = 0; x < 4; ++x)
                    sum += fast_exp2((float)(se.add_to(Cv[a][r][x], xa[r] - gl64) - bm64));
        }
        sum = wave_sum<WID>(sum);
        if (lane == 0) reds[wave] = sum;
        __syncthreads();   // also: every read of X_{T-1} done before the buffer is reused
        float tot = 0.f;
#pragma unroll
        for (int qq = 0; qq < kWaves; ++qq) tot += reds[qq];
        // log2 Z of the shifted energies (what the posterior offsets use), and the true one
        log2z = uniform64(G + bm64 + (double)fast_log2(tot));
        if (tid == 0) l2z[0] = log2z - Sh;
    }

    // ---------------- backward + posterior ----------------
    // The backward keeps more values live per step (the stash and the posterior sums), so
    // it holds the code values packed (PackedCodes): 32 registers instead of 64, which
    // keeps the step loop free of spills.
    PackedCodes<L, CODE> Ch;
    Ch.template init<CODE == kCodeXor || kSplitFwd>(tid, ca);
    // Y_{T-1} = 0
    derive(BwdSplit{});
#pragma unroll
    for (int r = 0; r < 4; ++r) lds_write4(buf, wrb(r), P, 0.0, 0.0, 0.0, 0.0);
    if (tid < kWaves) wmax[par][tid] = 0.f;
    __syncthreads();

    double Gm = G;     // G_t at the top of iteration t
    double H = 0.0;    // H_{t+1} at the top of iteration t
    // One backward step at t (t >= 1 produces Y_{t-1}); the posterior of step t is
    // accumulated on the way.  At t = 0 only the posterior is formed (X_0 = 0).
    auto bstep = [&](int t, bool produce) {
        derive(BwdRdSplit{});
        // Xn_t[(a, 4 tid + r)], r = 0..3, from the stash (Xn_0 = 0), prefetched one a
        // ahead; the first before the step's LDS reads and barrier
        auto stash_at = [&](int a) -> int4 {
            if (!produce) return make_int4(kFixZero, kFixZero, kFixZero, kFixZero);
            return xn_load<NT, VJP>(stash, (size_t)(t - 1), a, tid);
        };
        int4 xs_next = stash_at(0);
        float h = wmax[par][0];
#pragma unroll
        for (int q = 1; q < kWaves; ++q) h = __builtin_fmaxf(h, wmax[par][q]);
        const double h64 = (double)h;
        // inputs Y_t[(4 tid + r, x)] - h, x = 0..3, in fp64 (as forward)
        double yn[4][4];    // [r][x]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            lds_read4(buf, wrb_rd(r), P, yn[r]);
#pragma unroll
            for (int x = 0; x < 4; ++x) yn[r][x] -= h64;
            if constexpr (VJP && WIDE) {   // Yn_t[(4 tid + r, x)]
                double2* yw = reinterpret_cast<double2*>(ystash);
                yw[(((size_t)t * 4 + r) * 2 + 0) * NT + tid] = make_double2(yn[r][0], yn[r][1]);
                yw[(((size_t)t * 4 + r) * 2 + 1) * NT + tid] = make_double2(yn[r][2], yn[r][3]);
            } else if constexpr (VJP) {
                ystash[((size_t)t * 4 + r) * NT + tid] =
                    make_int4(to_fix(yn[r][0]), to_fix(yn[r][1]), to_fix(yn[r][2]), to_fix(yn[r][3]));
            }
        }
        if (produce) __syncthreads();   // every input read before any output overwrites it
        H = uniform64(H + h64);                       // H_t
        const double Ot = uniform64(log2z - Gm - H);  // log2 Z - G_t - H_t
        if (VJP && tid == 0) ofs[t] = Ot;
        const double OtS = uniform64(Ot + kStashShift);   // the stash decodes Xn + kStashShift
        Gm = uniform64(Gm - (double)gsh[t]);          // G_{t-1}
        const StepEnergy se = step_energy(t);
        float pg = 0.f, pc = 0.f;
        double ymax = -__builtin_inf();   // fp64 maximum, rounded to binary32 once below
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int4 xs = xs_next;
            if (a < 3) xs_next = stash_at(a + 1);
            asm volatile("" ::: "memory");    // no further hoisting of stash loads
            const int xsr[4] = {xs.x, xs.y, xs.z, xs.w};
#pragma unroll
            for (int h = 0; h < 2; ++h) {        // output pairs r = 2h, 2h + 1
                double y[2];
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const int r = 2 * h + rr;
                    float cx[4];
                    double v[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        cx[x] = Ch.at(a, r, x);
                        v[x] = se.add_to(cx[x], yn[r][x]);
                    }
                    // LSE over x (as lse2_4), whose exponentials q_x = 2^(v_x - m) also give
                    // the posterior of the four states (a, c, x): with the exponent
                    // X_t - O_t + (Y_t - h_t) - kappa e_t = xo + v_x, each is 2^(xo + m) q_x
                    const double m = max64(max64(v[0], v[1]), max64(v[2], v[3]));
                    float q[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) q[x] = fast_exp2((float)(v[x] - m));
                    const float sq = (q[0] + q[1]) + (q[2] + q[3]);
                    float qc = q[0] * cx[0];
#pragma unroll
                    for (int x = 1; x < 4; ++x) qc = __builtin_fmaf(q[x], cx[x], qc);
                    const double xo = from_fix_shifted(xsr[r]) - OtS;
                    const float pb = fast_exp2((float)(xo + m));
                    pg = __builtin_fmaf(pb, sq, pg);
                    pc = __builtin_fmaf(pb, qc, pc);
                    if (produce) {
                        y[rr] = m + (double)fast_log2(sq);
                        ymax = max64(ymax, y[rr]);
                    }
                }
                if (produce) *reinterpret_cast<double2*>(buf + rdb(a) + h * P) = make_double2(y[0], y[1]);
                __builtin_amdgcn_sched_barrier(0);   // bound live ranges
            }
        }
        pg = wave_sum<WID>(pg);
        pc = wave_sum<WID>(pc);
        if (lane == 0) {
            part[((size_t)t * kWaves + wave) * 2 + 0] = pg;
            part[((size_t)t * kWaves + wave) * 2 + 1] = pc;
        }
        if (produce) {
            // rounding is monotonic: the same value as the maximum of the rounded messages
            const float ymax32 = wave_max<WID>((float)ymax);
            if (lane == 0) wmax[par ^ 1][wave] = next_up(ymax32);
            par ^= 1;
            __syncthreads();
        }
    };
    for (int t = T - 1; t >= 1; --t) bstep(t, true);
    bstep(0, false);
}

// soft[b][t] = (sum_waves pc) / (sum_waves pg); log_z = ln 2 * log2 Z.  stride: the
// workspace bytes per sequence (bytes_per_seq or bytes_per_seq_vjp).
template <int L>
__global__ void __launch_bounds__(256)
bcjr_finalize(const char* __restrict__ ws, size_t stride, int T, int64_t n, int64_t b0,
              float* __restrict__ soft, float* __restrict__ logz)
{
    using Ly = BcjrLayout<L>;
    constexpr int kWaves = Ly::kWaves;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * T) return;
    const int64_t i = idx / T;
    const int t = (int)(idx - i * T);
    const char* base = ws + (size_t)i * stride;
    const float* part = reinterpret_cast<const float*>(base + Ly::off_part(T));
    float pg = 0.f, pc = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
        pg += part[((size_t)t * kWaves + q) * 2 + 0];
        pc += part[((size_t)t * kWaves + q) * 2 + 1];
    }
    if (soft) soft[(b0 + i) * T + t] = pc / pg;
    if (logz && t == 0) {
        const double l2z = *reinterpret_cast<const double*>(base);
        logz[b0 + i] = (float)(l2z * 0.69314718055994530942);
    }
}

}  // namespace qtcq
