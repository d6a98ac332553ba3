// viterbi.hpp -- Viterbi encoding on the bitshift trellis, gfx950.
//
// Trellis (QTIP blog, "The trellis: a stateful codebook"): 2^L states; j may follow i
// iff the top L-2 bits of j equal the bottom L-2 bits of i (k = 2), i.e. the state is
// a sliding L-bit window and the predecessors of j are (j >> 2) | (a << (L-2)),
// a = 0..3.  The search keeps the cheapest cost into every state and a backpointer per
// state and step, then reads the best walk back.
//
// Group structure used here (a consequence of the predecessor rule): the four states
// j = 4m + x (x = 0..3) share the same predecessor set {m + a*2^(L-2)}, so one 4-way
// minimum per group m serves four states, and the backpointer is per group.  With
// mu_t[m] = min_a cost_{t-1}[m + a*2^(L-2)] the recursion becomes
//     mu_t[(c << 2) | x] = min_a ( mu_{t-1}[(a << (L-4)) | c] + e_{t-1}((a, c, x)) )
// where c is an (L-4)-bit "butterfly" index and (a, c, x) the L-bit state
// (a << (L-2)) | (c << 2) | x: butterfly c reads 4 group minima and writes 4, touching
// 16 states.  The cost vector itself (2^L floats) is never stored: cost_{t-1}[i] =
// mu_{t-1}[i >> 2] + e_{t-1}(i) is rebuilt on the fly from the 2^(L-2) minima.
//
// Kernel layout (L = 16): one workgroup of 1024 threads (16 wave64) per sequence, one
// sequence per CU.  Thread tau owns butterflies c = 4*tau + r (r = 0..3): its 64 code
// values C[(a, c, x)] are computed once and live in VGPRs for the whole sequence.  The
// group minima (64 KiB) live in LDS, double-buffered (128 KiB of the 160 KiB); one
// barrier per step.  Reads are one ds_read_b128 per a (groups (a, 4*tau .. 4*tau+3)),
// writes one ds_write_b128 per r (groups (c, 0..3)); an XOR swizzle of the 16-byte
// chunk index keeps both patterns free of bank conflicts.  Each thread emits its 16
// groups' 2-bit argmins as one uint32 per step (coalesced 4 KiB per step per sequence
// to HBM).  Ties: strict comparisons keep the lowest a (the lowest predecessor), the
// final argmin keeps the lowest state.  Arithmetic: fl(fl(C - s)^2) [* w], then
// fl(mu + e) -- contraction is disabled at build time.
#pragma once

#include "codes.hpp"

namespace qtcq {

template <int L>
struct Trellis {
    static_assert(L >= 6 && L <= 16 && (L % 2) == 0, "k = 2 trellis with even 6 <= L <= 16");
    static constexpr int kStates = 1 << L;
    static constexpr int kGroups = kStates >> 2;        // predecessor sets, 2^(L-2)
    static constexpr int kButterflies = kGroups >> 2;   // 2^(L-4)
    static constexpr int kThreads = kButterflies / 4;   // 4 butterflies per thread
    static constexpr int kChunks = kGroups / 4;         // float4 chunks of a group vector
    // uint32 backpointer words per step: 16 groups x 2 bits per thread
    static constexpr int kBpWords = kThreads;
};

// XOR swizzle of a float4 chunk index: bits [3:0] ^= bits [5:2].  Bijective; makes
// both the read pattern (16 consecutive chunks per 16 lanes) and the write pattern
// (every 4th chunk per lane) hit 16 distinct chunk slots.
__device__ __forceinline__ int lds_chunk(int g)
{
    return g ^ ((g >> 2) & 15);
}

// A wave-uniform value copied into a VGPR (opaque to the compiler, so it is not folded
// back into an SGPR operand).
__device__ __forceinline__ float to_vgpr(float x)
{
    float v;
    asm("v_mov_b32 %0, %1" : "=v"(v) : "s"(x));
    return v;
}

// word * 2 + (this lane's bit of mask): one v_addc_co_u32 with the lane mask as the
// carry-in (the compiler would otherwise select, shift and OR).  All lanes of the wave
// must be active.
__device__ __forceinline__ uint32_t shift_in_bit(uint32_t word, uint64_t mask)
{
    uint32_t out;
    uint64_t carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(out), "=s"(carry_out) : "v"(word), "s"(mask));
    return out;
}

// Forward pass.  grid.x = number of sequences in the chunk, block = Trellis<L>::kThreads.
//   seq, wts : [*][T] (rows b0 .. b0 + gridDim.x - 1 are processed)
//   bp       : [gridDim.x][T-1][kBpWords] 2-bit argmins of each step
//   fin      : [gridDim.x] final state (uint32) ; fin_cost [gridDim.x]
//   mse      : [*] (row b0 + blockIdx.x) or nullptr
template <int L, int CODE, bool WEIGHTED>
__global__ void __launch_bounds__(Trellis<L>::kThreads)
viterbi_forward(const float* __restrict__ seq, const float* __restrict__ wts, int T, int64_t b0,
                uint32_t* __restrict__ bp, uint32_t* __restrict__ fin, float* __restrict__ fin_cost,
                float* __restrict__ mse)
{
    using Tr = Trellis<L>;
    constexpr int NB = Tr::kButterflies;
    constexpr int M = Tr::kGroups;
    __shared__ float4 mu[2][Tr::kChunks];

    const int tid = threadIdx.x;
    const int64_t row = b0 + blockIdx.x;
    const float* s = seq + row * T;
    const float* w = WEIGHTED ? wts + row * T : nullptr;
    uint32_t* bp_seq = bp + (int64_t)blockIdx.x * (T - 1) * Tr::kBpWords;

    // this thread's code values: state (a, c, x) = a*M + 16*tid + 4*r + x
    float Cv[4][4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int x = 0; x < 4; ++x)
                Cv[a][r][x] = code_value<CODE>((uint32_t)(a * M + 16 * tid + 4 * r + x));

    int rd[4], wr[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) rd[a] = lds_chunk(a * (NB / 4) + tid);   // groups (a, 4tid..4tid+3)
#pragma unroll
    for (int r = 0; r < 4; ++r) wr[r] = lds_chunk(4 * tid + r);          // groups (4tid+r, 0..3)

    // mu_0 = +0 everywhere, so cost_0 = fl(0 + e_0) = e_0
#pragma unroll
    for (int r = 0; r < 4; ++r) mu[0][wr[r]] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();

    // one ACS step: group minima of step t-1 in `src` -> group minima of step t in `dst`
    auto step = [&](int t, const float4* __restrict__ src, float4* __restrict__ dst) {
        // the step's target (and weight) are wave-uniform; keeping them in VGPRs lets
        // the sub/mul/add below issue as 2-operand VGPR ops, which gfx950 issues twice
        // as fast as ops reading an SGPR
        const float sp = to_vgpr(s[t - 1]);
        const float wp = WEIGHTED ? to_vgpr(w[t - 1]) : 1.0f;
        float in[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            float4 v = src[rd[a]];
            in[a][0] = v.x; in[a][1] = v.y; in[a][2] = v.z; in[a][3] = v.w;
        }
        uint32_t word = 0;
        float out[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                float v[4];
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    v[a] = in[a][r] + step_err<WEIGHTED>(Cv[a][r][x], sp, wp);
                const float m = __builtin_fminf(__builtin_fminf(v[0], v[1]), __builtin_fminf(v[2], v[3]));
                // lowest a attaining the minimum: 0 if v0 == m, else 1 if v1 == m, else
                // 2 if v2 == m, else 3.  The two bits are shifted in with add-with-carry
                // (word + word + bit), the compare masks serving as carries.
                const uint64_t n0 = __builtin_amdgcn_ballot_w64(v[0] != m);
                const uint64_t e1 = __builtin_amdgcn_ballot_w64(v[1] == m);
                const uint64_t n2 = __builtin_amdgcn_ballot_w64(v[2] != m);
                word = shift_in_bit(word, n0 & ~e1);          // a >= 2
                word = shift_in_bit(word, n0 & (e1 | n2));    // a odd
                out[r][x] = m;
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r)
            dst[wr[r]] = make_float4(out[r][0], out[r][1], out[r][2], out[r][3]);
        bp_seq[(int64_t)(t - 1) * Tr::kBpWords + tid] = word;
        __syncthreads();
    };

    // unrolled by two so that both buffers' LDS addresses stay loop-invariant
    int t = 1;
    for (; t + 1 < T; t += 2) {
        step(t, mu[0], mu[1]);
        step(t + 1, mu[1], mu[0]);
    }
    int cur = 0;
    if (t < T) {
        step(t, mu[0], mu[1]);
        cur = 1;
    }

    // final costs cost_{T-1}(i) = mu_{T-1}[i >> 2] + e_{T-1}(i); lowest i wins ties
    {
        const float sp = to_vgpr(s[T - 1]);
        const float wp = WEIGHTED ? to_vgpr(w[T - 1]) : 1.0f;
        float best = __builtin_inff();
        uint32_t bi = 0xFFFFFFFFu;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            float4 v = mu[cur][rd[a]];
            float in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    float c = in[r] + step_err<WEIGHTED>(Cv[a][r][x], sp, wp);
                    if (c < best) {   // states visited in increasing order
                        best = c;
                        bi = (uint32_t)(a * M + 16 * tid + 4 * r + x);
                    }
                }
        }
        // wave reduction of (best, bi), lexicographic, over the lanes that exist
        constexpr int kWidth = Tr::kThreads < 64 ? Tr::kThreads : 64;
#pragma unroll
        for (int off = kWidth / 2; off >= 1; off >>= 1) {
            float ob = __shfl_xor(best, off, 64);
            uint32_t oi = __shfl_xor(bi, off, 64);
            if (ob < best || (ob == best && oi < bi)) { best = ob; bi = oi; }
        }
        constexpr int kWaves = (Tr::kThreads + 63) / 64;
        if constexpr (kWaves > 1) {
            __shared__ float wbest[kWaves];
            __shared__ uint32_t wbi[kWaves];
            if ((tid & 63) == 0) { wbest[tid >> 6] = best; wbi[tid >> 6] = bi; }
            __syncthreads();
            if (tid == 0) {
                for (int q = 1; q < kWaves; ++q)
                    if (wbest[q] < best || (wbest[q] == best && wbi[q] < bi)) { best = wbest[q]; bi = wbi[q]; }
            }
        }
        if (tid == 0) {
            fin[blockIdx.x] = bi;
            fin_cost[blockIdx.x] = best;
            if (mse) mse[row] = best / (float)T;
        }
    }
}

// Traceback and pack.  One thread per sequence of the chunk: walks the backpointers
// from the final state to t = 0 and writes the stream (start state's L bits, then the
// 2 new bits of every later state, MSB first) and optionally the states.
template <int L>
__global__ void __launch_bounds__(256)
viterbi_traceback(const uint32_t* __restrict__ bp, const uint32_t* __restrict__ fin, int T,
                  int64_t n, int64_t b0, int W, uint32_t* __restrict__ bits,
                  uint32_t* __restrict__ states)
{
    using Tr = Trellis<L>;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t* bpq = bp + i * (int64_t)(T - 1) * Tr::kBpWords;
    uint32_t* out = bits + (b0 + i) * W;
    uint32_t* st = states ? states + (b0 + i) * (int64_t)T : nullptr;

    uint32_t j = fin[i];
    const int nbits = L + 2 * (T - 1);
    int curw = (nbits - 1) >> 5;
    uint32_t acc = 0;
    for (int t = T - 1; t >= 1; --t) {
        if (st) st[t] = j;
        const int p = L + 2 * (t - 1);              // stream position of st[t]'s new bits
        const int wi = p >> 5;
        if (wi != curw) { out[curw] = acc; curw = wi; acc = 0; }
        acc |= (j & 3u) << (30 - (p & 31));
        const uint32_t m = j >> 2;                   // group of j's predecessors
        const uint32_t word = bpq[(int64_t)(t - 1) * Tr::kBpWords + (m >> 4)];
        const uint32_t a = (word >> (30 - 2 * (m & 15))) & 3u;
        j = m | (a << (L - 2));
    }
    if (st) st[0] = j;
    if (curw != 0) { out[curw] = acc; acc = 0; }
    acc |= j << (32 - L);
    out[0] = acc;
}

}  // namespace qtcq
