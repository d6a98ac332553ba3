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
// sequence per CU.  Thread tau owns butterflies c = tau + r*NT (r = 0..3, NT = 1024
// threads): its 64 code values C[(a, c, x)] are computed once and live in VGPRs for the
// whole sequence.  The group minima (64 KiB) live in LDS, double-buffered (128 KiB of
// the 160 KiB); one barrier per step.  For each r the thread reads its four inputs
// (a, c), a = 0..3, as lane-contiguous ds_read_b32 and writes its four outputs (c, x),
// x = 0..3, as one lane-contiguous ds_write_b128 as soon as they are computed, so LDS
// traffic overlaps the arithmetic and no access pattern has bank conflicts.  Each
// thread emits its 16 groups' 2-bit argmins as one uint32 per step (coalesced 4 KiB
// per step per sequence to HBM).  Ties: strict comparisons keep the lowest a (the
// lowest predecessor), the final argmin keeps the lowest state.  Arithmetic:
// fl(fl(C - s)^2) [* w], then fl(mu + e) -- contraction is disabled at build time.
//
// Issue-rate notes (gfx950, measured): v_add/v_sub/v_mul_f32 with VGPR or constant
// operands issue at two wave64 instructions per CU cycle, while compares, min/min3,
// add-with-carry and any instruction reading an SGPR issue at one; hence the per-step
// target is copied into a VGPR and the argmin uses the fewest slow instructions
// (min3 + min, three compares, two add-with-carry per group of four candidates).
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
    // backpointer field of group m = 4c + x, c = tau + r*kThreads: word tau, field 4r + x
    __host__ __device__ static int bp_word(uint32_t m) { return (int)((m >> 2) % kThreads); }
    __host__ __device__ static int bp_shift(uint32_t m)
    {
        return 30 - 2 * (int)(4 * ((m >> 2) / kThreads) + (m & 3));
    }
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

// groups between a group's compares and the add-with-carry that packs its bits
constexpr int kBitDelay = 1;

// Forward pass over a pair of sequences per workgroup (or one, for batches that fit in
// one round of compute units).
//   grid.x = ceil(n / per_wg) for the n sequences of the chunk, block = Trellis<L>::kThreads.
//   per_wg   : sequences per workgroup, 2 (interleaved pair) or 1
//   seq, wts : [*][T]; the workgroup takes rows b0 + per_wg*blockIdx.x (+1 if per_wg = 2
//              and < b0 + n)
//   rot      : the search runs over the rotated targets s'[t] = s[(t + rot) mod T]
//              (0 <= rot < T; the tail-biting encoder's first search uses T/2)
//   pin      : PINNED only -- [n] overlap o per sequence (an (L-2)-bit value): the walk
//              must start in a state whose high L-2 bits are o (group o, so mu_0 = +inf
//              outside group o) and end in a state whose low L-2 bits are o (the final
//              minimum runs over the four states a*2^(L-2) + o)
//   bp       : [n][T-1][kBpWords] 2-bit argmins of each step
//   fin      : [n] final state (uint32) ; fin_cost [n]
//   mse      : [*] (row b0 + q) or nullptr
//   ca       : the code's run-time parameters
// The two sequences A and B are interleaved so that LDS latency hides behind
// arithmetic: each phase loads one sequence's inputs while it computes the other's
// step, with one barrier per phase.  Each sequence has a single 64 KiB buffer of group
// minima: a buffer is only written in the phase after every thread's reads of it have
// completed (a barrier in between), and only read after the barrier that follows its
// writes.  The code-value registers are shared by both sequences.
template <int L, int CODE, bool WEIGHTED, bool PINNED = false, bool SINGLE = false>
__global__ void __launch_bounds__(Trellis<L>::kThreads)
viterbi_forward(const float* __restrict__ seq, const float* __restrict__ wts, int T, int64_t b0,
                int64_t n, int per_wg, int rot, const uint32_t* __restrict__ pin,
                uint32_t* __restrict__ bp, uint32_t* __restrict__ fin, float* __restrict__ fin_cost,
                float* __restrict__ mse, CodeArg ca)
{
    using Tr = Trellis<L>;
    constexpr int NB = Tr::kButterflies;
    constexpr int M = Tr::kGroups;
    constexpr int NT = Tr::kThreads;
    __shared__ float4 muA[Tr::kChunks];   // group minima of sequence A, M / 4 float4
    __shared__ float4 muB[Tr::kChunks];   // and of sequence B

    const int tid = threadIdx.x;
    const int64_t qa = per_wg * (int64_t)blockIdx.x;     // index within the chunk
    const bool has_b = per_wg == 2 && qa + 1 < n;         // uniform over the workgroup
    const int64_t qb = has_b ? qa + 1 : qa;
    const float* sa = seq + (b0 + qa) * T;
    const float* sb = seq + (b0 + qb) * T;
    const float* wa = WEIGHTED ? wts + (b0 + qa) * T : nullptr;
    const float* wb = WEIGHTED ? wts + (b0 + qb) * T : nullptr;
    uint32_t* bpa = bp + qa * (T - 1) * Tr::kBpWords;
    uint32_t* bpb = bp + qb * (T - 1) * Tr::kBpWords;

    // this thread's code values: state (a, c, x) = a*M + 4*(tid + r*NT) + x, computed one
    // at a time (scheduling barriers) so the fp64 divisions do not pile up registers
    float Cv[4][4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                Cv[a][r][x] = code_value_prologue<CODE>((uint32_t)(a * M + 4 * (tid + r * NT) + x), ca);
                if constexpr (CODE == kCodeXor) Cv[a][r][x] = keep(Cv[a][r][x]);
                __builtin_amdgcn_sched_barrier(0);
            }

    // mu_0 = +0 everywhere, so cost_0 = fl(0 + e_0) = e_0; pinned: +inf outside group o,
    // so cost_0 = +inf for every start state outside the allowed four
    if constexpr (PINNED) {
        const uint32_t oA = pin[qa], oB = pin[qb];
        const float inf = __builtin_inff();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint32_t g = 4u * (uint32_t)(tid + r * NT);
            muA[tid + r * NT] = make_float4(g == oA ? 0.f : inf, g + 1 == oA ? 0.f : inf,
                                            g + 2 == oA ? 0.f : inf, g + 3 == oA ? 0.f : inf);
            muB[tid + r * NT] = make_float4(g == oB ? 0.f : inf, g + 1 == oB ? 0.f : inf,
                                            g + 2 == oB ? 0.f : inf, g + 3 == oB ? 0.f : inf);
        }
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            muA[tid + r * NT] = make_float4(0.f, 0.f, 0.f, 0.f);
            muB[tid + r * NT] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    __syncthreads();

    // inputs of this thread's butterflies: in[r][a] = mu_{t-1}[(a, tid + r*NT)]
    auto load_in = [&](const float4* src4, float (&in)[4][4]) {
        const float* src = reinterpret_cast<const float*>(src4);
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int a = 0; a < 4; ++a) in[r][a] = src[a * NB + tid + r * NT];
    };

    // one ACS step from registers: writes mu_t[(c, 0..3)] for c = tid + r*NT and
    // returns the 16 packed 2-bit argmins
    // sp, wp: the step's target and weight, wave-uniform but held in VGPRs so that the
    // sub/mul/add below issue as 2-operand VGPR ops
    auto acs = [&](const float (&in)[4][4], float sp, float wp, float4* dst) -> uint32_t {
        uint32_t word = 0;
        // a group's two argmin bits are shifted in two groups later, so the scalar mask
        // logic between its compares and its add-with-carry has time to complete
        uint64_t hi[16], lo[16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float out[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int g = 4 * r + x;
                float v[4];
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    v[a] = in[r][a] + step_err<WEIGHTED>(Cv[a][r][x], sp, wp);
                const float m = __builtin_fminf(__builtin_fminf(v[0], v[1]), __builtin_fminf(v[2], v[3]));
                // lowest a attaining the minimum: 0 if v0 == m, else 1 if v1 == m, else
                // 2 if v2 == m, else 3.  The two bits are shifted in with add-with-carry
                // (word + word + bit), the compare masks serving as carries.
                const uint64_t n0 = __builtin_amdgcn_ballot_w64(v[0] != m);
                const uint64_t e1 = __builtin_amdgcn_ballot_w64(v[1] == m);
                const uint64_t n2 = __builtin_amdgcn_ballot_w64(v[2] != m);
                hi[g] = n0 & ~e1;            // a >= 2
                lo[g] = n0 & (e1 | n2);      // a odd
                if (g >= kBitDelay) {
                    word = shift_in_bit(word, hi[g - kBitDelay]);
                    word = shift_in_bit(word, lo[g - kBitDelay]);
                }
                out[x] = m;
            }
            dst[tid + r * NT] = make_float4(out[0], out[1], out[2], out[3]);
        }
#pragma unroll
        for (int g = 16 - kBitDelay; g < 16; ++g) {
            word = shift_in_bit(word, hi[g]);
            word = shift_in_bit(word, lo[g]);
        }
        return word;
    };

    // A's first inputs: mu_0, formed in registers (+0 everywhere, or pinned: +0 in group
    // o only), the same values muA holds; no LDS read before the loop, so the pinned and
    // free kernels' step loops get the same register assignment.  (At L = 6, a one-thread
    // workgroup, the pinned kernel reads them back from muA instead: the register form
    // kept a stack array there.)
    float inA[4][4], inB[4][4];
    if constexpr (PINNED && L == 6) {
        load_in(muA, inA);
    } else if constexpr (PINNED) {
        const uint32_t oA = pin[qa];
        const float inf = __builtin_inff();
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                inA[r][a] = (uint32_t)(a * NB + tid + r * NT) == oA ? 0.f : inf;
    } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int a = 0; a < 4; ++a) inA[r][a] = 0.f;
    }

    // Targets (and weights) go through a small LDS ring of two 256-step chunks per
    // sequence and are read one phase ahead with the input loads: a per-step scalar
    // load would be waited on together with the LDS reads (one shared counter) and
    // stall every phase.  Chunk k + 1 is loaded at the start of step 256 k + 1 into the
    // slot chunk k - 1 used: the last reads of chunk k - 1 are A's target of step
    // 256 k - 1 (phase 2 of step 256 k - 1) and B's (phase 1 of step 256 k), both behind
    // a barrier by then; chunk k + 1 is first read at step 256 (k + 1).
    constexpr int kChunk = 256;
    constexpr int kRing = WEIGHTED ? 4 : 2;    // sa, sb [, wa, wb]
    __shared__ float ring[kRing][2][kChunk];
    auto fill = [&](int k) {   // chunk k of every stream into slot k & 1
        const int j = k * kChunk;
        for (int i = tid; i < kChunk; i += NT) {
            const bool ok = j + i < T;
            int src = j + i + rot;             // rotated step index, < 2T
            if (src >= T) src -= T;
            ring[0][k & 1][i] = ok ? sa[src] : 0.f;
            ring[1][k & 1][i] = ok ? sb[src] : 0.f;
            if constexpr (WEIGHTED) {
                ring[2][k & 1][i] = ok ? wa[src] : 0.f;
                ring[3][k & 1][i] = ok ? wb[src] : 0.f;
            }
        }
    };
    auto ring_at = [&](int stream, int j) -> float {   // LDS read, lands in a VGPR
        return ring[stream][(j / kChunk) & 1][j % kChunk];
    };
    fill(0);
    if (T > kChunk) fill(1);
    __syncthreads();

    float spA = ring_at(0, 0), spB = 0.f;
    float wpA = WEIGHTED ? ring_at(2, 0) : 1.0f, wpB = 1.0f;
    if constexpr (SINGLE) {
        // One sequence per workgroup (per_wg = 1): muB is free, so the group minima
        // alternate between the two buffers (mu_t in muB for odd t, muA for even t) and one
        // barrier per step orders both the reads of mu_{t-1} before the writes that reuse
        // its buffer one step later and the writes of mu_t before their reads.  Each step
        // reads its inputs at its start, so every use waits only for its own read, and
        // then the next step's target.  Target ring: index t is read during step t, and
        // chunk k + 1 is loaded into the slot of chunk k - 1 at the start of step
        // 256 k + 1, two barriers after its last read (step 256 k - 1) and a barrier
        // before its first (step 256 (k + 1)).  Step 1 takes mu_0 from the registers.
        float spN = 0.f, wpN = 1.0f;   // the next step's target and weight
        if (T > 1) {
            if (T > 2) {
                spN = ring_at(0, 1);
                if constexpr (WEIGHTED) wpN = ring_at(2, 1);
            }
            const uint32_t wordA = acs(inA, spA, wpA, muB);
            bpa[tid] = wordA;
            __syncthreads();
        }
        for (int t = 2; t < T; ++t) {
            if (t > kChunk && t % kChunk == 1 && (t / kChunk + 1) * kChunk < T) fill(t / kChunk + 1);
            load_in((t & 1) ? muA : muB, inA);          // mu_{t-1}
            spA = spN;
            wpA = wpN;
            if (t + 1 < T) {
                spN = ring_at(0, t);
                if constexpr (WEIGHTED) wpN = ring_at(2, t);
            }
            const uint32_t wordA = acs(inA, spA, wpA, (t & 1) ? muB : muA);
            bpa[(int64_t)(t - 1) * Tr::kBpWords + tid] = wordA;
            __syncthreads();
        }
    } else {
    for (int t = 1; t < T; ++t) {
        if (t > kChunk && t % kChunk == 1 && (t / kChunk + 1) * kChunk < T) fill(t / kChunk + 1);
        // phase 1: fetch B's inputs and target, step A
        load_in(muB, inB);
        spB = ring_at(1, t - 1);
        if constexpr (WEIGHTED) wpB = ring_at(3, t - 1);
        const uint32_t wordA = acs(inA, spA, wpA, muA);
        bpa[(int64_t)(t - 1) * Tr::kBpWords + tid] = wordA;
        __syncthreads();
        // phase 2: fetch A's next inputs and target, step B
        if (t + 1 < T) {
            load_in(muA, inA);
            spA = ring_at(0, t);
            if constexpr (WEIGHTED) wpA = ring_at(2, t);
        }
        if (has_b) {
            const uint32_t wordB = acs(inB, spB, wpB, muB);
            bpb[(int64_t)(t - 1) * Tr::kBpWords + tid] = wordB;
        }
        __syncthreads();
    }
    }

    // final costs cost_{T-1}(i) = mu_{T-1}[i >> 2] + e_{T-1}(i); lowest i wins ties
    const int last = (T - 1 + rot) % T;    // the last step's target index
    auto finish = [&](const float4* mu4, const float* s, const float* w, int64_t q) {
        const float* fin_mu = reinterpret_cast<const float*>(mu4);
        // the thread index through an opaque move: keeps the epilogue's address
        // arithmetic from being hoisted above the step loop (where it would be spilled)
        int tid = threadIdx.x;
        asm volatile("v_mov_b32 %0, %0" : "+v"(tid));
        const float sp = to_vgpr(s[last]);
        const float wp = WEIGHTED ? to_vgpr(w[last]) : 1.0f;
        const uint32_t o = PINNED ? pin[q] : 0u;
        float best = __builtin_inff();
        uint32_t bi = 0xFFFFFFFFu;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float in = fin_mu[a * NB + tid + r * NT];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    float c = in + step_err<WEIGHTED>(Cv[a][r][x], sp, wp);
                    // pinned: only the end states whose low L-2 bits are o take part
                    if (PINNED && (uint32_t)(4 * (tid + r * NT) + x) != o) continue;
                    // states are visited in increasing order; the first one is taken
                    // whatever its cost, so a row whose costs are all +inf (finite inputs
                    // whose squared errors overflow binary32) still ends in its lowest
                    // allowed state
                    if (c < best || bi == 0xFFFFFFFFu) {
                        best = c;
                        bi = (uint32_t)(a * M + 4 * (tid + r * NT) + x);
                    }
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
                for (int k = 1; k < kWaves; ++k)
                    if (wbest[k] < best || (wbest[k] == best && wbi[k] < bi)) { best = wbest[k]; bi = wbi[k]; }
            }
            __syncthreads();   // the slots are reused by the next call
        }
        if (tid == 0) {
            fin[q] = bi;
            fin_cost[q] = best;
            if (mse) mse[b0 + q] = best / (float)T;
        }
    };
    // mu_{T-1}: in muA, or with one sequence per workgroup in the buffer of step T - 1
    finish(SINGLE && ((T - 1) & 1) ? muB : muA, sa, wa, qa);
    if (has_b) finish(muB, sb, wb, qb);
}

// Traceback and pack.  One thread per sequence of the chunk: walks the backpointers
// from the final state to t = 0 and writes the stream and optionally the states.
//   plain (TB = false): the start state's L bits, then the 2 new bits of every later
//     state, MSB first -- L + 2(T-1) bits;
//   tail-biting (TB = true): the 2 high bits of every state st[t] at stream bits
//     [2t, 2t + 2) -- exactly 2T bits; the cyclic window rule restores every state.
template <int L, bool TB = false>
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
    const int nbits = TB ? 2 * T : L + 2 * (T - 1);
    int curw = (nbits - 1) >> 5;
    uint32_t acc = 0;
    for (int t = T - 1; t >= 1; --t) {
        if (st) st[t] = j;
        // stream position of the 2 bits st[t] contributes: its high bits (tail-biting)
        // or the bits that entered its window (plain)
        const int p = TB ? 2 * t : L + 2 * (t - 1);
        const int wi = p >> 5;
        if (wi != curw) { out[curw] = acc; curw = wi; acc = 0; }
        acc |= ((TB ? j >> (L - 2) : j) & 3u) << (30 - (p & 31));
        const uint32_t m = j >> 2;                   // group of j's predecessors
        const uint32_t word = bpq[(int64_t)(t - 1) * Tr::kBpWords + Tr::bp_word(m)];
        const uint32_t a = (word >> Tr::bp_shift(m)) & 3u;
        j = m | (a << (L - 2));
    }
    if (st) st[0] = j;
    if (curw != 0) { out[curw] = acc; acc = 0; }
    acc |= TB ? (j >> (L - 2)) << 30 : j << (32 - L);
    out[0] = acc;
}

// Seam of the tail-biting encoder's first (rotated) search: walks back from the final
// state to step pos and stores the high L-2 bits of that state (the overlap the second
// search pins both ends to).  One thread per sequence of the chunk; 0 <= pos < T.
template <int L>
__global__ void __launch_bounds__(256)
viterbi_seam(const uint32_t* __restrict__ bp, const uint32_t* __restrict__ fin, int T,
             int64_t n, int pos, uint32_t* __restrict__ overlap)
{
    using Tr = Trellis<L>;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t* bpq = bp + i * (int64_t)(T - 1) * Tr::kBpWords;
    uint32_t j = fin[i];
    for (int t = T - 1; t > pos; --t) {
        const uint32_t m = j >> 2;
        const uint32_t word = bpq[(int64_t)(t - 1) * Tr::kBpWords + Tr::bp_word(m)];
        j = m | (((word >> Tr::bp_shift(m)) & 3u) << (L - 2));
    }
    overlap[i] = j >> 2;
}

}  // namespace qtcq
