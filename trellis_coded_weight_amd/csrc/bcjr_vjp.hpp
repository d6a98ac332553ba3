// bcjr_vjp.hpp -- vector-Jacobian product of the BCJR soft codeword, gfx950.
//
// BCJR-QAT abstract: the soft codeword is the Boltzmann expectation of the
// reconstruction over trellis walks at temperature tau, and the relaxation is exactly
// differentiable.  With p(walk) ~ exp(-E / tau) and dE/ds_u = -2 w_u (C(state_u) - s_u),
//     d soft_t / d s_u = (2 w_u / tau) Cov( C(state_t), C(state_u) ),
// so for an upstream gradient g (g_t = dLoss / dsoft_t)
//     grad_u = (2 w_u / tau) Cov( F, C(state_u) ),   F = sum_t g_t C(state_t).
// Given state_u = j the walk's past and future are independent, so
//     E[F | state_u = j] - Fbar = Phi_u(j >> 2) + g_u (C_j - soft_u) + Psi_u(j mod M)
// with Fbar = sum_t g_t soft_t and two linear recursions over the same trellis groups as
// the soft pass, centred on soft (which keeps their values O(1) and fp32 adequate):
//     Phi_0 = 0,  Phi_t[(c, x)] = sum_a P_a (Phi_{t-1}[(a, c)] + g_{t-1} (C_(a,c,x) - soft_{t-1}))
//                 P_a ~ 2^( Xn_{t-1}[(a, c)] - kappa e_{t-1}((a, c, x)) )
//     Psi_{T-1} = 0,  Psi_{u-1}[(a, c)] = sum_x Q_x (g_u (C_(a,c,x) - soft_u) + Psi_u[(c, x)])
//                 Q_x ~ 2^( Yn_u[(c, x)] - kappa e_u((a, c, x)) )
// where Xn, Yn are the soft pass's normalised forward / backward messages (32-bit
// stash, to_fix) and kappa = log2(e) / tau.  At every u the posterior gamma_u(j) =
// 2^(Xn_u + Yn_u - kappa e_u - O_u) gives the four sums S0 = sum gamma, S1 = sum gamma c,
// S2 = sum gamma f, S3 = sum gamma c f (c = C_j - soft_u, f = the bracket above), and
//     Cov = S3 / S0 - (S1 / S0)(S2 / S0).
// Kernel: one workgroup per sequence, thread tau owns butterflies c = 4 tau + r as in
// the soft pass, handled in two halves (r = 2h, 2h + 1) so that only half of the
// messages are live at once.  Phi / Psi live in a double-buffered fp32 LDS buffer (one
// barrier per step).  While step t + 1 reads Phi_t it also stores it to HBM
// ([t][a][h][tau] float2, lane-contiguous) for the backward; per-wave partial sums per
// step go to the workspace and bcjr_vjp_finalize forms the gradient.
#pragma once

#include <type_traits>

#include "bcjr.hpp"

namespace qtcq {

// grid.x = sequences in the chunk; block = Trellis<L>::kThreads.  ws: the chunk's VJP
// workspace as left by bcjr_sweep<..., VJP = true> (bytes_per_seq_vjp(T) per sequence).
// gup: [*][T] upstream gradient; row b0 + blockIdx.x.
// WIDE: the soft pass stashed fp64 values (bcjr_sweep<..., VJP = true, WIDE = true>).
template <int L, int CODE, bool WEIGHTED, bool WIDE = false>
__global__ void __launch_bounds__(Trellis<L>::kThreads)
bcjr_vjp_sweep(const float* __restrict__ seq, const float* __restrict__ wts,
               const float* __restrict__ gup, int T, int64_t b0, double kappa,
               char* __restrict__ ws, CodeArg ca)
{
    using Tr = Trellis<L>;
    using Ly = BcjrLayout<L>;
    constexpr int NT = Tr::kThreads;
    constexpr int NB = Tr::kButterflies;
    constexpr int kWaves = Ly::kWaves;
    constexpr int WID = NT < 64 ? NT : 64;
    // expectation messages, double-buffered: chunk g (4 consecutive groups) keeps its two
    // halves (groups 0-1 and 2-3) in separate planes, so that the half accesses (8 bytes
    // per lane) are as lane-contiguous as the whole-chunk ones (16 bytes as two halves)
    __shared__ float2 bufp[2][2][NB];
    __shared__ float softs[kBcjrMaxT];   // soft_t, formed as the soft pass's finalize forms it

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t row = b0 + blockIdx.x;
    const float* s = seq + row * T;
    const float* w = WEIGHTED ? wts + row * T : nullptr;
    const float* gu = gup + row * T;
    char* base = ws + (size_t)blockIdx.x * Ly::bytes_per_seq_vjp(T);
    const float* part = reinterpret_cast<const float*>(base + Ly::off_part(T));
    using SV = StashVal<WIDE>;
    using ST = typename SV::T;
    struct Pair { ST x, y; };
    const int2* xst = reinterpret_cast<const int2*>(base + Ly::off_stash(T));    // [t-1][a][h][tau]
    const int4* yst = reinterpret_cast<const int4*>(base + Ly::off_ystash(T));   // [t][r][tau]
    const double2* xsw = reinterpret_cast<const double2*>(base + Ly::off_xwide(T));   // WIDE
    const double2* ysw = reinterpret_cast<const double2*>(base + Ly::off_ystash(T));  // WIDE: [t][r][hh][tau]
    // Xn_t[(a, 4 tau + 2h + i)], i = 0, 1, for t >= 1
    auto x_pair = [&](int t, int a, int h) -> Pair {
        const size_t k = (((size_t)(t - 1) * 4 + a) * 2 + h) * NT + tid;
        if constexpr (WIDE) {
            const double2 q = xsw[k];
            return Pair{q.x, q.y};
        } else {
            const int2 q = xst[k];
            return Pair{q.x, q.y};
        }
    };
    const double* ofs = reinterpret_cast<const double*>(base + Ly::off_ofs(T));
    float2* phs = reinterpret_cast<float2*>(base + Ly::off_phi(T));              // [t][a][h][tau]
    float* vpart = reinterpret_cast<float*>(base + Ly::off_vpart(T));

    for (int t = tid; t < T; t += NT) {
        float pg = 0.f, pc = 0.f;
#pragma unroll
        for (int q = 0; q < kWaves; ++q) {
            pg += part[((size_t)t * kWaves + q) * 2 + 0];
            pc += part[((size_t)t * kWaves + q) * 2 + 1];
        }
        softs[t] = pc / pg;
    }
    PackedCodes<L, CODE> Cp;   // code values of the states (a, c = 4 tid + r, x)
    Cp.init(tid, ca);

    // chunk indices of the groups (a, 4tid + r) and (4tid + r, x).  With at least 64
    // threads (L >= 12) the swizzle leaves a * NT alone: rd(a) = c0 + a NT and
    // wr(r) = c1 XOR r, from two bases derived once per step (derive()) from an opaque copy
    // of the thread index, so that neither they nor eight loop-invariant indices are
    // carried across steps.  Smaller workgroups recompute each index at its use, and so
    // does the palette code's weighted wide-stash sweep, whose registers are full (it
    // would spill).
    constexpr bool kSplit = NT >= 64 && !(CODE == kCodeXor && WEIGHTED && WIDE);
    auto opaque_tid = [&]() {
        int v = tid;
        asm volatile("v_mov_b32 %0, %0" : "+v"(v));
        return v;
    };
    int c0 = 0, c1 = 0;
    auto derive = [&]() {
        if constexpr (kSplit) {
            const int t = opaque_tid();
            c0 = lds_chunk(t);
            c1 = lds_chunk(4 * t);
        }
    };
    auto rd = [&](int a) {   // groups (a, 4tid + r)
        if constexpr (kSplit) return c0 + a * NT;
        else return lds_chunk(a * NT + opaque_tid());
    };
    auto wr = [&](int r) {   // groups (4tid + r, x)
        if constexpr (kSplit) return c1 ^ r;
        else return lds_chunk(4 * opaque_tid() + r);
    };
    auto put4 = [&](int cur, int chunk, float4 v) {
        bufp[cur][0][chunk] = make_float2(v.x, v.y);
        bufp[cur][1][chunk] = make_float2(v.z, v.w);
    };
    auto get4 = [&](int cur, int chunk) -> float4 {
        const float2 lo = bufp[cur][0][chunk], hi = bufp[cur][1][chunk];
        return make_float4(lo.x, lo.y, hi.x, hi.y);
    };
    auto half = [&](int cur, int chunk, int h) -> float2& {
        return bufp[cur][h][chunk];
    };
    // the soft pass's (shifted) energy terms: its posterior offsets O_u were formed with them
    auto step_energy = [&](int t) { return StepEnergy(kappa, s[t], WEIGHTED ? w[t] : 1.0f); };
    auto phi_slot = [&](int t, int a, int h) -> size_t {
        return (((size_t)t * 4 + a) * 2 + h) * NT + tid;
    };

    // ---------------- forward: Phi ----------------
    derive();
#pragma unroll
    for (int r = 0; r < 4; ++r) put4(0, wr(r), make_float4(0.f, 0.f, 0.f, 0.f));
    __syncthreads();
    int cur = 0;
    // One forward step at t (1 <= t < T): Phi_t from Phi_{t-1}.  HAS_X: Xn_{t-1} comes from
    // the stash (t >= 2); the step with t = 1 (Xn_0 = 0) is peeled so that the loop body
    // has no branches.
    auto fstep = [&](int t, auto has_x_tag) {
        constexpr bool HAS_X = decltype(has_x_tag)::value;
        derive();
        const StepEnergy se = step_energy(t - 1);
        const float gp = gu[t - 1];
        const float sft = softs[t - 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float ph[4][2];   // Phi_{t-1}[(a, 4 tid + 2h + i)]
            ST xq[4][2];      // Xn_{t-1}[(a, 4 tid + 2h + i)]
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float2 v = half(cur, rd(a), h);
                phs[phi_slot(t - 1, a, h)] = v;
                ph[a][0] = v.x; ph[a][1] = v.y;
                Pair q{SV::kZero, SV::kZero};   // Xn_0 = 0
                if constexpr (HAS_X) q = x_pair(t - 1, a, h);
                xq[a][0] = q.x; xq[a][1] = q.y;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 2 * h + i;
                float out[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    double lw[4];
                    float cx[4];
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        cx[a] = Cp.at(a, r, x);
                        lw[a] = se.add_to(cx[a], SV::get(xq[a][i]));
                    }
                    const double m = max64(max64(lw[0], lw[1]), max64(lw[2], lw[3]));
                    float num = 0.f, den = 0.f;
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const float p = fast_exp2((float)(lw[a] - m));
                        den += p;
                        num = __builtin_fmaf(p, __builtin_fmaf(gp, cx[a] - sft, ph[a][i]), num);
                    }
                    out[x] = num * __builtin_amdgcn_rcpf(den);   // den >= 1: its largest term is 2^0
                }
                put4(cur ^ 1, wr(r), make_float4(out[0], out[1], out[2], out[3]));
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        cur ^= 1;
        __syncthreads();
    };
    if (T >= 2) fstep(1, std::false_type{});
    for (int t = 2; t < T; ++t) fstep(t, std::true_type{});
    // Phi_{T-1}
    derive();
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int a = 0; a < 4; ++a) phs[phi_slot(T - 1, a, h)] = half(cur, rd(a), h);

    // ---------------- backward: Psi and the covariance sums ----------------
    // Psi_{T-1} = 0 (the buffer not read by the last forward step)
    derive();
#pragma unroll
    for (int r = 0; r < 4; ++r) put4(cur ^ 1, wr(r), make_float4(0.f, 0.f, 0.f, 0.f));
    cur ^= 1;
    __syncthreads();   // also orders this workgroup's Phi stores before their reads
    // One backward step at u: the covariance sums of step u and, if PRODUCE (u >= 1),
    // Psi_{u-1}.  The step with u = 0 is peeled so that the loop body has no branches.
    auto bstep = [&](int u, auto produce_tag) {
        constexpr bool PRODUCE = decltype(produce_tag)::value;
        derive();
        const StepEnergy se = step_energy(u);
        const float gp = gu[u];
        const float sft = softs[u];
        const double OuS = ofs[u] + 2.0 * SV::kShift;
        float S0 = 0.f, S1 = 0.f, S2 = 0.f, S3 = 0.f;
        // Xn_u and Phi_u of the groups (a, 4 tid + 2h + i), loaded one (h, a) ahead of use
        auto load_xp = [&](int h, int a, Pair& xq, float2& ph) {
            xq = Pair{SV::kZero, SV::kZero};   // Xn_0 = 0
            if constexpr (PRODUCE) xq = x_pair(u, a, h);
            ph = phs[phi_slot(u, a, h)];
        };
        Pair xq_next;
        float2 ph_next;
        load_xp(0, 0, xq_next, ph_next);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float ps[2][4];   // Psi_u[(4 tid + 2h + i, x)]
            ST yq[2][4];      // Yn_u[(4 tid + 2h + i, x)]
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float4 v = get4(cur, wr(2 * h + i));
                ps[i][0] = v.x; ps[i][1] = v.y; ps[i][2] = v.z; ps[i][3] = v.w;
                if constexpr (WIDE) {
                    const size_t k = ((size_t)u * 4 + 2 * h + i) * 2;
                    const double2 lo = ysw[(k + 0) * NT + tid], hi = ysw[(k + 1) * NT + tid];
                    yq[i][0] = lo.x; yq[i][1] = lo.y; yq[i][2] = hi.x; yq[i][3] = hi.y;
                } else {
                    const int4 q = yst[((size_t)u * 4 + 2 * h + i) * NT + tid];
                    yq[i][0] = q.x; yq[i][1] = q.y; yq[i][2] = q.z; yq[i][3] = q.w;
                }
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const Pair xq = xq_next;
                const float2 ph = ph_next;
                if (a < 3)
                    load_xp(h, a + 1, xq_next, ph_next);
                else if (h == 0)
                    load_xp(1, 0, xq_next, ph_next);
                const ST xqi[2] = {xq.x, xq.y};
                const float phi[2] = {ph.x, ph.y};
                float outp[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int r = 2 * h + i;
                    double lq[4];
                    float cx[4];
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        cx[x] = Cp.at(a, r, x);
                        lq[x] = se.add_to(cx[x], SV::get(yq[i][x]));
                    }
                    // Q_x = 2^(lq_x - m) / den; the posterior of state (a, c, x) is
                    // 2^(Xn_u - O_u + lq_x) = 2^(Xn_u - O_u + m) * 2^(lq_x - m)
                    const double m = max64(max64(lq[0], lq[1]), max64(lq[2], lq[3]));
                    // with f = phi + bk (bk = g_u c + Psi_u, the future's part):
                    //   sum q f = phi den + sum q bk,  sum q c f = phi sum q c + sum q c bk
                    float den = 0.f, num = 0.f, s1 = 0.f, t3 = 0.f;
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const float q = fast_exp2((float)(lq[x] - m));
                        const float cj = cx[x] - sft;
                        const float bk = __builtin_fmaf(gp, cj, ps[i][x]);
                        const float qc = q * cj;
                        den += q;
                        num = __builtin_fmaf(q, bk, num);
                        s1 += qc;
                        t3 = __builtin_fmaf(qc, bk, t3);
                    }
                    // SV::get and m (through lq) both carry SV::kShift: OuS = O_u + 2 kShift
                    const float pb = fast_exp2((float)((SV::get(xqi[i]) - OuS) + m));
                    S0 = __builtin_fmaf(pb, den, S0);
                    S1 = __builtin_fmaf(pb, s1, S1);
                    S2 = __builtin_fmaf(pb, __builtin_fmaf(phi[i], den, num), S2);
                    S3 = __builtin_fmaf(pb, __builtin_fmaf(phi[i], s1, t3), S3);
                    if constexpr (PRODUCE) outp[i] = num * __builtin_amdgcn_rcpf(den);
                }
                if constexpr (PRODUCE) half(cur ^ 1, rd(a), h) = make_float2(outp[0], outp[1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        S0 = wave_sum<WID>(S0);
        S1 = wave_sum<WID>(S1);
        S2 = wave_sum<WID>(S2);
        S3 = wave_sum<WID>(S3);
        if (lane == 0) {
            float* vp = vpart + ((size_t)u * kWaves + wave) * 4;
            vp[0] = S0; vp[1] = S1; vp[2] = S2; vp[3] = S3;
        }
        if constexpr (PRODUCE) {
            cur ^= 1;
            __syncthreads();
        }
    };
    for (int u = T - 1; u >= 1; --u) bstep(u, std::true_type{});
    bstep(0, std::false_type{});
}

// grad[b][u] = (2 w_u / tau) (S3 / S0 - (S1 / S0)(S2 / S0)), the S's summed over waves.
template <int L>
__global__ void __launch_bounds__(256)
bcjr_vjp_finalize(const char* __restrict__ ws, const float* __restrict__ wts, int T, int64_t n,
                  int64_t b0, double two_over_tau, float* __restrict__ grad)
{
    using Ly = BcjrLayout<L>;
    constexpr int kWaves = Ly::kWaves;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * T) return;
    const int64_t i = idx / T;
    const int u = (int)(idx - i * T);
    const char* base = ws + (size_t)i * Ly::bytes_per_seq_vjp(T);
    const float* vp = reinterpret_cast<const float*>(base + Ly::off_vpart(T));
    double S[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int q = 0; q < kWaves; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k) S[k] += (double)vp[((size_t)u * kWaves + q) * 4 + k];
    const double cov = S[3] / S[0] - (S[1] / S[0]) * (S[2] / S[0]);
    const double wu = wts ? (double)wts[(b0 + i) * T + u] : 1.0;
    grad[(b0 + i) * T + u] = (float)(two_over_tau * wu * cov);
}

}  // namespace qtcq
