// bcjr.hpp -- BCJR soft relaxation on the bitshift trellis, gfx950.
//
// BCJR-QAT abstract: replace the Viterbi argmax by the forward-backward sum-product
// recursion at temperature tau; the soft codeword is the Boltzmann expectation of the
// reconstructed value over trellis walks, weight exp(-E / tau) with E the search's path
// cost.  Start state uniform (plain trellis), so the recursion is the Viterbi one with
// (min, +) replaced by (log-sum-exp, +).
//
// Log2 domain, fp32.  kappa = log2(e) / tau and every code value is pre-scaled by
// sqrt(kappa), so kappa * e_t(j) = w_t * (C'_j - s'_t)^2 with C' = sqrt(kappa) C,
// s' = sqrt(kappa) s: two VALU ops per state (sub, fma) unweighted.
//
// Forward messages per group (as in the search, a group m = j >> 2 shares its
// predecessors): A_t[(c, x)] = LSE2_a( A_{t-1}[(a, c)] - kappa e_{t-1}((a, c, x)) ),
// A_0 = 0.  Stored values X_t = A_t - G_{t-1} where g_t = max X_t is subtracted on the
// next read and G accumulates the g's (in fp64).  Every X_t goes to an HBM stash.
// Backward messages per low-(L-2)-bit group: B_{t-1}[(a, c)] = LSE2_x( B_t[(c, x)] -
// kappa e_t((a, c, x)) ), B_{T-1} = 0, normalised the same way (h_t, H_t).  The same
// 16 states (a, c, x) and code values serve both directions, so the thread mapping,
// LDS layout and swizzle are the search kernel's (see viterbi.hpp).
// Posterior at t: gamma_t(j) = 2^( la_t(j) + lb_t(j) - log2 Z ), computed in the
// backward sweep from the stash value X_t[(a, c)], the backward input Y_t[(c, x)] and
// the step energy, with the exact offset O_t = log2 Z - G_{t-1} - H_t, so the largest
// exponent is <= 0 and >= -L.  soft_t = sum gamma C / sum gamma: per-wave partial sums
// per step go to the workspace and a small kernel divides them.
#pragma once

#include "codes.hpp"
#include "viterbi.hpp"

namespace qtcq {

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float lse2_4(float v0, float v1, float v2, float v3)
{
    const float m = __builtin_fmaxf(__builtin_fmaxf(v0, v1), __builtin_fmaxf(v2, v3));
    const float s = (fast_exp2(v0 - m) + fast_exp2(v1 - m)) + (fast_exp2(v2 - m) + fast_exp2(v3 - m));
    return m + fast_log2(s);
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
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = WIDTH / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <int L>
struct BcjrLayout {
    using Tr = Trellis<L>;
    static constexpr int kWaves = (Tr::kThreads + 63) / 64;
    // Per-sequence workspace, each part 256-byte aligned:
    //   log2 Z (double) | g_0..g_{T-1} (float) | posterior partial sums [T][kWaves][2]
    //   | stash X_1..X_{T-1} ([T-1][4][kThreads] float4: chunk 4*tau + r at [r][tau])
    __host__ __device__ static size_t up(size_t b) { return (b + 255) / 256 * 256; }
    __host__ __device__ static size_t off_g() { return 256; }
    __host__ __device__ static size_t off_part(int T) { return off_g() + up((size_t)T * 4); }
    __host__ __device__ static size_t off_stash(int T) { return off_part(T) + up((size_t)T * kWaves * 8); }
    __host__ __device__ static size_t bytes_per_seq(int T) { return off_stash(T) + up((size_t)(T - 1) * Tr::kGroups * 4); }
};

inline size_t bcjr_bytes_per_seq(int T, int L)
{
    switch (L) {
    case 6: return BcjrLayout<6>::bytes_per_seq(T);
    case 8: return BcjrLayout<8>::bytes_per_seq(T);
    case 10: return BcjrLayout<10>::bytes_per_seq(T);
    case 12: return BcjrLayout<12>::bytes_per_seq(T);
    case 14: return BcjrLayout<14>::bytes_per_seq(T);
    default: return BcjrLayout<16>::bytes_per_seq(T);
    }
}

// grid.x = sequences in the chunk; block = Trellis<L>::kThreads.  ws points at the
// chunk's workspace, bytes_per_seq(T) per sequence.
template <int L, int CODE, bool WEIGHTED>
__global__ void __launch_bounds__(Trellis<L>::kThreads)
bcjr_sweep(const float* __restrict__ seq, const float* __restrict__ wts, int T, int64_t b0,
           float sk, char* __restrict__ ws)
{
    using Tr = Trellis<L>;
    using Ly = BcjrLayout<L>;
    constexpr int NB = Tr::kButterflies;
    constexpr int M = Tr::kGroups;
    constexpr int NT = Tr::kThreads;
    constexpr int kWaves = Ly::kWaves;
    constexpr int WID = NT < 64 ? NT : 64;
    __shared__ float4 buf[2][Tr::kChunks];
    __shared__ float wmax[2][kWaves];
    __shared__ float redm[kWaves], reds[kWaves];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t row = b0 + blockIdx.x;
    const float* s = seq + row * T;
    const float* w = WEIGHTED ? wts + row * T : nullptr;
    char* base = ws + (size_t)blockIdx.x * Ly::bytes_per_seq(T);
    double* l2z = reinterpret_cast<double*>(base);
    float* gnorm = reinterpret_cast<float*>(base + Ly::off_g());
    float* part = reinterpret_cast<float*>(base + Ly::off_part(T));
    float4* stash = reinterpret_cast<float4*>(base + Ly::off_stash(T));

    float Cs[4][4][4];   // sqrt(kappa) * code value of state (a, c = 4 tid + r, x)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int x = 0; x < 4; ++x)
                Cs[a][r][x] = sk * code_value<CODE>((uint32_t)(a * M + 16 * tid + 4 * r + x));

    int rd[4], wr[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) rd[a] = lds_chunk(a * (NB / 4) + tid);
#pragma unroll
    for (int r = 0; r < 4; ++r) wr[r] = lds_chunk(4 * tid + r);

    // ---------------- forward ----------------
#pragma unroll
    for (int r = 0; r < 4; ++r) buf[0][wr[r]] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < kWaves) wmax[0][tid] = 0.f;
    __syncthreads();

    double G = 0.0;   // sum of g_0 .. g_{t-1}
    int cur = 0;
    for (int t = 1; t < T; ++t) {
        float g = wmax[cur][0];
#pragma unroll
        for (int q = 1; q < kWaves; ++q) g = __builtin_fmaxf(g, wmax[cur][q]);
        G += (double)g;
        if (tid == 0) gnorm[t - 1] = g;
        const float sp = sk * s[t - 1];
        const float wp = WEIGHTED ? w[t - 1] : 1.0f;
        float u[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            float4 v = buf[cur][rd[a]];
            u[a][0] = v.x - g; u[a][1] = v.y - g; u[a][2] = v.z - g; u[a][3] = v.w - g;
        }
        float lmax = -__builtin_inff();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float o[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                float v[4];
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float d = Cs[a][r][x] - sp;
                    v[a] = WEIGHTED ? __builtin_fmaf(-(wp * d), d, u[a][r]) : __builtin_fmaf(-d, d, u[a][r]);
                }
                o[x] = lse2_4(v[0], v[1], v[2], v[3]);
                lmax = __builtin_fmaxf(lmax, o[x]);
            }
            const float4 ov = make_float4(o[0], o[1], o[2], o[3]);
            buf[cur ^ 1][wr[r]] = ov;
            stash[((size_t)(t - 1) * 4 + r) * NT + tid] = ov;
        }
        lmax = wave_max<WID>(lmax);
        if (lane == 0) wmax[cur ^ 1][wave] = lmax;
        __syncthreads();
        cur ^= 1;
    }

    // log2 Z = G_{T-1} + LSE2_j( X_{T-1}[j >> 2] - g_{T-1} - kappa e_{T-1}(j) )
    float gl = wmax[cur][0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) gl = __builtin_fmaxf(gl, wmax[cur][q]);
    G += (double)gl;
    if (tid == 0) gnorm[T - 1] = gl;
    double log2z;
    {
        const float sp = sk * s[T - 1];
        const float wp = WEIGHTED ? w[T - 1] : 1.0f;
        float q[4][4][4];
        float m = -__builtin_inff();
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            float4 v = buf[cur][rd[a]];
            float in[4] = {v.x - gl, v.y - gl, v.z - gl, v.w - gl};
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float d = Cs[a][r][x] - sp;
                    q[a][r][x] = WEIGHTED ? __builtin_fmaf(-(wp * d), d, in[r]) : __builtin_fmaf(-d, d, in[r]);
                    m = __builtin_fmaxf(m, q[a][r][x]);
                }
        }
        float wm = wave_max<WID>(m);
        if (lane == 0) redm[wave] = wm;
        __syncthreads();
        float bm = redm[0];
#pragma unroll
        for (int qq = 1; qq < kWaves; ++qq) bm = __builtin_fmaxf(bm, redm[qq]);
        float sum = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int x = 0; x < 4; ++x) sum += fast_exp2(q[a][r][x] - bm);
        sum = wave_sum<WID>(sum);
        if (lane == 0) reds[wave] = sum;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int qq = 0; qq < kWaves; ++qq) tot += reds[qq];
        log2z = G + (double)bm + (double)fast_log2(tot);
        if (tid == 0) l2z[0] = log2z;
    }

    // ---------------- backward + posterior ----------------
    // Y_{T-1} = 0 in the buffer not holding X_{T-1}
    int cb = cur ^ 1;
#pragma unroll
    for (int a = 0; a < 4; ++a) buf[cb][rd[a]] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < kWaves) wmax[cb][tid] = 0.f;
    __syncthreads();

    double Gm = G;     // G_{t} at the top of iteration t (sum g_0..g_t)
    double H = 0.0;    // H_{t+1} at the top of iteration t
    for (int t = T - 1; t >= 0; --t) {
        float h = wmax[cb][0];
#pragma unroll
        for (int q = 1; q < kWaves; ++q) h = __builtin_fmaxf(h, wmax[cb][q]);
        H += (double)h;                        // H_t
        Gm -= (double)gnorm[t];                // G_{t-1}
        const float Ot = (float)(log2z - Gm - H);
        // X_t[(a, 4 tid + r)] - O_t from the stash (X_0 = 0)
        float xo[4][4];
        if (t > 0) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const int g = a * (NB / 4) + tid;      // logical chunk index
                const float4 v = stash[((size_t)(t - 1) * 4 + (g & 3)) * NT + (g >> 2)];
                xo[a][0] = v.x - Ot; xo[a][1] = v.y - Ot; xo[a][2] = v.z - Ot; xo[a][3] = v.w - Ot;
            }
        } else {
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int r = 0; r < 4; ++r) xo[a][r] = -Ot;
        }
        float u[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float4 v = buf[cb][wr[r]];
            u[r][0] = v.x - h; u[r][1] = v.y - h; u[r][2] = v.z - h; u[r][3] = v.w - h;
        }
        const float sp = sk * s[t];
        const float wp = WEIGHTED ? w[t] : 1.0f;
        float pg = 0.f, pc = 0.f;
        float ymax = -__builtin_inff();
        float yo[4][4];   // Y_{t-1}[(a, 4 tid + r)]
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v[4];
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float d = Cs[a][r][x] - sp;
                    v[x] = WEIGHTED ? __builtin_fmaf(-(wp * d), d, u[r][x]) : __builtin_fmaf(-d, d, u[r][x]);
                    const float p = fast_exp2(xo[a][r] + v[x]);
                    pg += p;
                    pc = __builtin_fmaf(p, Cs[a][r][x], pc);
                }
                if (t > 0) {
                    yo[a][r] = lse2_4(v[0], v[1], v[2], v[3]);
                    ymax = __builtin_fmaxf(ymax, yo[a][r]);
                }
            }
        }
        pg = wave_sum<WID>(pg);
        pc = wave_sum<WID>(pc);
        if (lane == 0) {
            part[((size_t)t * kWaves + wave) * 2 + 0] = pg;
            part[((size_t)t * kWaves + wave) * 2 + 1] = pc;
        }
        if (t == 0) break;
#pragma unroll
        for (int a = 0; a < 4; ++a)
            buf[cb ^ 1][rd[a]] = make_float4(yo[a][0], yo[a][1], yo[a][2], yo[a][3]);
        ymax = wave_max<WID>(ymax);
        if (lane == 0) wmax[cb ^ 1][wave] = ymax;
        __syncthreads();
        cb ^= 1;
    }
}

// soft[b][t] = (sum_waves pc) / (sum_waves pg) / sqrt(kappa); log_z = ln 2 * log2 Z.
template <int L>
__global__ void __launch_bounds__(256)
bcjr_finalize(const char* __restrict__ ws, int T, int64_t n, int64_t b0, float inv_sk,
              float* __restrict__ soft, float* __restrict__ logz)
{
    using Ly = BcjrLayout<L>;
    constexpr int kWaves = Ly::kWaves;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= n * T) return;
    const int64_t i = idx / T;
    const int t = (int)(idx - i * T);
    const char* base = ws + (size_t)i * Ly::bytes_per_seq(T);
    const float* part = reinterpret_cast<const float*>(base + Ly::off_part(T));
    float pg = 0.f, pc = 0.f;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
        pg += part[((size_t)t * kWaves + q) * 2 + 0];
        pc += part[((size_t)t * kWaves + q) * 2 + 1];
    }
    soft[(b0 + i) * T + t] = (pc / pg) * inv_sk;
    if (logz && t == 0) {
        const double l2z = *reinterpret_cast<const double*>(base);
        logz[b0 + i] = (float)(l2z * 0.69314718055994530942);
    }
}

}  // namespace qtcq
