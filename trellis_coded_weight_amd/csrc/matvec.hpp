// matvec.hpp -- decode -> matrix-vector product straight from trellis streams, gfx950.
//
// QTIP blog, "What it buys end to end": every 16x16 tile of a weight matrix is one
// 256-long sequence that decodes straight into the matrix operand, and at batch 1 the
// product streams 2-bit weights; "The trellis: a stateful codebook": weight t of a
// sequence is the code of the window of stream bits [2t, 2t + L).  Tiles are numbered
// row-major (sequence I * (N/16) + J is tile (I, J)) and weight t = 16 r + c of a tile is
// W[16 I + r][16 J + c].
//
// One workgroup per band of 16 output rows (tile row I).  Thread (r, js), r = tid & 15,
// js = tid >> 4, owns row r of tiles J = js, js + NJS, ...: the 16 weights of a tile row
// are stream bits [32 r, 32 r + 30 + L), i.e. inside words r and r + 1 (word 16 of a
// tail-biting stream is word 0 again), so each weight is one funnel shift of those two
// words, then the code.  The 16 weights are multiplied into the batch rows' running
// sums by FMA in c order.  The NJS partial sums of an output row are then added in a
// fixed order (lanes r, r+16, r+32, r+48 of a wave by two xor-shuffles, then the 16
// waves in sequence), so results are bit-deterministic, and a one-hot x reproduces a
// column of W exactly.
//
// Rounding: every output is a sum of N products; along its longest chain there are
// 16 * ceil((N/16) / NJS) FMAs, 2 shuffle additions and 15 wave additions, so
//     |y - W x| <= (16 ceil(N / (16 NJS)) + 17) * 2^-24 * sum_n |W[m][n] x[n]|  (to first order).
//
// This path is decode-ALU-bound on this chip, not HBM-bound: at 2 bits per weight the
// HBM streams ~3.2e13 weights/s, while the window + LCG + byte sum + exact rescale of a
// computed code costs ~9 CU cycles per 64 weights (~4.4e12 weights/s at 2.4 GHz).  The
// products are fp32 VALU FMAs: fp32 MFMA runs at the same rate as fp32 VALU FMA here and
// an fp16 / bf16 MFMA would round the decoded weights.
#pragma once

#include "codes.hpp"

namespace qtcq {

struct MatvecShape {
    static constexpr int kThreads = 1024;
    static constexpr int kJSlots = kThreads / 16;   // NJS: tile columns in flight per band
    static constexpr int kWaves = kThreads / 64;
    static constexpr int kMaxBatch = 8;
};

// grid.x = M / 16, block = MatvecShape::kThreads.  bits [(M/16)(N/16)][Wd]; x [batch][N];
// y [batch][M].  TB: tail-biting streams (Wd = 16 words, windows wrap to word 0).
template <int L, int CODE, bool TB>
__global__ void __launch_bounds__(MatvecShape::kThreads)
decode_matvec(const uint32_t* __restrict__ bits, int M, int N, int Wd,
              const float* __restrict__ x, int batch, float* __restrict__ y)
{
    constexpr int NJS = MatvecShape::kJSlots;
    constexpr int NB = MatvecShape::kMaxBatch;
    __shared__ float red[MatvecShape::kWaves][NB][16];

    const int tid = threadIdx.x;
    const int r = tid & 15, js = tid >> 4;
    const int lane = tid & 63, wave = tid >> 6;
    const int I = blockIdx.x;
    const int NTJ = N >> 4;
    const uint32_t* band = bits + (size_t)I * NTJ * Wd;

    float acc[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[i] = 0.0f;

    for (int J = js; J < NTJ; J += NJS) {
        const uint32_t* sw = band + (size_t)J * Wd;
        const uint32_t hi = sw[r];
        const uint32_t lo = sw[(TB && r == 15) ? 0 : r + 1];
        float wv[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            // stream bits [32 r + 2c, 32 r + 2c + 32) of the 64-bit funnel hi:lo
            const uint32_t top = c == 0 ? hi : __builtin_amdgcn_alignbit(hi, lo, 32 - 2 * c);
            wv[c] = code_value<CODE>(top >> (32 - L));
        }
        const float* xj = x + 16 * (size_t)J;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (i < batch) {
                const float4* xv = reinterpret_cast<const float4*>(xj + (size_t)i * N);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float4 v = xv[q];
                    acc[i] = __builtin_fmaf(wv[4 * q + 0], v.x, acc[i]);
                    acc[i] = __builtin_fmaf(wv[4 * q + 1], v.y, acc[i]);
                    acc[i] = __builtin_fmaf(wv[4 * q + 2], v.z, acc[i]);
                    acc[i] = __builtin_fmaf(wv[4 * q + 3], v.w, acc[i]);
                }
            }
        }
    }

    // partial sums of row r: lanes r, r + 16, r + 32, r + 48 of every wave
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if (i < batch) {
            float v = acc[i];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if (lane < 16) red[wave][i][lane] = v;
        }
    }
    __syncthreads();
    if (tid < 16 * batch) {
        const int i = tid >> 4, rr = tid & 15;
        float s = red[0][i][rr];
#pragma unroll
        for (int q = 1; q < MatvecShape::kWaves; ++q) s += red[q][i][rr];
        y[(size_t)i * M + 16 * I + rr] = s;
    }
}

}  // namespace qtcq
