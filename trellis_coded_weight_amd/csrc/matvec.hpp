// matvec.hpp -- decode -> matrix-vector product straight from trellis streams, gfx950.
//
// QTIP blog, "What it buys end to end": every 16x16 tile of a weight matrix is one
// 256-long sequence that decodes straight into the matrix operand, and at batch 1 the
// product streams 2-bit weights; "The trellis: a stateful codebook": weight t of a
// sequence is the code of the window of stream bits [2t, 2t + L).  Tiles are numbered
// row-major (sequence I * (N/16) + J is tile (I, J)) and weight t = 16 r + c of a tile is
// W[16 I + r][16 J + c].
//
// One workgroup per band of 16 output rows (tile row I).  A thread owns the 4x4 block
// (rows 4 rq + a, columns 4 cq + b) of tiles J = js, js + NJS, ... (lane bits: cq = 1:0,
// rq = 3:2, tile 5:4; js = tid >> 4).  Row 4 rq + a of a tile is stream bits
// [32 (4 rq + a), ... + 30 + L), inside words 4 rq + a and 4 rq + a + 1 (word 16 of a
// tail-biting stream is word 0 again), so a thread reads words 4 rq .. 4 rq + 4, one
// funnel shift per row gives the bits of its four columns and each weight is a bit-field
// of that, then the code.  The thread needs x[16 J + 4 cq .. + 3] of each batch row (one
// float4) and accumulates its four rows by FMA in b order.  The products use the code
// before its rescale (1MAD: S - 510; 3INST: the fp16 sum -- both exact in binary32) and
// each output is rescaled once at the end (code_rescale: exact for any raw value, so a
// one-hot x still reproduces a column of W bit for bit).  The stream words of the next
// tile are loaded while the current one is decoded.  Partial sums of a row are then
// added in a fixed order (the 4 column groups and the 4 tiles of a wave by xor-shuffles,
// then the 16 waves in sequence), so results are bit-deterministic, and a one-hot x
// reproduces a column of W exactly.
//
// Rounding: every output is a sum of N products; along its longest chain there are
// 4 * ceil((N/16) / NJS) FMAs, 4 shuffle additions and 15 wave additions; the raw code
// differs from W * D (D the code's divisor) by at most one rounding of W, and the final
// rescale adds at most 1.5 more, so
//     |y - W x| <= (4 ceil(N / (16 NJS)) + 22) * 2^-24 * sum_n |W[m][n] x[n]|  (to first order).
//
// This path is decode-ALU-bound on this chip, not HBM-bound: at 2 bits per weight the
// HBM streams ~3.2e13 weights/s, while the window, LCG, byte sum and exact rescale of a
// computed code cost ~7 CU cycles per 64 weights (~5e12 weights/s at 2.4 GHz).  The
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

// grid.x = M / 16, block = MatvecShape::kThreads.  bits [(M/16)(N/16)][Wd]; x [batch][N]
// (16-byte aligned); y [batch][M].  TB: tail-biting streams (Wd = 16, windows wrap).
// NB: batch rows the kernel is compiled for (1, 2, 4, 8), batch <= NB.
template <int L, int CODE, bool TB, int NB>
__global__ void __launch_bounds__(MatvecShape::kThreads)
decode_matvec(const uint32_t* __restrict__ bits, int M, int N, int Wd,
              const float* __restrict__ x, int batch, float* __restrict__ y, CodeArg ca)
{
    constexpr int NJS = MatvecShape::kJSlots;
    static_assert(NB >= 1 && NB <= MatvecShape::kMaxBatch, "batch width");
    // the LCG's three-instruction form where it measured faster: 1MAD at eight rows
    // (132 against 146 us on 28672x8192); 3INST at eight rows is slower with it
    constexpr bool kSplitLcg = CODE == kCode1Mad && NB >= 8;
    __shared__ float red[MatvecShape::kWaves][NB][16];

    const int tid = threadIdx.x;
    const int cq = tid & 3, rq = (tid >> 2) & 3, js = tid >> 4;
    const int lane = tid & 63, wave = tid >> 6;
    const int I = blockIdx.x;
    const int NTJ = N >> 4;
    const uint32_t* band = bits + (size_t)I * NTJ * Wd;
    // funnel shift that brings bit 8 cq of a row to the top (cq = 0: the row's first word)
    const int sh = (32 - 8 * cq) & 31;

    float acc[4][NB];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < NB; ++i) acc[a][i] = 0.0f;

    auto load_words = [&](int J, uint32_t (&w)[5]) {
        const uint32_t* sw = band + (size_t)J * Wd + 4 * rq;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = sw[q];
        w[4] = (TB && rq == 3) ? sw[-12] : sw[4];
    };
    uint32_t wn[5] = {0u, 0u, 0u, 0u, 0u};
    if (js < NTJ) load_words(js, wn);
    for (int J = js; J < NTJ; J += NJS) {
        uint32_t w[5];
#pragma unroll
        for (int q = 0; q < 5; ++q) w[q] = wn[q];
        if (J + NJS < NTJ) load_words(J + NJS, wn);
        // rows i >= batch re-read the last row: their sums are never stored, and the
        // products need no per-row guard
        float4 xv[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int ii = i < batch ? i : batch - 1;
            xv[i] = *reinterpret_cast<const float4*>(x + (size_t)ii * N + 16 * (size_t)J + 4 * cq);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            // bits [8 cq, 8 cq + 32) of row 4 rq + a
            const uint32_t f = cq == 0 ? w[a] : __builtin_amdgcn_alignbit(w[a], w[a + 1], sh);
            float wv[4];
#pragma unroll
            for (int b = 0; b < 4; ++b)
                wv[b] = code_raw<CODE, kSplitLcg>((f >> (32 - L - 2 * b)) & ((1u << L) - 1u), ca);
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                acc[a][i] = __builtin_fmaf(wv[0], xv[i].x, acc[a][i]);
                acc[a][i] = __builtin_fmaf(wv[1], xv[i].y, acc[a][i]);
                acc[a][i] = __builtin_fmaf(wv[2], xv[i].z, acc[a][i]);
                acc[a][i] = __builtin_fmaf(wv[3], xv[i].w, acc[a][i]);
            }
        }
    }

    // partial sums of row 4 rq + a: lanes differing in cq (bits 1:0) and tile (bits 5:4)
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        if (i < batch) {
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                float v = acc[a][i];
                v += __shfl_xor(v, 1, 64);
                v += __shfl_xor(v, 2, 64);
                v += __shfl_xor(v, 16, 64);
                v += __shfl_xor(v, 32, 64);
                if ((lane & 0x33) == 0) red[wave][i][4 * rq + a] = v;
            }
        }
    }
    __syncthreads();
    if (tid < 16 * batch) {
        const int i = tid >> 4, rr = tid & 15;
        float s = red[0][i][rr];
#pragma unroll
        for (int q = 1; q < MatvecShape::kWaves; ++q) s += red[q][i][rr];
        y[(size_t)i * M + 16 * I + rr] = code_rescale<CODE>(s);
    }
}

}  // namespace qtcq
