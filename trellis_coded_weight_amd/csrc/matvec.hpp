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
// tail-biting stream is word 0 again), so a thread reads five words of its four rows,
// one funnel shift per row gives the bits of its four columns and each weight is a
// bit-field of that, then the code.  The thread needs x[16 J + 4 cq .. + 3] of each batch
// row (one float4) and accumulates its four rows by FMA in b order.  The products use the
// code before its rescale (1MAD: S - 510; 3INST: the fp16 sum -- both exact in binary32)
// and each output is rescaled once at the end (code_rescale: exact for any raw value, so
// a one-hot x still reproduces a column of W bit for bit).  The stream words of the next
// tile are loaded while the current one is decoded, into two register sets in turn.
// Partial sums of a row are then added in a fixed order (the 4 column groups and the 4
// tiles of a wave by xor-shuffles, then the 16 waves in sequence), so results are
// bit-deterministic, and a one-hot x reproduces a column of W exactly.
//
// Rounding: every output is a sum of N products; along its longest chain there are
// 4 * ceil((N/16) / NJS) FMAs, 4 shuffle additions and 15 wave additions; the raw code
// differs from W * D (D the code's divisor) by at most one rounding of W, and the final
// rescale adds at most 1.5 more, so
//     |y - W x| <= (4 ceil(N / (16 NJS)) + 22) * 2^-24 * sum_n |W[m][n] x[n]|  (to first order).
//
// This path is decode-ALU-bound on this chip, not HBM-bound: at 2 bits per weight the
// HBM streams ~3.2e13 weights/s, while the window, LCG, byte sum, conversion and FMA of a
// computed code take 6 VALU instructions per weight, mostly of the one-per-cycle kind:
// ~6 CU cycles per 64 weights, ~6.5e12 weights/s at 2.4 GHz on 256 CUs.  The
// products are fp32 VALU FMAs: fp32 MFMA runs at the same rate as fp32 VALU FMA here and
// an fp16 / bf16 MFMA would round the decoded weights.
#pragma once

#include "codes.hpp"

namespace qtcq {

typedef float mv4f __attribute__((ext_vector_type(4)));

struct MatvecShape {
    static constexpr int kThreads = 1024;
    static constexpr int kJSlots = kThreads / 16;   // NJS: tile columns in flight per band
    static constexpr int kWaves = kThreads / 64;
    static constexpr int kMaxBatch = 8;
    // columns: keeps the buffer descriptors' sizes and offsets within 32-bit integers
    static constexpr int kMaxN = 1 << 22;
};

// grid.x = M / 16, block = MatvecShape::kThreads.  bits [(M/16)(N/16)][Wd]; x [batch][N]
// (16-byte aligned); y [batch][M].  TB: tail-biting streams (Wd = 16, windows wrap).
// NB: batch rows the kernel is compiled for (1, 2, 4, 8), batch <= NB.
//
// TABLE (the XOR palette code): the workgroup first writes the code of every L-bit state
// in fp16 into a 2^L-entry LDS table (xor_table_f16), then takes bands blockIdx.x,
// + gridDim.x, ... in turn (any grid), reading each window's code from the table: one
// LDS read and a conversion per weight instead of the parity arithmetic.  The values,
// products and their order are the arithmetic decode's, so results are the same bits.
// Dynamic LDS: matvec_table_lds_bytes<L, NB>(), the table first, at LDS address 0.
template <int L, int NB>
constexpr size_t matvec_table_lds_bytes()
{
    return ((size_t)2 << L) + sizeof(float) * MatvecShape::kWaves * NB * 16;
}

template <int L, int CODE, bool TB, int NB, bool TABLE = false>
__global__ void __launch_bounds__(MatvecShape::kThreads)
decode_matvec(const uint32_t* __restrict__ bits, int M, int N, int Wd,
              const float* __restrict__ x, int batch, float* __restrict__ y, CodeArg ca)
{
    constexpr int NJS = MatvecShape::kJSlots;
    static_assert(NB >= 1 && NB <= MatvecShape::kMaxBatch, "batch width");
    static_assert(!TABLE || CODE == kCodeXor, "the LDS table serves the palette code");
    // the LCG's three-instruction form where it measured faster: 1MAD at eight rows
    // (132 against 146 us on 28672x8192); 3INST at eight rows is slower with it
    constexpr bool kSplitLcg = CODE == kCode1Mad && NB >= 8;
    // per-wave partial sums; with a table they follow it in dynamic LDS, so the table
    // starts at LDS address 0 and a window's table address is just twice the window
    typedef float Red[MatvecShape::kWaves][NB][16];
    __shared__ float red_static[TABLE ? 1 : MatvecShape::kWaves * NB * 16];
    extern __shared__ __align__(16) uint32_t mv_table[];   // TABLE: 2^(L-1) fp16 pairs
    Red& red = *reinterpret_cast<Red*>(TABLE ? reinterpret_cast<float*>(mv_table + (1 << (L - 1)))
                                             : red_static);

    const int tid = threadIdx.x;
    const int cq = tid & 3, rq = (tid >> 2) & 3, js = tid >> 4;
    const int lane = tid & 63, wave = tid >> 6;
    const int NTJ = N >> 4;
    if constexpr (TABLE) {
        xor_table_f16<L>(mv_table, ca, tid, MatvecShape::kThreads);
        __syncthreads();
    }
    typedef const __attribute__((address_space(3))) _Float16 LdsHalf;
    LdsHalf* tab16 = reinterpret_cast<LdsHalf*>(static_cast<uintptr_t>(0));

    // The four windows of row 4 rq + a in column quarter cq span row bits
    // [8 cq, 8 cq + 6 + L).  The funnel f_a holds row bits [8 cq - 4, 8 cq + 28): for
    // cq >= 1 the pair (word 4 rq + a, word 4 rq + a + 1) shifted by 36 - 8 cq, for cq = 0
    // the pair (word 4 rq + a - 1, word 4 rq + a) shifted by 4, whose first word only
    // lends f_a its top 4 bits, which no window reads.  So every lane takes
    // f_a = alignbit(v[a], v[a + 1], s) with its own five words v and one shift, and window
    // b of f_a sits 4 + 2 b bits below its top.  v[0] of a cq = 0 lane is therefore any
    // word: it reads word 4 rq.  Word 16 of a tail-biting stream is word 0 again.
    const int c1 = cq != 0 ? 1 : 0;
    // byte offsets of a lane's words within its tile
    const int o0 = 4 * (js * Wd + 4 * rq);                                  // v[0]
    const int o1 = o0 + 4 * c1;                                              // v[1..3]
    const int o4 = (TB && rq == 3 && c1) ? 4 * js * Wd : o1 + 12;           // v[4]
    const uint32_t s = (uint32_t)(36 - 8 * cq) & 31u;
    const int ox = 4 * (16 * js + 4 * cq);                                  // x[16 J + 4 cq]
    // The streams of the band and x are read through buffer descriptors: the lane offsets
    // above stay in registers, and a thread's k-th tile J = js + k NJS adds the uniform
    // k NJS Wd words (x: 16 k NJS floats) as the scalar offset, so stepping to the next
    // tile takes no vector instruction.  Every access is inside the descriptors' ranges.
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(x), (short)0, batch * N * 4, kRawBufferWord3);
    // tiles of this thread in a band (the loop below runs the workgroup's largest count,
    // so k and the scalar offsets are uniform; each lane works on its own tiles only)
    const int ntiles = js < NTJ ? (NTJ - js + NJS - 1) / NJS : 0;
    const int kmax = (NTJ + NJS - 1) / NJS;

    auto run_band = [&](int I) {
        const uint32_t* band = bits + (size_t)I * NTJ * Wd;
        const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t*>(band), (short)0, NTJ * Wd * 4, kRawBufferWord3);

        float acc[4][NB];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < NB; ++i) acc[a][i] = 0.0f;

        auto load_words = [&](int k, uint32_t (&v)[5]) {
            const int so = k * (NJS * Wd * 4);
            v[0] = __builtin_amdgcn_raw_buffer_load_b32(br, o0, so, 0);
            v[1] = __builtin_amdgcn_raw_buffer_load_b32(br, o1, so, 0);
            v[2] = __builtin_amdgcn_raw_buffer_load_b32(br, o1 + 4, so, 0);
            v[3] = __builtin_amdgcn_raw_buffer_load_b32(br, o1 + 8, so, 0);
            v[4] = __builtin_amdgcn_raw_buffer_load_b32(br, o4, so, 0);
        };
        auto tile = [&](int k, const uint32_t (&v)[5]) {
            // rows i >= batch re-read the last row: their sums are never stored, and the
            // products need no per-row guard
            mv4f xv[NB];
#pragma unroll
            for (int i = 0; i < NB; ++i) {
                const int ii = i < batch ? i : batch - 1;
                xv[i] = __builtin_bit_cast(mv4f, __builtin_amdgcn_raw_buffer_load_b128(
                    xr, ox, (ii * N + 16 * NJS * k) * 4, 0));
            }
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const uint32_t f = __builtin_amdgcn_alignbit(v[a], v[a + 1], s);
                float wv[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t win = (f >> (28 - L - 2 * b)) & ((1u << L) - 1u);
                    if constexpr (TABLE)
                        wv[b] = (float)tab16[win];
                    else
                        wv[b] = code_raw<CODE, kSplitLcg>(win, ca);
                }
#pragma unroll
                for (int i = 0; i < NB; ++i) {
                    acc[a][i] = __builtin_fmaf(wv[0], xv[i][0], acc[a][i]);
                    acc[a][i] = __builtin_fmaf(wv[1], xv[i][1], acc[a][i]);
                    acc[a][i] = __builtin_fmaf(wv[2], xv[i][2], acc[a][i]);
                    acc[a][i] = __builtin_fmaf(wv[3], xv[i][3], acc[a][i]);
                }
            }
        };
        // two word buffers in turn: the next tile's words load while this one decodes
        uint32_t va[5], vb[5];
        if (ntiles > 0) load_words(0, va);
        int k = 0;
        for (; k + 1 < kmax; k += 2) {
            if (k + 1 < ntiles) load_words(k + 1, vb);
            if (k < ntiles) tile(k, va);
            if (k + 2 < ntiles) load_words(k + 2, va);
            if (k + 1 < ntiles) tile(k + 1, vb);
        }
        if (k < ntiles) tile(k, va);

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
            float sum = red[0][i][rr];
#pragma unroll
            for (int q = 1; q < MatvecShape::kWaves; ++q) sum += red[q][i][rr];
            y[(size_t)i * M + 16 * I + rr] = code_rescale<CODE>(sum);
        }
    };

    if constexpr (TABLE) {
        const int nbands = M >> 4;
        for (int I = blockIdx.x; I < nbands; I += gridDim.x) {
            run_band(I);
            if (I + (int)gridDim.x < nbands) __syncthreads();   // red is rewritten next
        }
    } else {
        run_band(blockIdx.x);
    }
}

}  // namespace qtcq
