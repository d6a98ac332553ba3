// matvec_mfma.hpp -- decode -> matrix-vector product with the products on the matrix
// cores (v_mfma_f32_16x16x32_f16), gfx950.
//
// Same operation and tile numbering as decode_matvec (QTIP blog, "What it buys end to
// end": every 16x16 tile of W is one 256-long sequence decoded straight into the matrix
// operand; "The trellis: a stateful codebook": weight t of a sequence is the code of the
// stream window [2t, 2t + L)).  The VALU only decodes: the products and their sums move
// to the matrix cores, so at batch 8 the VALU no longer spends eight FMAs per weight.
//
// Operands.  The code before its rescale is exact in fp16 (1MAD: the integer S - 510,
// |S - 510| <= 510; 3INST: the fp16 sum itself), so W needs one fp16 operand.  x does
// not fit fp16, so each batch row i is scaled by a power of two 2^s_i (chosen from
// max_n |x[i][n]| so the largest element lands in [2^14, 2^15)) and split into two fp16
// parts, x' = x 2^s_i = xh + xl + d with xh = rn16(x'), xl = rn16(x' - xh) (the
// difference is exact in fp32) and |d| <= 2^-22 |x'| + 2^-25.  The 16 columns of the
// MFMA's B operand hold xh of batch rows 0..7 (columns 0..7) and xl (columns 8..15), so
// one MFMA multiplies 16 rows x 32 columns of W by both parts of all eight rows.  A
// small first kernel writes the split, in the B operand's lane order, to the workspace.
//
// Layout of v_mfma_f32_16x16x32_f16 (checked on the device): lane l holds
//   A[l % 16][8 (l / 16) + e], B[8 (l / 16) + e][l % 16] for e = 0..7, and
//   D[4 (l / 16) + v][l % 16] for v = 0..3.
// Here A row r = l % 16 is row 16 I + r of W and A column 8 g + e (g = l / 16) of k-block
// kb is column 32 kb + 8 g + e: tile J = 2 kb + (g >> 1), tile column 8 (g & 1) + e.
// That row's eight windows lie in stream bits [32 r + 16 (g & 1), + 14 + L), inside
// words r and r + 1 (word 16 of a tail-biting stream is word 0): one funnel shift and
// one bit-field extract per weight.
//
// Mapping.  One workgroup of 16 waves per band of 16 output rows (tile row I); wave w
// takes k-blocks w, w + 16, ...  Each MFMA starts from zero and its 4 outputs per lane
// are added to the lane's accumulators in k-block order; then hi + lo (lanes l and
// l ^ 8), the 16 waves in sequence, the power of two 2^-s_i (exact) and the code's
// rescale.  Results are bit-deterministic and a one-hot x (scale 2^14, xl = 0) returns
// a column of W bit for bit.
//
// Rounding: with K = ceil(ceil(N / 32) / 16) k-blocks per wave, u = 2^-24, and allowing
// each addition inside an MFMA one unit in the last place (2u),
//   |y - W x| <= (4 + 62 + K + 1 + 15 + 2.5) u sum_n |W[m][n] x[n]|
//               + 2^-39 max_n |x[n]| sum_n |W[m][n]|          (to first order).
#pragma once

#include "codes.hpp"

namespace qtcq {

typedef _Float16 mv_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 mv_half2 __attribute__((ext_vector_type(2)));
typedef float mv_float4 __attribute__((ext_vector_type(4)));

struct MatvecMfmaShape {
    static constexpr int kThreads = 1024;
    static constexpr int kWaves = kThreads / 64;
    static constexpr int kMaxBatch = 8;
    static constexpr int kSplitThreads = 1024;
    // one k-block (32 columns of x): the B operand of one MFMA, 64 lanes x 8 halves
    static constexpr size_t kBlockBytes = 64 * 16;
    static constexpr int kExpAlign = 256;
    // byte offsets into the split x stay below 2^31 (twice its size)
    static constexpr int kMaxN = 1 << 24;
    // workspace: [ceil(N/32)][64 lanes][8 halves] split x, then int s_i[8]
    static size_t workspace_bytes(int N)
    {
        const size_t nkb = (size_t)((N / 16 + 1) / 2);
        return nkb * kBlockBytes + kExpAlign;
    }
};

// Split of x into the B operand.  grid.x = batch, block = kSplitThreads.
//   x [batch][N] (16-byte aligned, N a multiple of 16); xs [nkb][64] 16-byte fragments;
//   sexp [batch] the exponent s_i.  Writes columns i (xh) and 8 + i (xl) of every
//   k-block; k >= N (the half k-block after an odd N / 16) is written as zero.
__global__ void __launch_bounds__(MatvecMfmaShape::kSplitThreads)
matvec_split_x(const float* __restrict__ x, int N, int nkb, uint4* __restrict__ xs,
               int* __restrict__ sexp)
{
    constexpr int NT = MatvecMfmaShape::kSplitThreads;
    __shared__ float wmax[NT / 64];
    const int i = blockIdx.x, tid = threadIdx.x;
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)i * N);
    const int ng = N >> 3;            // groups of 8 consecutive columns
    float m = 0.0f;
    for (int q = tid; q < ng; q += NT) {
        const float4 a = xr[2 * q], b = xr[2 * q + 1];
        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(a.x), __builtin_fabsf(a.y)),
                                               __builtin_fmaxf(__builtin_fabsf(a.z), __builtin_fabsf(a.w))));
        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(b.x), __builtin_fabsf(b.y)),
                                               __builtin_fmaxf(__builtin_fabsf(b.z), __builtin_fabsf(b.w))));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
    if ((tid & 63) == 0) wmax[tid >> 6] = m;
    __syncthreads();
    m = wmax[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) m = __builtin_fmaxf(m, wmax[w]);
    // max = f 2^e with f in [1/2, 1): x 2^(15 - e) has its largest magnitude in
    // [2^14, 2^15).  A zero or non-finite maximum keeps s = 0 (non-finite inputs give
    // non-finite outputs either way).
    int s = 0;
    if (m > 0.0f && m <= 3.402823466e38f) s = 15 - __builtin_amdgcn_frexp_expf(m);
    if (tid == 0) sexp[i] = s;

    for (int q = tid; q < 4 * nkb; q += NT) {
        float v[8];
        if (q < ng) {
            const float4 a = xr[2 * q], b = xr[2 * q + 1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
            v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0.0f;
        }
        mv_half8 h, l;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float xp = __builtin_ldexpf(v[e], s);
            const _Float16 hh = (_Float16)xp;          // round to nearest even
            h[e] = hh;
            l[e] = (_Float16)(xp - (float)hh);         // the difference is exact
        }
        const int kb = q >> 2, g = q & 3;
        xs[(size_t)kb * 64 + 16 * g + i] = __builtin_bit_cast(uint4, h);
        xs[(size_t)kb * 64 + 16 * g + 8 + i] = __builtin_bit_cast(uint4, l);
    }
}

// Two windows' codes before their rescale, as one packed pair of fp16.
template <int CODE>
__device__ __forceinline__ uint32_t code_raw_pair_f16(uint32_t w0, uint32_t w1)
{
    if constexpr (CODE == kCode1Mad) {
        // v_sad_u8 into an accumulator 0x6400 (fp16 1024): the halves read 1024 + S
        // exactly (S <= 1020), and one packed fp16 subtraction of 1534 gives S - 510
        const uint32_t t0 = __builtin_amdgcn_sad_u8(lcg_step(w0), 0u, 0x6400u);
        const uint32_t t1 = __builtin_amdgcn_sad_u8(lcg_step(w1), 0u, 0x6400u);
        const mv_half2 p = __builtin_bit_cast(mv_half2, t0 | (t1 << 16));
        const mv_half2 bias = {(_Float16)-1534.0f, (_Float16)-1534.0f};
        return __builtin_bit_cast(uint32_t, p + bias);
    } else {
        // the two halves of each (u & 0x8FFF8FFF) ^ 0x3B603B60, gathered as (lo0, lo1)
        // and (hi0, hi1), added by one packed fp16 add (round to nearest even)
        const uint32_t v0 = (lcg_step(w0) & 0x8FFF8FFFu) ^ 0x3B603B60u;
        const uint32_t v1 = (lcg_step(w1) & 0x8FFF8FFFu) ^ 0x3B603B60u;
        const uint32_t lo = __builtin_amdgcn_perm(v1, v0, 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(v1, v0, 0x07060302u);
        return __builtin_bit_cast(uint32_t, __builtin_bit_cast(mv_half2, hi) + __builtin_bit_cast(mv_half2, lo));
    }
}

// grid.x = M / 16, block = MatvecMfmaShape::kThreads.  bits [(M/16)(N/16)][Wd];
// xs, sexp as written by matvec_split_x for this x; y [batch][M].
template <int L, int CODE, bool TB>
__global__ void __launch_bounds__(MatvecMfmaShape::kThreads)
decode_matvec_mfma(const uint32_t* __restrict__ bits, int M, int N, int Wd,
                   const uint4* __restrict__ xs, const int* __restrict__ sexp, int batch,
                   float* __restrict__ y)
{
    constexpr int NW = MatvecMfmaShape::kWaves;
    __shared__ float red[NW][8][16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int I = blockIdx.x;
    const int NTJ = N >> 4, nkb = (NTJ + 1) >> 1;
    const uint32_t* band = bits + (size_t)I * NTJ * Wd;
    // f = bits [16 (g & 1), + 32) of words (r, r + 1): alignbit(w_hi, w_lo, sh); for even
    // g the lane's "lo" word is word r itself and the shift is 0
    const uint32_t sh = (g & 1) ? 16u : 0u;
    const int o_hi = r;
    const int o_lo = (g & 1) ? ((TB && r == 15) ? 0 : r + 1) : r;
    // The split x is read through a buffer descriptor sized to its k-blocks; the lanes
    // of batch rows beyond the batch read at an offset past that size, which the buffer
    // unit returns as zero without touching memory.
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint4*>(xs), (short)0, nkb * (int)MatvecMfmaShape::kBlockBytes, 0x00020000);
    const int boff = ((r & 7) < batch) ? lane * 16 : nkb * (int)MatvecMfmaShape::kBlockBytes;

    // Loads of k-block kb: the stream words of this lane's row and the B fragment.  A
    // tile past the last one (the second half of the last k-block after an odd N / 16)
    // is replaced by the last tile: its products meet the zero columns k >= N of x.
    // A k-block past the last one (prefetch after the last iteration) re-reads the last.
    auto load = [&](int kb, uint32_t& wh, uint32_t& wl, uint4& bx) {
        kb = kb < nkb ? kb : nkb - 1;
        int J = 2 * kb + (g >> 1);
        J = J < NTJ ? J : NTJ - 1;
        const uint32_t* sw = band + (size_t)J * Wd;
        wh = sw[o_hi];
        wl = sw[o_lo];
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, boff + kb * (int)MatvecMfmaShape::kBlockBytes, 0, 0);
        bx = __builtin_bit_cast(uint4, v);
    };
    mv_float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto step = [&](uint32_t wh, uint32_t wl, const uint4& bx) {
        const uint32_t f = __builtin_amdgcn_alignbit(wh, wl, sh);
        uint32_t a[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t w0 = (f >> (32 - L - 4 * p)) & ((1u << L) - 1u);
            const uint32_t w1 = (f >> (30 - L - 4 * p)) & ((1u << L) - 1u);
            a[p] = code_raw_pair_f16<CODE>(w0, w1);
        }
        const mv_half8 av = __builtin_bit_cast(mv_half8, make_uint4(a[0], a[1], a[2], a[3]));
        const mv_float4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        acc += __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(mv_half8, bx), zero, 0, 0, 0);
    };

    // two register sets, k-blocks alternating between them; every load is in range
    // (past the last k-block it re-reads the last), so none of them is conditional
    if (wave < nkb) {
        uint32_t h0, l0, h1, l1;
        uint4 b0, b1;
        int kb = wave;
        load(kb, h0, l0, b0);
        for (; kb + NW < nkb; kb += 2 * NW) {
            load(kb + NW, h1, l1, b1);
            step(h0, l0, b0);
            load(kb + 2 * NW, h0, l0, b0);
            step(h1, l1, b1);
        }
        if (kb < nkb) step(h0, l0, b0);
    }

    // lane l holds rows 4 g + v of column r: xh products of batch row r (r < 8) or xl
    // products of batch row r - 8; add the two parts, then the waves in order
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const float s = acc[v] + __shfl_xor(acc[v], 8, 64);
        if (r < batch) red[wave][r][4 * g + v] = s;
    }
    __syncthreads();
    if (tid < 16 * batch) {
        const int i = tid >> 4, rr = tid & 15;
        float s = red[0][i][rr];
#pragma unroll
        for (int q = 1; q < NW; ++q) s += red[q][i][rr];
        y[(size_t)i * M + 16 * I + rr] = code_rescale<CODE>(__builtin_ldexpf(s, -sexp[i]));
    }
}

}  // namespace qtcq
