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
// not fit fp16, so each batch row i is cut into k-blocks of 32 columns, each scaled by
// a power of two 2^s (chosen from the block's largest magnitude, which lands in
// [2^14, 2^15)) and split into two fp16 parts, x' = x 2^s = xh + xl + d with
// xh = rn16(x'), xl = rn16(x' - xh) (the difference is exact in fp32) and
// |d| <= 2^-22 |x'| + 2^-25.  The 16 columns of one B operand (a fragment) hold xh of 8
// batch rows (columns 0..7) and their xl (columns 8..15), so one MFMA multiplies 16 rows
// x 32 columns of W by both parts of eight rows; up to four fragments (32 rows) share
// each decoded A operand.  A small first kernel writes the split, in the B operand's
// lane order, and the factors 2^-s to the workspace.
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
// Mapping.  One workgroup of 16 waves per band of 16 output rows (tile row I), or per two
// bands at wide batches on tall matrices (with the LDS code table, each resident
// workgroup loops over bands); wave w takes k-blocks w, w + 16, ...  Each MFMA starts
// from zero; its 4 outputs per lane, times the block's 2^-s (exact), are added to the
// lane's accumulators in k-block order by FMA; then hi + lo (lanes l and l ^ 8), the 16
// waves in sequence and the code's rescale.  Results are bit-deterministic and a one-hot x (its block scaled to 2^14,
// xl = 0) returns a column of W bit for bit.
//
// Rounding: with K = ceil(ceil(N / 32) / 16) k-blocks per wave, u = 2^-24, and allowing
// each addition inside an MFMA one unit in the last place (2u),
//   |y - W x| <= (4 + 62 + K + 1 + 15 + 2.5) u sum_n |W[m][n] x[n]|
//               + 2^-39 max_n |x[n]| sum_n |W[m][n]|
// to first order (no underflow: blocks whose largest |x| is below 2^-111 are scaled by
// at most 2^126 and keep less precision).
#pragma once

#include "codes.hpp"

namespace qtcq {

typedef _Float16 mv_half8 __attribute__((ext_vector_type(8)));
typedef _Float16 mv_half2 __attribute__((ext_vector_type(2)));
typedef float mv_float4 __attribute__((ext_vector_type(4)));

struct MatvecMfmaShape {
    static constexpr int kThreads = 1024;
    static constexpr int kWaves = kThreads / 64;
    // batch rows per B fragment (hi and lo of 8 rows fill its 16 columns) and fragments
    static constexpr int kRowsPerFrag = 8;
    static constexpr int kMaxFrags = 4;
    static constexpr int kMaxBatch = kRowsPerFrag * kMaxFrags;
    // one B fragment (32 columns of x for 8 rows): 64 lanes x 8 halves
    static constexpr size_t kBlockBytes = 64 * 16;
    // per fragment and k-block: 8 row scales 2^-s (float)
    static constexpr size_t kScaleBytes = 8 * 4;
    static constexpr int kSplitBlock = 256;
    // byte offsets into the workspace (at most twice its size) stay below 2^31
    static constexpr int kMaxN = 1 << 22;
    // uint32 words of one T = 256 stream: L + 2 * 255 bits, or 512 tail-biting
    template <int L, bool TB>
    static constexpr int stream_words() { return TB ? 16 : (L + 2 * 255 + 31) / 32; }
    __host__ __device__ static int kblocks(int N) { return (N / 16 + 1) / 2; }
    __host__ __device__ static int frags(int batch) { return (batch + kRowsPerFrag - 1) / kRowsPerFrag; }
    // workspace (sized for the largest batch): split x [nkb][frags][64 lanes][8 halves],
    // then float scale [nkb][frags][8]
    static size_t workspace_bytes(int N)
    {
        const size_t nkb = (size_t)kblocks(N);
        return ((nkb * kMaxFrags * (kBlockBytes + kScaleBytes) + 255) / 256) * 256 + 256;
    }
};

// Split of x into the B operand, one scale per batch row and k-block (32 columns).
//   grid.x = ceil(nkb * nf * 64 / kSplitBlock), block = kSplitBlock, nf = frags(batch);
//   thread t writes lane slot l = t % 64 of fragment f of k-block kb (t / 64 = kb nf + f),
//   i.e. the 8 halves B[8 g + e][j] (g = l / 16, j = l % 16): xh (j < 8) or xl (j >= 8)
//   of batch row 8 f + (j & 7) at columns 32 kb + 8 g + e, so a wave writes one
//   fragment's kilobyte contiguously.  The four slots of a (row, block) pair (g = 0..3)
//   are lanes 16 apart in one wave and share the block's maximum by two shuffles.
//   x [batch][N] (16-byte aligned, N a multiple of 16); xs [nkb][nf][64] 16-byte
//   fragments; sc [nkb][nf][8] the factor 2^-s of each row's block.  Columns k >= N (the
//   half k-block after an odd N / 16) are written as zero; slots of rows >= batch are not
//   written (the product kernel never reads them).
__global__ void __launch_bounds__(MatvecMfmaShape::kSplitBlock)
matvec_split_x(const float* __restrict__ x, int N, int nkb, int batch, uint4* __restrict__ xs,
               float* __restrict__ sc)
{
    const int nf = MatvecMfmaShape::frags(batch);
    const int t = blockIdx.x * MatvecMfmaShape::kSplitBlock + threadIdx.x;
    const int kf = t >> 6, l = t & 63, g = l >> 4, j = l & 15;
    const int kb = kf / nf, i = 8 * (kf - kb * nf) + (j & 7);
    // whole waves share (kb, f), and the shuffle partners (l ^ 16, l ^ 32) share i: a lane
    // that leaves here takes its partners with it
    if (kb >= nkb || i >= batch) return;
    const int n0 = 32 * kb + 8 * g;
    float v[8];
    if (n0 < N) {
        const float4* xr = reinterpret_cast<const float4*>(x + (size_t)i * N + n0);
        const float4 a = xr[0], b = xr[1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
    m = __builtin_fmaxf(m, __shfl_xor(m, 16, 64));
    m = __builtin_fmaxf(m, __shfl_xor(m, 32, 64));
    // max = f 2^e with f in [1/2, 1): x 2^(15 - e) has its largest magnitude in
    // [2^14, 2^15).  s <= 126 keeps the factor 2^-s a normal float (blocks below 2^-111
    // lose precision, as fp32 products there underflow anyway).  A zero or non-finite
    // maximum keeps s = 0 (non-finite inputs give non-finite outputs either way).
    int s = 0;
    if (m > 0.0f && m <= 3.402823466e38f) {
        s = 15 - __builtin_amdgcn_frexp_expf(m);
        s = s < 126 ? s : 126;
    }
    mv_half8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float xp = __builtin_ldexpf(v[e], s);
        const _Float16 hh = (_Float16)xp;                  // round to nearest even
        h[e] = j < 8 ? hh : (_Float16)(xp - (float)hh);    // the difference is exact
    }
    xs[(size_t)kf * 64 + l] = __builtin_bit_cast(uint4, h);
    if (l < 8) sc[(size_t)kf * 8 + l] = __builtin_ldexpf(1.0f, -s);
}

// A constant copied into a VGPR (opaque to the compiler, so it stays a VGPR operand).
__device__ __forceinline__ uint32_t vgpr_u32(uint32_t c)
{
    uint32_t v;
    asm("v_mov_b32 %0, %1" : "=v"(v) : "s"(c));
    return v;
}

// Two windows' codes before their rescale, as one packed pair of fp16.
//   kbias: fp16 -1534 in both halves, in a VGPR
template <int CODE>
__device__ __forceinline__ uint32_t code_raw_pair_f16(uint32_t w0, uint32_t w1, uint32_t kbias,
                                                      const CodeArg& ca)
{
    if constexpr (CODE == kCodeXor) {
        // palette values, exact in fp16 (so the round-toward-zero pack is exact)
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(code_xor(w0, ca), code_xor(w1, ca)));
    } else if constexpr (CODE == kCode1Mad) {
        // byte sums into both halves of an accumulator 0x64006400 (fp16 1024 twice):
        // v_sad_u8 adds S0 to the low half, v_sad_hi_u8 adds S1 << 16, so the halves read
        // 1024 + S0 and 1024 + S1 exactly (S <= 1020, no carry between them); one packed
        // fp16 subtraction of 1534 gives S - 510
        const uint32_t t0 = __builtin_amdgcn_sad_u8(lcg_step(w0), 0u, 0x64006400u);
        const uint32_t t = __builtin_amdgcn_sad_hi_u8(lcg_step(w1), 0u, t0);
        return __builtin_bit_cast(uint32_t, __builtin_bit_cast(mv_half2, t) + __builtin_bit_cast(mv_half2, kbias));
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

// grid.x = ceil((M / 16) / BANDS) (any grid.x >= 1 is correct: workgroup g takes band
// groups g, g + grid.x, ...), block = MatvecMfmaShape::kThreads.  bits
// [(M/16)(N/16)][Wd] with Wd = MatvecMfmaShape::stream_words<L, TB>(); xs, sc as written
// by matvec_split_x for this x; y [batch][M].  NF = frags(batch) B fragments per k-block.
// BANDS = 2: a workgroup takes bands 2 blockIdx.x and 2 blockIdx.x + 1 (the second may be
// absent when M / 16 is odd), and every B fragment it loads serves both, which halves
// the split x's reads from L2 at wide batches.
//
// TABLE: the workgroup first writes the code of every L-bit state (before its rescale, in
// fp16) into a 2^L-entry LDS table, then takes bands BANDS blockIdx.x, + BANDS gridDim.x,
// ... in turn, reading every window's code from the table: one LDS read and two and a
// half VALU operations (shift, mask, half a pack of two halves) per weight.  The values,
// the products and their order are those of the arithmetic decode, so results are the
// same bits.  It pays for the XOR palette
// code, whose arithmetic decode takes several times that; a random 16-bit LDS read costs
// the compute unit about as much as the 1MAD or 3INST arithmetic it would replace.
// Dynamic LDS (TABLE): mv_table_lds_bytes<L, NF, BANDS>(), of which the table is the
// first 2^(L+1) bytes.
template <int L, int NF, int BANDS>
constexpr size_t mv_table_lds_bytes()
{
    return ((size_t)2 << L) + sizeof(float) * MatvecMfmaShape::kWaves * BANDS * 8 * NF * 16;
}

template <int L, int CODE, bool TB, int NF, int BANDS, bool TABLE = false>
__global__ void __launch_bounds__(MatvecMfmaShape::kThreads)
decode_matvec_mfma(const uint32_t* __restrict__ bits, int M, int N,
                   const uint4* __restrict__ xs, const float* __restrict__ sc, int batch,
                   float* __restrict__ y, CodeArg ca)
{
    constexpr int NW = MatvecMfmaShape::kWaves;
    constexpr int Wd = MatvecMfmaShape::stream_words<L, TB>();
    constexpr int FB = (int)MatvecMfmaShape::kBlockBytes;     // bytes of one fragment
    constexpr int SB = (int)MatvecMfmaShape::kScaleBytes;     // bytes of its scales
    static_assert(NF >= 1 && NF <= MatvecMfmaShape::kMaxFrags, "fragments");
    static_assert(BANDS == 1 || BANDS == 2, "bands");
    // one MFMA result per band and fragment held back a k-block (hides its latency)
    // when there are few of them; with more, the later MFMAs cover the earlier ones
    constexpr bool DEFER = NF * BANDS <= 2;
    // per-wave partial sums; with a table they follow it in dynamic LDS, so the table
    // starts at LDS address 0 and a window's table address is just twice the window
    typedef float Red[NW][BANDS * 8 * NF][16];
    __shared__ float red_static[TABLE ? 1 : NW * BANDS * 8 * NF * 16];
    extern __shared__ __align__(16) uint32_t mv_table[];   // TABLE: 2^(L-1) fp16 pairs
    Red& red = *reinterpret_cast<Red*>(TABLE ? reinterpret_cast<float*>(mv_table + (1 << (L - 1)))
                                             : red_static);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 15, g = lane >> 4;
    const int NTJ = N >> 4, nkb = (NTJ + 1) >> 1;
    const int nbands = M >> 4;
    // loop-invariant operands held in VGPRs (an SGPR operand halves a VALU op's issue rate)
    const uint32_t kbias = vgpr_u32(0xE5FEE5FEu);   // fp16 -1534 in both halves
    if constexpr (TABLE) {
        // entry x holds the raw code of state x (pair e: states 2e, 2e + 1)
        if constexpr (CODE == kCodeXor) {
            xor_table_f16<L>(mv_table, ca, tid, MatvecMfmaShape::kThreads);
        } else {
            for (int e = tid; e < (1 << (L - 1)); e += MatvecMfmaShape::kThreads)
                mv_table[e] = code_raw_pair_f16<CODE>(2u * e, 2u * e + 1u, kbias, ca);
        }
        __syncthreads();
    }
    // the table read through a literal LDS address (the dynamic area starts at 0: the
    // kernel has no static LDS with TABLE), so the window times two is the whole address
    // and no base is added per read
    typedef const __attribute__((address_space(3))) _Float16 LdsHalf;
    LdsHalf* tab16 = reinterpret_cast<LdsHalf*>(static_cast<uintptr_t>(0));
    for (int I0 = BANDS * blockIdx.x; I0 < nbands; I0 += BANDS * gridDim.x) {
    // f = bits [16 (g & 1), + 32) of words (r, r + 1): alignbit(w_hi, w_lo, sh); for even
    // g the lane's "lo" word is word r itself and the shift is 0
    const uint32_t sh = (g & 1) ? 16u : 0u;
    const int o_hi = r;
    const int o_lo = (g & 1) ? ((TB && r == 15) ? 0 : r + 1) : r;
    // Both operands are read through buffer descriptors sized to each band's streams and
    // to the split x: an offset past the end reads as zero without touching memory.  So
    // the tile after the last one (the second half of the last k-block when N / 16 is
    // odd) decodes as the all-zero window, whose finite codes meet the zero columns
    // k >= N of the split x; the prefetch after a wave's last k-block reads zeros; the
    // lanes of the last fragment's rows beyond the batch start past the end; and an
    // absent second band has an empty descriptor.
    __amdgpu_buffer_rsrc_t wr[BANDS];
#pragma unroll
    for (int b = 0; b < BANDS; ++b) {
        const bool has = I0 + b < nbands;
        wr[b] = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint32_t*>(bits + (size_t)(has ? I0 + b : 0) * NTJ * Wd), (short)0,
            has ? NTJ * Wd * 4 : 0, kRawBufferWord3);
    }
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint4*>(xs), (short)0, nkb * NF * FB, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(sc), (short)0, nkb * NF * SB, kRawBufferWord3);
    // Byte offsets of k-block kb = wave + 2 NW j (tiles 2 kb and 2 kb + 1); the second
    // register set (kb + NW, 2 NW tiles further) adds a constant to the stream offsets
    // and has its own B and scale offsets.  Fragment f of a k-block is f FB (f SB) bytes
    // after fragment 0 (an immediate offset); the last fragment has offsets of its own,
    // past the end for the lanes of rows beyond the batch.
    constexpr int dstr = 4 * NW * Wd * 4;        // stream bytes of 2 NW k-blocks
    constexpr int dstr1 = 2 * NW * Wd * 4;       // of NW k-blocks
    const int dx = 2 * NF * FB * NW, dsc = 2 * NF * SB * NW;
    int oh = ((2 * wave + (g >> 1)) * Wd + o_hi) * 4;
    int ol = ((2 * wave + (g >> 1)) * Wd + o_lo) * 4;
    const bool live_last = 8 * (NF - 1) + (r & 7) < batch;
    int ob0 = wave * NF * FB + lane * 16;
    int ob1 = ob0 + NF * FB * NW;
    int obl0 = live_last ? ob0 + (NF - 1) * FB : nkb * NF * FB;
    int obl1 = obl0 + NF * FB * NW;
    int os0 = wave * NF * SB + (r & 7) * 4;
    int os1 = os0 + NF * SB * NW;
    int osl0 = live_last ? os0 + (NF - 1) * SB : nkb * NF * SB;
    int osl1 = osl0 + NF * SB * NW;
    struct Set { uint32_t wh[BANDS], wl[BANDS]; uint4 b[NF]; float sc[NF]; };
    auto load = [&](int d, int ob, int obl, int os, int osl, Set& q) {
#pragma unroll
        for (int b = 0; b < BANDS; ++b) {
            q.wh[b] = __builtin_amdgcn_raw_buffer_load_b32(wr[b], oh + d, 0, 0);
            q.wl[b] = __builtin_amdgcn_raw_buffer_load_b32(wr[b], ol + d, 0, 0);
        }
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int o = f == NF - 1 ? obl : ob + f * FB;
            const int os_ = f == NF - 1 ? osl : os + f * SB;
            q.b[f] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, o, 0, 0));
            q.sc[f] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, os_, 0, 0));
        }
    };
    // loop-invariant operands held in VGPRs (an SGPR operand halves a VALU op's issue rate)
    const uint32_t kbias = vgpr_u32(0xE5FEE5FEu);   // fp16 -1534 in both halves
    // Each MFMA's result, times its block's 2^-s (exact), is added to the accumulators
    // by FMA, in k-block order (DEFER: one k-block later, so its latency hides behind the
    // next block's decode).
    mv_float4 acc[BANDS][NF], pend[BANDS][NF];
    float pscl[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) {
#pragma unroll
        for (int b = 0; b < BANDS; ++b) {
            acc[b][f] = mv_float4{0.0f, 0.0f, 0.0f, 0.0f};
            pend[b][f] = mv_float4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        pscl[f] = 0.0f;
    }
    auto settle = [&]() {
#pragma unroll
        for (int b = 0; b < BANDS; ++b)
#pragma unroll
            for (int f = 0; f < NF; ++f)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[b][f][v] = __builtin_fmaf(pend[b][f][v], pscl[f], acc[b][f][v]);
    };
    auto step = [&](const Set& q) {
        mv_half8 av[BANDS];
#pragma unroll
        for (int b = 0; b < BANDS; ++b) {
            const uint32_t fw = __builtin_amdgcn_alignbit(q.wh[b], q.wl[b], sh);
            uint32_t a[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t w0 = (fw >> (32 - L - 4 * p)) & ((1u << L) - 1u);
                const uint32_t w1 = (fw >> (30 - L - 4 * p)) & ((1u << L) - 1u);
                if constexpr (TABLE) {
                    const mv_half2 h = {tab16[w0], tab16[w1]};
                    a[p] = __builtin_bit_cast(uint32_t, h);
                } else {
                    a[p] = code_raw_pair_f16<CODE>(w0, w1, kbias, ca);
                }
            }
            av[b] = __builtin_bit_cast(mv_half8, make_uint4(a[0], a[1], a[2], a[3]));
        }
        const mv_float4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (DEFER) settle();
#pragma unroll
        for (int f = 0; f < NF; ++f) {
#pragma unroll
            for (int b = 0; b < BANDS; ++b)
                pend[b][f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[b], __builtin_bit_cast(mv_half8, q.b[f]), zero, 0, 0, 0);
            pscl[f] = q.sc[f];
        }
        if constexpr (!DEFER) settle();
    };

    // two register sets, k-blocks alternating between them; no load is conditional
    if (wave < nkb) {
        Set q0, q1;
        int kb = wave;
        load(0, ob0, obl0, os0, osl0, q0);
        for (; kb + NW < nkb; kb += 2 * NW) {
            load(dstr1, ob1, obl1, os1, osl1, q1);
            step(q0);
            oh += dstr;
            ol += dstr;
            ob0 += dx;
            ob1 += dx;
            obl0 += dx;
            obl1 += dx;
            os0 += dsc;
            os1 += dsc;
            osl0 += dsc;
            osl1 += dsc;
            load(0, ob0, obl0, os0, osl0, q0);
            step(q1);
        }
        if (kb < nkb) step(q0);
        if constexpr (DEFER) settle();
    }

    // lane l holds rows 4 g + v of column r of each band's fragment f: xh products of
    // batch row 8 f + r (r < 8) or xl products of batch row 8 f + r - 8; add the two
    // parts, then the waves in order
#pragma unroll
    for (int b = 0; b < BANDS; ++b)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float s = acc[b][f][v] + __shfl_xor(acc[b][f][v], 8, 64);
                if (r < 8 && 8 * f + r < batch) red[wave][b * 8 * NF + 8 * f + r][4 * g + v] = s;
            }
    __syncthreads();
    for (int o = tid; o < BANDS * 16 * batch; o += MatvecMfmaShape::kThreads) {
        const int b = o / (16 * batch), io = o - b * 16 * batch;
        const int i = io >> 4, rr = io & 15;
        if (I0 + b >= nbands) continue;
        float s = red[0][b * 8 * NF + i][rr];
#pragma unroll
        for (int q = 1; q < NW; ++q) s += red[q][b * 8 * NF + i][rr];
        y[(size_t)i * M + 16 * (I0 + b) + rr] = code_rescale<CODE>(s);
    }
    if (I0 + BANDS * (int)gridDim.x < nbands) __syncthreads();   // red is rewritten next
    }
}

}  // namespace qtcq
