// decode.hpp -- parallel window decode of bitshift-trellis streams, gfx950.
//
// QTIP blog, "The trellis: a stateful codebook": the state at weight t is the L-bit
// window of the MSB-first stream starting at bit t*k, so every weight decodes on its
// own, with no graph and no serial walk.
//
// One workgroup decodes a tile of SB whole sequences (SB*T <= 4096 weights): the tile's
// stream words are staged in LDS (one coalesced read), then every thread decodes weights
// of the tile in flattened order -- a 64-bit funnel of the two words the window can
// touch, a shift and a mask, then the code -- and writes them coalesced.  When the MSE
// is wanted the same thread forms the step error against the (coalesced) target and
// leaves it in LDS; the path cost must be summed in t order to reproduce the encoder
// bit for bit, so after a barrier one thread per sequence adds its row sequentially.
#pragma once

#include "codes.hpp"

namespace qtcq {

// Tile geometry, shared by the kernel and its launcher.
struct DecodeTile {
    static constexpr int kThreads = 256;
    static constexpr int kMaxWeights = 4096;     // SB * T
    static constexpr int kBitsWords = 1024;      // bound on SB * W (L <= 16, T <= 4096)
    static constexpr int kErrFloats = 5888;      // bound on SB * err_stride(T)
    // sequences per tile: SB*T <= 4096 and one summing thread per sequence
    static int seqs(int T)
    {
        const int sb = kMaxWeights / T;
        return sb < 1 ? 1 : (sb > kThreads ? kThreads : sb);
    }
    // row stride of the step errors: a multiple of 4 (16-byte reads), offset by 4 words
    // per row so that the summing threads' reads fall in different banks
    __host__ __device__ static int err_stride(int T) { return ((T + 3) & ~3) + 4; }
    static size_t lds_bytes(int T, int W, bool with_mse)
    {
        const int sb = seqs(T);
        return 4 * (size_t)((with_mse ? sb * err_stride(T) : 0) + sb * W);
    }
};

// grid.x = ceil(B / SB), block = 256.  recon may be NULL (MSE only); mse may be NULL
// (decode only, MSE_ = false).  TB: tail-biting streams of exactly 2T bits, whose
// windows are read cyclically (a window running past the end continues at bit 0;
// 2T >= L, so it wraps at most once).
template <int L, int CODE, bool MSE_, bool WEIGHTED, bool TB = false>
__global__ void __launch_bounds__(DecodeTile::kThreads)
decode_tile(const uint32_t* __restrict__ bits, const float* __restrict__ seq,
            const float* __restrict__ wts, int64_t B, int T, int W, int SB,
            float* __restrict__ recon, float* __restrict__ mse, CodeArg ca)
{
    constexpr int NT = DecodeTile::kThreads;
    // dynamic LDS, DecodeTile::lds_bytes: step errors [SB][err_stride] (MSE only), then
    // the tile's stream words [SB][W]
    extern __shared__ __align__(16) char dyn_lds[];
    float* lerr = reinterpret_cast<float*>(dyn_lds);
    uint32_t* lbits = reinterpret_cast<uint32_t*>(dyn_lds) + (MSE_ ? SB * DecodeTile::err_stride(T) : 0);

    const int tid = threadIdx.x;
    const int64_t b0 = (int64_t)blockIdx.x * SB;
    const int n = (int)((B - b0) < SB ? (B - b0) : SB);
    const int total = n * T;                  // <= kMaxWeights: at most U per thread
    const int64_t base = b0 * T;
    constexpr int U = DecodeTile::kMaxWeights / NT;

    // every target (and weight) this thread needs, in flight before the staging barrier;
    // targets, weights and reconstructions are touched once, so they bypass the caches'
    // retention (non-temporal), which streams ~12% faster
    float sv[U], wv[U];
    if constexpr (MSE_) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = tid + u * NT;
            sv[u] = i < total ? __builtin_nontemporal_load(seq + base + i) : 0.0f;
            wv[u] = (WEIGHTED && i < total) ? __builtin_nontemporal_load(wts + base + i) : 1.0f;
        }
    }
    const int nw = n * W;
    const uint32_t* gb = bits + b0 * W;
    for (int i = tid; i < nw; i += NT) lbits[i] = gb[i];
    __syncthreads();

    const int ES = DecodeTile::err_stride(T);
    // flattened element i = r * T + t, advanced by NT per iteration without a division
    int r = tid / T, t = tid - r * T;
    const int dr = NT / T, dt = NT - dr * T;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = tid + u * NT;
        if (i >= total) break;
        const int p = 2 * t;                  // first stream bit of the window (k = 2)
        const int wi = p >> 5;
        const uint32_t hi = lbits[r * W + wi];
        const uint32_t lo = (wi + 1 < W) ? lbits[r * W + wi + 1] : 0u;
        // bits [p, p + 32) of the stream, then the top L of them
        const uint32_t top = __builtin_amdgcn_alignbit(hi, lo, (32 - (p & 31)) & 31);
        uint32_t win = ((p & 31) ? top : hi) >> (32 - L);
        if constexpr (TB) {
            const int nf = 2 * T - p;          // stream bits left from p
            if (nf < L) {                      // the first nf bits, then L - nf from bit 0
                const uint32_t head = lbits[r * W];
                win = ((((p & 31) ? top : hi) >> (32 - nf)) << (L - nf)) | (head >> (32 - (L - nf)));
            }
        }
        const float c = code_value<CODE>(win, ca);
        if (recon) __builtin_nontemporal_store(c, recon + base + i);
        if constexpr (MSE_) lerr[r * ES + t] = step_err<WEIGHTED>(c, sv[u], wv[u]);
        r += dr;
        t += dt;
        if (t >= T) { t -= T; ++r; }
    }
    if constexpr (MSE_) {
        __syncthreads();
        if (tid < n) {
            const float* e = lerr + tid * ES;
            float acc = 0.0f;
            int u = 0;
            for (; u + 4 <= T; u += 4) {
                const float4 q = *reinterpret_cast<const float4*>(e + u);
                acc = acc + q.x;
                acc = acc + q.y;
                acc = acc + q.z;
                acc = acc + q.w;
            }
            for (; u < T; ++u) acc = acc + e[u];
            mse[b0 + tid] = acc / (float)T;
        }
    }
}

// The same tile decode four consecutive weights at a time, for T % 4 == 0 and targets,
// weights and reconstructions 16-byte aligned: quad q of the tile is row q / (T/4),
// steps t0 .. t0 + 3 with t0 = 4 (q mod T/4).  Their windows start at bits 2 t0 .. 2 t0 + 6
// (2 t0 a multiple of 8), so one funnel of the two stream words around bit 2 t0 holds all
// four (L + 6 <= 32): one shift and mask each, instead of a funnel, two LDS reads and
// the index steps per weight.  Targets, weights and reconstructions move as float4, the
// step errors go to LDS as float4; the per-sequence sum in t order is decode_tile's.
// Tail-biting windows that run past the end of the stream (the last L/2 steps of a row)
// take their last bits from the head, as in decode_tile.  Same grid, block and LDS.
template <int L, int CODE, bool MSE_, bool WEIGHTED, bool TB = false>
__global__ void __launch_bounds__(DecodeTile::kThreads)
decode_tile4(const uint32_t* __restrict__ bits, const float* __restrict__ seq,
             const float* __restrict__ wts, int64_t B, int T, int W, int SB,
             float* __restrict__ recon, float* __restrict__ mse, CodeArg ca)
{
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int NT = DecodeTile::kThreads;
    extern __shared__ __align__(16) char dyn_lds[];
    float* lerr = reinterpret_cast<float*>(dyn_lds);
    uint32_t* lbits = reinterpret_cast<uint32_t*>(dyn_lds) + (MSE_ ? SB * DecodeTile::err_stride(T) : 0);

    const int tid = threadIdx.x;
    const int64_t b0 = (int64_t)blockIdx.x * SB;
    const int n = (int)((B - b0) < SB ? (B - b0) : SB);
    const int TQ = T >> 2;                    // quads per row
    const int nq = n * TQ;                    // <= kMaxWeights / 4: at most U per thread
    const int64_t base = b0 * T;
    constexpr int U = DecodeTile::kMaxWeights / 4 / NT;

    f4 sv[U], wv[U];
    if constexpr (MSE_) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = tid + u * NT;
            const f4 zero = {0.0f, 0.0f, 0.0f, 0.0f}, one = {1.0f, 1.0f, 1.0f, 1.0f};
            sv[u] = q < nq ? __builtin_nontemporal_load(reinterpret_cast<const f4*>(seq + base) + q) : zero;
            wv[u] = (WEIGHTED && q < nq) ? __builtin_nontemporal_load(reinterpret_cast<const f4*>(wts + base) + q) : one;
        }
    }
    const int nw = n * W;
    const uint32_t* gb = bits + b0 * W;
    for (int i = tid; i < nw; i += NT) lbits[i] = gb[i];
    __syncthreads();

    const int ES = DecodeTile::err_stride(T);
    int r = tid / TQ, tq = tid - r * TQ;      // quad q = r * TQ + tq, advanced by NT
    const int dr = NT / TQ, dq = NT - dr * TQ;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int q = tid + u * NT;
        if (q >= nq) break;
        const int t0 = 4 * tq;
        const int p = 2 * t0;                 // first stream bit of the quad's first window
        const int wi = p >> 5;
        const uint32_t hi = lbits[r * W + wi];
        const uint32_t lo = (wi + 1 < W) ? lbits[r * W + wi + 1] : 0u;
        const uint32_t f = (p & 31) ? __builtin_amdgcn_alignbit(hi, lo, 32 - (p & 31)) : hi;
        float c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t win = (f >> (32 - L - 2 * j)) & ((1u << L) - 1u);
            if constexpr (TB) {
                const int nf = 2 * T - (p + 2 * j);   // stream bits left from the window's start
                if (nf < L) {                          // the first nf bits, then L - nf from bit 0
                    const uint32_t head = lbits[r * W];
                    win = (((f << (2 * j)) >> (32 - nf)) << (L - nf)) | (head >> (32 - (L - nf)));
                }
            }
            c[j] = code_value<CODE>(win, ca);
        }
        if (recon) {
            const f4 cv = {c[0], c[1], c[2], c[3]};
            __builtin_nontemporal_store(cv, reinterpret_cast<f4*>(recon + base) + q);
        }
        if constexpr (MSE_) {
            const f4 e = {step_err<WEIGHTED>(c[0], sv[u].x, wv[u].x), step_err<WEIGHTED>(c[1], sv[u].y, wv[u].y),
                          step_err<WEIGHTED>(c[2], sv[u].z, wv[u].z), step_err<WEIGHTED>(c[3], sv[u].w, wv[u].w)};
            *reinterpret_cast<f4*>(lerr + r * ES + t0) = e;
        }
        r += dr;
        tq += dq;
        if (tq >= TQ) { tq -= TQ; ++r; }
    }
    if constexpr (MSE_) {
        __syncthreads();
        if (tid < n) {
            const float* e = lerr + tid * ES;
            float acc = 0.0f;
            int u = 0;
            for (; u + 4 <= T; u += 4) {
                const float4 qv = *reinterpret_cast<const float4*>(e + u);
                acc = acc + qv.x;
                acc = acc + qv.y;
                acc = acc + qv.z;
                acc = acc + qv.w;
            }
            mse[b0 + tid] = acc / (float)T;
        }
    }
}

// Code table: out[x] = code(x) for x < n.
template <int CODE>
__global__ void __launch_bounds__(256)
code_table_kernel(float* __restrict__ out, int64_t n, CodeArg ca)
{
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x < n) out[x] = code_value<CODE>((uint32_t)x, ca);
}

}  // namespace qtcq
