// decode.hpp -- parallel window decode of bitshift-trellis streams, gfx950.
//
// QTIP blog, "The trellis: a stateful codebook": the state at weight t is the L-bit
// window of the MSB-first stream starting at bit t*k, so every weight decodes on its
// own, with no graph and no serial walk.  One thread per weight: a 64-bit funnel of
// the two stream words the window can touch, a shift and a mask, then the code.
//
// The path cost of the reconstruction (the encoder's mse) must be summed in t order to
// reproduce the encoder bit for bit, so it runs as its own kernel with one thread per
// sequence that slides the window along the stream.
#pragma once

#include "codes.hpp"

namespace qtcq {

template <int L, int CODE>
__global__ void __launch_bounds__(256)
window_decode(const uint32_t* __restrict__ bits, int64_t total, int T, int W,
              float* __restrict__ recon)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= total) return;
    const int64_t b = idx / T;
    const int t = (int)(idx - b * T);
    const int p = 2 * t;                 // first stream bit of the window (k = 2)
    const int wi = p >> 5;
    const uint32_t* row = bits + b * W;
    const uint64_t hi = row[wi];
    const uint64_t lo = (wi + 1 < W) ? row[wi + 1] : 0u;
    const uint64_t f = (hi << 32) | lo;
    const uint32_t win = (uint32_t)(f >> (64 - (p & 31) - L)) & ((1u << L) - 1u);
    recon[idx] = code_value<CODE>(win);
}

// One thread per sequence: walks its stream's windows in t order (each new window is
// the previous one shifted left by 2 with the next 2 stream bits entering at the
// bottom) and sums the binary32 path cost against seq (and weights), divided by T.
template <int L, int CODE, bool WEIGHTED>
__global__ void __launch_bounds__(256)
decode_path_mse(const uint32_t* __restrict__ bits, const float* __restrict__ seq,
                const float* __restrict__ wts, int64_t B, int T, int W, float* __restrict__ mse)
{
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const uint32_t* row = bits + b * W;
    const float* s = seq + b * T;
    const float* w = WEIGHTED ? wts + b * T : nullptr;
    uint32_t word = row[0];
    uint32_t win = word >> (32 - L);
    int p = L;                                 // next unread stream bit
    float acc = 0.0f;
    for (int t = 0; t < T; ++t) {
        if (t > 0) {
            if ((p & 31) == 0) word = row[p >> 5];
            const uint32_t nb = (word >> (30 - (p & 31))) & 3u;
            win = ((win << 2) | nb) & ((1u << L) - 1u);
            p += 2;
        }
        acc = acc + step_err<WEIGHTED>(code_value<CODE>(win), s[t], WEIGHTED ? w[t] : 1.0f);
    }
    mse[b] = acc / (float)T;
}

// Code table: out[x] = code(x) for x < n.
template <int CODE>
__global__ void __launch_bounds__(256)
code_table_kernel(float* __restrict__ out, int64_t n)
{
    const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (x < n) out[x] = code_value<CODE>((uint32_t)x);
}

}  // namespace qtcq
