// qtcq.hip -- host side of the C ABI declared in include/qtcq.h: argument validation,
// workspace sizing, batch chunking and kernel launches on the caller's stream.
// Everything the path computes runs in the kernels included below.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "qtcq.h"
#include "codes.hpp"
#include "viterbi.hpp"
#include "decode.hpp"
#include "bcjr.hpp"
#include "bcjr_vjp.hpp"
#include "matvec.hpp"
#include "matvec_mfma.hpp"

namespace {

using namespace qtcq;

constexpr int kMaxT = 4096;
static_assert(kMaxT <= kBcjrMaxT, "the BCJR kernels stage T per-step values in LDS");

bool supported_trellis(int L, int k)
{
    return k == 2 && L >= 6 && L <= 16 && (L % 2) == 0;
}

bool valid_code(int code) { return code == QTCQ_CODE_1MAD || code == QTCQ_CODE_3INST; }

int64_t stream_words(int L, int k, int T)
{
    return ((int64_t)L + (int64_t)k * (T - 1) + 31) / 32;
}

// tail-biting: exactly k*T bits, and at least one window long
bool tailbiting_ok(int L, int k, int T) { return (int64_t)k * T >= L; }
int64_t tb_stream_words(int k, int T) { return ((int64_t)k * T + 31) / 32; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

qtcq_status launch_status()
{
    return hipGetLastError() == hipSuccess ? QTCQ_OK : QTCQ_ERR_DEVICE;
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

// ---- encode ------------------------------------------------------------------------

size_t encode_bytes_per_seq(int T, int L)
{
    // backpointer words per step = 2^(L-6); final state + final cost
    const size_t words = (size_t)(T - 1) * ((size_t)1 << (L - 6));
    return words * 4 + 8;
}

template <int L, int CODE, bool W>
qtcq_status encode_chunk(const float* seq, const float* w, int64_t b0, int64_t n, int T,
                         uint32_t* bits, float* mse, uint32_t* states, char* ws, hipStream_t st)
{
    using Tr = Trellis<L>;
    uint32_t* bp = reinterpret_cast<uint32_t*>(ws);
    uint32_t* fin = bp + (size_t)n * (T - 1) * Tr::kBpWords;
    float* fin_cost = reinterpret_cast<float*>(fin + n);
    hipLaunchKernelGGL((viterbi_forward<L, CODE, W>), dim3((unsigned)((n + 1) / 2)), dim3(Tr::kThreads),
                       0, st, seq, w, T, b0, n, 0, nullptr, bp, fin, fin_cost, mse);
    qtcq_status rc = launch_status();
    if (rc != QTCQ_OK) return rc;
    const int Wd = (int)stream_words(L, 2, T);
    hipLaunchKernelGGL((viterbi_traceback<L>), dim3(blocks_for(n, 256)), dim3(256), 0, st,
                       bp, fin, T, n, b0, Wd, bits, states);
    return launch_status();
}

template <int L, int CODE, bool W>
qtcq_status encode_all(const float* seq, const float* w, int64_t B, int T, uint32_t* bits,
                       float* mse, uint32_t* states, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t per_chunk = (int64_t)(ws_bytes / encode_bytes_per_seq(T, L));
    for (int64_t b0 = 0; b0 < B; b0 += per_chunk) {
        const int64_t n = (B - b0 < per_chunk) ? B - b0 : per_chunk;
        qtcq_status rc = encode_chunk<L, CODE, W>(seq, w, b0, n, T, bits, mse, states,
                                                  static_cast<char*>(ws), st);
        if (rc != QTCQ_OK) return rc;
    }
    return QTCQ_OK;
}

// ---- tail-biting encode -------------------------------------------------------------
// Two searches per sequence: the free-start search over the targets rotated by T/2, the
// seam (the overlap read off the state of original position 0), then the search over
// the original targets with both ends pinned to the overlap, traced back and packed
// as a 2T-bit cyclic stream.  Workspace per sequence: the encode layout plus the
// overlap word.

size_t tb_bytes_per_seq(int T, int L) { return encode_bytes_per_seq(T, L) + 4; }

template <int L, int CODE, bool W>
qtcq_status tb_chunk(const float* seq, const float* w, int64_t b0, int64_t n, int T,
                     uint32_t* bits, float* mse, uint32_t* states, char* ws, hipStream_t st)
{
    using Tr = Trellis<L>;
    uint32_t* bp = reinterpret_cast<uint32_t*>(ws);
    uint32_t* fin = bp + (size_t)n * (T - 1) * Tr::kBpWords;
    float* fin_cost = reinterpret_cast<float*>(fin + n);
    uint32_t* overlap = reinterpret_cast<uint32_t*>(fin_cost + n);
    const dim3 grid((unsigned)((n + 1) / 2)), block(Tr::kThreads);
    const int rot = T / 2;
    hipLaunchKernelGGL((viterbi_forward<L, CODE, W, false>), grid, block, 0, st, seq, w, T, b0, n,
                       rot, nullptr, bp, fin, fin_cost, nullptr);
    qtcq_status rc = launch_status();
    if (rc != QTCQ_OK) return rc;
    hipLaunchKernelGGL((viterbi_seam<L>), dim3(blocks_for(n, 256)), dim3(256), 0, st, bp, fin, T, n,
                       (T - rot) % T, overlap);
    rc = launch_status();
    if (rc != QTCQ_OK) return rc;
    hipLaunchKernelGGL((viterbi_forward<L, CODE, W, true>), grid, block, 0, st, seq, w, T, b0, n, 0,
                       overlap, bp, fin, fin_cost, mse);
    rc = launch_status();
    if (rc != QTCQ_OK) return rc;
    hipLaunchKernelGGL((viterbi_traceback<L, true>), dim3(blocks_for(n, 256)), dim3(256), 0, st,
                       bp, fin, T, n, b0, (int)tb_stream_words(2, T), bits, states);
    return launch_status();
}

template <int L, int CODE, bool W>
qtcq_status tb_all(const float* seq, const float* w, int64_t B, int T, uint32_t* bits,
                   float* mse, uint32_t* states, void* ws, size_t ws_bytes, hipStream_t st)
{
    const int64_t per_chunk = (int64_t)(ws_bytes / tb_bytes_per_seq(T, L));
    for (int64_t b0 = 0; b0 < B; b0 += per_chunk) {
        const int64_t n = (B - b0 < per_chunk) ? B - b0 : per_chunk;
        qtcq_status rc = tb_chunk<L, CODE, W>(seq, w, b0, n, T, bits, mse, states,
                                              static_cast<char*>(ws), st);
        if (rc != QTCQ_OK) return rc;
    }
    return QTCQ_OK;
}

template <int L>
qtcq_status tb_dispatch_code(int code, bool weighted, const float* seq, const float* w,
                             int64_t B, int T, uint32_t* bits, float* mse, uint32_t* states,
                             void* ws, size_t wsb, hipStream_t st)
{
    if (code == QTCQ_CODE_1MAD)
        return weighted ? tb_all<L, kCode1Mad, true>(seq, w, B, T, bits, mse, states, ws, wsb, st)
                        : tb_all<L, kCode1Mad, false>(seq, w, B, T, bits, mse, states, ws, wsb, st);
    return weighted ? tb_all<L, kCode3Inst, true>(seq, w, B, T, bits, mse, states, ws, wsb, st)
                    : tb_all<L, kCode3Inst, false>(seq, w, B, T, bits, mse, states, ws, wsb, st);
}

template <int L>
qtcq_status encode_dispatch_code(int code, bool weighted, const float* seq, const float* w,
                                 int64_t B, int T, uint32_t* bits, float* mse, uint32_t* states,
                                 void* ws, size_t wsb, hipStream_t st)
{
    if (code == QTCQ_CODE_1MAD)
        return weighted ? encode_all<L, kCode1Mad, true>(seq, w, B, T, bits, mse, states, ws, wsb, st)
                        : encode_all<L, kCode1Mad, false>(seq, w, B, T, bits, mse, states, ws, wsb, st);
    return weighted ? encode_all<L, kCode3Inst, true>(seq, w, B, T, bits, mse, states, ws, wsb, st)
                    : encode_all<L, kCode3Inst, false>(seq, w, B, T, bits, mse, states, ws, wsb, st);
}

// ---- decode ------------------------------------------------------------------------

template <int L, int CODE, bool TB>
qtcq_status decode_impl(const uint32_t* bits, int64_t B, int T, float* recon, const float* seq,
                        const float* w, float* mse, hipStream_t st)
{
    const int Wd = (int)(TB ? tb_stream_words(2, T) : stream_words(L, 2, T));
    const int SB = DecodeTile::seqs(T);
    if (SB * Wd > DecodeTile::kBitsWords || SB * DecodeTile::err_stride(T) > DecodeTile::kErrFloats)
        return QTCQ_ERR_UNSUPPORTED;      // not reachable for T <= 4096, L <= 16
    const dim3 grid(blocks_for(B, SB)), block(DecodeTile::kThreads);
    const size_t lds = DecodeTile::lds_bytes(T, Wd, mse != nullptr);
    if (!mse)
        hipLaunchKernelGGL((decode_tile<L, CODE, false, false, TB>), grid, block, lds, st, bits,
                           seq, w, B, T, Wd, SB, recon, mse);
    else if (w)
        hipLaunchKernelGGL((decode_tile<L, CODE, true, true, TB>), grid, block, lds, st, bits, seq,
                           w, B, T, Wd, SB, recon, mse);
    else
        hipLaunchKernelGGL((decode_tile<L, CODE, true, false, TB>), grid, block, lds, st, bits,
                           seq, w, B, T, Wd, SB, recon, mse);
    return launch_status();
}

template <int L>
qtcq_status decode_dispatch_code(int code, bool tb, const uint32_t* bits, int64_t B, int T,
                                 float* recon, const float* seq, const float* w, float* mse,
                                 hipStream_t st)
{
    if (code == QTCQ_CODE_1MAD)
        return tb ? decode_impl<L, kCode1Mad, true>(bits, B, T, recon, seq, w, mse, st)
                  : decode_impl<L, kCode1Mad, false>(bits, B, T, recon, seq, w, mse, st);
    return tb ? decode_impl<L, kCode3Inst, true>(bits, B, T, recon, seq, w, mse, st)
              : decode_impl<L, kCode3Inst, false>(bits, B, T, recon, seq, w, mse, st);
}

// ---- bcjr --------------------------------------------------------------------------

template <int L, int CODE, bool W>
qtcq_status bcjr_all(const float* seq, const float* w, int64_t B, int T, float temperature,
                     float* soft, float* log_z, void* ws, size_t ws_bytes, hipStream_t st)
{
    using Tr = Trellis<L>;
    const size_t per = BcjrLayout<L>::bytes_per_seq(T);
    const int64_t per_chunk = (int64_t)(ws_bytes / per);
    const double kappa = 1.4426950408889634074 / (double)temperature;   // log2(e) / tau
    char* wsc = static_cast<char*>(ws);
    for (int64_t b0 = 0; b0 < B; b0 += per_chunk) {
        const int64_t n = (B - b0 < per_chunk) ? B - b0 : per_chunk;
        hipLaunchKernelGGL((bcjr_sweep<L, CODE, W>), dim3((unsigned)n), dim3(Tr::kThreads), 0, st,
                           seq, w, T, b0, kappa, wsc);
        qtcq_status rc = launch_status();
        if (rc != QTCQ_OK) return rc;
        hipLaunchKernelGGL((bcjr_finalize<L>), dim3(blocks_for(n * T, 256)), dim3(256), 0, st,
                           wsc, per, T, n, b0, soft, log_z);
        rc = launch_status();
        if (rc != QTCQ_OK) return rc;
    }
    return QTCQ_OK;
}

// ---- BCJR gradient (vector-Jacobian product) ------------------------------------------
// Per chunk: the soft pass in VJP mode (stashes both message directions and the posterior
// offsets), its finalize when soft / log Z are wanted, the Phi / Psi sweep, the gradient.
// Below tau = 0.01 the stashes keep fp64 values (WIDE); the 32-bit stash's fp32 range
// below -1024 log2 units is too coarse for the states the backward messages lift there.
constexpr float kWideStashBelowTau = 0.01f;

template <int L, int CODE, bool W, bool WIDE>
qtcq_status vjp_all(const float* seq, const float* w, const float* gup, int64_t B, int T,
                    float temperature, float* grad, float* soft, float* log_z, void* ws,
                    size_t ws_bytes, hipStream_t st)
{
    using Tr = Trellis<L>;
    const size_t per = BcjrLayout<L>::bytes_per_seq_vjp(T);
    const int64_t per_chunk = (int64_t)(ws_bytes / per);
    const double kappa = 1.4426950408889634074 / (double)temperature;
    const double two_over_tau = 2.0 / (double)temperature;
    char* wsc = static_cast<char*>(ws);
    for (int64_t b0 = 0; b0 < B; b0 += per_chunk) {
        const int64_t n = (B - b0 < per_chunk) ? B - b0 : per_chunk;
        hipLaunchKernelGGL((bcjr_sweep<L, CODE, W, true, WIDE>), dim3((unsigned)n), dim3(Tr::kThreads), 0,
                           st, seq, w, T, b0, kappa, wsc);
        qtcq_status rc = launch_status();
        if (rc != QTCQ_OK) return rc;
        if (soft || log_z) {
            hipLaunchKernelGGL((bcjr_finalize<L>), dim3(blocks_for(n * T, 256)), dim3(256), 0, st,
                               wsc, per, T, n, b0, soft, log_z);
            rc = launch_status();
            if (rc != QTCQ_OK) return rc;
        }
        hipLaunchKernelGGL((bcjr_vjp_sweep<L, CODE, W, WIDE>), dim3((unsigned)n), dim3(Tr::kThreads), 0,
                           st, seq, w, gup, T, b0, kappa, wsc);
        rc = launch_status();
        if (rc != QTCQ_OK) return rc;
        hipLaunchKernelGGL((bcjr_vjp_finalize<L>), dim3(blocks_for(n * T, 256)), dim3(256), 0, st,
                           wsc, w, T, n, b0, two_over_tau, grad);
        rc = launch_status();
        if (rc != QTCQ_OK) return rc;
    }
    return QTCQ_OK;
}

template <int L>
qtcq_status vjp_dispatch_code(int code, bool weighted, const float* seq, const float* w,
                              const float* gup, int64_t B, int T, float temperature, float* grad,
                              float* soft, float* log_z, void* ws, size_t wsb, hipStream_t st)
{
#define QTCQ_VJP(C_, W_) (temperature < kWideStashBelowTau                                              \
        ? vjp_all<L, C_, W_, true>(seq, w, gup, B, T, temperature, grad, soft, log_z, ws, wsb, st)      \
        : vjp_all<L, C_, W_, false>(seq, w, gup, B, T, temperature, grad, soft, log_z, ws, wsb, st))
    if (code == QTCQ_CODE_1MAD)
        return weighted ? QTCQ_VJP(kCode1Mad, true) : QTCQ_VJP(kCode1Mad, false);
    return weighted ? QTCQ_VJP(kCode3Inst, true) : QTCQ_VJP(kCode3Inst, false);
#undef QTCQ_VJP
}

template <int L>
qtcq_status bcjr_dispatch_code(int code, bool weighted, const float* seq, const float* w,
                               int64_t B, int T, float temperature, float* soft, float* log_z,
                               void* ws, size_t wsb, hipStream_t st)
{
    if (code == QTCQ_CODE_1MAD)
        return weighted ? bcjr_all<L, kCode1Mad, true>(seq, w, B, T, temperature, soft, log_z, ws, wsb, st)
                        : bcjr_all<L, kCode1Mad, false>(seq, w, B, T, temperature, soft, log_z, ws, wsb, st);
    return weighted ? bcjr_all<L, kCode3Inst, true>(seq, w, B, T, temperature, soft, log_z, ws, wsb, st)
                    : bcjr_all<L, kCode3Inst, false>(seq, w, B, T, temperature, soft, log_z, ws, wsb, st);
}

// L dispatch: instantiate every supported trellis size.
template <template <int> class F, typename... Args>
qtcq_status by_L(int L, Args&&... args)
{
    switch (L) {
    case 6: return F<6>::run(args...);
    case 8: return F<8>::run(args...);
    case 10: return F<10>::run(args...);
    case 12: return F<12>::run(args...);
    case 14: return F<14>::run(args...);
    case 16: return F<16>::run(args...);
    default: return QTCQ_ERR_UNSUPPORTED;
    }
}

// ---- decode -> matrix-vector product --------------------------------------------------

template <int L, int CODE, bool TB>
qtcq_status matvec_impl(const uint32_t* bits, int M, int N, const float* x, int batch, float* y,
                        hipStream_t st)
{
    const int Wd = (int)(TB ? tb_stream_words(2, 256) : stream_words(L, 2, 256));
    const dim3 grid((unsigned)(M / 16)), block(MatvecShape::kThreads);
    if (batch <= 1)
        hipLaunchKernelGGL((decode_matvec<L, CODE, TB, 1>), grid, block, 0, st, bits, M, N, Wd, x, batch, y);
    else if (batch <= 2)
        hipLaunchKernelGGL((decode_matvec<L, CODE, TB, 2>), grid, block, 0, st, bits, M, N, Wd, x, batch, y);
    else if (batch <= 4)
        hipLaunchKernelGGL((decode_matvec<L, CODE, TB, 4>), grid, block, 0, st, bits, M, N, Wd, x, batch, y);
    else
        hipLaunchKernelGGL((decode_matvec<L, CODE, TB, 8>), grid, block, 0, st, bits, M, N, Wd, x, batch, y);
    return launch_status();
}

template <int L>
qtcq_status matvec_dispatch_code(int code, bool tb, const uint32_t* bits, int M, int N,
                                 const float* x, int batch, float* y, hipStream_t st)
{
    if (code == QTCQ_CODE_1MAD)
        return tb ? matvec_impl<L, kCode1Mad, true>(bits, M, N, x, batch, y, st)
                  : matvec_impl<L, kCode1Mad, false>(bits, M, N, x, batch, y, st);
    return tb ? matvec_impl<L, kCode3Inst, true>(bits, M, N, x, batch, y, st)
              : matvec_impl<L, kCode3Inst, false>(bits, M, N, x, batch, y, st);
}

// the split x of the matrix-core product: fragments, then block scales, in the workspace
uint4* split_frags(void* ws) { return static_cast<uint4*>(ws); }
float* split_scales(void* ws, int N, int batch)
{
    return reinterpret_cast<float*>(static_cast<char*>(ws) + (size_t)MatvecMfmaShape::kblocks(N) *
                                    MatvecMfmaShape::frags(batch) * MatvecMfmaShape::kBlockBytes);
}

qtcq_status split_x_launch(const float* x, int N, int batch, void* ws, hipStream_t st)
{
    const int nkb = MatvecMfmaShape::kblocks(N);
    if (nkb == 0) return QTCQ_OK;
    const int threads = nkb * MatvecMfmaShape::frags(batch) * 64;
    const int bs = MatvecMfmaShape::kSplitBlock;
    hipLaunchKernelGGL(matvec_split_x, dim3((unsigned)((threads + bs - 1) / bs)), dim3(bs), 0, st,
                       x, N, nkb, batch, split_frags(ws), split_scales(ws, N, batch));
    return launch_status();
}

// the same product with the decoded weights and the split x on the matrix cores; x ==
// nullptr: the workspace already holds the split of this (N, batch)
template <int L, int CODE, bool TB>
qtcq_status matvec_mfma_impl(const uint32_t* bits, int M, int N, const float* x, int batch,
                             float* y, void* workspace, hipStream_t st)
{
    static_assert(MatvecMfmaShape::stream_words<L, TB>() == (TB ? 16 : 17), "stream words");
    const int nf = MatvecMfmaShape::frags(batch);
    if (x) {
        const qtcq_status rc = split_x_launch(x, N, batch, workspace, st);
        if (rc != QTCQ_OK) return rc;
    }
    const uint4* xs = split_frags(workspace);
    const float* sc = split_scales(workspace, N, batch);
    // Two bands per workgroup once the batch spans three or four fragments (reading the
    // split x then dominates: each fragment costs a kilobyte per k-block and wave) and
    // M / 16 >= 1024, so the grid keeps >= 512 workgroups (two per CU).  Results do not
    // depend on the choice (same arithmetic, same order).
    const int nb = M / 16;
    const bool two = nf >= 3 && nb >= 1024;
    const dim3 grid1((unsigned)nb), grid2((unsigned)((nb + 1) / 2)), block(MatvecMfmaShape::kThreads);
#define QTCQ_MV(NF_, B_, G_) hipLaunchKernelGGL((decode_matvec_mfma<L, CODE, TB, NF_, B_>), G_, block, 0, st, \
                                               bits, M, N, xs, sc, batch, y)
    switch (nf) {
    case 1: QTCQ_MV(1, 1, grid1); break;
    case 2: if (two) QTCQ_MV(2, 2, grid2); else QTCQ_MV(2, 1, grid1); break;
    case 3: if (two) QTCQ_MV(3, 2, grid2); else QTCQ_MV(3, 1, grid1); break;
    default: if (two) QTCQ_MV(4, 2, grid2); else QTCQ_MV(4, 1, grid1); break;
    }
#undef QTCQ_MV
    return launch_status();
}

template <int L>
qtcq_status matvec_mfma_dispatch_code(int code, bool tb, const uint32_t* bits, int M, int N,
                                      const float* x, int batch, float* y, void* workspace,
                                      hipStream_t st)
{
    if (code == QTCQ_CODE_1MAD)
        return tb ? matvec_mfma_impl<L, kCode1Mad, true>(bits, M, N, x, batch, y, workspace, st)
                  : matvec_mfma_impl<L, kCode1Mad, false>(bits, M, N, x, batch, y, workspace, st);
    return tb ? matvec_mfma_impl<L, kCode3Inst, true>(bits, M, N, x, batch, y, workspace, st)
              : matvec_mfma_impl<L, kCode3Inst, false>(bits, M, N, x, batch, y, workspace, st);
}

template <int L>
struct MatvecMfmaF {
    template <typename... A>
    static qtcq_status run(A... a) { return matvec_mfma_dispatch_code<L>(a...); }
};

template <int L>
struct MatvecF {
    template <typename... A>
    static qtcq_status run(A... a) { return matvec_dispatch_code<L>(a...); }
};

template <int L>
struct EncodeF {
    template <typename... A>
    static qtcq_status run(A... a) { return encode_dispatch_code<L>(a...); }
};
template <int L>
struct TailBitingF {
    template <typename... A>
    static qtcq_status run(A... a) { return tb_dispatch_code<L>(a...); }
};
template <int L>
struct DecodeF {
    template <typename... A>
    static qtcq_status run(A... a) { return decode_dispatch_code<L>(a...); }
};
template <int L>
struct VjpF {
    template <typename... A>
    static qtcq_status run(A... a) { return vjp_dispatch_code<L>(a...); }
};
template <int L>
struct BcjrF {
    template <typename... A>
    static qtcq_status run(A... a) { return bcjr_dispatch_code<L>(a...); }
};

}  // namespace

extern "C" {

const char* qtcq_status_string(qtcq_status s)
{
    switch (s) {
    case QTCQ_OK: return "ok";
    case QTCQ_ERR_INVALID_ARG: return "invalid argument";
    case QTCQ_ERR_UNSUPPORTED: return "unsupported trellis or code";
    case QTCQ_ERR_WORKSPACE: return "workspace too small or misaligned";
    case QTCQ_ERR_DEVICE: return "device launch failed";
    }
    return "unknown status";
}

int64_t qtcq_bitstream_words(int L, int k, int T)
{
    if (k < 1 || L < k || L > 32 || T < 1) return -1;
    return stream_words(L, k, T);
}

size_t qtcq_encode_workspace_bytes(int64_t B, int T, int L, int k)
{
    if (!supported_trellis(L, k) || T < 1 || T > kMaxT || B < 0) return 0;
    return (size_t)(B > 0 ? B : 1) * encode_bytes_per_seq(T, L);
}

size_t qtcq_bcjr_workspace_bytes(int64_t B, int T, int L, int k)
{
    if (!supported_trellis(L, k) || T < 1 || T > kMaxT || B < 0) return 0;
    return (size_t)(B > 0 ? B : 1) * bcjr_bytes_per_seq(T, L);
}

size_t qtcq_bcjr_vjp_workspace_bytes(int64_t B, int T, int L, int k)
{
    if (!supported_trellis(L, k) || T < 1 || T > kMaxT || B < 0) return 0;
    return (size_t)(B > 0 ? B : 1) * bcjr_bytes_per_seq(T, L, true);
}

qtcq_status qtcq_code_table(int code, int L, float* out, void* stream)
{
    if (!out || L < 1 || L > 24) return QTCQ_ERR_INVALID_ARG;
    if (!valid_code(code)) return QTCQ_ERR_UNSUPPORTED;
    const int64_t n = (int64_t)1 << L;
    if (code == QTCQ_CODE_1MAD)
        hipLaunchKernelGGL((code_table_kernel<kCode1Mad>), dim3(blocks_for(n, 256)), dim3(256), 0,
                           as_stream(stream), out, n);
    else
        hipLaunchKernelGGL((code_table_kernel<kCode3Inst>), dim3(blocks_for(n, 256)), dim3(256), 0,
                           as_stream(stream), out, n);
    return launch_status();
}

qtcq_status qtcq_viterbi_encode(const float* seq, const float* err_w, int64_t B, int T, int L,
                                int k, int code, uint32_t* bits, float* mse, uint32_t* states,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k) || !valid_code(code)) return QTCQ_ERR_UNSUPPORTED;
    if (B == 0) return QTCQ_OK;
    if (!seq || !bits) return QTCQ_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < encode_bytes_per_seq(T, L))
        return QTCQ_ERR_WORKSPACE;
    return by_L<EncodeF>(L, code, err_w != nullptr, seq, err_w, B, T, bits, mse, states, workspace,
                         workspace_bytes, as_stream(stream));
}

qtcq_status qtcq_decode(const uint32_t* bits, int64_t B, int T, int L, int k, int code,
                        float* recon, const float* seq, const float* err_w, float* mse,
                        void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k) || !valid_code(code)) return QTCQ_ERR_UNSUPPORTED;
    if (!recon && !mse) return QTCQ_ERR_INVALID_ARG;
    if (mse && !seq) return QTCQ_ERR_INVALID_ARG;
    if (B == 0) return QTCQ_OK;
    if (!bits) return QTCQ_ERR_INVALID_ARG;
    return by_L<DecodeF>(L, code, false, bits, B, T, recon, seq, err_w, mse, as_stream(stream));
}

int64_t qtcq_tailbiting_words(int L, int k, int T)
{
    if (k < 1 || L < k || L > 32 || T < 1 || !tailbiting_ok(L, k, T)) return -1;
    return tb_stream_words(k, T);
}

size_t qtcq_tailbiting_workspace_bytes(int64_t B, int T, int L, int k)
{
    if (!supported_trellis(L, k) || T < 1 || T > kMaxT || B < 0 || !tailbiting_ok(L, k, T))
        return 0;
    return (size_t)(B > 0 ? B : 1) * tb_bytes_per_seq(T, L);
}

qtcq_status qtcq_tailbiting_encode(const float* seq, const float* err_w, int64_t B, int T, int L,
                                   int k, int code, uint32_t* bits, float* mse, uint32_t* states,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k) || !valid_code(code)) return QTCQ_ERR_UNSUPPORTED;
    if (!tailbiting_ok(L, k, T)) return QTCQ_ERR_INVALID_ARG;
    if (B == 0) return QTCQ_OK;
    if (!seq || !bits) return QTCQ_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < tb_bytes_per_seq(T, L))
        return QTCQ_ERR_WORKSPACE;
    return by_L<TailBitingF>(L, code, err_w != nullptr, seq, err_w, B, T, bits, mse, states,
                             workspace, workspace_bytes, as_stream(stream));
}

qtcq_status qtcq_tailbiting_decode(const uint32_t* bits, int64_t B, int T, int L, int k, int code,
                                   float* recon, const float* seq, const float* err_w, float* mse,
                                   void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k) || !valid_code(code)) return QTCQ_ERR_UNSUPPORTED;
    if (!tailbiting_ok(L, k, T)) return QTCQ_ERR_INVALID_ARG;
    if (!recon && !mse) return QTCQ_ERR_INVALID_ARG;
    if (mse && !seq) return QTCQ_ERR_INVALID_ARG;
    if (B == 0) return QTCQ_OK;
    if (!bits) return QTCQ_ERR_INVALID_ARG;
    return by_L<DecodeF>(L, code, true, bits, B, T, recon, seq, err_w, mse, as_stream(stream));
}

qtcq_status qtcq_bcjr_soft(const float* seq, const float* err_w, int64_t B, int T, int L, int k,
                           int code, float temperature, float* soft, float* log_z,
                           void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!(temperature > 0.0f) || !__builtin_isfinite(temperature)) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k) || !valid_code(code)) return QTCQ_ERR_UNSUPPORTED;
    if (B == 0) return QTCQ_OK;
    if (!seq || !soft) return QTCQ_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < bcjr_bytes_per_seq(T, L))
        return QTCQ_ERR_WORKSPACE;
    return by_L<BcjrF>(L, code, err_w != nullptr, seq, err_w, B, T, temperature, soft, log_z,
                       workspace, workspace_bytes, as_stream(stream));
}

qtcq_status qtcq_bcjr_vjp(const float* seq, const float* err_w, int64_t B, int T, int L, int k,
                          int code, float temperature, const float* grad_soft, float* grad_seq,
                          float* soft, float* log_z, void* workspace, size_t workspace_bytes,
                          void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!(temperature > 0.0f) || !__builtin_isfinite(temperature)) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k) || !valid_code(code)) return QTCQ_ERR_UNSUPPORTED;
    if (B == 0) return QTCQ_OK;
    if (!seq || !grad_soft || !grad_seq) return QTCQ_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < bcjr_bytes_per_seq(T, L, true))
        return QTCQ_ERR_WORKSPACE;
    return by_L<VjpF>(L, code, err_w != nullptr, seq, err_w, grad_soft, B, T, temperature,
                      grad_seq, soft, log_z, workspace, workspace_bytes, as_stream(stream));
}

qtcq_status qtcq_decode_matvec(const uint32_t* bits, int M, int N, int L, int k, int code,
                               int tailbiting, const float* x, int batch, float* y, void* stream)
{
    if (M < 0 || N < 0 || (M % 16) != 0 || (N % 16) != 0 || batch < 0) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k) || !valid_code(code)) return QTCQ_ERR_UNSUPPORTED;
    if (batch > MatvecShape::kMaxBatch) return QTCQ_ERR_UNSUPPORTED;
    if (M == 0 || batch == 0) return QTCQ_OK;
    if (!y || (N > 0 && (!x || !aligned16(x) || !bits))) return QTCQ_ERR_INVALID_ARG;
    return by_L<MatvecF>(L, code, tailbiting != 0, bits, M, N, x, batch, y, as_stream(stream));
}

size_t qtcq_decode_matvec_mfma_workspace_bytes(int N)
{
    if (N < 0 || (N % 16) != 0 || N > MatvecMfmaShape::kMaxN) return 0;
    return MatvecMfmaShape::workspace_bytes(N);
}

qtcq_status qtcq_decode_matvec_mfma(const uint32_t* bits, int M, int N, int L, int k, int code,
                                    int tailbiting, const float* x, int batch, float* y,
                                    void* workspace, size_t workspace_bytes, void* stream)
{
    if (M < 0 || N < 0 || (M % 16) != 0 || (N % 16) != 0 || batch < 0) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k) || !valid_code(code)) return QTCQ_ERR_UNSUPPORTED;
    if (batch > MatvecMfmaShape::kMaxBatch || N > MatvecMfmaShape::kMaxN) return QTCQ_ERR_UNSUPPORTED;
    if (M == 0 || batch == 0) return QTCQ_OK;
    if (!y || (N > 0 && (!x || !aligned16(x) || !bits))) return QTCQ_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < MatvecMfmaShape::workspace_bytes(N))
        return QTCQ_ERR_WORKSPACE;
    return by_L<MatvecMfmaF>(L, code, tailbiting != 0, bits, M, N, x, batch, y, workspace,
                             as_stream(stream));
}

qtcq_status qtcq_matvec_mfma_split_x(const float* x, int N, int batch, void* workspace,
                                     size_t workspace_bytes, void* stream)
{
    if (N < 0 || (N % 16) != 0 || batch < 0) return QTCQ_ERR_INVALID_ARG;
    if (batch > MatvecMfmaShape::kMaxBatch || N > MatvecMfmaShape::kMaxN) return QTCQ_ERR_UNSUPPORTED;
    if (!workspace || !aligned16(workspace) || workspace_bytes < MatvecMfmaShape::workspace_bytes(N))
        return QTCQ_ERR_WORKSPACE;
    if (batch == 0 || N == 0) return QTCQ_OK;
    if (!x || !aligned16(x)) return QTCQ_ERR_INVALID_ARG;
    return split_x_launch(x, N, batch, workspace, as_stream(stream));
}

qtcq_status qtcq_decode_matvec_mfma_presplit(const uint32_t* bits, int M, int N, int L, int k,
                                             int code, int tailbiting, const void* split,
                                             size_t split_bytes, int batch, float* y,
                                             void* stream)
{
    if (M < 0 || N < 0 || (M % 16) != 0 || (N % 16) != 0 || batch < 0) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k) || !valid_code(code)) return QTCQ_ERR_UNSUPPORTED;
    if (batch > MatvecMfmaShape::kMaxBatch || N > MatvecMfmaShape::kMaxN) return QTCQ_ERR_UNSUPPORTED;
    if (!split || !aligned16(split) || split_bytes < MatvecMfmaShape::workspace_bytes(N))
        return QTCQ_ERR_WORKSPACE;
    if (M == 0 || batch == 0) return QTCQ_OK;
    if (!y || (N > 0 && !bits)) return QTCQ_ERR_INVALID_ARG;
    return by_L<MatvecMfmaF>(L, code, tailbiting != 0, bits, M, N, (const float*)nullptr, batch, y,
                             const_cast<void*>(split), as_stream(stream));
}

}  // extern "C"
