// host.hpp -- host-side helpers shared by the C ABI (qtcq.hip) and the launch units
// (launch_*.hip, one per kernel family, compiled separately): argument predicates, sizes,
// the trellis-size dispatch, and the launch entry point of each family.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include "qtcq.h"

namespace qtcq {
namespace host {

constexpr int kMaxT = 4096;

inline bool supported_trellis(int L, int k)
{
    return k == 2 && L >= 6 && L <= 16 && (L % 2) == 0;
}

inline bool valid_code(int code) { return code == QTCQ_CODE_1MAD || code == QTCQ_CODE_3INST; }

inline int64_t stream_words(int L, int k, int T)
{
    return ((int64_t)L + (int64_t)k * (T - 1) + 31) / 32;
}

// tail-biting: exactly k*T bits, and at least one window long
inline bool tailbiting_ok(int L, int k, int T) { return (int64_t)k * T >= L; }
inline int64_t tb_stream_words(int k, int T) { return ((int64_t)k * T + 31) / 32; }

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline qtcq_status launch_status()
{
    return hipGetLastError() == hipSuccess ? QTCQ_OK : QTCQ_ERR_DEVICE;
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

// Sequences per search workgroup.  A workgroup holds its group minima in LDS, so one
// runs per compute unit.  Two interleaved sequences per workgroup hide each other's LDS
// latency and barriers; when the whole chunk fits in one round of compute units on its
// own, one sequence per workgroup uses twice as many of them instead.
inline int search_seqs_per_wg(int64_t n)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 2;
    return n <= cus ? 1 : 2;
}

inline size_t encode_bytes_per_seq(int T, int L)
{
    // backpointer words per step = 2^(L-6); final state + final cost
    const size_t words = (size_t)(T - 1) * ((size_t)1 << (L - 6));
    return words * 4 + 8;
}

inline size_t tb_bytes_per_seq(int T, int L) { return encode_bytes_per_seq(T, L) + 4; }

// L dispatch: instantiate every supported trellis size.
template <template <int> class F, typename... Args>
inline qtcq_status by_L(int L, Args&&... args)
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

// ---- launch entry points (arguments validated by the caller) -------------------------
// launch_encode.hip
qtcq_status launch_viterbi_encode(int L, int code, bool weighted, const float* seq, const float* w,
                           int64_t B, int T, uint32_t* bits, float* mse, uint32_t* states,
                           void* ws, size_t wsb, hipStream_t st);
qtcq_status launch_tailbiting_encode(int L, int code, bool weighted, const float* seq, const float* w,
                              int64_t B, int T, uint32_t* bits, float* mse, uint32_t* states,
                              void* ws, size_t wsb, hipStream_t st);
// launch_decode.hip
qtcq_status launch_decode(int L, int code, bool tb, const uint32_t* bits, int64_t B, int T, float* recon,
                   const float* seq, const float* w, float* mse, hipStream_t st);
qtcq_status launch_code_table(int code, int L, float* out, hipStream_t st);
// launch_bcjr.hip
size_t bcjr_seq_bytes(int T, int L, bool vjp);
qtcq_status launch_bcjr_soft(int L, int code, bool weighted, const float* seq, const float* w, int64_t B,
                      int T, float temperature, float* soft, float* log_z, void* ws, size_t wsb,
                      hipStream_t st);
// launch_vjp.hip
qtcq_status launch_bcjr_vjp(int L, int code, bool weighted, const float* seq, const float* w,
                     const float* gup, int64_t B, int T, float temperature, float* grad,
                     float* soft, float* log_z, void* ws, size_t wsb, hipStream_t st);
// launch_matvec.hip
int matvec_max_batch();
int matvec_mfma_max_batch();
int matvec_mfma_max_n();
size_t matvec_mfma_workspace_bytes(int N);
qtcq_status launch_decode_matvec(int L, int code, bool tb, const uint32_t* bits, int M, int N,
                          const float* x, int batch, float* y, hipStream_t st);
qtcq_status launch_decode_matvec_mfma(int L, int code, bool tb, const uint32_t* bits, int M, int N,
                               const float* x, int batch, float* y, void* ws, hipStream_t st);
qtcq_status launch_split_x(const float* x, int N, int batch, void* ws, hipStream_t st);

}  // namespace host
}  // namespace qtcq
