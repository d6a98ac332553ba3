// host.hpp -- host-side helpers shared by the C ABI (qtcq.hip) and the launch units
// (launch_*.hip, one per kernel family, compiled separately): argument predicates, sizes,
// the trellis-size dispatch, and the launch entry point of each family.
#pragma once

#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

#include <type_traits>

#include "qtcq.h"
#include "codes.hpp"

namespace qtcq {
namespace host {

constexpr int kMaxT = 4096;

inline bool supported_trellis(int L, int k)
{
    return k == 2 && L >= 6 && L <= 16 && (L % 2) == 0;
}


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

// A code as the launch units take it: its id (kCode1Mad, kCode3Inst, kCodeXor) and its
// run-time parameters (the XOR palette code's parity masks).
struct CodeSel {
    int id;
    CodeArg arg;
};

template <int V> using int_c = std::integral_constant<int, V>;
template <bool V> using bool_c = std::integral_constant<bool, V>;

// f(int_c<L>{}, int_c<CODE>{}) for every supported trellis size and code: the one place
// where run-time (L, code) become template arguments.
template <typename F>
inline qtcq_status with_L_code(int L, int code, F&& f)
{
    auto by_code = [&](auto l) -> qtcq_status {
        switch (code) {
        case kCode1Mad: return f(l, int_c<kCode1Mad>{});
        case kCode3Inst: return f(l, int_c<kCode3Inst>{});
        case kCodeXor: return f(l, int_c<kCodeXor>{});
        default: return QTCQ_ERR_UNSUPPORTED;
        }
    };
    switch (L) {
    case 6: return by_code(int_c<6>{});
    case 8: return by_code(int_c<8>{});
    case 10: return by_code(int_c<10>{});
    case 12: return by_code(int_c<12>{});
    case 14: return by_code(int_c<14>{});
    case 16: return by_code(int_c<16>{});
    default: return QTCQ_ERR_UNSUPPORTED;
    }
}

// f(bool_c<b>{})
template <typename F>
inline qtcq_status with_bool(bool b, F&& f)
{
    return b ? f(bool_c<true>{}) : f(bool_c<false>{});
}

// The code descriptor of the C ABI (qtcq.h): the id in bits 0-7 and, for the XOR
// palette code, four 14-bit parity masks at bits 8, 22, 36 and 50.  Fills *out and
// returns QTCQ_OK; QTCQ_ERR_UNSUPPORTED for an unknown id or parameter bits on a code
// that takes none; QTCQ_ERR_INVALID_ARG for an XOR code whose masks reach beyond the
// L - 2 history bits (or L < 2).
inline qtcq_status parse_code(qtcq_code code, int L, CodeSel* out)
{
    const uint64_t id = code & 0xFFu;
    const uint64_t params = code >> 8;
    out->arg = CodeArg{{0u, 0u, 0u, 0u}};
    if (id == QTCQ_CODE_1MAD || id == QTCQ_CODE_3INST) {
        if (params != 0) return QTCQ_ERR_UNSUPPORTED;
        out->id = id == QTCQ_CODE_1MAD ? kCode1Mad : kCode3Inst;
        return QTCQ_OK;
    }
    if (id != QTCQ_CODE_XOR) return QTCQ_ERR_UNSUPPORTED;
    if (L < 2) return QTCQ_ERR_INVALID_ARG;
    out->id = kCodeXor;
    for (int i = 0; i < 4; ++i) {
        const uint32_t m = (uint32_t)((params >> (14 * i)) & 0x3FFFu);
        if (L - 2 < 14 && (m >> (L - 2)) != 0) return QTCQ_ERR_INVALID_ARG;
        out->arg.m[i] = m;
    }
    return QTCQ_OK;
}

// ---- launch entry points (arguments validated by the caller) -------------------------
// launch_encode.hip
qtcq_status launch_viterbi_encode(int L, const CodeSel& code, bool weighted, const float* seq, const float* w,
                           int64_t B, int T, uint32_t* bits, float* mse, uint32_t* states,
                           void* ws, size_t wsb, hipStream_t st);
qtcq_status launch_tailbiting_encode(int L, const CodeSel& code, bool weighted, const float* seq, const float* w,
                              int64_t B, int T, uint32_t* bits, float* mse, uint32_t* states,
                              void* ws, size_t wsb, hipStream_t st);
// launch_decode.hip
qtcq_status launch_decode(int L, const CodeSel& code, bool tb, const uint32_t* bits, int64_t B, int T, float* recon,
                   const float* seq, const float* w, float* mse, hipStream_t st);
qtcq_status launch_code_table(const CodeSel& code, int L, float* out, hipStream_t st);
// launch_bcjr.hip
size_t bcjr_seq_bytes(int T, int L, bool vjp);
qtcq_status launch_bcjr_soft(int L, const CodeSel& code, bool weighted, const float* seq, const float* w, int64_t B,
                      int T, float temperature, float* soft, float* log_z, void* ws, size_t wsb,
                      hipStream_t st);
// launch_vjp.hip
qtcq_status launch_bcjr_vjp(int L, const CodeSel& code, bool weighted, const float* seq, const float* w,
                     const float* gup, int64_t B, int T, float temperature, float* grad,
                     float* soft, float* log_z, void* ws, size_t wsb, hipStream_t st);
// launch_matvec.hip
int matvec_max_batch();
int matvec_max_n();
int matvec_mfma_max_batch();
int matvec_mfma_max_n();
size_t matvec_mfma_workspace_bytes(int N);
qtcq_status launch_decode_matvec(int L, const CodeSel& code, bool tb, const uint32_t* bits, int M, int N,
                          const float* x, int batch, float* y, hipStream_t st);
qtcq_status launch_decode_matvec_mfma(int L, const CodeSel& code, bool tb, const uint32_t* bits, int M, int N,
                               const float* x, int batch, float* y, void* ws, hipStream_t st);
// the same product with the split x in the library's per-device scratch array
// (kNoAllocScratchBytes; QTCQ_ERR_WORKSPACE when the split of N needs more)
constexpr size_t kNoAllocScratchBytes = QTCQ_NOALLOC_SCRATCH_BYTES;
qtcq_status launch_decode_matvec_mfma_noalloc(int L, const CodeSel& code, bool tb,
                                              const uint32_t* bits, int M, int N, const float* x,
                                              int batch, float* y, hipStream_t st);
qtcq_status launch_split_x(const float* x, int N, int batch, void* ws, hipStream_t st);

}  // namespace host
}  // namespace qtcq
