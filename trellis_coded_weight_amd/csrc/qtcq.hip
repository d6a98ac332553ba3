// qtcq.hip -- the C ABI declared in include/qtcq.h: argument validation and workspace
// sizing; every accepted call goes to the launch unit of its kernel family
// (launch_*.hip), which chunks the batch and enqueues the kernels on the caller's
// stream.  Everything the path computes runs in those kernels.
#include "host.hpp"

namespace host = qtcq::host;
using namespace qtcq::host;
using qtcq::kCodeXor;

extern "C" {

const char* qtcq_status_string(int status)
{
    switch (status) {
    case QTCQ_OK: return "ok";
    case QTCQ_ERR_INVALID_ARG: return "invalid argument";
    case QTCQ_ERR_UNSUPPORTED: return "unsupported trellis or code";
    case QTCQ_ERR_WORKSPACE: return "workspace too small or misaligned";
    case QTCQ_ERR_DEVICE: return "device launch failed";
    }
    return "unknown status";
}

qtcq_code qtcq_xor_code(uint32_t m0, uint32_t m1, uint32_t m2, uint32_t m3)
{
    if ((m0 | m1 | m2 | m3) > 0x3FFFu) return QTCQ_CODE_INVALID;
    return (qtcq_code)QTCQ_CODE_XOR | ((qtcq_code)m0 << 8) | ((qtcq_code)m1 << 22) |
           ((qtcq_code)m2 << 36) | ((qtcq_code)m3 << 50);
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
    return (size_t)(B > 0 ? B : 1) * host::bcjr_seq_bytes(T, L, false);
}

size_t qtcq_bcjr_vjp_workspace_bytes(int64_t B, int T, int L, int k)
{
    if (!supported_trellis(L, k) || T < 1 || T > kMaxT || B < 0) return 0;
    return (size_t)(B > 0 ? B : 1) * host::bcjr_seq_bytes(T, L, true);
}

qtcq_status qtcq_code_table(qtcq_code code, int L, float* out, void* stream)
{
    if (!out || L < 1 || L > 24) return QTCQ_ERR_INVALID_ARG;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (cs.id == kCodeXor && L > 16) return QTCQ_ERR_INVALID_ARG;
    return host::launch_code_table(cs, L, out, as_stream(stream));
}

qtcq_status qtcq_viterbi_encode(const float* seq, const float* err_w, int64_t B, int T, int L,
                                int k, qtcq_code code, uint32_t* bits, float* mse, uint32_t* states,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k)) return QTCQ_ERR_UNSUPPORTED;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (B == 0) return QTCQ_OK;
    if (!seq || !bits) return QTCQ_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < encode_bytes_per_seq(T, L))
        return QTCQ_ERR_WORKSPACE;
    return host::launch_viterbi_encode(L, cs, err_w != nullptr, seq, err_w, B, T, bits, mse, states, workspace,
                         workspace_bytes, as_stream(stream));
}

qtcq_status qtcq_decode(const uint32_t* bits, int64_t B, int T, int L, int k, qtcq_code code,
                        float* recon, const float* seq, const float* err_w, float* mse,
                        void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k)) return QTCQ_ERR_UNSUPPORTED;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (!recon && !mse) return QTCQ_ERR_INVALID_ARG;
    if (mse && !seq) return QTCQ_ERR_INVALID_ARG;
    if (B == 0) return QTCQ_OK;
    if (!bits) return QTCQ_ERR_INVALID_ARG;
    return host::launch_decode(L, cs, false, bits, B, T, recon, seq, err_w, mse, as_stream(stream));
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
                                   int k, qtcq_code code, uint32_t* bits, float* mse, uint32_t* states,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k)) return QTCQ_ERR_UNSUPPORTED;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (!tailbiting_ok(L, k, T)) return QTCQ_ERR_INVALID_ARG;
    if (B == 0) return QTCQ_OK;
    if (!seq || !bits) return QTCQ_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < tb_bytes_per_seq(T, L))
        return QTCQ_ERR_WORKSPACE;
    return host::launch_tailbiting_encode(L, cs, err_w != nullptr, seq, err_w, B, T, bits, mse, states,
                             workspace, workspace_bytes, as_stream(stream));
}

qtcq_status qtcq_tailbiting_decode(const uint32_t* bits, int64_t B, int T, int L, int k, qtcq_code code,
                                   float* recon, const float* seq, const float* err_w, float* mse,
                                   void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k)) return QTCQ_ERR_UNSUPPORTED;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (!tailbiting_ok(L, k, T)) return QTCQ_ERR_INVALID_ARG;
    if (!recon && !mse) return QTCQ_ERR_INVALID_ARG;
    if (mse && !seq) return QTCQ_ERR_INVALID_ARG;
    if (B == 0) return QTCQ_OK;
    if (!bits) return QTCQ_ERR_INVALID_ARG;
    return host::launch_decode(L, cs, true, bits, B, T, recon, seq, err_w, mse, as_stream(stream));
}

qtcq_status qtcq_bcjr_soft(const float* seq, const float* err_w, int64_t B, int T, int L, int k,
                           qtcq_code code, float temperature, float* soft, float* log_z,
                           void* workspace, size_t workspace_bytes, void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!(temperature > 0.0f) || !__builtin_isfinite(temperature)) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k)) return QTCQ_ERR_UNSUPPORTED;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (B == 0) return QTCQ_OK;
    if (!seq || !soft) return QTCQ_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < host::bcjr_seq_bytes(T, L, false))
        return QTCQ_ERR_WORKSPACE;
    return host::launch_bcjr_soft(L, cs, err_w != nullptr, seq, err_w, B, T, temperature, soft, log_z,
                       workspace, workspace_bytes, as_stream(stream));
}

qtcq_status qtcq_bcjr_vjp(const float* seq, const float* err_w, int64_t B, int T, int L, int k,
                          qtcq_code code, float temperature, const float* grad_soft, float* grad_seq,
                          float* soft, float* log_z, void* workspace, size_t workspace_bytes,
                          void* stream)
{
    if (B < 0 || T < 1 || T > kMaxT) return QTCQ_ERR_INVALID_ARG;
    if (!(temperature > 0.0f) || !__builtin_isfinite(temperature)) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k)) return QTCQ_ERR_UNSUPPORTED;
    if (temperature < QTCQ_VJP_MIN_TEMPERATURE) return QTCQ_ERR_UNSUPPORTED;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (B == 0) return QTCQ_OK;
    if (!seq || !grad_soft || !grad_seq) return QTCQ_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < host::bcjr_seq_bytes(T, L, true))
        return QTCQ_ERR_WORKSPACE;
    return host::launch_bcjr_vjp(L, cs, err_w != nullptr, seq, err_w, grad_soft, B, T, temperature,
                      grad_seq, soft, log_z, workspace, workspace_bytes, as_stream(stream));
}

qtcq_status qtcq_decode_matvec(const uint32_t* bits, int M, int N, int L, int k, qtcq_code code,
                               int tailbiting, const float* x, int batch, float* y, void* stream)
{
    if (M < 0 || N < 0 || (M % 16) != 0 || (N % 16) != 0 || batch < 0) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k)) return QTCQ_ERR_UNSUPPORTED;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (batch > host::matvec_max_batch() || N > host::matvec_max_n()) return QTCQ_ERR_UNSUPPORTED;
    if (M == 0 || batch == 0) return QTCQ_OK;
    if (!y || (N > 0 && (!x || !aligned16(x) || !bits))) return QTCQ_ERR_INVALID_ARG;
    return host::launch_decode_matvec(L, cs, tailbiting != 0, bits, M, N, x, batch, y, as_stream(stream));
}

size_t qtcq_decode_matvec_mfma_workspace_bytes(int N)
{
    if (N < 0 || (N % 16) != 0 || N > host::matvec_mfma_max_n()) return 0;
    return host::matvec_mfma_workspace_bytes(N);
}

qtcq_status qtcq_decode_matvec_mfma(const uint32_t* bits, int M, int N, int L, int k, qtcq_code code,
                                    int tailbiting, const float* x, int batch, float* y,
                                    void* workspace, size_t workspace_bytes, void* stream)
{
    if (M < 0 || N < 0 || (M % 16) != 0 || (N % 16) != 0 || batch < 0) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k)) return QTCQ_ERR_UNSUPPORTED;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (batch > host::matvec_mfma_max_batch() || N > host::matvec_mfma_max_n()) return QTCQ_ERR_UNSUPPORTED;
    if (M == 0 || batch == 0) return QTCQ_OK;
    if (!y || (N > 0 && (!x || !aligned16(x) || !bits))) return QTCQ_ERR_INVALID_ARG;
    if (!workspace || !aligned16(workspace) || workspace_bytes < host::matvec_mfma_workspace_bytes(N))
        return QTCQ_ERR_WORKSPACE;
    return host::launch_decode_matvec_mfma(L, cs, tailbiting != 0, bits, M, N, x, batch, y, workspace,
                             as_stream(stream));
}

qtcq_status qtcq_decode_matvec_mfma_noalloc(const uint32_t* bits, int M, int N, int L, int k,
                                            qtcq_code code, int tailbiting, const float* x,
                                            int batch, float* y, void* stream)
{
    if (M < 0 || N < 0 || (M % 16) != 0 || (N % 16) != 0 || batch < 0) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k)) return QTCQ_ERR_UNSUPPORTED;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (batch > host::matvec_mfma_max_batch() || N > host::matvec_mfma_max_n()) return QTCQ_ERR_UNSUPPORTED;
    if (host::matvec_mfma_workspace_bytes(N) > host::kNoAllocScratchBytes) return QTCQ_ERR_WORKSPACE;
    if (M == 0 || batch == 0) return QTCQ_OK;
    if (!y || (N > 0 && (!x || !aligned16(x) || !bits))) return QTCQ_ERR_INVALID_ARG;
    return host::launch_decode_matvec_mfma_noalloc(L, cs, tailbiting != 0, bits, M, N, x, batch, y,
                                                   as_stream(stream));
}

qtcq_status qtcq_matvec_mfma_split_x(const float* x, int N, int batch, void* workspace,
                                     size_t workspace_bytes, void* stream)
{
    if (N < 0 || (N % 16) != 0 || batch < 0) return QTCQ_ERR_INVALID_ARG;
    if (batch > host::matvec_mfma_max_batch() || N > host::matvec_mfma_max_n()) return QTCQ_ERR_UNSUPPORTED;
    if (!workspace || !aligned16(workspace) || workspace_bytes < host::matvec_mfma_workspace_bytes(N))
        return QTCQ_ERR_WORKSPACE;
    if (batch == 0 || N == 0) return QTCQ_OK;
    if (!x || !aligned16(x)) return QTCQ_ERR_INVALID_ARG;
    return host::launch_split_x(x, N, batch, workspace, as_stream(stream));
}

qtcq_status qtcq_decode_matvec_mfma_presplit(const uint32_t* bits, int M, int N, int L, int k,
                                             qtcq_code code, int tailbiting, const void* split,
                                             size_t split_bytes, int batch, float* y,
                                             void* stream)
{
    if (M < 0 || N < 0 || (M % 16) != 0 || (N % 16) != 0 || batch < 0) return QTCQ_ERR_INVALID_ARG;
    if (!supported_trellis(L, k)) return QTCQ_ERR_UNSUPPORTED;
    CodeSel cs;
    if (const qtcq_status pc = parse_code(code, L, &cs); pc != QTCQ_OK) return pc;
    if (batch > host::matvec_mfma_max_batch() || N > host::matvec_mfma_max_n()) return QTCQ_ERR_UNSUPPORTED;
    if (!split || !aligned16(split) || split_bytes < host::matvec_mfma_workspace_bytes(N))
        return QTCQ_ERR_WORKSPACE;
    if (M == 0 || batch == 0) return QTCQ_OK;
    if (!y || (N > 0 && !bits)) return QTCQ_ERR_INVALID_ARG;
    return host::launch_decode_matvec_mfma(L, cs, tailbiting != 0, bits, M, N, (const float*)nullptr, batch, y,
                             const_cast<void*>(split), as_stream(stream));
}

}  // extern "C"
