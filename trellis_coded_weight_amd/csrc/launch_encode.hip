// launch_encode.hip -- launches of the Viterbi search, its traceback and the
// tail-biting encoder (viterbi.hpp): batch chunking over the caller's workspace.
#include "host.hpp"
#include "viterbi.hpp"

namespace qtcq {
namespace host {
namespace {

// The search over n sequences of the chunk: pairs of sequences per workgroup, or one
// (its minima then double-buffered in the kernel) when the batch is small enough that
// pairs would leave compute units idle.
template <int L, int CODE, bool W, bool PINNED>
void launch_forward(const float* seq, const float* w, int T, int64_t b0, int64_t n, int rot,
                    const uint32_t* pin, uint32_t* bp, uint32_t* fin, float* fin_cost, float* mse,
                    const CodeArg& ca, hipStream_t st)
{
    using Tr = Trellis<L>;
    const int per_wg = search_seqs_per_wg(n);
    const dim3 grid(blocks_for(n, per_wg)), block(Tr::kThreads);
    if (per_wg == 1)
        hipLaunchKernelGGL((viterbi_forward<L, CODE, W, PINNED, true>), grid, block, 0, st, seq, w, T,
                           b0, n, per_wg, rot, pin, bp, fin, fin_cost, mse, ca);
    else
        hipLaunchKernelGGL((viterbi_forward<L, CODE, W, PINNED, false>), grid, block, 0, st, seq, w, T,
                           b0, n, per_wg, rot, pin, bp, fin, fin_cost, mse, ca);
}

template <int L, int CODE, bool W>
qtcq_status encode_chunk(const float* seq, const float* w, int64_t b0, int64_t n, int T,
                         uint32_t* bits, float* mse, uint32_t* states, char* ws,
                         const CodeArg& ca, hipStream_t st)
{
    using Tr = Trellis<L>;
    uint32_t* bp = reinterpret_cast<uint32_t*>(ws);
    uint32_t* fin = bp + (size_t)n * (T - 1) * Tr::kBpWords;
    float* fin_cost = reinterpret_cast<float*>(fin + n);
    launch_forward<L, CODE, W, false>(seq, w, T, b0, n, 0, nullptr, bp, fin, fin_cost, mse, ca, st);
    qtcq_status rc = launch_status();
    if (rc != QTCQ_OK) return rc;
    const int Wd = (int)stream_words(L, 2, T);
    hipLaunchKernelGGL((viterbi_traceback<L>), dim3(blocks_for(n, 256)), dim3(256), 0, st,
                       bp, fin, T, n, b0, Wd, bits, states);
    return launch_status();
}

template <int L, int CODE, bool W>
qtcq_status encode_all(const float* seq, const float* w, int64_t B, int T, uint32_t* bits,
                       float* mse, uint32_t* states, void* ws, size_t ws_bytes, const CodeArg& ca,
                       hipStream_t st)
{
    const int64_t per_chunk = (int64_t)(ws_bytes / encode_bytes_per_seq(T, L));
    for (int64_t b0 = 0; b0 < B; b0 += per_chunk) {
        const int64_t n = (B - b0 < per_chunk) ? B - b0 : per_chunk;
        qtcq_status rc = encode_chunk<L, CODE, W>(seq, w, b0, n, T, bits, mse, states,
                                                  static_cast<char*>(ws), ca, st);
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

template <int L, int CODE, bool W>
qtcq_status tb_chunk(const float* seq, const float* w, int64_t b0, int64_t n, int T,
                     uint32_t* bits, float* mse, uint32_t* states, char* ws, const CodeArg& ca,
                     hipStream_t st)
{
    using Tr = Trellis<L>;
    uint32_t* bp = reinterpret_cast<uint32_t*>(ws);
    uint32_t* fin = bp + (size_t)n * (T - 1) * Tr::kBpWords;
    float* fin_cost = reinterpret_cast<float*>(fin + n);
    uint32_t* overlap = reinterpret_cast<uint32_t*>(fin_cost + n);
    const int rot = T / 2;
    launch_forward<L, CODE, W, false>(seq, w, T, b0, n, rot, nullptr, bp, fin, fin_cost, nullptr, ca, st);
    qtcq_status rc = launch_status();
    if (rc != QTCQ_OK) return rc;
    hipLaunchKernelGGL((viterbi_seam<L>), dim3(blocks_for(n, 256)), dim3(256), 0, st, bp, fin, T, n,
                       (T - rot) % T, overlap);
    rc = launch_status();
    if (rc != QTCQ_OK) return rc;
    launch_forward<L, CODE, W, true>(seq, w, T, b0, n, 0, overlap, bp, fin, fin_cost, mse, ca, st);
    rc = launch_status();
    if (rc != QTCQ_OK) return rc;
    hipLaunchKernelGGL((viterbi_traceback<L, true>), dim3(blocks_for(n, 256)), dim3(256), 0, st,
                       bp, fin, T, n, b0, (int)tb_stream_words(2, T), bits, states);
    return launch_status();
}

template <int L, int CODE, bool W>
qtcq_status tb_all(const float* seq, const float* w, int64_t B, int T, uint32_t* bits,
                   float* mse, uint32_t* states, void* ws, size_t ws_bytes, const CodeArg& ca,
                   hipStream_t st)
{
    const int64_t per_chunk = (int64_t)(ws_bytes / tb_bytes_per_seq(T, L));
    for (int64_t b0 = 0; b0 < B; b0 += per_chunk) {
        const int64_t n = (B - b0 < per_chunk) ? B - b0 : per_chunk;
        qtcq_status rc = tb_chunk<L, CODE, W>(seq, w, b0, n, T, bits, mse, states,
                                              static_cast<char*>(ws), ca, st);
        if (rc != QTCQ_OK) return rc;
    }
    return QTCQ_OK;
}

}  // namespace

qtcq_status launch_viterbi_encode(int L, const CodeSel& code, bool weighted, const float* seq,
                                  const float* w, int64_t B, int T, uint32_t* bits, float* mse,
                                  uint32_t* states, void* ws, size_t wsb, hipStream_t st)
{
    return with_L_code(L, code.id, [&](auto l, auto c) {
        return with_bool(weighted, [&](auto wt) {
            return encode_all<decltype(l)::value, decltype(c)::value, decltype(wt)::value>(
                seq, w, B, T, bits, mse, states, ws, wsb, code.arg, st);
        });
    });
}

qtcq_status launch_tailbiting_encode(int L, const CodeSel& code, bool weighted, const float* seq,
                                     const float* w, int64_t B, int T, uint32_t* bits, float* mse,
                                     uint32_t* states, void* ws, size_t wsb, hipStream_t st)
{
    return with_L_code(L, code.id, [&](auto l, auto c) {
        return with_bool(weighted, [&](auto wt) {
            return tb_all<decltype(l)::value, decltype(c)::value, decltype(wt)::value>(
                seq, w, B, T, bits, mse, states, ws, wsb, code.arg, st);
        });
    });
}

}  // namespace host
}  // namespace qtcq
