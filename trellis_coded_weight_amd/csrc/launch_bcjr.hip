// launch_bcjr.hip -- launches of the BCJR soft pass and its finalize (bcjr.hpp).
#include "host.hpp"
#include "viterbi.hpp"
#include "bcjr.hpp"

namespace qtcq {
namespace host {
namespace {

static_assert(kMaxT <= kBcjrMaxT, "the BCJR kernels stage T per-step values in LDS");

template <int L, int CODE, bool W>
qtcq_status bcjr_all(const float* seq, const float* w, int64_t B, int T, float temperature,
                     float* soft, float* log_z, void* ws, size_t ws_bytes, const CodeArg& ca,
                     hipStream_t st)
{
    using Tr = Trellis<L>;
    const size_t per = BcjrLayout<L>::bytes_per_seq(T);
    const int64_t per_chunk = (int64_t)(ws_bytes / per);
    const double kappa = 1.4426950408889634074 / (double)temperature;   // log2(e) / tau
    char* wsc = static_cast<char*>(ws);
    for (int64_t b0 = 0; b0 < B; b0 += per_chunk) {
        const int64_t n = (B - b0 < per_chunk) ? B - b0 : per_chunk;
        hipLaunchKernelGGL((bcjr_sweep<L, CODE, W>), dim3((unsigned)n), dim3(Tr::kThreads), 0, st,
                           seq, w, T, b0, kappa, wsc, ca);
        qtcq_status rc = launch_status();
        if (rc != QTCQ_OK) return rc;
        hipLaunchKernelGGL((bcjr_finalize<L>), dim3(blocks_for(n * T, 256)), dim3(256), 0, st,
                           wsc, per, T, n, b0, soft, log_z);
        rc = launch_status();
        if (rc != QTCQ_OK) return rc;
    }
    return QTCQ_OK;
}

}  // namespace

size_t bcjr_seq_bytes(int T, int L, bool vjp) { return bcjr_bytes_per_seq(T, L, vjp); }

qtcq_status launch_bcjr_soft(int L, const CodeSel& code, bool weighted, const float* seq,
                             const float* w, int64_t B, int T, float temperature, float* soft,
                             float* log_z, void* ws, size_t wsb, hipStream_t st)
{
    return with_L_code(L, code.id, [&](auto l, auto c) {
        return with_bool(weighted, [&](auto wt) {
            return bcjr_all<decltype(l)::value, decltype(c)::value, decltype(wt)::value>(
                seq, w, B, T, temperature, soft, log_z, ws, wsb, code.arg, st);
        });
    });
}

}  // namespace host
}  // namespace qtcq
