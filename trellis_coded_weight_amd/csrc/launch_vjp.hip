// launch_vjp.hip -- launches of the BCJR gradient: the soft pass in gradient mode,
// the expectation-message sweep and the gradient finalize (bcjr.hpp, bcjr_vjp.hpp).
#include "host.hpp"
#include "viterbi.hpp"
#include "bcjr.hpp"
#include "bcjr_vjp.hpp"

namespace qtcq {
namespace host {
namespace {

// Per chunk: the soft pass in VJP mode (stashes both message directions and the posterior
// offsets), its finalize when soft / log Z are wanted, the Phi / Psi sweep, the gradient.
// Below tau = 0.01 the stashes keep fp64 values (WIDE); the 32-bit stash's binary32 range
// below -1024 log2 units is too coarse for the states the backward messages lift there.
constexpr float kWideStashBelowTau = 0.01f;

template <int L, int CODE, bool W, bool WIDE>
qtcq_status vjp_all(const float* seq, const float* w, const float* gup, int64_t B, int T,
                    float temperature, float* grad, float* soft, float* log_z, void* ws,
                    size_t ws_bytes, const CodeArg& ca, hipStream_t st)
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
                           st, seq, w, T, b0, kappa, wsc, ca);
        qtcq_status rc = launch_status();
        if (rc != QTCQ_OK) return rc;
        if (soft || log_z) {
            hipLaunchKernelGGL((bcjr_finalize<L>), dim3(blocks_for(n * T, 256)), dim3(256), 0, st,
                               wsc, per, T, n, b0, soft, log_z);
            rc = launch_status();
            if (rc != QTCQ_OK) return rc;
        }
        hipLaunchKernelGGL((bcjr_vjp_sweep<L, CODE, W, WIDE>), dim3((unsigned)n), dim3(Tr::kThreads), 0,
                           st, seq, w, gup, T, b0, kappa, wsc, ca);
        rc = launch_status();
        if (rc != QTCQ_OK) return rc;
        hipLaunchKernelGGL((bcjr_vjp_finalize<L>), dim3(blocks_for(n * T, 256)), dim3(256), 0, st,
                           wsc, w, T, n, b0, two_over_tau, grad);
        rc = launch_status();
        if (rc != QTCQ_OK) return rc;
    }
    return QTCQ_OK;
}

}  // namespace

qtcq_status launch_bcjr_vjp(int L, const CodeSel& code, bool weighted, const float* seq,
                            const float* w, const float* gup, int64_t B, int T, float temperature,
                            float* grad, float* soft, float* log_z, void* ws, size_t wsb,
                            hipStream_t st)
{
    return with_L_code(L, code.id, [&](auto l, auto c) {
        return with_bool(weighted, [&](auto wt) {
            return with_bool(temperature < kWideStashBelowTau, [&](auto wide) {
                return vjp_all<decltype(l)::value, decltype(c)::value, decltype(wt)::value,
                               decltype(wide)::value>(seq, w, gup, B, T, temperature, grad, soft,
                                                      log_z, ws, wsb, code.arg, st);
            });
        });
    });
}

}  // namespace host
}  // namespace qtcq
