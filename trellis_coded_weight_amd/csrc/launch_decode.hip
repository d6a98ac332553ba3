// launch_decode.hip -- launches of the window decode and the code table (decode.hpp).
#include "host.hpp"
#include "decode.hpp"

namespace qtcq {
namespace host {
namespace {

template <int L, int CODE, bool TB>
qtcq_status decode_impl(const uint32_t* bits, int64_t B, int T, float* recon, const float* seq,
                        const float* w, float* mse, const CodeArg& ca, hipStream_t st)
{
    const int Wd = (int)(TB ? tb_stream_words(2, T) : stream_words(L, 2, T));
    const int SB = DecodeTile::seqs(T);
    if (SB * Wd > DecodeTile::kBitsWords || SB * DecodeTile::err_stride(T) > DecodeTile::kErrFloats)
        return QTCQ_ERR_UNSUPPORTED;      // not reachable for T <= 4096, L <= 16
    const dim3 grid(blocks_for(B, SB)), block(DecodeTile::kThreads);
    const size_t lds = DecodeTile::lds_bytes(T, Wd, mse != nullptr);
    // four weights per step of a thread when rows are whole float4s (same results)
    const bool quads = T % 4 == 0 && aligned16(seq) && aligned16(w) && aligned16(recon);
    auto go = [&](auto mse_c, auto w_c) {
        constexpr bool MSE_ = decltype(mse_c)::value, WEIGHTED = decltype(w_c)::value;
        if (quads)
            hipLaunchKernelGGL((decode_tile4<L, CODE, MSE_, WEIGHTED, TB>), grid, block, lds, st, bits, seq, w,
                               B, T, Wd, SB, recon, mse, ca);
        else
            hipLaunchKernelGGL((decode_tile<L, CODE, MSE_, WEIGHTED, TB>), grid, block, lds, st, bits, seq, w,
                               B, T, Wd, SB, recon, mse, ca);
    };
    if (!mse)
        go(bool_c<false>{}, bool_c<false>{});
    else if (w)
        go(bool_c<true>{}, bool_c<true>{});
    else
        go(bool_c<true>{}, bool_c<false>{});
    return launch_status();
}

}  // namespace

qtcq_status launch_decode(int L, const CodeSel& code, bool tb, const uint32_t* bits, int64_t B,
                          int T, float* recon, const float* seq, const float* w, float* mse,
                          hipStream_t st)
{
    return with_L_code(L, code.id, [&](auto l, auto c) {
        return with_bool(tb, [&](auto t) {
            return decode_impl<decltype(l)::value, decltype(c)::value, decltype(t)::value>(
                bits, B, T, recon, seq, w, mse, code.arg, st);
        });
    });
}

qtcq_status launch_code_table(const CodeSel& code, int L, float* out, hipStream_t st)
{
    const int64_t n = (int64_t)1 << L;
    const dim3 grid(blocks_for(n, 256)), block(256);
    switch (code.id) {
    case kCode1Mad:
        hipLaunchKernelGGL((code_table_kernel<kCode1Mad>), grid, block, 0, st, out, n, code.arg);
        break;
    case kCode3Inst:
        hipLaunchKernelGGL((code_table_kernel<kCode3Inst>), grid, block, 0, st, out, n, code.arg);
        break;
    case kCodeXor:
        hipLaunchKernelGGL((code_table_kernel<kCodeXor>), grid, block, 0, st, out, n, code.arg);
        break;
    default:
        return QTCQ_ERR_UNSUPPORTED;
    }
    return launch_status();
}

}  // namespace host
}  // namespace qtcq
