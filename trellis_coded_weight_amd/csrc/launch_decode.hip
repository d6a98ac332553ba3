// launch_decode.hip -- launches of the window decode and the code table (decode.hpp).
#include "host.hpp"
#include "codes.hpp"
#include "decode.hpp"

namespace qtcq {
namespace host {
namespace {

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

template <int L>
struct DecodeF {
    template <typename... A>
    static qtcq_status run(A... a) { return decode_dispatch_code<L>(a...); }
};

}  // namespace

qtcq_status launch_decode(int L, int code, bool tb, const uint32_t* bits, int64_t B, int T, float* recon,
                   const float* seq, const float* w, float* mse, hipStream_t st)
{
    return by_L<DecodeF>(L, code, tb, bits, B, T, recon, seq, w, mse, st);
}

qtcq_status launch_code_table(int code, int L, float* out, hipStream_t st)
{
    const int64_t n = (int64_t)1 << L;
    if (code == QTCQ_CODE_1MAD)
        hipLaunchKernelGGL((code_table_kernel<kCode1Mad>), dim3(blocks_for(n, 256)), dim3(256), 0, st,
                           out, n);
    else
        hipLaunchKernelGGL((code_table_kernel<kCode3Inst>), dim3(blocks_for(n, 256)), dim3(256), 0, st,
                           out, n);
    return launch_status();
}

}  // namespace host
}  // namespace qtcq
