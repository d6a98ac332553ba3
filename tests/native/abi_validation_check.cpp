// Host-side check of the C ABI's validation layer (csrc/qtcq.hip), built host-only with
// AddressSanitizer and UndefinedBehaviorSanitizer by the test suite.  The kernel-launch
// entry points of the launch units are replaced by stand-ins that count their calls and
// return a sentinel status, so every path runs without a GPU:
//   - each rejected call returns its documented status and reaches no launch;
//   - one accepted call per entry point reaches exactly one launch (the sentinel);
//   - the size queries and the code descriptors give their documented values.
// Prints "ok" and exits 0, or the first failure and exits 1.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "host.hpp"
#include "viterbi.hpp"
#include "bcjr.hpp"
#include "matvec.hpp"

namespace qtcq {
namespace host {

static int g_launches = 0;
// a status no entry point returns, inside the enumeration's value range (0..7)
constexpr qtcq_status kLaunched = (qtcq_status)7;

static qtcq_status stand_in()
{
    ++g_launches;
    return kLaunched;
}

qtcq_status launch_viterbi_encode(int, const CodeSel&, bool, const float*, const float*, int64_t, int,
                                  uint32_t*, float*, uint32_t*, void*, size_t, hipStream_t)
{ return stand_in(); }
qtcq_status launch_tailbiting_encode(int, const CodeSel&, bool, const float*, const float*, int64_t, int,
                                     uint32_t*, float*, uint32_t*, void*, size_t, hipStream_t)
{ return stand_in(); }
qtcq_status launch_decode(int, const CodeSel&, bool, const uint32_t*, int64_t, int, float*,
                          const float*, const float*, float*, hipStream_t)
{ return stand_in(); }
qtcq_status launch_code_table(const CodeSel&, int, float*, hipStream_t) { return stand_in(); }
size_t bcjr_seq_bytes(int T, int L, bool vjp) { return bcjr_bytes_per_seq(T, L, vjp); }
qtcq_status launch_bcjr_soft(int, const CodeSel&, bool, const float*, const float*, int64_t, int, float,
                             float*, float*, void*, size_t, hipStream_t)
{ return stand_in(); }
qtcq_status launch_bcjr_vjp(int, const CodeSel&, bool, const float*, const float*, const float*, int64_t,
                            int, float, float*, float*, float*, void*, size_t, hipStream_t)
{ return stand_in(); }
int matvec_max_batch() { return MatvecShape::kMaxBatch; }
int matvec_max_n() { return MatvecShape::kMaxN; }
// the matrix-core shapes (matvec_mfma.hpp holds a kernel, so its constants are restated
// here from its declaration: 4 fragments of 8 rows, N up to 2^22, 4224 bytes per
// 32-column block, 256-byte rounding plus 256)
int matvec_mfma_max_batch() { return 32; }
int matvec_mfma_max_n() { return 1 << 22; }
size_t matvec_mfma_workspace_bytes(int N)
{
    const size_t nkb = (size_t)((N / 16 + 1) / 2);
    return ((nkb * 4 * (1024 + 32) + 255) / 256) * 256 + 256;
}
qtcq_status launch_decode_matvec(int, const CodeSel&, bool, const uint32_t*, int, int, const float*, int,
                                 float*, hipStream_t)
{ return stand_in(); }
qtcq_status launch_decode_matvec_mfma(int, const CodeSel&, bool, const uint32_t*, int, int, const float*,
                                      int, float*, void*, hipStream_t)
{ return stand_in(); }
qtcq_status launch_decode_matvec_mfma_noalloc(int, const CodeSel&, bool, const uint32_t*, int, int,
                                              const float*, int, float*, hipStream_t)
{ return stand_in(); }
qtcq_status launch_split_x(const float*, int, int, void*, hipStream_t) { return stand_in(); }

}  // namespace host
}  // namespace qtcq

using qtcq::host::g_launches;
using qtcq::host::kLaunched;

static int failures = 0;

static void expect(const char* what, int got, int want, int launches_before, bool launched)
{
    const int dl = g_launches - launches_before;
    if (got != want || dl != (launched ? 1 : 0)) {
        std::printf("FAIL %s: status %d (want %d), launches %d (want %d)\n", what, got, want, dl,
                    launched ? 1 : 0);
        ++failures;
    }
}

#define CHECK(what, call, want)                                                       \
    do {                                                                              \
        const int before_ = g_launches;                                               \
        const int got_ = (int)(call);                                                 \
        expect(what, got_, (int)(want), before_, (int)(want) == (int)kLaunched);      \
    } while (0)

int main()
{
    // fake device addresses: never dereferenced by validation (16-byte aligned)
    float* f = reinterpret_cast<float*>(uintptr_t(1) << 20);
    uint32_t* u = reinterpret_cast<uint32_t*>(uintptr_t(1) << 21);
    void* ws = reinterpret_cast<void*>(uintptr_t(1) << 22);
    void* ws_mis = reinterpret_cast<void*>((uintptr_t(1) << 22) + 8);
    const size_t enc_ws = qtcq_encode_workspace_bytes(1, 256, 16, 2);
    const size_t bcjr_ws = qtcq_bcjr_workspace_bytes(1, 256, 16, 2);
    const size_t vjp_ws = qtcq_bcjr_vjp_workspace_bytes(1, 256, 16, 2);
    const size_t mv_ws = qtcq_decode_matvec_mfma_workspace_bytes(64);
    const qtcq_code xc = qtcq_xor_code(0x2D35, 0x1ACB, 0x34AE, 0x0F53);

    // sizes and descriptors
    if (qtcq_bitstream_words(16, 2, 256) != 17 || qtcq_tailbiting_words(16, 2, 256) != 16 ||
        qtcq_bitstream_words(16, 0, 256) != -1 || enc_ws != 255u * 1024u * 4u + 8u ||
        qtcq_encode_workspace_bytes(1, 256, 7, 2) != 0 || qtcq_xor_code(1u << 14, 0, 0, 0) != QTCQ_CODE_INVALID ||
        (xc & 0xFF) != QTCQ_CODE_XOR || qtcq_decode_matvec_mfma_workspace_bytes(40) != 0) {
        std::printf("FAIL sizes or descriptors\n");
        ++failures;
    }
    for (int s = -1; s < 6; ++s)
        if (!qtcq_status_string(s)) ++failures;
    if (qtcq_status_string(99)[0] != 'u') ++failures;   // "unknown status"

    // encode
    CHECK("encode ok", qtcq_viterbi_encode(f, nullptr, 4, 256, 16, 2, QTCQ_CODE_1MAD, u, f, nullptr, ws, enc_ws, nullptr), kLaunched);
    CHECK("encode xor ok", qtcq_viterbi_encode(f, f, 4, 256, 16, 2, xc, u, f, u, ws, enc_ws, nullptr), kLaunched);
    CHECK("encode B<0", qtcq_viterbi_encode(f, nullptr, -1, 256, 16, 2, 0, u, f, nullptr, ws, enc_ws, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("encode B=0", qtcq_viterbi_encode(nullptr, nullptr, 0, 256, 16, 2, 0, nullptr, nullptr, nullptr, nullptr, 0, nullptr), QTCQ_OK);
    CHECK("encode T=0", qtcq_viterbi_encode(f, nullptr, 4, 0, 16, 2, 0, u, f, nullptr, ws, enc_ws, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("encode T big", qtcq_viterbi_encode(f, nullptr, 4, 4097, 16, 2, 0, u, f, nullptr, ws, enc_ws, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("encode L=7", qtcq_viterbi_encode(f, nullptr, 4, 256, 7, 2, 0, u, f, nullptr, ws, enc_ws, nullptr), QTCQ_ERR_UNSUPPORTED);
    CHECK("encode code 3", qtcq_viterbi_encode(f, nullptr, 4, 256, 16, 2, 3, u, f, nullptr, ws, enc_ws, nullptr), QTCQ_ERR_UNSUPPORTED);
    CHECK("encode 1mad params", qtcq_viterbi_encode(f, nullptr, 4, 256, 16, 2, 1u << 8, u, f, nullptr, ws, enc_ws, nullptr), QTCQ_ERR_UNSUPPORTED);
    CHECK("encode xor masks", qtcq_viterbi_encode(f, nullptr, 4, 256, 12, 2, xc, u, f, nullptr, ws, enc_ws, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("encode seq null", qtcq_viterbi_encode(nullptr, nullptr, 4, 256, 16, 2, 0, u, f, nullptr, ws, enc_ws, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("encode ws small", qtcq_viterbi_encode(f, nullptr, 4, 256, 16, 2, 0, u, f, nullptr, ws, enc_ws - 1, nullptr), QTCQ_ERR_WORKSPACE);
    CHECK("encode ws misaligned", qtcq_viterbi_encode(f, nullptr, 4, 256, 16, 2, 0, u, f, nullptr, ws_mis, enc_ws, nullptr), QTCQ_ERR_WORKSPACE);
    // tail-biting
    CHECK("tb ok", qtcq_tailbiting_encode(f, nullptr, 4, 256, 16, 2, 1, u, f, nullptr, ws, enc_ws + 4, nullptr), kLaunched);
    CHECK("tb short", qtcq_tailbiting_encode(f, nullptr, 4, 7, 16, 2, 1, u, f, nullptr, ws, enc_ws + 4, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("tb decode ok", qtcq_tailbiting_decode(u, 4, 256, 16, 2, 0, f, nullptr, nullptr, nullptr, nullptr), kLaunched);
    // decode
    CHECK("decode ok", qtcq_decode(u, 4, 256, 16, 2, 0, f, f, nullptr, f, nullptr), kLaunched);
    CHECK("decode nothing", qtcq_decode(u, 4, 256, 16, 2, 0, nullptr, nullptr, nullptr, nullptr, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("decode mse no seq", qtcq_decode(u, 4, 256, 16, 2, 0, f, nullptr, nullptr, f, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("decode bits null", qtcq_decode(nullptr, 4, 256, 16, 2, 0, f, nullptr, nullptr, nullptr, nullptr), QTCQ_ERR_INVALID_ARG);
    // code table
    CHECK("table ok", qtcq_code_table(0, 20, f, nullptr), kLaunched);
    CHECK("table xor ok", qtcq_code_table(xc, 16, f, nullptr), kLaunched);
    CHECK("table xor L", qtcq_code_table(xc, 20, f, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("table L 25", qtcq_code_table(0, 25, f, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("table null", qtcq_code_table(0, 16, nullptr, nullptr), QTCQ_ERR_INVALID_ARG);
    // BCJR and its gradient
    CHECK("bcjr ok", qtcq_bcjr_soft(f, nullptr, 4, 256, 16, 2, 0, 0.1f, f, f, ws, bcjr_ws, nullptr), kLaunched);
    CHECK("bcjr tau 0", qtcq_bcjr_soft(f, nullptr, 4, 256, 16, 2, 0, 0.0f, f, f, ws, bcjr_ws, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("bcjr tau nan", qtcq_bcjr_soft(f, nullptr, 4, 256, 16, 2, 0, NAN, f, f, ws, bcjr_ws, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("bcjr tau inf", qtcq_bcjr_soft(f, nullptr, 4, 256, 16, 2, 0, INFINITY, f, f, ws, bcjr_ws, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("bcjr ws", qtcq_bcjr_soft(f, nullptr, 4, 256, 16, 2, 0, 0.1f, f, f, ws, bcjr_ws - 1, nullptr), QTCQ_ERR_WORKSPACE);
    CHECK("vjp ok", qtcq_bcjr_vjp(f, nullptr, 4, 256, 16, 2, 0, 0.1f, f, f, nullptr, nullptr, ws, vjp_ws, nullptr), kLaunched);
    CHECK("vjp floor ok", qtcq_bcjr_vjp(f, nullptr, 4, 256, 16, 2, 0, QTCQ_VJP_MIN_TEMPERATURE, f, f, nullptr, nullptr, ws, vjp_ws, nullptr), kLaunched);
    CHECK("vjp below floor", qtcq_bcjr_vjp(f, nullptr, 4, 256, 16, 2, 0, 1e-3f, f, f, nullptr, nullptr, ws, vjp_ws, nullptr), QTCQ_ERR_UNSUPPORTED);
    CHECK("vjp grad null", qtcq_bcjr_vjp(f, nullptr, 4, 256, 16, 2, 0, 0.1f, f, nullptr, nullptr, nullptr, ws, vjp_ws, nullptr), QTCQ_ERR_INVALID_ARG);
    // matvec products
    CHECK("matvec ok", qtcq_decode_matvec(u, 32, 64, 16, 2, 0, 0, f, 8, f, nullptr), kLaunched);
    CHECK("matvec batch 9", qtcq_decode_matvec(u, 32, 64, 16, 2, 0, 0, f, 9, f, nullptr), QTCQ_ERR_UNSUPPORTED);
    CHECK("matvec N > 2^22", qtcq_decode_matvec(u, 32, (1 << 22) + 16, 16, 2, 0, 0, f, 1, f, nullptr), QTCQ_ERR_UNSUPPORTED);
    CHECK("matvec M odd", qtcq_decode_matvec(u, 33, 64, 16, 2, 0, 0, f, 1, f, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("matvec x misaligned", qtcq_decode_matvec(u, 32, 64, 16, 2, 0, 0, f + 1, 1, f, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("mfma ok", qtcq_decode_matvec_mfma(u, 32, 64, 16, 2, 0, 1, f, 32, f, ws, mv_ws, nullptr), kLaunched);
    CHECK("mfma batch 33", qtcq_decode_matvec_mfma(u, 32, 64, 16, 2, 0, 1, f, 33, f, ws, mv_ws, nullptr), QTCQ_ERR_UNSUPPORTED);
    CHECK("mfma ws", qtcq_decode_matvec_mfma(u, 32, 64, 16, 2, 0, 1, f, 1, f, ws, mv_ws - 1, nullptr), QTCQ_ERR_WORKSPACE);
    CHECK("split ok", qtcq_matvec_mfma_split_x(f, 64, 4, ws, mv_ws, nullptr), kLaunched);
    CHECK("split x null", qtcq_matvec_mfma_split_x(nullptr, 64, 4, ws, mv_ws, nullptr), QTCQ_ERR_INVALID_ARG);
    CHECK("presplit ok", qtcq_decode_matvec_mfma_presplit(u, 32, 64, 16, 2, 0, 0, ws, mv_ws, 4, f, nullptr), kLaunched);
    CHECK("presplit small", qtcq_decode_matvec_mfma_presplit(u, 32, 64, 16, 2, 0, 0, ws, mv_ws - 16, 4, f, nullptr), QTCQ_ERR_WORKSPACE);
    CHECK("noalloc ok", qtcq_decode_matvec_mfma_noalloc(u, 32, 63520, 16, 2, 0, 0, f, 32, f, nullptr), kLaunched);
    CHECK("noalloc too wide", qtcq_decode_matvec_mfma_noalloc(u, 32, 63536, 16, 2, 0, 0, f, 1, f, nullptr), QTCQ_ERR_WORKSPACE);
    CHECK("noalloc batch 0", qtcq_decode_matvec_mfma_noalloc(u, 32, 64, 16, 2, 0, 0, f, 0, f, nullptr), QTCQ_OK);

    if (failures) return 1;
    std::printf("ok\n");
    return 0;
}
