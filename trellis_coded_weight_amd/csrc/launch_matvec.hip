// launch_matvec.hip -- launches of the decode -> matrix-vector products (matvec.hpp,
// matvec_mfma.hpp).
#include <mutex>

#include "host.hpp"
#include "matvec.hpp"
#include "matvec_mfma.hpp"

namespace qtcq {
namespace host {
namespace {

// ---- the LDS-table kernel's grid --------------------------------------------------------
// The table kernel loops over bands (16-row tile rows), one workgroup per resident slot.
// Per device and kernel, once: raise its dynamic-LDS limit and read how many of its
// workgroups one compute unit holds; 0 when the runtime refuses either query.
constexpr int kGridMaxDevices = 64;

struct ResidentState {
    std::once_flag once[kGridMaxDevices];
    int per_cu[kGridMaxDevices] = {};
};

inline int resident_per_cu(const void* kernel, int threads, size_t dyn_lds, ResidentState& state)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kGridMaxDevices) return 0;
    std::call_once(state.once[dev], [&]() {
        int occ = 0;
        hipError_t e = hipSuccess;
        if (dyn_lds > 0)
            e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn_lds);
        if (e == hipSuccess)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, threads, dyn_lds);
        if (e == hipSuccess)
            state.per_cu[dev] = occ > 0 ? occ : 0;
        else
            (void)hipGetLastError();   // a refused query leaves no error behind for the launch
    });
    return state.per_cu[dev];
}

inline int device_cus()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return cus;
}

// The fp32 VALU product of the XOR code through its LDS table (decode_matvec<..., TABLE>),
// when each workgroup gets at least 2^(L-9) tiles, the same threshold as the matrix-core
// table kernel's below; otherwise launches nothing and returns false.
template <int L, bool TB, int NB>
bool launch_valu_table(const uint32_t* bits, int M, int N, int Wd, const float* x, int batch,
                       float* y, const CodeArg& ca, hipStream_t st)
{
    static ResidentState state;
    const auto kernel = decode_matvec<L, kCodeXor, TB, NB, true>;
    constexpr size_t lds = matvec_table_lds_bytes<L, NB>();
    const int per_cu = resident_per_cu(reinterpret_cast<const void*>(kernel), MatvecShape::kThreads, lds, state);
    const int cus = device_cus();
    if (per_cu < 1 || cus < 1) return false;
    const int nb = M / 16;
    const int grid = (int)((int64_t)per_cu * cus < nb ? (int64_t)per_cu * cus : nb);
    const int64_t tiles_per_wg = (int64_t)((nb + grid - 1) / grid) * (N / 16);
    constexpr int need_log2 = L - 9;
    if (tiles_per_wg < ((int64_t)1 << (need_log2 > 0 ? need_log2 : 0))) return false;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(MatvecShape::kThreads), lds, st, bits, M, N, Wd,
                       x, batch, y, ca);
    return true;
}

template <int L, int CODE, bool TB>
qtcq_status matvec_impl(const uint32_t* bits, int M, int N, const float* x, int batch, float* y,
                        const CodeArg& ca, hipStream_t st)
{
    const int Wd = (int)(TB ? tb_stream_words(2, 256) : stream_words(L, 2, 256));
    if constexpr (CODE == kCodeXor) {
        bool done;
        if (batch <= 1)
            done = launch_valu_table<L, TB, 1>(bits, M, N, Wd, x, batch, y, ca, st);
        else if (batch <= 2)
            done = launch_valu_table<L, TB, 2>(bits, M, N, Wd, x, batch, y, ca, st);
        else if (batch <= 4)
            done = launch_valu_table<L, TB, 4>(bits, M, N, Wd, x, batch, y, ca, st);
        else
            done = launch_valu_table<L, TB, 8>(bits, M, N, Wd, x, batch, y, ca, st);
        if (done) return launch_status();
    }
    const dim3 grid((unsigned)(M / 16)), block(MatvecShape::kThreads);
    if (batch <= 1)
        hipLaunchKernelGGL((decode_matvec<L, CODE, TB, 1>), grid, block, 0, st, bits, M, N, Wd, x, batch, y, ca);
    else if (batch <= 2)
        hipLaunchKernelGGL((decode_matvec<L, CODE, TB, 2>), grid, block, 0, st, bits, M, N, Wd, x, batch, y, ca);
    else if (batch <= 4)
        hipLaunchKernelGGL((decode_matvec<L, CODE, TB, 4>), grid, block, 0, st, bits, M, N, Wd, x, batch, y, ca);
    else
        hipLaunchKernelGGL((decode_matvec<L, CODE, TB, 8>), grid, block, 0, st, bits, M, N, Wd, x, batch, y, ca);
    return launch_status();
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

// Launches the table kernel and returns true when it pays: writing the table costs each
// workgroup about as much as the arithmetic decode of 2^(L-9) tiles saves (measured on
// MI355X at L = 12, 14 and 16, batch 1 to 32: 1.05-1.5x at the threshold and above,
// 0.6-1.0x below it).  Otherwise launches nothing and returns false.
template <int L, int CODE, bool TB, int NF>
bool launch_table(const uint32_t* bits, int M, int N, const uint4* xs, const float* sc, int batch,
                  float* y, const CodeArg& ca, hipStream_t st)
{
    static ResidentState state;
    const auto kernel = decode_matvec_mfma<L, CODE, TB, NF, 1, true>;
    constexpr size_t lds = mv_table_lds_bytes<L, NF, 1>();
    const int per_cu = resident_per_cu(reinterpret_cast<const void*>(kernel), MatvecMfmaShape::kThreads, lds, state);
    const int cus = device_cus();
    if (per_cu < 1 || cus < 1) return false;
    const int nb = M / 16;
    const int grid = (int)((int64_t)per_cu * cus < nb ? (int64_t)per_cu * cus : nb);
    const int64_t tiles_per_wg = (int64_t)((nb + grid - 1) / grid) * (N / 16);
    constexpr int need_log2 = L - 9;
    if (tiles_per_wg < ((int64_t)1 << (need_log2 > 0 ? need_log2 : 0))) return false;
    hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(MatvecMfmaShape::kThreads), lds, st, bits, M, N,
                       xs, sc, batch, y, ca);
    return true;
}

// the same product with the decoded weights and the split x on the matrix cores; x ==
// nullptr: the workspace already holds the split of this (N, batch)
template <int L, int CODE, bool TB>
qtcq_status matvec_mfma_impl(const uint32_t* bits, int M, int N, const float* x, int batch,
                             float* y, void* workspace, const CodeArg& ca, hipStream_t st)
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
    if constexpr (CODE == kCodeXor) {
        bool done = false;
        switch (nf) {
        case 1: done = launch_table<L, CODE, TB, 1>(bits, M, N, xs, sc, batch, y, ca, st); break;
        case 2: done = launch_table<L, CODE, TB, 2>(bits, M, N, xs, sc, batch, y, ca, st); break;
        case 3: done = launch_table<L, CODE, TB, 3>(bits, M, N, xs, sc, batch, y, ca, st); break;
        default: done = launch_table<L, CODE, TB, 4>(bits, M, N, xs, sc, batch, y, ca, st); break;
        }
        if (done) return launch_status();
    }
    const bool two = nf >= 3 && nb >= 1024;
    auto go = [&](auto nf_c, auto bands_c) {
        constexpr int NF = decltype(nf_c)::value, BANDS = decltype(bands_c)::value;
        const dim3 grid((unsigned)((nb + BANDS - 1) / BANDS));
        hipLaunchKernelGGL((decode_matvec_mfma<L, CODE, TB, NF, BANDS>), grid, dim3(MatvecMfmaShape::kThreads), 0, st,
                           bits, M, N, xs, sc, batch, y, ca);
    };
    switch (nf) {
    case 1: go(int_c<1>{}, int_c<1>{}); break;
    case 2: if (two) go(int_c<2>{}, int_c<2>{}); else go(int_c<2>{}, int_c<1>{}); break;
    case 3: if (two) go(int_c<3>{}, int_c<2>{}); else go(int_c<3>{}, int_c<1>{}); break;
    default: if (two) go(int_c<4>{}, int_c<2>{}); else go(int_c<4>{}, int_c<1>{}); break;
    }
    return launch_status();
}

// ---- the matrix-core product without allocation ---------------------------------------
// For callers that cannot allocate device memory (graph capture with a fixed memory
// plan, serving loops): the split x lives in this file-scope device array instead of a
// caller workspace.  Every GPU the library runs on holds its own copy until the process
// ends.  Host code never passes `scratch` itself to a kernel (on the host it is a
// stand-in, not a device address): each device's address comes from
// hipGetSymbolAddress, resolved once per device, with that device current, on the first
// call there.
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kNoAllocMaxDevices];

// the current device's scratch address, or nullptr (device index out of range, or the
// symbol lookup failed)
void* scratch_for_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return nullptr;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&slot]() {
        void* p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess) slot.ptr = p;
    });
    return slot.err == hipSuccess ? slot.ptr : nullptr;
}

}  // namespace

int matvec_max_batch() { return MatvecShape::kMaxBatch; }
int matvec_max_n() { return MatvecShape::kMaxN; }
int matvec_mfma_max_batch() { return MatvecMfmaShape::kMaxBatch; }
int matvec_mfma_max_n() { return MatvecMfmaShape::kMaxN; }
size_t matvec_mfma_workspace_bytes(int N) { return MatvecMfmaShape::workspace_bytes(N); }

qtcq_status launch_decode_matvec(int L, const CodeSel& code, bool tb, const uint32_t* bits, int M,
                                 int N, const float* x, int batch, float* y, hipStream_t st)
{
    return with_L_code(L, code.id, [&](auto l, auto c) {
        return with_bool(tb, [&](auto t) {
            return matvec_impl<decltype(l)::value, decltype(c)::value, decltype(t)::value>(
                bits, M, N, x, batch, y, code.arg, st);
        });
    });
}

qtcq_status launch_decode_matvec_mfma(int L, const CodeSel& code, bool tb, const uint32_t* bits,
                                      int M, int N, const float* x, int batch, float* y, void* ws,
                                      hipStream_t st)
{
    return with_L_code(L, code.id, [&](auto l, auto c) {
        return with_bool(tb, [&](auto t) {
            return matvec_mfma_impl<decltype(l)::value, decltype(c)::value, decltype(t)::value>(
                bits, M, N, x, batch, y, ws, code.arg, st);
        });
    });
}

qtcq_status launch_decode_matvec_mfma_noalloc(int L, const CodeSel& code, bool tb,
                                              const uint32_t* bits, int M, int N, const float* x,
                                              int batch, float* y, hipStream_t st)
{
    if (MatvecMfmaShape::workspace_bytes(N) > kNoAllocScratchBytes) return QTCQ_ERR_WORKSPACE;
    void* ws = scratch_for_current_device();
    if (!ws) return QTCQ_ERR_DEVICE;
    return launch_decode_matvec_mfma(L, code, tb, bits, M, N, x, batch, y, ws, st);
}

qtcq_status launch_split_x(const float* x, int N, int batch, void* ws, hipStream_t st)
{
    return split_x_launch(x, N, batch, ws, st);
}

}  // namespace host
}  // namespace qtcq
