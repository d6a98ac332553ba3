"""GPU parity of the XOR-Trellis palette code (XOR-Trellis explainer, "The sign at each
junction has to be cheap") through every entry point, against the CPU oracle's own
implementation of the code, with the parity masks as inputs.

Bars as for the other codes: code tables, states, bitstreams, reconstructions and MSEs
bit-exact (plain and tail-biting, weighted and not); the soft codeword, log Z and the
gradient within 1e-5 * RMS of the binary64 oracle; the decode -> matvec products within
their stated rounding bounds, one-hot columns exact.  Targets are N(0, 1) scaled to the
palettes' spread (inputs.xor_targets).
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs

from helpers import bcjr_err, dev, oracle_vjp_par, say, u32
from test_gpu_bcjr import run_and_compare as bcjr_compare
from test_gpu_bcjr_vjp import run_and_compare as vjp_compare, upstream
from test_gpu_encode import check_encode
from test_gpu_matvec import check as matvec_check, random_words
from test_gpu_matvec import matrix as mfma_matrix
from test_gpu_matvec_mfma import bound as mfma_bound, check as mfma_check
from test_gpu_tailbiting import check_tb

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    from trellis_coded_weight_amd import api as a
    return a


def sync():
    import torch
    torch.cuda.synchronize()


def xcode(L, masks=None):
    return ("xor", inputs.xor_masks(L) if masks is None else masks)


@pytest.mark.parametrize("L", [2, 6, 10, 16])
def test_code_table_exhaustive(api, L):
    rng = np.random.default_rng(L)
    sets = [inputs.xor_masks(L), (0, 0, 0, 0)] + \
        [tuple(int(m) for m in rng.integers(0, 1 << max(L - 2, 0), 4)) for _ in range(3)]
    for masks in sets:
        say("xor code_table L=%d masks=%s" % (L, masks))
        got = api.code_table(("xor", masks), L)
        sync()
        want = oracle.code_table(("xor", masks), L)
        assert np.array_equal(u32(got), want.view(np.uint32))


@pytest.mark.parametrize("L", [6, 8, 12, 14])
@pytest.mark.parametrize("T", [1, 37, 256])
@pytest.mark.parametrize("weighted", [False, True])
def test_encode_decode_small_trellis(api, L, T, weighted):
    seed = 4000 + 10 * L + T
    s = inputs.xor_targets(5, T, seed)
    w = inputs.weights(5, T, seed + 1) if weighted else None
    check_encode(api, s, w, L, xcode(L))


def test_encode_decode_L16(api):
    s = inputs.xor_targets(16, 256, 4100)
    check_encode(api, s, None, 16, xcode(16))
    w = inputs.weights(3, 256, 4101)
    check_encode(api, s[:3], w, 16, xcode(16))


def test_encode_paired_workgroups(api):
    """More sequences than compute units: two interleaved sequences per workgroup."""
    s = inputs.xor_targets(301, 64, 4200)
    check_encode(api, s, None, 8, xcode(8))


def test_decode_random_streams(api):
    import torch
    L, T, B = 16, 256, 64
    W = oracle.stream_words(L, 2, T)
    words = np.random.default_rng(4300).integers(0, 1 << 32, size=(B, W), dtype=np.uint32)
    nbits = oracle.stream_bits(L, 2, T)
    pad = W * 32 - nbits
    words[:, -1] &= np.uint32((0xFFFFFFFF << pad) & 0xFFFFFFFF)
    say("xor decode random streams")
    recon, _ = api.decode(torch.from_numpy(words.view(np.int32)).cuda(), T, L=L, code=xcode(L))
    sync()
    _, rec_o = oracle.decode(words, T, oracle.code_table(xcode(L), L), L, 2)
    assert np.array_equal(u32(recon), rec_o.view(np.uint32))


@pytest.mark.parametrize("L,T", [(6, 7), (8, 37), (12, 256), (16, 256)])
@pytest.mark.parametrize("weighted", [False, True])
def test_tailbiting(api, L, T, weighted):
    B = 5 if L < 16 else 3
    s = inputs.xor_targets(B, T, 4400 + L + T)
    w = inputs.weights(B, T, 4401) if weighted else None
    check_tb(api, s, w, L, xcode(L))


@pytest.mark.parametrize("L", [8, 12])
@pytest.mark.parametrize("tau", [1.0, 0.1, 0.01])
def test_bcjr_soft(api, L, tau):
    s = inputs.xor_targets(4, 64, 4500 + L)
    bcjr_compare(api, s, None, tau, L, xcode(L))


def test_bcjr_soft_weighted_L16(api):
    s = inputs.xor_targets(2, 256, 4510)
    w = inputs.weights(2, 256, 4511)
    bcjr_compare(api, s, w, 0.1, 16, xcode(16))


@pytest.mark.parametrize("L", [8, 12])
@pytest.mark.parametrize("tau", [0.1, 0.01, 3e-3])
def test_bcjr_vjp(api, L, tau):
    s = inputs.xor_targets(3, 48, 4600 + L)
    w = inputs.weights(3, 48, 4601)
    vjp_compare(api, s, w, upstream(3, 48, 4602), tau, L, xcode(L))


@pytest.mark.parametrize("tb", [False, True])
@pytest.mark.parametrize("L", [16, 8])
@pytest.mark.parametrize("M,N,batch", [(16, 16, 1), (48, 1040, 8), (64, 2064, 3)])
def test_matvec_both_products(api, tb, L, M, N, batch):
    words = random_words(M, N, L, tb, 4700 + M + N + L)
    x = inputs.targets(batch, N, 4701 + N)
    matvec_check(api, words, M, N, L, xcode(L), tb, x, "xor")
    mfma_check(api, words, M, N, L, xcode(L), tb, x, "xor")


def test_matvec_one_hot_columns_exact(api):
    import torch
    M, N, L = 32, 64, 16
    words = random_words(M, N, L, True, 4800)
    C = oracle.code_table(xcode(L), L)
    _, rec = oracle.tb_decode(words, 256, C, L, 2)
    Wm = oracle.tiles_to_matrix(rec, M, N)
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    for n in (0, 17, 63):
        x = np.zeros((1, N), dtype=np.float32)
        x[0, n] = 1.0
        say("xor matvec one-hot column %d" % n)
        y = api.decode_matvec(bd, M, N, dev(x), L=L, code=xcode(L), tailbiting=True)
        ym = api.decode_matvec_mfma(bd, M, N, dev(x), L=L, code=xcode(L), tailbiting=True)
        sync()
        assert np.array_equal(y.cpu().numpy()[0], Wm[:, n].astype(np.float32))
        assert np.array_equal(ym.cpu().numpy()[0], Wm[:, n].astype(np.float32))


def test_invalid_masks_rejected(api):
    import torch
    from trellis_coded_weight_amd import _native as nat
    s = torch.zeros((2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(nat.QtcqError):
        api.encode(s, L=8, code=("xor", (1 << 6, 0, 0, 0)))     # history has 6 bits at L = 8
    with pytest.raises(ValueError):
        api.encode(s, L=16, code=("xor", (1 << 14, 0, 0, 0)))
    sync()


# ---- the LDS-table decode of the matrix-core product ------------------------------------
# For the XOR code the product reads each window's code from a 2^L-entry table in LDS
# once a workgroup has enough tiles to pay for writing it: 2^(L-9) tiles (one workgroup
# per compute unit at L = 16, looping over bands).  The values and their order are the
# arithmetic decode's, so the bits match.

def cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("tb", [False, True])
@pytest.mark.parametrize("L,M,N,batch", [(16, 32, 4096, 1), (16, 48, 4112, 8), (16, 16, 8192, 20),
                                         (16, 16, 8208, 32), (14, 64, 1040, 3), (12, 64, 1040, 32),
                                         (10, 48, 272, 9), (6, 32, 48, 2)])
def test_matvec_table_path_oracle(api, tb, L, M, N, batch):
    words = random_words(M, N, L, tb, 4900 + M + N + L + batch)
    x = inputs.targets(batch, N, 4901 + N + batch)
    mfma_check(api, words, M, N, L, xcode(L), tb, x, "xor table")


@pytest.mark.parametrize("batch", [1, 20])
def test_matvec_table_path_matches_arithmetic_path(api, batch):
    """At L = 16 a workgroup needs 128 tiles before the table pays.  With N = 1024 a band
    is 64 tiles: 256 bands (one per workgroup on 256 compute units) run the arithmetic
    decode, 512 bands (two per workgroup) the table.  The first 256 bands are the same
    streams in both, and their outputs the same bits."""
    import torch
    if cus() != 256:
        pytest.skip("the split between the two paths assumes 256 compute units")
    L, N = 16, 1024
    words = random_words(512 * 16, N, L, True, 4950 + batch)
    x = inputs.targets(batch, N, 4951 + batch)
    say("xor matvec table vs arithmetic, batch %d" % batch)
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    y_tab = api.decode_matvec_mfma(bd, 512 * 16, N, dev(x), L=L, code=xcode(L), tailbiting=True)
    n_half = 256 * (N // 16)          # tiles of the first 256 bands
    y_ar = api.decode_matvec_mfma(bd[:n_half], 256 * 16, N, dev(x), L=L, code=xcode(L), tailbiting=True)
    sync()
    assert np.array_equal(u32(y_tab)[:, :256 * 16], u32(y_ar))
    # and the table run's second half of the rows against the oracle
    C = oracle.code_table(xcode(L), L)
    y_o = oracle.decode_matvec(words[n_half:], 256 * 16, N, C, x, L, 2, tailbiting=True)
    Wm = mfma_matrix(words[n_half:], 256 * 16, N, C, L, True)
    err = np.abs(y_tab.cpu().numpy()[:, 256 * 16:].astype(np.float64) - y_o)
    assert np.all(err <= mfma_bound(x, Wm, N))


def test_matvec_table_path_bands_per_workgroup(api):
    """700 bands over the resident workgroups (several bands each at L = 16): every band's
    outputs equal the same band computed in a 16-band matrix, bit for bit, and the whole
    product meets the oracle bound."""
    import torch
    L, N, M = 16, 4096, 700 * 16
    words = random_words(M, N, L, False, 4960)
    x = inputs.targets(3, N, 4961)
    y = mfma_check(api, words, M, N, L, xcode(L), False, x, "xor 700 bands")
    Wd = oracle.stream_words(L, 2, 256)
    for b0 in (0, 300, 684):
        part = words[b0 * (N // 16):(b0 + 16) * (N // 16)]
        bd = torch.from_numpy(part.view(np.int32)).cuda()
        say("xor matvec bands %d..%d alone" % (b0, b0 + 15))
        yp = api.decode_matvec_mfma(bd, 256, N, dev(x), L=L, code=xcode(L), tailbiting=False)
        sync()
        assert part.shape[1] == Wd
        assert np.array_equal(u32(y)[:, b0 * 16:(b0 + 16) * 16], u32(yp))


def test_matvec_table_path_one_hot_columns_exact(api):
    import torch
    M, N, L = 32, 4096, 16
    words = random_words(M, N, L, True, 4970)
    C = oracle.code_table(xcode(L), L)
    _, rec = oracle.tb_decode(words, 256, C, L, 2)
    Wm = oracle.tiles_to_matrix(rec, M, N)
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    for n in (0, 1234, 4095):
        x = np.zeros((1, N), dtype=np.float32)
        x[0, n] = 1.0
        say("xor table matvec one-hot column %d" % n)
        ym = api.decode_matvec_mfma(bd, M, N, dev(x), L=L, code=xcode(L), tailbiting=True)
        sync()
        assert np.array_equal(ym.cpu().numpy()[0], Wm[:, n].astype(np.float32))


@pytest.mark.parametrize("product,batch", [("valu", 1), ("valu", 8), ("mfma", 1), ("mfma", 8), ("mfma", 32)])
def test_matvec_full_size_sampled_bands(api, product, batch):
    """The benchmark's XOR shape, 28672x8192 tail-biting with random streams, through both
    products in the benchmark's launch (the matrix-core product through its LDS code
    table): 16 sampled bands of 16 output rows (first, last and seeded) against the
    oracle on those bands' streams, each at its product's bar."""
    import torch
    L, M, N = 16, 28672, 8192
    words = random_words(M, N, L, True, 5100 + batch)
    rng = np.random.default_rng(5101 + batch)
    x = inputs.targets(batch, N, 5102 + batch)
    say("xor matvec full size, %s batch %d" % (product, batch))
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    if product == "valu":
        y = api.decode_matvec(bd, M, N, dev(x), L=L, k=2, code=xcode(L), tailbiting=True)
    else:
        y = api.decode_matvec_mfma(bd, M, N, dev(x), L=L, code=xcode(L), tailbiting=True)
    sync()
    yh = y.cpu().numpy()
    bands = sorted({0, M // 16 - 1} | set(rng.choice(M // 16, size=14, replace=False).tolist()))
    NTJ = N // 16
    sub = np.concatenate([words[I * NTJ:(I + 1) * NTJ] for I in bands])
    Ms = 16 * len(bands)
    C = oracle.code_table(xcode(L), L)
    y_o = oracle.decode_matvec(sub, Ms, N, C, x, L, 2, tailbiting=True)
    Wm = mfma_matrix(sub, Ms, N, C, L, True)
    if product == "valu":
        bar = (4 * -(-N // 1024) + 23) * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(Wm).T)
    else:
        bar = mfma_bound(x, Wm, N)
    cols = np.concatenate([np.arange(16 * I, 16 * I + 16) for I in bands])
    err = np.abs(yh[:, cols].astype(np.float64) - y_o)
    assert np.all(err <= bar), "worst err/bar %g" % (err / np.maximum(bar, 1e-300)).max()
