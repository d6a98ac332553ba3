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
from test_gpu_matvec_mfma import check as mfma_check
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
