"""GPU parity of the decode -> matrix-vector product on the matrix cores
(qtcq_decode_matvec_mfma) against the oracle (binary64 matmul over the oracle's window
decode, row-major 16x16 tiles).

Bar, per output (u = 2^-24, K = ceil(ceil(N/32)/16) k-blocks per wave):
    |y_gpu - y_oracle| <= (86 + K) u sum_n |W x| + 2^-38 max_n |x| sum_n |W|,
the kernel's stated bound -- x split per 32-column block into two scaled fp16 parts (4u),
each addition in a 32-product matrix instruction allowed 2u (62u), K accumulator
additions, hi + lo, 15 wave additions, the code's rescale (2.5u) -- plus one unit for the
comparison, and twice the split's absolute term.  A one-hot x must return the decoded column bit for bit.  Streams
are random words (every bit pattern is a valid stream) and the encoder's own streams of
the 4096x4096 matrix.  Inner dimensions with N/16 odd cover the half k-block.
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs

from helpers import dev, say, u32
from test_gpu_matvec import matrix, random_words

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    from trellis_coded_weight_amd import api as a
    return a


def sync():
    import torch
    torch.cuda.synchronize()


def bound(x, Wm, N):
    K = -(-(-(-N // 32)) // 16)
    x64 = x.astype(np.float64)
    mag = np.abs(x64) @ np.abs(Wm).T
    amax = np.abs(x64).max(axis=1, initial=0.0)[:, None]
    return (86 + K) * U32 * mag + 2.0 ** -38 * amax * np.abs(Wm).sum(axis=1)[None, :]


def check(api, words, M, N, L, code, tb, x, tag):
    import torch
    say("matvec_mfma %s M=%d N=%d L=%d code=%s tb=%s batch=%d" % (tag, M, N, L, code, tb, x.shape[0]))
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    y = api.decode_matvec_mfma(bd, M, N, dev(x), L=L, k=2, code=code, tailbiting=tb)
    sync()
    C = oracle.code_table(code, L)
    y_o = oracle.decode_matvec(words, M, N, C, x, L, 2, tailbiting=tb)
    Wm = matrix(words, M, N, C, L, tb)
    b = bound(x, Wm, N)
    err = np.abs(y.cpu().numpy().astype(np.float64) - y_o)
    assert np.all(err <= b), "worst err/bound %g" % (err / np.maximum(b, 1e-300)).max()
    return y


@pytest.mark.parametrize("tb", [False, True])
@pytest.mark.parametrize("L,code", [(16, "1mad"), (16, "3inst"), (12, "1mad"), (6, "3inst")])
@pytest.mark.parametrize("M,N,batch", [(16, 16, 1), (32, 48, 3), (48, 1040, 8), (64, 2064, 2),
                                       (16, 1024, 8)])
def test_matvec_mfma_random_streams(api, tb, L, code, M, N, batch):
    words = random_words(M, N, L, tb, M + N + L)
    x = inputs.targets(batch, N, 7 + N)
    check(api, words, M, N, L, code, tb, x, "random")


@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 16, 17, 24, 25, 31, 32])
def test_matvec_mfma_every_batch_width(api, batch):
    """Batch widths over one to four B fragments of 8 rows, full and partial; each row
    equals the same row computed alone, bit for bit (the row's block scales and
    matrix-core column do not depend on the other rows or on how many fragments run)."""
    import torch
    M, N, L = 32, 1040, 16
    words = random_words(M, N, L, False, 900 + batch)
    x = inputs.targets(batch, N, 910 + batch)
    y = check(api, words, M, N, L, "1mad", False, x, "batch")
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    for i in sorted({0, 7 % batch, 8 % batch, batch - 1}):
        yi = api.decode_matvec_mfma(bd, M, N, dev(x[i:i + 1]), L=L)
        sync()
        assert torch.equal(yi[0], y[i])


@pytest.mark.parametrize("tb", [False, True])
@pytest.mark.parametrize("code", ["1mad", "3inst"])
def test_matvec_mfma_batch_32(api, tb, code):
    """Four fragments, ragged N / 16, both codes and stream kinds."""
    words = random_words(48, 2064, 16, tb, 70)
    x = inputs.targets(32, 2064, 71)
    check(api, words, 48, 2064, 16, code, tb, x, "batch 32")


@pytest.mark.parametrize("tb", [False, True])
@pytest.mark.parametrize("code", ["1mad", "3inst"])
def test_matvec_mfma_one_hot_columns_exact(api, tb, code):
    import torch
    L, M, N = 16, 48, 1056
    words = random_words(M, N, L, tb, 99)
    C = oracle.code_table(code, L)
    Wm = matrix(words, M, N, C, L, tb).astype(np.float32)
    cols = np.array([0, 15, 16, 31, 32, 511, 1024, N - 1])
    x = np.zeros((len(cols), N), dtype=np.float32)
    x[np.arange(len(cols)), cols] = 1.0
    x[3] *= -0.375                     # its block scaled by 2^16 to an exact fp16 -24576
    say("matvec_mfma one-hot tb=%s code=%s" % (tb, code))
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    y = api.decode_matvec_mfma(bd, M, N, dev(x), L=L, code=code, tailbiting=tb).cpu().numpy()
    want = Wm[:, cols].T.astype(np.float64) * x[np.arange(len(cols)), cols][:, None]
    # rows with x = 1 are W's columns bit for bit; the -3/8 row's sum is exact, and its
    # rescale rounds raw * (-3/8) / D once where W * (-3/8) rounded raw / D
    ones = [i for i in range(len(cols)) if i != 3]
    assert np.array_equal(y[ones].view(np.uint32), want[ones].astype(np.float32).view(np.uint32))
    assert np.all(np.abs(y[3] - want[3]) <= 3 * U32 * np.abs(want[3]))


@pytest.mark.parametrize("scale", [2.0 ** 100, 2.0 ** -100, 1e-30, 3e30])
def test_matvec_mfma_scaled_rows(api, scale):
    """The per-block power-of-two scale keeps fp16 in range whatever the magnitude of x."""
    M, N = 32, 2064
    words = random_words(M, N, 16, False, 31)
    x = (inputs.targets(3, N, 32).astype(np.float64) * scale).astype(np.float32)
    check(api, words, M, N, 16, "1mad", False, x, "scale %g" % scale)


def test_matvec_mfma_mixed_magnitudes(api):
    """Elements spanning many binades within a row (the small ones lose nothing but the
    split's absolute term against their block's maximum), a zero row and a one-element
    row."""
    M, N = 48, 1040
    words = random_words(M, N, 16, True, 41)
    rng = np.random.default_rng(42)
    x = inputs.targets(4, N, 43)
    x[0] *= (10.0 ** rng.uniform(-12, 6, size=N)).astype(np.float32)
    x[1] = 0.0
    x[2] = 0.0
    x[2, 517] = 3.0e-7
    x[3] *= (2.0 ** rng.integers(-60, 60, size=N)).astype(np.float32)
    y = check(api, words, M, N, 16, "1mad", True, x, "mixed")
    assert not np.any(y.cpu().numpy()[1])


def test_matvec_mfma_nonfinite_row(api):
    """inf / NaN in a row of x give non-finite outputs in that row only."""
    import torch
    M, N = 32, 1024
    words = random_words(M, N, 16, False, 51)
    x = inputs.targets(3, N, 52)
    x[0, 5] = np.inf
    x[2, 700] = np.nan
    say("matvec_mfma non-finite rows")
    y = api.decode_matvec_mfma(torch.from_numpy(words.view(np.int32)).cuda(), M, N, dev(x))
    sync()
    yh = y.cpu().numpy()
    assert not np.isfinite(yh[0]).any() and not np.isfinite(yh[2]).any()
    C = oracle.code_table("1mad", 16)
    y_o = oracle.decode_matvec(words, M, N, C, x[1:2], 16, 2)
    Wm = matrix(words, M, N, C, 16, False)
    assert np.all(np.abs(yh[1:2] - y_o) <= bound(x[1:2], Wm, N))


def test_matvec_mfma_empty_and_degenerate(api):
    import torch
    say("matvec_mfma N=0, M=0, batch=0")
    x = torch.empty((2, 0), dtype=torch.float32, device="cuda")
    bd = torch.empty((0, 17), dtype=torch.int32, device="cuda")
    y = api.decode_matvec_mfma(bd, 32, 0, x)
    sync()
    assert torch.count_nonzero(y).item() == 0 and tuple(y.shape) == (2, 32)
    y0 = api.decode_matvec_mfma(torch.empty((0, 17), dtype=torch.int32, device="cuda"), 0, 64,
                                torch.ones((3, 64), device="cuda"))
    xb = torch.empty((0, 64), dtype=torch.float32, device="cuda")
    yb = api.decode_matvec_mfma(torch.zeros((4 * 4, 17), dtype=torch.int32, device="cuda"), 64, 64, xb)
    sync()
    assert tuple(y0.shape) == (3, 0) and tuple(yb.shape) == (0, 64)


def test_matvec_mfma_deterministic_and_workspace_reuse(api):
    """Two calls give the same bits; a workspace reused after a wider call (stale split
    values of other rows and columns in it) changes nothing."""
    import torch
    M, N = 64, 4096
    words = random_words(M, N, 16, False, 5)
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    ws = api.matvec_mfma_workspace(N)
    x32 = dev(inputs.targets(32, N, 6))
    x2 = dev(inputs.targets(2, N, 7))
    say("matvec_mfma determinism")
    a = api.decode_matvec_mfma(bd, M, N, x2, workspace=ws)
    api.decode_matvec_mfma(bd, M, N, x32, workspace=ws)
    b = api.decode_matvec_mfma(bd, M, N, x2, workspace=ws)
    c = api.decode_matvec_mfma(bd, M, N, x2)
    sync()
    assert torch.equal(a, b) and torch.equal(a, c)


def test_matvec_mfma_wide_inner_dimension(api):
    M, N, L = 32, 65536, 16
    words = random_words(M, N, L, False, 4748)
    x = inputs.targets(8, N, 4749)
    check(api, words, M, N, L, "1mad", False, x, "wide")


@pytest.mark.parametrize("tb", [False, True])
def test_matvec_mfma_encoded_4096x4096(api, tb):
    """The encoder's streams of the 4096x4096 matrix, batch 8, every output against the
    oracle, and against the fp32 VALU product within the sum of both bounds."""
    import torch
    s, _, code = inputs.workload("enc4096x4096_1mad")
    M = N = 4096
    say("matvec_mfma encoded 4096x4096 tb=%s" % tb)
    sd = dev(s)
    if tb:
        bits, _, _ = api.tailbiting_encode(sd, L=16, k=2, code=code,
                                           workspace=api.tailbiting_workspace(65536, max_bytes=64 << 30))
    else:
        bits, _, _ = api.encode(sd, L=16, k=2, code=code,
                                workspace=api.encode_workspace(65536, max_bytes=64 << 30))
    sync()
    x = inputs.targets(8, N, 12)
    y = check(api, u32(bits), M, N, 16, code, tb, x, "encoded")
    yv = api.decode_matvec(bits, M, N, dev(x), L=16, k=2, code=code, tailbiting=tb)
    sync()
    C = oracle.code_table(code, 16)
    Wm = matrix(u32(bits), M, N, C, 16, tb)
    mag = np.abs(x.astype(np.float64)) @ np.abs(Wm).T
    both = bound(x, Wm, N) + (4 * -(-N // 1024) + 23) * U32 * mag
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - yv.cpu().numpy()) <= both)
    del bits
    torch.cuda.empty_cache()


@pytest.mark.parametrize("batch", [8, 32])
@pytest.mark.parametrize("code,M,N", [("1mad", 28672, 8192), ("3inst", 4096, 14336)])
def test_matvec_mfma_full_size_sampled_bands(api, code, M, N, batch):
    """The benchmark's tail-biting shapes at batch 8 and 32 (random streams; 28672x8192 at
    batch 32 runs two bands per workgroup): 16 sampled bands of 16 output rows (first,
    last and seeded) against the oracle on those bands' streams."""
    import torch
    L, W = 16, 16
    rng = np.random.default_rng(60 + M)
    words = rng.integers(0, 1 << 32, size=((M // 16) * (N // 16), W), dtype=np.uint32)
    x = inputs.targets(batch, N, 61)
    say("matvec_mfma full size %dx%d %s batch %d" % (M, N, code, batch))
    y = api.decode_matvec_mfma(torch.from_numpy(words.view(np.int32)).cuda(), M, N, dev(x),
                               L=L, code=code, tailbiting=True)
    sync()
    yh = y.cpu().numpy()
    bands = sorted({0, M // 16 - 1} | set(rng.choice(M // 16, size=14, replace=False).tolist()))
    NTJ = N // 16
    sub = np.concatenate([words[I * NTJ:(I + 1) * NTJ] for I in bands])
    Ms = 16 * len(bands)
    C = oracle.code_table(code, L)
    y_o = oracle.decode_matvec(sub, Ms, N, C, x, L, 2, tailbiting=True)
    Wm = matrix(sub, Ms, N, C, L, True)
    cols = np.concatenate([np.arange(16 * I, 16 * I + 16) for I in bands])
    err = np.abs(yh[:, cols].astype(np.float64) - y_o)
    assert np.all(err <= bound(x, Wm, N))


@pytest.mark.parametrize("M,batch", [(16384, 9), (16400, 32), (16400, 16)])
def test_matvec_mfma_two_bands_per_workgroup(api, M, batch):
    """M / 16 >= 1024 with more than 8 rows: each workgroup takes two bands (the last one
    alone when M / 16 is odd); every output against the oracle."""
    N = 80
    words = random_words(M, N, 16, True, M + batch)
    x = inputs.targets(batch, N, 72)
    check(api, words, M, N, 16, "3inst", True, x, "two bands")


@pytest.mark.parametrize("batch", [1, 8, 20, 32])
def test_matvec_mfma_presplit_equals_one_call(api, batch):
    """One split of x serves three matrices of different heights (plain and tail-biting,
    both codes): each product equals the one-call product bit for bit, and the split is
    not modified by the products."""
    import torch
    N = 1040
    x = dev(inputs.targets(batch, N, 80 + batch))
    say("matvec_mfma presplit batch=%d" % batch)
    split = api.matvec_mfma_split_x(x)
    assert (split.N, split.batch) == (N, batch)
    sync()
    before = split.workspace.clone()
    for M, code, tb, seed in [(48, "1mad", False, 1), (16400, "3inst", True, 2), (4096, "1mad", True, 3)]:
        words = random_words(M, N, 16, tb, 300 + seed)
        bd = torch.from_numpy(words.view(np.int32)).cuda()
        y1 = api.decode_matvec_mfma_presplit(bd, M, N, split, code=code, tailbiting=tb)
        y2 = api.decode_matvec_mfma(bd, M, N, x, code=code, tailbiting=tb)
        sync()
        assert torch.equal(y1, y2), "M=%d" % M
    assert torch.equal(split.workspace, before)


@pytest.mark.parametrize("batch", [1, 8, 32])
@pytest.mark.parametrize("code", ["1mad", "3inst"])
def test_matvec_mfma_bands_per_workgroup(api, code, batch):
    """1100 bands (two per workgroup at batch 32): every output against the oracle, and
    sampled bands equal the same bands computed as a 16-band matrix, bit for bit (a
    band's outputs depend on its own streams only)."""
    import torch
    M, N, L = 1100 * 16, 272, 16
    words = random_words(M, N, L, True, 1100 + batch)
    x = inputs.targets(batch, N, 1101 + batch)
    y = check(api, words, M, N, L, code, True, x, "1100 bands")
    NTJ = N // 16
    for b0 in (0, 517, 1084):
        part = torch.from_numpy(words[b0 * NTJ:(b0 + 16) * NTJ].view(np.int32)).cuda()
        yp = api.decode_matvec_mfma(part, 256, N, dev(x), L=L, code=code, tailbiting=True)
        sync()
        assert np.array_equal(u32(y)[:, 16 * b0:16 * (b0 + 16)], u32(yp)), "bands %d.." % b0
