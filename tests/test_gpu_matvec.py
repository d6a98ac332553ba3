"""GPU parity of the decode -> matrix-vector product against the oracle (binary64 matmul
over the oracle's window decode, row-major 16x16 tiles).

Bar, per output: |y_gpu - y_oracle| <= (4 ceil(N / 1024) + 23) * 2^-24 * sum_n |W x|, the
kernel's fp32 rounding bound (4 FMAs per tile row segment, ceil((N/16)/64) tiles per
thread, 4 shuffle and 15 wave additions, products of the code before its rescale and
one final rescale) plus one unit for the comparison.
A one-hot x must return the decoded column bit for bit (every
other product is an exact zero).  Streams are random words (every bit pattern is a
valid stream) and, at full size, the encoder's own streams of the 4096x4096 matrix.
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs

from helpers import dev, say, u32

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


def words_for(M, N, L, tb):
    W = oracle.tb_stream_words(L, 2, 256) if tb else oracle.stream_words(L, 2, 256)
    return (M // 16) * (N // 16), W


def random_words(M, N, L, tb, seed):
    n, W = words_for(M, N, L, tb)
    return np.random.default_rng(seed).integers(0, 1 << 32, size=(n, W), dtype=np.uint32)


def matrix(words, M, N, C, L, tb):
    dec = oracle.tb_decode if tb else oracle.decode
    _, rec = dec(words, 256, C, L, 2)
    return oracle.tiles_to_matrix(rec, M, N).astype(np.float64)


def check(api, words, M, N, L, code, tb, x, tag):
    import torch
    say("matvec %s M=%d N=%d L=%d code=%s tb=%s batch=%d" % (tag, M, N, L, code, tb, x.shape[0]))
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    y = api.decode_matvec(bd, M, N, dev(x), L=L, k=2, code=code, tailbiting=tb)
    sync()
    C = oracle.code_table(code, L)
    y_o = oracle.decode_matvec(words, M, N, C, x, L, 2, tailbiting=tb)
    Wm = matrix(words, M, N, C, L, tb)
    mag = np.abs(x.astype(np.float64)) @ np.abs(Wm).T
    bound = (4 * -(-N // 1024) + 23) * U32 * mag
    err = np.abs(y.cpu().numpy().astype(np.float64) - y_o)
    assert np.all(err <= bound), "worst err/bound %g" % (err / np.maximum(bound, 1e-300)).max()
    return y


@pytest.mark.parametrize("tb", [False, True])
@pytest.mark.parametrize("L,code", [(16, "1mad"), (16, "3inst"), (12, "1mad"), (6, "3inst")])
@pytest.mark.parametrize("M,N,batch", [(16, 16, 1), (32, 48, 3), (48, 1040, 8), (64, 2064, 2)])
def test_matvec_random_streams(api, tb, L, code, M, N, batch):
    words = random_words(M, N, L, tb, M + N + L)
    x = inputs.targets(batch, N, 7 + N)
    check(api, words, M, N, L, code, tb, x, "random")


# every batch width (the kernel is compiled for 1, 2, 4 and 8 rows; the rows beyond the
# batch re-read its last row and are never stored)
@pytest.mark.parametrize("batch", [4, 5, 6, 7])
def test_matvec_every_batch_width(api, batch):
    M, N, L = 32, 1040, 16
    words = random_words(M, N, L, False, 900 + batch)
    x = inputs.targets(batch, N, 910 + batch)
    y = check(api, words, M, N, L, "1mad", False, x, "batch")
    # each row equals the same row computed alone
    import torch
    for i in (0, batch - 1):
        yi = api.decode_matvec(torch.from_numpy(words.view(np.int32)).cuda(), M, N, dev(x[i:i + 1]),
                               L=L, k=2, code="1mad", tailbiting=False)
        sync()
        assert torch.equal(yi[0], y[i])


@pytest.mark.parametrize("tb", [False, True])
def test_matvec_one_hot_columns_exact(api, tb):
    import torch
    L, M, N = 16, 48, 1056
    words = random_words(M, N, L, tb, 99)
    C = oracle.code_table("1mad", L)
    Wm = matrix(words, M, N, C, L, tb).astype(np.float32)
    cols = np.array([0, 15, 16, 511, 1024, N - 1])
    x = np.zeros((len(cols), N), dtype=np.float32)
    x[np.arange(len(cols)), cols] = 1.0
    say("matvec one-hot tb=%s" % tb)
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    chunks = [x[i:i + 8] for i in range(0, len(cols), 8)]
    ys = [api.decode_matvec(bd, M, N, dev(c), L=L, tailbiting=tb) for c in chunks]
    sync()
    y = np.concatenate([v.cpu().numpy() for v in ys])
    assert np.array_equal(y.view(np.uint32), Wm[:, cols].T.copy().view(np.uint32))


def test_matvec_empty_inner_dimension(api):
    import torch
    x = torch.empty((2, 0), dtype=torch.float32, device="cuda")
    bd = torch.empty((0, 17), dtype=torch.int32, device="cuda")
    say("matvec N=0")
    y = api.decode_matvec(bd, 32, 0, x)
    sync()
    assert torch.count_nonzero(y).item() == 0 and tuple(y.shape) == (2, 32)


def test_matvec_deterministic(api):
    import torch
    M, N = 64, 4096
    words = random_words(M, N, 16, False, 5)
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    x = dev(inputs.targets(4, N, 6))
    say("matvec determinism")
    a = api.decode_matvec(bd, M, N, x)
    b = api.decode_matvec(bd, M, N, x)
    sync()
    assert torch.equal(a, b)


@pytest.mark.parametrize("tb", [False, True])
def test_matvec_encoded_4096x4096(api, tb):
    """The encoder's streams of the 4096x4096 matrix (65,536 sequences as 16x16 tiles):
    the product of the quantized matrix with a batch of 8 activations, every output
    against the oracle."""
    import torch
    s, _, code = inputs.workload("enc4096x4096_1mad")
    M = N = 4096
    say("matvec encoded 4096x4096 tb=%s" % tb)
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
    # the quantized matrix approximates the targets: W x ~ S x with relative error ~ sqrt(MSE)
    S = oracle.tiles_to_matrix(s, M, N).astype(np.float64)
    ys = x.astype(np.float64) @ S.T
    rel = np.linalg.norm(y.cpu().numpy() - ys) / np.linalg.norm(ys)
    assert 0.2 < rel < 0.3
    del bits
    torch.cuda.empty_cache()


@pytest.mark.parametrize("batch", [1, 8])
@pytest.mark.parametrize("code", ["1mad", "3inst"])
def test_matvec_bands_per_workgroup(api, code, batch):
    """1100 bands, one workgroup each: every output against the oracle, and sampled bands
    equal the same bands computed as a 16-band matrix, bit for bit (a band's outputs
    depend on its own streams only)."""
    import torch
    M, N, L = 1100 * 16, 272, 16
    words = random_words(M, N, L, True, 1200 + batch)
    x = inputs.targets(batch, N, 1201 + batch)
    y = check(api, words, M, N, L, code, True, x, "1100 bands")
    NTJ = N // 16
    for b0 in (0, 517, 1084):
        part = torch.from_numpy(words[b0 * NTJ:(b0 + 16) * NTJ].view(np.int32)).cuda()
        yp = api.decode_matvec(part, 256, N, dev(x), L=L, code=code, tailbiting=True)
        sync()
        assert np.array_equal(u32(y)[:, 16 * b0:16 * (b0 + 16)], u32(yp)), "bands %d.." % b0


@pytest.mark.parametrize("batch", [1, 8])
@pytest.mark.parametrize("code,M,N,tb", [("1mad", 28672, 8192, True), ("3inst", 4096, 14336, True),
                                         ("1mad", 4096, 4096, False)])
def test_matvec_full_size_sampled_bands(api, code, M, N, tb, batch):
    """The benchmark's shapes and launch (one workgroup per band of 16 rows, the whole
    matrix in one call) at batch 1 and 8, random streams: 16 sampled bands (first, last
    and seeded) against the oracle on those bands' streams, at the bar above."""
    import torch
    L = 16
    n, W = words_for(M, N, L, tb)
    rng = np.random.default_rng(70 + M + N + batch)
    words = rng.integers(0, 1 << 32, size=(n, W), dtype=np.uint32)
    x = inputs.targets(batch, N, 71 + batch)
    say("matvec full size %dx%d %s tb=%s batch %d" % (M, N, code, tb, batch))
    y = api.decode_matvec(torch.from_numpy(words.view(np.int32)).cuda(), M, N, dev(x), L=L, k=2,
                          code=code, tailbiting=tb)
    sync()
    yh = y.cpu().numpy()
    bands = sorted({0, M // 16 - 1} | set(rng.choice(M // 16, size=14, replace=False).tolist()))
    NTJ = N // 16
    sub = np.concatenate([words[I * NTJ:(I + 1) * NTJ] for I in bands])
    Ms = 16 * len(bands)
    C = oracle.code_table(code, L)
    y_o = oracle.decode_matvec(sub, Ms, N, C, x, L, 2, tailbiting=tb)
    Wm = matrix(sub, Ms, N, C, L, tb)
    bound = (4 * -(-N // 1024) + 23) * U32 * (np.abs(x.astype(np.float64)) @ np.abs(Wm).T)
    cols = np.concatenate([np.arange(16 * I, 16 * I + 16) for I in bands])
    err = np.abs(yh[:, cols].astype(np.float64) - y_o)
    assert np.all(err <= bound), "worst err/bound %g" % (err / np.maximum(bound, 1e-300)).max()
