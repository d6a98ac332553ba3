"""The entry points can be captured in a HIP graph: they launch kernels on the caller's
stream and allocate nothing, and no call records a memset.  Each captured sequence is
replayed several times, with the inputs changed by eager work and the device synchronised
between replays, and every replay is compared with the same calls run eagerly."""
import numpy as np
import pytest

from trellis_coded_weight_amd import inputs

from helpers import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    from trellis_coded_weight_amd import api as a
    return a


def capture(fn):
    """Warm up on a side stream, then capture fn() into a graph; returns (graph, outputs)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def test_graph_encode_decode_bcjr(api):
    import torch
    L, T, B = 12, 256, 64
    seq = dev(inputs.targets(B, T, 81))
    ws = api.encode_workspace(B, T, L, 2)
    bws = api.bcjr_workspace(B, T, L, 2)

    def step():
        bits, mse, _ = api.encode(seq, L=L, workspace=ws)
        recon, mse2 = api.decode(bits, T, L=L, seq=seq, want_mse=True)
        soft, lz = api.bcjr_soft(seq, 0.1, L=L, workspace=bws)
        return bits, mse, recon, mse2, soft, lz

    say("graph: encode + decode + bcjr L=%d B=%d" % (L, B))
    g, out = capture(step)
    for rep in range(3):
        seq.copy_(dev(inputs.targets(B, T, 90 + rep)))     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = step()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b), "replay %d differs from the eager calls" % rep


def test_graph_decode_matvec(api):
    import torch
    M, N, L = 256, 1024, 16
    rng = np.random.default_rng(82)
    words = rng.integers(0, 1 << 32, size=((M // 16) * (N // 16), 17), dtype=np.uint32)
    bits = torch.from_numpy(words.view(np.int32)).cuda()
    x = dev(inputs.targets(4, N, 83))

    def step():
        return [api.decode_matvec(bits, M, N, x, L=L) for _ in range(8)]

    say("graph: 8 x decode_matvec M=%d N=%d batch 4" % (M, N))
    g, out = capture(step)
    for rep in range(3):
        x.copy_(dev(inputs.targets(4, N, 84 + rep)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = api.decode_matvec(bits, M, N, x, L=L)
        torch.cuda.synchronize()
        for y in out:
            assert torch.equal(y, ref), "replay %d differs from the eager call" % rep


def test_graph_decode_matvec_mfma(api):
    """The matrix-core product (split kernel + product kernel, one shared workspace)
    captured 8 times over, replays equal to the eager call."""
    import torch
    M, N, L = 256, 1040, 16
    rng = np.random.default_rng(85)
    words = rng.integers(0, 1 << 32, size=((M // 16) * (N // 16), 16), dtype=np.uint32)
    bits = torch.from_numpy(words.view(np.int32)).cuda()
    x = dev(inputs.targets(8, N, 86))
    ws = api.matvec_mfma_workspace(N)

    def step():
        return [api.decode_matvec_mfma(bits, M, N, x, L=L, code="3inst", tailbiting=True,
                                       workspace=ws) for _ in range(8)]

    say("graph: 8 x decode_matvec_mfma M=%d N=%d batch 8" % (M, N))
    g, out = capture(step)
    for rep in range(3):
        x.copy_(dev(inputs.targets(8, N, 87 + rep)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = api.decode_matvec_mfma(bits, M, N, x, L=L, code="3inst", tailbiting=True)
        torch.cuda.synchronize()
        for y in out:
            assert torch.equal(y, ref), "replay %d differs from the eager call" % rep


def test_graph_matvec_mfma_split_once_wide_batch(api):
    """One split and three products of 32 rows (four fragments; the tall matrix runs two
    bands per workgroup) captured together; replays equal the eager one-call products."""
    import torch
    N, L = 1040, 16
    rng = np.random.default_rng(88)
    shapes = [(16400, True), (64, False), (4096, True)]
    mats = []
    for M, tb in shapes:
        W = 16 if tb else 17
        words = rng.integers(0, 1 << 32, size=((M // 16) * (N // 16), W), dtype=np.uint32)
        mats.append((torch.from_numpy(words.view(np.int32)).cuda(), M, tb))
    x = dev(inputs.targets(32, N, 89))
    ws = api.matvec_mfma_workspace(N)

    def step():
        sp = api.matvec_mfma_split_x(x, workspace=ws)
        return [api.decode_matvec_mfma_presplit(b, M, N, sp, L=L, tailbiting=tb)
                for b, M, tb in mats]

    say("graph: split + 3 x decode_matvec_mfma_presplit batch 32")
    g, out = capture(step)
    for rep in range(3):
        x.copy_(dev(inputs.targets(32, N, 90 + rep)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        refs = [api.decode_matvec_mfma(b, M, N, x, L=L, tailbiting=tb) for b, M, tb in mats]
        torch.cuda.synchronize()
        for y, ref in zip(out, refs):
            assert torch.equal(y, ref), "replay %d differs from the eager call" % rep
