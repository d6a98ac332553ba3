"""The window decode's two kernels give the same bits: four weights per thread step
(T % 4 == 0, targets, weights and reconstructions 16-byte aligned) and one weight per step
(any T or alignment).  The same call is made with the targets (and weights) in aligned
buffers and at a 4-byte offset, which selects the one-weight kernel; reconstructions and
path-cost MSEs must agree bit for bit, and both equal the oracle's decode.  Covers every
code, plain and tail-biting streams (windows wrapping past the end of a tail-biting
stream), weighted and unweighted path costs, and the shortest tail-biting rows."""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs

from helpers import dev, say, u32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    from trellis_coded_weight_amd import api as a
    return a


def offset_copy(a):
    """a (float32 [B][T]) in device memory 4 bytes past a 16-byte boundary"""
    import torch
    buf = torch.empty(a.size + 4, dtype=torch.float32, device="cuda")
    v = buf[1:1 + a.size].view(a.shape)
    v.copy_(torch.from_numpy(a))
    assert v.data_ptr() % 16 == 4
    return v


def code_of(name, L):
    return ("xor", inputs.xor_masks(L)) if name == "xor" else name


@pytest.mark.parametrize("code", ["1mad", "3inst", "xor"])
@pytest.mark.parametrize("tb", [False, True])
@pytest.mark.parametrize("weighted", [False, True])
@pytest.mark.parametrize("L,T,B", [(16, 256, 37), (12, 64, 50), (8, 4, 9), (16, 8, 5), (14, 1024, 6)])
def test_quad_and_single_kernels_agree(api, code, tb, weighted, L, T, B):
    import torch
    if tb and 2 * T < L:
        pytest.skip("a tail-biting row needs 2T >= L")
    cd = code_of(code, L)
    W = oracle.tb_stream_words(L, 2, T) if tb else oracle.stream_words(L, 2, T)
    rng = np.random.default_rng(7000 + L + T + B + tb)
    words = rng.integers(0, 1 << 32, size=(B, W), dtype=np.uint32)
    nbits = oracle.tb_stream_bits(L, 2, T) if tb else oracle.stream_bits(L, 2, T)
    pad = W * 32 - nbits
    if pad:
        words[:, -1] &= np.uint32((0xFFFFFFFF << pad) & 0xFFFFFFFF)
    s = inputs.targets(B, T, 7001 + T)
    w = inputs.weights(B, T, 7002 + T) if weighted else None
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    dec = api.tailbiting_decode if tb else api.decode
    say("decode kernels code=%s tb=%s weighted=%s L=%d T=%d B=%d" % (code, tb, weighted, L, T, B))
    r4, m4 = dec(bd, T, L=L, code=cd, seq=dev(s), weights=None if w is None else dev(w), want_mse=True)
    r1, m1 = dec(bd, T, L=L, code=cd, seq=offset_copy(s), weights=None if w is None else offset_copy(w),
                 want_mse=True)
    torch.cuda.synchronize()
    assert np.array_equal(u32(r4), u32(r1))
    assert np.array_equal(u32(m4), u32(m1))
    C = oracle.code_table(cd, L)
    odec = oracle.tb_decode if tb else oracle.decode
    _, rec_o = odec(words, T, C, L, 2)
    assert np.array_equal(u32(r4), rec_o.view(np.uint32))
    # the path cost in t order, binary32, as the encoder accumulates it
    for b in range(B):
        assert m4.cpu().numpy()[b] == np.float32(oracle.path_cost(rec_o[b], s[b], None if w is None else w[b]) / T)
