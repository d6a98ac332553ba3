"""GPU parity: computed codes, Viterbi encode and window decode through the C ABI,
element by element against the CPU oracle on the same seeded inputs.  Bar: bit-exact
states, bitstreams, reconstructions and MSEs (integer and tie decisions are taken in
binary32 on both sides).
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs

from helpers import dev, oracle_viterbi_par, say, u32

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


@pytest.mark.parametrize("code", ["1mad", "3inst"])
def test_code_table_exhaustive(api, code):
    for L in (16, 20):
        say("code_table %s L=%d" % (code, L))
        got = api.code_table(code, L)
        sync()
        want = oracle.code_table(code, L)
        assert np.array_equal(u32(got), want.view(np.uint32))


def check_encode(api, s, w, L, code, workspace=None):
    B, T = s.shape
    say("encode L=%d T=%d B=%d code=%s weighted=%s" % (L, T, B, code, w is not None))
    sd = dev(s)
    wd = None if w is None else dev(w)
    bits, mse, states = api.encode(sd, wd, L=L, k=2, code=code, want_states=True,
                                   workspace=workspace)
    recon, mse2 = api.decode(bits, T, L=L, k=2, code=code, seq=sd, weights=wd, want_mse=True)
    sync()
    C = oracle.code_table(code, L)
    st_o, cost_o, mse_o = oracle_viterbi_par(C, s, w, L=L)
    words_o = oracle.pack(st_o, L, 2)
    _, rec_o = oracle.decode(words_o, T, C, L, 2)
    assert np.array_equal(u32(states), st_o)
    assert np.array_equal(u32(bits), words_o)
    assert np.array_equal(mse.cpu().numpy().view(np.uint32), mse_o.view(np.uint32))
    assert np.array_equal(recon.cpu().numpy().view(np.uint32), rec_o.view(np.uint32))
    assert np.array_equal(mse2.cpu().numpy().view(np.uint32), mse_o.view(np.uint32))
    return bits, mse, states


@pytest.mark.parametrize("L", [6, 8, 10, 12, 14])
@pytest.mark.parametrize("T", [1, 2, 17, 256])
@pytest.mark.parametrize("code,weighted", [("1mad", False), ("3inst", False), ("1mad", True)])
def test_encode_small_trellis(api, L, T, code, weighted):
    B = 5 if L <= 12 else 2
    seed = 1000 * L + T
    s = inputs.targets(B, T, seed)
    w = inputs.weights(B, T, seed + 1) if weighted else None
    check_encode(api, s, w, L, code)


def test_encode_L16_sixteen_sequences(api):
    s, w, code = inputs.workload("enc16_1mad")
    check_encode(api, s, w, 16, code)


@pytest.mark.parametrize("T", [1, 2, 33, 256])
@pytest.mark.parametrize("code,weighted", [("3inst", False), ("1mad", True)])
def test_encode_L16_variants(api, T, code, weighted):
    B = 3
    s = inputs.targets(B, T, 77 + T)
    w = inputs.weights(B, T, 78 + T) if weighted else None
    check_encode(api, s, w, 16, code)


def test_encode_chunked_workspace_matches(api):
    # a workspace holding 3 sequences forces chunks of 3, 3, 2
    import torch
    s = inputs.targets(8, 256, 91)
    say("encode chunked B=8 ws=3 sequences")
    sd = dev(s)
    ws = api.encode_workspace(3, 256, 16, 2)
    b1, m1, s1 = api.encode(sd, want_states=True, workspace=ws)
    b2, m2, s2 = api.encode(sd, want_states=True)
    sync()
    assert torch.equal(b1, b2) and torch.equal(m1, m2) and torch.equal(s1, s2)


def test_encode_deterministic(api):
    import torch
    s = inputs.targets(32, 256, 92)
    sd = dev(s)
    say("encode determinism B=32")
    r1 = api.encode(sd, want_states=True)
    r2 = api.encode(sd, want_states=True)
    sync()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_encode_empty_batch(api):
    import torch
    sd = torch.empty((0, 256), dtype=torch.float32, device="cuda")
    bits, mse, _ = api.encode(sd)
    sync()
    assert bits.shape == (0, 17) and mse.shape == (0,)


@pytest.mark.parametrize("L,T,code", [(16, 256, "1mad"), (16, 256, "3inst"), (12, 100, "1mad"),
                                      (6, 1, "3inst"), (8, 3, "1mad")])
def test_decode_random_streams(api, L, T, code):
    # every bit pattern of the right length is a valid plain-trellis stream
    rng = np.random.default_rng(L * 7 + T)
    B = 64
    W = oracle.stream_words(L, 2, T)
    nb = oracle.stream_bits(L, 2, T)
    words = rng.integers(0, 2 ** 32, size=(B, W), dtype=np.uint64).astype(np.uint32)
    tail = 32 * W - nb
    if tail:
        words[:, -1] &= np.uint32((0xFFFFFFFF << tail) & 0xFFFFFFFF)
    s = inputs.targets(B, T, 5 + T)
    say("decode random streams L=%d T=%d code=%s" % (L, T, code))
    recon, mse = api.decode(dev(words.view(np.int32)), T, L=L, k=2, code=code, seq=dev(s),
                            want_mse=True)
    sync()
    C = oracle.code_table(code, L)
    _, rec_o = oracle.decode(words, T, C, L, 2)
    assert np.array_equal(recon.cpu().numpy().view(np.uint32), rec_o.view(np.uint32))
    mse_o = np.array([np.float32(oracle.path_cost(rec_o[b], s[b]) / np.float32(T)) for b in range(B)])
    assert np.array_equal(mse.cpu().numpy().view(np.uint32), mse_o.view(np.uint32))
