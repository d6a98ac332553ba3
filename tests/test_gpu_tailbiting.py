"""GPU parity of the tail-biting encoder (two searches per sequence) and the cyclic
window decode, through the C ABI, element by element against the CPU oracle on the
same seeded inputs.  Bar: bit-exact states, streams, reconstructions and MSEs.
Full-size: the 4096x4096 (1MAD) and 4096x14336 (3INST) matrices as 65,536 / 229,376
sequences of 256, sampled rows against the oracle plus properties of every row.
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs

from helpers import N_WORKERS, _split, dev, say, u32

pytestmark = pytest.mark.gpu

WS_CAP = 64 << 30


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    from trellis_coded_weight_amd import api as a
    return a


def sync():
    import torch
    torch.cuda.synchronize()


def oracle_tb_par(C, s, w=None, L=16, k=2):
    from concurrent.futures import ThreadPoolExecutor
    B, T = s.shape
    st = np.empty((B, T), dtype=np.uint32)
    cost = np.empty(B, dtype=np.float32)
    mse = np.empty(B, dtype=np.float32)

    def job(r):
        a, b = r
        st[a:b], cost[a:b], mse[a:b] = oracle.tailbiting(C, s[a:b], None if w is None else w[a:b],
                                                         L=L, k=k)

    with ThreadPoolExecutor(N_WORKERS) as ex:
        list(ex.map(job, _split(B, N_WORKERS * 2)))
    return st, cost, mse


def check_tb(api, s, w, L, code, workspace=None):
    B, T = s.shape
    say("tail-biting encode L=%d T=%d B=%d code=%s weighted=%s" % (L, T, B, code, w is not None))
    sd = dev(s)
    wd = None if w is None else dev(w)
    bits, mse, states = api.tailbiting_encode(sd, wd, L=L, k=2, code=code, want_states=True,
                                              workspace=workspace)
    recon, mse2 = api.tailbiting_decode(bits, T, L=L, k=2, code=code, seq=sd, weights=wd,
                                        want_mse=True)
    sync()
    C = oracle.code_table(code, L)
    st_o, _, mse_o = oracle_tb_par(C, s, w, L=L)
    words_o = oracle.tb_pack(st_o, L, 2)
    _, rec_o = oracle.tb_decode(words_o, T, C, L, 2)
    assert np.array_equal(u32(states), st_o)
    assert np.array_equal(u32(bits), words_o)
    assert np.array_equal(mse.cpu().numpy().view(np.uint32), mse_o.view(np.uint32))
    assert np.array_equal(recon.cpu().numpy().view(np.uint32), rec_o.view(np.uint32))
    assert np.array_equal(mse2.cpu().numpy().view(np.uint32), mse_o.view(np.uint32))


@pytest.mark.parametrize("L", [6, 8, 10, 12, 14])
@pytest.mark.parametrize("Tsel", ["min", "odd", "256"])
@pytest.mark.parametrize("code,weighted", [("1mad", False), ("3inst", False), ("1mad", True)])
def test_tailbiting_small_trellis(api, L, Tsel, code, weighted):
    T = {"min": L // 2, "odd": 37, "256": 256}[Tsel]
    B = 5 if L <= 12 else 2
    seed = 2000 * L + T
    s = inputs.targets(B, T, seed)
    w = inputs.weights(B, T, seed + 1) if weighted else None
    check_tb(api, s, w, L, code)


@pytest.mark.parametrize("T", [8, 9, 33, 256])
@pytest.mark.parametrize("code,weighted", [("1mad", False), ("3inst", False), ("1mad", True)])
def test_tailbiting_L16(api, T, code, weighted):
    s = inputs.targets(3, T, 3000 + T)
    w = inputs.weights(3, T, 3001 + T) if weighted else None
    check_tb(api, s, w, 16, code)


def test_tailbiting_chunked_workspace(api):
    import torch
    s = inputs.targets(7, 256, 3100)
    sd = dev(s)
    say("tail-biting chunked B=7 ws=3 sequences")
    ws = api.tailbiting_workspace(3, 256, 16, 2)
    r1 = api.tailbiting_encode(sd, want_states=True, workspace=ws)
    r2 = api.tailbiting_encode(sd, want_states=True)
    sync()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


def test_tailbiting_rejects_short_streams(api):
    import torch
    from trellis_coded_weight_amd import _native as nat
    sd = torch.zeros((2, 7), dtype=torch.float32, device="cuda")   # 2*7 < 16
    with pytest.raises(ValueError):
        api.tailbiting_encode(sd, L=16)
    assert nat.qtcq_tailbiting_words(16, 2, 7) == -1


@pytest.mark.parametrize("L,T,code", [(16, 256, "1mad"), (16, 256, "3inst"), (16, 8, "1mad"),
                                      (12, 100, "3inst"), (6, 3, "1mad"), (10, 17, "1mad")])
def test_tailbiting_decode_random_streams(api, L, T, code):
    # every bit pattern of kT bits is a valid tail-biting stream
    rng = np.random.default_rng(L * 11 + T)
    B = 64
    W = oracle.tb_stream_words(L, 2, T)
    words = rng.integers(0, 2 ** 32, size=(B, W), dtype=np.uint64).astype(np.uint32)
    tail = 32 * W - 2 * T
    if tail:
        words[:, -1] &= np.uint32((0xFFFFFFFF << tail) & 0xFFFFFFFF)
    s = inputs.targets(B, T, 9 + T)
    say("tail-biting decode random streams L=%d T=%d code=%s" % (L, T, code))
    recon, mse = api.tailbiting_decode(dev(words.view(np.int32)), T, L=L, k=2, code=code,
                                       seq=dev(s), want_mse=True)
    sync()
    C = oracle.code_table(code, L)
    _, rec_o = oracle.tb_decode(words, T, C, L, 2)
    assert np.array_equal(recon.cpu().numpy().view(np.uint32), rec_o.view(np.uint32))
    mse_o = np.array([np.float32(oracle.path_cost(rec_o[b], s[b]) / np.float32(T)) for b in range(B)])
    assert np.array_equal(mse.cpu().numpy().view(np.uint32), mse_o.view(np.uint32))


@pytest.mark.parametrize("name,mse_ref", [("tb4096x4096_1mad", 0.0697),
                                          ("tb4096x14336_3inst", 0.0696)])
def test_tailbiting_full_size(api, name, mse_ref):
    import torch
    s, w, code = inputs.workload(name)
    B, T = s.shape
    say("full-size tail-biting %s B=%d" % (name, B))
    sd = dev(s)
    ws = api.tailbiting_workspace(B, T, 16, 2, max_bytes=WS_CAP)
    bits, mse, _ = api.tailbiting_encode(sd, L=16, k=2, code=code, workspace=ws)
    del ws
    recon, mse2 = api.tailbiting_decode(bits, T, L=16, k=2, code=code, seq=sd, want_mse=True)
    sync()
    assert bits.shape == (B, 16)
    assert torch.equal(mse, mse2)
    m = mse.cpu().numpy()
    assert abs(float(m.mean()) - mse_ref) <= 0.002
    rng = np.random.default_rng(11)
    rows = np.array(sorted(set([0, B - 1]) | set(rng.choice(B, size=1022, replace=False).tolist())))
    C = oracle.code_table(code, 16)
    st_o, _, mse_o = oracle_tb_par(C, s[rows], L=16)
    assert np.array_equal(u32(bits)[rows], oracle.tb_pack(st_o, 16, 2))
    assert np.array_equal(m[rows].view(np.uint32), mse_o.view(np.uint32))
    _, rec_o = oracle.tb_decode(oracle.tb_pack(st_o, 16, 2), T, C, 16, 2)
    assert np.array_equal(recon.cpu().numpy()[rows].view(np.uint32), rec_o.view(np.uint32))
