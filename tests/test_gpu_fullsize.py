"""GPU checks at the full workload sizes, in the launch configuration the benchmark
times (64 GiB encode workspace cap, the library's default BCJR / gradient caps): sampled
sequences (first, last and seeded random rows: 4,096 per encode configuration, 256 per
BCJR temperature, 16 for the gradient) against the oracle, bit for bit for the encodes,
and properties that hold for every sequence --
decoding the stream reproduces the encoder's MSE bit for bit, the stream's pad bits are
zero, and the mean MSE matches the pages' free-start value (0.065 +- 0.002 at L = 16).
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs

from helpers import bcjr_err, dev, oracle_bcjr_par, oracle_viterbi_par, oracle_vjp_par, say, u32

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


def sample_rows(B, n, seed):
    rng = np.random.default_rng(seed)
    rows = set([0, B - 1]) | set(rng.choice(B, size=n - 2, replace=False).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", ["enc4096x4096_1mad", "enc4096x14336_3inst",
                                  "enc4096x4096_1mad_weighted"])
def test_encode_decode_full(api, name):
    import torch
    s, w, code = inputs.workload(name)
    B, T = s.shape
    say("full-size encode+decode %s B=%d" % (name, B))
    sd = dev(s)
    wd = None if w is None else dev(w)
    ws = api.encode_workspace(B, T, 16, 2, max_bytes=WS_CAP)
    bits, mse, _ = api.encode(sd, wd, L=16, k=2, code=code, workspace=ws)
    del ws
    recon, mse2 = api.decode(bits, T, L=16, k=2, code=code, seq=sd, weights=wd, want_mse=True)
    sync()
    assert torch.equal(mse, mse2)
    bits_h = u32(bits)
    assert np.all(bits_h[:, -1] & np.uint32((1 << 18) - 1) == 0)      # 526 bits, 18 pad
    m = mse.cpu().numpy()
    if w is None:
        assert abs(float(m.mean()) - 0.065) <= 0.002
    rows = sample_rows(B, 4096, 7)
    C = oracle.code_table(code, 16)
    st_o, _, mse_o = oracle_viterbi_par(C, s[rows], None if w is None else w[rows], L=16)
    words_o = oracle.pack(st_o, 16, 2)
    assert np.array_equal(bits_h[rows], words_o)
    assert np.array_equal(m[rows].view(np.uint32), mse_o.view(np.uint32))
    _, rec_o = oracle.decode(words_o, T, C, 16, 2)
    assert np.array_equal(recon.cpu().numpy()[rows].view(np.uint32), rec_o.view(np.uint32))


def test_bcjr_full(api):
    s, _, code = inputs.workload("bcjr4096x4096_1mad")
    B, T = s.shape
    sd = dev(s)
    rows = sample_rows(B, 256, 8)
    C = oracle.code_table(code, 16)
    for tau in (1.0, 0.1, 0.01):
        say("full-size bcjr B=%d tau=%g" % (B, tau))
        soft, logz = api.bcjr_soft(sd, tau, L=16, k=2, code=code)
        sync()
        sh = soft.cpu().numpy()
        assert np.isfinite(sh).all() and np.isfinite(logz.cpu().numpy()).all()
        soft_o, logz_o = oracle_bcjr_par(C, s[rows], tau, L=16)
        err = bcjr_err(sh[rows], soft_o)
        assert err.max() <= 1e-5, "tau %g err %g" % (tau, err.max())
        lz = logz.cpu().numpy()[rows].astype(np.float64)
        assert np.all(np.abs(lz - logz_o) <= 1e-5 * np.maximum(1.0, np.abs(logz_o)))


def test_bcjr_vjp_full(api):
    s, _, code = inputs.workload("bcjr4096x4096_1mad")
    B, T = s.shape
    g = np.random.default_rng(9).standard_normal((B, T), dtype=np.float32)
    say("full-size bcjr vjp B=%d tau=0.1" % B)
    grad, soft, _ = api.bcjr_vjp(dev(s), 0.1, dev(g), L=16, k=2, code=code, want_soft=True)
    sync()
    gh = grad.cpu().numpy()
    assert np.isfinite(gh).all()
    rows = sample_rows(B, 16, 10)
    C = oracle.code_table(code, 16)
    grad_o, soft_o = oracle_vjp_par(C, s[rows], 0.1, g[rows].astype(np.float64), L=16)
    assert bcjr_err(soft.cpu().numpy()[rows], soft_o).max() <= 1e-5
    err = bcjr_err(gh[rows], grad_o)
    assert err.max() <= 1e-5, "grad err %g" % err.max()
