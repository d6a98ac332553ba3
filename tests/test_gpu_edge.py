"""GPU parity at the edges of the input domain and of the launch shapes, through the C ABI,
against the CPU oracle:

* rows whose step errors overflow binary32 (finite targets of magnitude 1e20): every path
  cost is +inf, and both sides end in the lowest allowed state (plain and tail-biting);
* the search's two launch shapes: one sequence per workgroup when the chunk fits in one
  round of compute units, an interleaved pair otherwise (odd counts leave the last
  workgroup a single sequence) -- bit-exact on both sides of the switch;
* the soft relaxation at temperatures of 1e-9 and 1e-8, where the messages reach ~1e10
  log2 units (the largest scale the 32-bit stash resolves): log Z is finite, and the
  soft codeword must equal the Viterbi code wherever the best walk with a
  different value at that step is more than 1e-6 above the optimum (the tau -> 0 limit of
  the BCJR-QAT abstract), to the rounding of the posterior mean's one division.
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


@pytest.mark.parametrize("L", [8, 16])
@pytest.mark.parametrize("weighted", [False, True])
def test_overflowing_rows_match_oracle(api, L, weighted):
    T = 32
    s = inputs.targets(5, T, 900)
    s[1] = 1e20
    s[3, ::2] = -3e19
    s[3, 1::2] = 1e20
    w = inputs.weights(5, T, 901) if weighted else None
    C = oracle.code_table("1mad", L)
    say("overflowing rows L=%d weighted=%s" % (L, weighted))
    bits, mse, st = api.encode(dev(s), None if w is None else dev(w), L=L, code="1mad",
                               want_states=True)
    sync()
    st_o, _, mse_o = oracle.viterbi(C, s, w, L=L)
    assert np.isinf(mse_o[1]) and np.isinf(mse_o[3])
    assert np.array_equal(u32(st), st_o)
    assert np.array_equal(u32(bits), oracle.pack(st_o, L, 2))
    assert np.array_equal(mse.cpu().numpy(), mse_o)

    say("overflowing rows tail-biting L=%d weighted=%s" % (L, weighted))
    tbits, tmse, tst = api.tailbiting_encode(dev(s), None if w is None else dev(w), L=L,
                                             code="1mad", want_states=True)
    sync()
    tst_o, _, tmse_o = oracle.tailbiting(C, s, w, L=L)
    assert np.array_equal(u32(tst), tst_o)
    assert np.array_equal(u32(tbits), oracle.tb_pack(tst_o, L, 2))
    assert np.array_equal(tmse.cpu().numpy(), tmse_o)


@pytest.mark.parametrize("B", [1, 255, 256, 257, 513])
def test_search_launch_shapes(api, B):
    """Around the switch between one and two sequences per workgroup (256 compute units):
    every row bit-exact, whichever shape ran it."""
    L, T = 8, 40
    s = inputs.targets(B, T, 910 + B)
    C = oracle.code_table("3inst", L)
    say("search launch shape B=%d" % B)
    bits, mse, st = api.encode(dev(s), L=L, code="3inst", want_states=True)
    sync()
    st_o, _, mse_o = oracle_viterbi_par(C, s, L=L)
    assert np.array_equal(u32(st), st_o)
    assert np.array_equal(u32(bits), oracle.pack(st_o, L, 2))
    assert np.array_equal(mse.cpu().numpy(), mse_o)


@pytest.mark.parametrize("weighted,tau", [(False, 1e-9), (True, 1e-8)])
def test_bcjr_tiny_temperature_is_viterbi(api, weighted, tau):
    """Messages of ~1e10 log2 units (|log2 Z| ~ 7e9 here), the largest scale the 32-bit
    stash resolves: tau = 1e-9 on N(0,1) targets, tau = 1e-8 with weights 10 x
    log-normal."""
    L, T = 8, 48
    s = inputs.targets(6, T, 920)
    w = (inputs.weights(6, T, 921) * 10.0).astype(np.float32) if weighted else None
    C = oracle.code_table("1mad", L)
    say("bcjr tau=%g weighted=%s" % (tau, weighted))
    soft, logz = api.bcjr_soft(dev(s), tau, None if w is None else dev(w), L=L, code="1mad")
    sync()
    soft = soft.cpu().numpy()
    assert np.all(np.isfinite(soft)) and np.all(np.isfinite(logz.cpu().numpy()))
    st_o, _, _ = oracle.viterbi(C, s, w, L=L)
    Cd = C.astype(np.float64)
    checked = 0
    for b in range(s.shape[0]):
        best = oracle.minsum_marginals(C, s[b], None if w is None else w[b], L=L)
        estar = best.min(axis=1)
        for t in range(T):
            other = Cd != Cd[st_o[b, t]]
            gap = best[t][other].min() - estar[t]
            if gap > 1e-6:
                # one state carries the posterior: soft = fl(fl(p C) / p), within a unit
                want = float(C[st_o[b, t]])
                assert abs(soft[b, t] - want) <= 2.0 ** -23 * abs(want), (b, t, soft[b, t], want)
                checked += 1
    assert checked >= 0.9 * s.size
