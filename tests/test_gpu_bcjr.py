"""GPU parity of the fp32 BCJR soft relaxation against the binary64 oracle.

Tolerance (fp32 against an exact reference): per sequence,
    max_t |soft_gpu - soft_oracle| <= 1e-5 * RMS_t(soft_oracle)
(element-wise relative error is ill-posed where the soft value crosses 0), and
|log Z_gpu - log Z_oracle| <= 1e-5 * max(1, |log Z_oracle|).
Also: the tau -> 0 limit against the GPU's own Viterbi code, where the best walk with
a different value at t lies a positive gap above the optimum (gap from the oracle's
binary64 min-sum marginals).
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs

from helpers import bcjr_err, dev, oracle_bcjr_par, say, u32

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    from trellis_coded_weight_amd import api as a
    return a


def sync():
    import torch
    torch.cuda.synchronize()


def run_and_compare(api, s, w, tau, L, code):
    B, T = s.shape
    say("bcjr L=%d T=%d B=%d tau=%g code=%s weighted=%s" % (L, T, B, tau, code, w is not None))
    soft, logz = api.bcjr_soft(dev(s), tau, None if w is None else dev(w), L=L, k=2, code=code)
    sync()
    C = oracle.code_table(code, L)
    soft_o, logz_o = oracle_bcjr_par(C, s, tau, w, L=L)
    err = bcjr_err(soft.cpu().numpy(), soft_o)
    assert err.max() <= TOL, "max err/rms %g" % err.max()
    lz = logz.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(lz - logz_o) <= TOL * np.maximum(1.0, np.abs(logz_o)))
    return soft, err


@pytest.mark.parametrize("L", [6, 8, 12])
@pytest.mark.parametrize("tau", [1.0, 0.1, 0.01])
@pytest.mark.parametrize("T", [1, 2, 37, 256])
def test_bcjr_small_trellis(api, L, tau, T):
    s = inputs.targets(4, T, 500 + L + T)
    run_and_compare(api, s, None, tau, L, "1mad")


@pytest.mark.parametrize("code,weighted", [("3inst", False), ("1mad", True)])
def test_bcjr_variants_L12(api, code, weighted):
    s = inputs.targets(3, 256, 41)
    w = inputs.weights(3, 256, 42) if weighted else None
    run_and_compare(api, s, w, 0.1, 12, code)


@pytest.mark.parametrize("tau", [1.0, 0.1, 0.01])
def test_bcjr_L16(api, tau):
    s, _, code = inputs.workload("bcjr4096x4096_1mad", B=3)
    run_and_compare(api, s, None, tau, 16, code)


# Below the configurations' temperatures: the soft codeword and log Z keep the same bar
# (measured <= 2e-6 * RMS and <= 1e-7 relative down to tau = 3e-4), although the messages
# there carry ~1e-4 log2 of accumulated fp32 exp2/log2 rounding.
@pytest.mark.parametrize("L", [12, 16])
@pytest.mark.parametrize("tau", [3e-3, 1e-3, 3e-4])
def test_bcjr_low_temperature(api, L, tau):
    s = inputs.targets(3, 256, 920 + L)
    run_and_compare(api, s, None, tau, L, "1mad")


def test_bcjr_L16_3inst_weighted(api):
    s = inputs.targets(2, 256, 44)
    w = inputs.weights(2, 256, 45)
    run_and_compare(api, s, w, 0.1, 16, "3inst")


@pytest.mark.parametrize("tau", [1.0, 0.1, 0.01])
def test_bcjr_large_targets(api, tau):
    # targets far outside the codebook's range (|s| up to ~15) and log-normal weights: the
    # per-step energies and their shifts are thousands of log2 units
    s = (4.0 + 3.0 * inputs.targets(3, 256, 46)).astype(np.float32)
    w = inputs.weights(3, 256, 47)
    run_and_compare(api, s, w, tau, 12, "1mad")


def test_bcjr_chunked_workspace(api):
    import torch
    s = inputs.targets(5, 64, 43)
    sd = dev(s)
    say("bcjr chunked L=12 B=5")
    ws = api.bcjr_workspace(2, 64, 12, 2)
    a1, z1 = api.bcjr_soft(sd, 0.3, L=12, workspace=ws)
    a2, z2 = api.bcjr_soft(sd, 0.3, L=12)
    sync()
    assert torch.equal(a1, a2) and torch.equal(z1, z2)


@pytest.mark.parametrize("L,T", [(8, 64), (16, 256)])
def test_bcjr_zero_temperature_limit(api, L, T):
    B = 2
    s = inputs.targets(B, T, 600 + L)
    say("bcjr tau->0 L=%d" % L)
    sd = dev(s)
    _, _, states = api.encode(sd, L=L, k=2, code="1mad", want_states=True)
    sync()
    C = oracle.code_table("1mad", L)
    C64 = C.astype(np.float64)
    # the limit is the oracle's Viterbi code (the GPU search returns the same states)
    st_o, _, _ = oracle.viterbi(C, s, L=L, k=2)
    assert np.array_equal(u32(states), st_o)
    hard = C64[st_o]
    errs = []
    for tau in (1e-3, 1e-4, 1e-5):
        soft, _ = api.bcjr_soft(sd, tau, L=L, k=2, code="1mad")
        sync()
        errs.append(np.abs(soft.cpu().numpy().astype(np.float64) - hard))
    nwalks_log = (L + 2 * (T - 1)) * np.log(2.0)
    for b in range(B):
        best = oracle.minsum_marginals(C, s[b], L=L)
        estar = best.min(axis=1)[0]
        gap = np.empty(T)
        for t in range(T):
            other = best[t][C64 != hard[b, t]]
            gap[t] = other.min() - estar if other.size else np.inf
        ok = gap > 1e-9
        assert ok.sum() >= T - 4
        spread = C64.max() - C64.min()
        for tau, err in zip((1e-3, 1e-4, 1e-5), errs):
            # P(value at t differs from the hard code) <= #walks * exp(-gap / tau); fp32
            # resolution floors the comparison at 1e-6
            bound = spread * np.exp(np.minimum(0.0, nwalks_log - gap[ok] / tau))
            assert np.all(err[b][ok] <= np.maximum(bound, 1e-6))
        # at tau = 1e-5 every position with a clear gap carries the hard value
        clear = ok & (nwalks_log - gap / 1e-5 < np.log(1e-7))
        assert errs[2][b][clear].max() <= 1e-6


@pytest.mark.parametrize("L", [8, 16])
def test_bcjr_high_temperature(api, L):
    """tau -> infinity: every walk weighs the same, so the soft codeword is the mean code
    value (about -0.002 / -0.0004 at L = 8 / 16) at every step.  The soft values then
    cancel to near 0 while the sums behind them average code values of unit scale, so the
    bound is taken against that scale (the error of a sum with cancellation is relative
    to the magnitude of its terms): |soft_gpu - soft_oracle| <= 1e-5 * RMS(C)."""
    import torch
    B, T, tau = 2, 64, 1e6
    s = inputs.targets(B, T, 620 + L)
    say("bcjr high temperature L=%d" % L)
    soft, logz = api.bcjr_soft(dev(s), tau, L=L)
    sync()
    C = oracle.code_table("1mad", L).astype(np.float64)
    soft_o, logz_o = oracle_bcjr_par(C.astype(np.float32), s, tau, L=L)
    rms_c = np.sqrt((C ** 2).mean())
    assert np.abs(soft.cpu().numpy() - soft_o).max() <= 1e-5 * rms_c
    assert np.abs(soft_o - C.mean()).max() <= 1e-4
    lz = logz.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(lz - logz_o) <= TOL * np.maximum(1.0, np.abs(logz_o)))
