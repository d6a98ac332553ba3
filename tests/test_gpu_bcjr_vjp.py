"""GPU parity of the BCJR gradient (vector-Jacobian product of the soft codeword with
respect to the targets) against the binary64 oracle.

Tolerance (fp32 against an exact reference), per sequence:
    max_u |grad_gpu - grad_oracle| <= 1e-5 * RMS_u(grad_oracle) + 2^-100,
the bound used for the soft codeword itself, plus an absolute floor above binary32's
underflow range (posterior weights below 2^-126 lose their relative precision; the
floor decides only for gradients that are numerically zero); the kernel keeps the messages it needs in
fixed point (2^-21 log2 units; below tau = 0.01 in fp64) and its expectation messages
centred on the soft codeword, which a CPU emulation of this arithmetic puts at <= 6e-6
at tau = 0.01 and <= 1.1e-6 at tau = 1e-3 (the entry point refuses temperatures below 3e-3).
Also: the soft codeword that the gradient call returns is bit-identical to the soft
pass's, a zero upstream gradient gives exactly zero, the product is linear in the
upstream gradient, and a chunked workspace gives the same bits.
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs

from helpers import bcjr_err, dev, oracle_vjp_par, say

pytestmark = pytest.mark.gpu

TOL = 1e-5
# absolute floor: the kernels form the gradient from binary32 posterior weights, and a
# gradient below ~2^-100 is carried by weights near or below binary32's normal range
# (2^-126), whose products underflow -- it is numerically zero (e.g. ~1e-33 for an XOR
# sequence at tau = 3e-3 whose competing walks have weights near 2^-120)
FLOOR = 2.0 ** -100


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    from trellis_coded_weight_amd import api as a
    return a


def sync():
    import torch
    torch.cuda.synchronize()


def upstream(B, T, seed):
    return np.random.default_rng(seed).standard_normal((B, T)).astype(np.float32)


def run_and_compare(api, s, w, g, tau, L, code, tol=TOL):
    import torch
    B, T = s.shape
    say("bcjr_vjp L=%d T=%d B=%d tau=%g code=%s weighted=%s" % (L, T, B, tau, code, w is not None))
    sd, gd = dev(s), dev(g)
    wd = None if w is None else dev(w)
    grad, soft, logz = api.bcjr_vjp(sd, tau, gd, wd, L=L, k=2, code=code, want_soft=True)
    soft2, logz2 = api.bcjr_soft(sd, tau, wd, L=L, k=2, code=code)
    sync()
    assert torch.equal(soft, soft2) and torch.equal(logz, logz2)
    C = oracle.code_table(code, L)
    grad_o, soft_o = oracle_vjp_par(C, s, tau, g.astype(np.float64), w, L=L)
    assert bcjr_err(soft.cpu().numpy(), soft_o).max() <= TOL
    err = bcjr_err(grad.cpu().numpy(), grad_o)
    # each sequence's bar is tol * RMS plus FLOOR (it matters only for a gradient that is
    # numerically zero, e.g. ~1e-48 at tau = 0.01 far from any near-tie)
    dmax = np.abs(grad.cpu().numpy().astype(np.float64) - grad_o).max(axis=1)
    rms = np.sqrt((grad_o ** 2).mean(axis=1))
    assert np.all(dmax <= tol * rms + FLOOR), "max grad err/rms %g" % err.max()
    return err


@pytest.mark.parametrize("L", [6, 8, 12])
@pytest.mark.parametrize("tau", [1.0, 0.1, 0.01])
@pytest.mark.parametrize("T", [1, 2, 37, 256])
def test_vjp_small_trellis(api, L, tau, T):
    s = inputs.targets(3, T, 700 + L + T)
    g = upstream(3, T, 800 + L + T)
    run_and_compare(api, s, None, g, tau, L, "1mad")


@pytest.mark.parametrize("code,weighted", [("3inst", False), ("1mad", True), ("3inst", True)])
def test_vjp_variants_L12(api, code, weighted):
    s = inputs.targets(3, 256, 51)
    w = inputs.weights(3, 256, 52) if weighted else None
    run_and_compare(api, s, w, upstream(3, 256, 53), 0.1, 12, code)


@pytest.mark.parametrize("tau", [1.0, 0.1, 0.01])
def test_vjp_L16(api, tau):
    s, _, code = inputs.workload("bcjr4096x4096_1mad", B=2)
    run_and_compare(api, s, None, upstream(2, 256, 54), tau, 16, code)


# Below tau = 0.01 the soft pass stashes fp64 messages for the gradient (the 32-bit
# stash keeps only fp32 resolution below -1024 log2 units, where a backward message can
# lift a state back at low temperature).  The entry point refuses temperatures below
# 3e-3 (QTCQ_VJP_MIN_TEMPERATURE): at L = 16 and tau = 1e-3 the gradient of a sequence
# collapses onto two positions (14x and 7x its RMS) and the fp32 expectation messages
# and exp2 weights leave 1.2e-6 relative on them, 1.7e-5 * RMS.  At the floor every
# workload below meets the bar.
@pytest.mark.parametrize("L,B,tau", [(12, 3, 0.009), (16, 2, 0.009), (12, 3, 3e-3), (16, 2, 3e-3)])
def test_vjp_low_temperature(api, L, B, tau):
    s = inputs.targets(B, 256, 900 + L)
    run_and_compare(api, s, None, upstream(B, 256, 901), tau, L, "1mad")


@pytest.mark.parametrize("code", ["1mad", "3inst"])
@pytest.mark.parametrize("L", [12, 16])
def test_vjp_low_temperature_weighted(api, code, L):
    """Log-normal weights scale some positions' energies by 10 and more, i.e. a lower
    effective temperature: at the floor, tau = 3e-3."""
    s = inputs.targets(2, 256, 910 + L)
    w = inputs.weights(2, 256, 911)
    run_and_compare(api, s, w, upstream(2, 256, 912), 3e-3, L, code)


def test_vjp_refuses_below_temperature_floor(api):
    import torch
    from trellis_coded_weight_amd import _native as nat
    s = dev(inputs.targets(2, 64, 913))
    g = dev(upstream(2, 64, 914))
    for tau in (2.9e-3, 1e-3, 1e-6):
        with pytest.raises(nat.QtcqError) as e:
            api.bcjr_vjp(s, tau, g, L=12)
        assert e.value.status == nat.QTCQ_ERR_UNSUPPORTED
    grad, _, _ = api.bcjr_vjp(s, 3e-3, g, L=12)      # the floor itself runs
    torch.cuda.synchronize()
    assert torch.isfinite(grad).all()


def test_vjp_L16_3inst_weighted(api):
    s = inputs.targets(2, 256, 58)
    w = inputs.weights(2, 256, 59)
    run_and_compare(api, s, w, upstream(2, 256, 60), 0.1, 16, "3inst")


# Targets far outside the codebook's range (4 + 3 N(0,1), |s| up to ~15) with log-normal
# weights: energy gaps of thousands of log2 units, where the candidate that wins an LSE is
# often far below the largest input (the case that needs every input in fp64).  At
# tau = 0.01 one of these sequences has gradient RMS ~1e-8, below what a relative bound
# can measure, so the test stops at 0.1.
@pytest.mark.parametrize("tau,tol", [(1.0, TOL), (0.1, TOL)])
def test_vjp_large_targets(api, tau, tol):
    s = (4.0 + 3.0 * inputs.targets(3, 256, 61)).astype(np.float32)
    w = inputs.weights(3, 256, 62)
    run_and_compare(api, s, w, upstream(3, 256, 63), tau, 12, "1mad", tol=tol)


def test_vjp_zero_and_linear(api):
    import torch
    L, T, B = 12, 256, 4
    s = dev(inputs.targets(B, T, 55))
    g1 = dev(upstream(B, T, 56))
    g2 = dev(upstream(B, T, 57))
    say("bcjr_vjp zero / linearity L=12")
    z, _, _ = api.bcjr_vjp(s, 0.1, torch.zeros_like(s), L=L)
    a, _, _ = api.bcjr_vjp(s, 0.1, g1, L=L)
    b, _, _ = api.bcjr_vjp(s, 0.1, g2, L=L)
    c, _, _ = api.bcjr_vjp(s, 0.1, g1 + 2.0 * g2, L=L)
    sync()
    assert torch.count_nonzero(z).item() == 0
    ref = (a + 2.0 * b).double().cpu().numpy()
    err = np.abs(c.double().cpu().numpy() - ref).max(axis=1) / np.sqrt((ref ** 2).mean(axis=1))
    assert err.max() <= 2 * TOL


def test_vjp_chunked_workspace(api):
    import torch
    s = dev(inputs.targets(5, 64, 58))
    g = dev(upstream(5, 64, 59))
    say("bcjr_vjp chunked L=12 B=5")
    ws = api.bcjr_vjp_workspace(2, 64, 12, 2)
    a1, s1, z1 = api.bcjr_vjp(s, 0.3, g, L=12, want_soft=True, workspace=ws)
    a2, s2, z2 = api.bcjr_vjp(s, 0.3, g, L=12, want_soft=True)
    sync()
    assert torch.equal(a1, a2) and torch.equal(s1, s2) and torch.equal(z1, z2)


def test_vjp_chunked_workspace_wide_stash(api):
    """The fp64 stash (tau < 0.01) in a workspace of two sequences over five: same bits."""
    import torch
    s = dev(inputs.targets(5, 64, 68))
    g = dev(upstream(5, 64, 69))
    say("bcjr_vjp chunked wide stash L=12 B=5")
    ws = api.bcjr_vjp_workspace(2, 64, 12, 2)
    a1, s1, z1 = api.bcjr_vjp(s, 0.004, g, L=12, want_soft=True, workspace=ws)
    a2, s2, z2 = api.bcjr_vjp(s, 0.004, g, L=12, want_soft=True)
    sync()
    assert torch.equal(a1, a2) and torch.equal(s1, s2) and torch.equal(z1, z2)
