"""Pins for the oracle's binary64 BCJR soft relaxation.  CPU only.

Source: BCJR-QAT abstract -- forward-backward sum-product at temperature tau; the soft
codeword is the Boltzmann expectation over trellis paths, it recovers the hard (Viterbi)
code as tau -> 0, and the computation is a transfer-matrix product of a 1D chain.
Energy reading: a walk's energy is its search cost (sum of weighted squared errors), its
weight exp(-E / tau), start state uniform (plain trellis).

Pins:
* explicit enumeration of every walk at L = 6, k = 2, T <= 6 (relative error 1e-12);
* the transfer-matrix product (dense 64 x 64 matrices) gives the same log Z;
* C = 1 everywhere gives soft = 1 (the posterior is normalised);
* tau -> infinity gives soft_t -> mean(C) (uniform walks have uniform marginals);
* tau -> 0 gives the value of the minimum-energy walk wherever the best walk with a
  different value at t lies a gap g_t > 0 above it, within #walks * exp(-g_t / tau);
* the free-energy bracket E* - tau ln(#walks) <= -tau log Z <= E*;
* d(-tau log Z)/d s_t = 2 w_t (s_t - soft_t), by central differences.
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs


@pytest.mark.parametrize("T", [1, 2, 4, 6])
@pytest.mark.parametrize("tau", [1.0, 0.1, 0.01])
def test_bruteforce_L6(T, tau):
    L, k = 6, 2
    C = oracle.code_table("1mad", L)
    for seed in range(3):
        s = inputs.targets(1, T, 300 + seed)[0]
        soft, lz = oracle.bcjr(C, s, tau, L=L, k=k)
        bsoft, blz = oracle.brute_bcjr(C, s, tau, L=L, k=k)
        assert np.allclose(soft, bsoft, rtol=1e-12, atol=1e-12 * np.abs(C).max())
        assert abs(lz - blz) <= 1e-12 * max(1.0, abs(blz))


@pytest.mark.parametrize("T", [3, 5])
def test_bruteforce_weighted_3inst_L6(T):
    L, k = 6, 2
    C = oracle.code_table("3inst", L)
    s = inputs.targets(1, T, 17)[0]
    w = inputs.weights(1, T, 18)[0]
    soft, lz = oracle.bcjr(C, s, 0.3, w, L=L, k=k)
    bsoft, blz = oracle.brute_bcjr(C, s, 0.3, w, L=L, k=k)
    assert np.allclose(soft, bsoft, rtol=1e-12, atol=1e-12)
    assert abs(lz - blz) <= 1e-12 * max(1.0, abs(blz))


def test_transfer_matrix_logz_L6():
    L, k, T, tau = 6, 2, 12, 0.7
    N = 1 << L
    C = oracle.code_table("1mad", L)
    s = inputs.targets(1, T, 9)[0]
    _, lz = oracle.bcjr(C, s, tau, L=L, k=k)
    A = np.zeros((N, N))
    for i in range(N):
        for b in range(1 << k):
            A[i, ((i << k) | b) & (N - 1)] = 1.0
    E = (C.astype(np.float64)[None, :] - s.astype(np.float64)[:, None]) ** 2   # [T][N]
    v = np.exp(-E[0] / tau)
    for t in range(1, T):
        v = (v @ A) * np.exp(-E[t] / tau)
    assert abs(np.log(v.sum()) - lz) <= 1e-12 * abs(lz)


def test_normalised_posterior():
    L = 8
    s = inputs.targets(1, 40, 4)[0]
    ones = np.ones(1 << L, dtype=np.float32)
    for tau in (2.0, 0.05):
        soft, _ = oracle.bcjr(ones, s, tau, L=L)
        assert np.allclose(soft, 1.0, rtol=0, atol=1e-13)


def test_high_temperature_limit():
    L = 8
    C = oracle.code_table("1mad", L)
    s = inputs.targets(1, 30, 5)[0]
    soft, _ = oracle.bcjr(C, s, 1e9, L=L)
    assert np.allclose(soft, C.astype(np.float64).mean(), atol=1e-7)


def test_low_temperature_limit_matches_hard_code():
    L, k, T = 8, 2, 48
    C = oracle.code_table("1mad", L)
    s = inputs.targets(1, T, 6)[0]
    best = oracle.minsum_marginals(C, s, L=L, k=k)          # [T][N]
    estar = best.min(axis=1)
    assert np.allclose(estar, estar[0], rtol=0, atol=1e-9)  # same optimum at every t
    nwalks_log = (L + k * (T - 1)) * np.log(2.0)
    C64 = C.astype(np.float64)
    hard = np.empty(T)
    gap = np.empty(T)
    for t in range(T):
        opt = np.nonzero(best[t] <= estar[0] + 1e-12)[0]
        vals = np.unique(C64[opt])
        if len(vals) > 1:
            gap[t] = 0.0
            hard[t] = np.nan
            continue
        hard[t] = vals[0]
        other = best[t][C64 != vals[0]]
        gap[t] = other.min() - estar[0]
    ok = gap > 0
    assert ok.sum() >= T - 2
    # the fp32 Viterbi walk has the same values where the optimum is strict
    st, _, _ = oracle.viterbi(C, s, L=L, k=k)
    assert np.array_equal(C64[st][ok], hard[ok])
    spread = C64.max() - C64.min()
    errs = []
    for tau in (1e-3, 1e-4, 1e-5):
        soft, _ = oracle.bcjr(C, s, tau, L=L, k=k)
        err = np.abs(soft - hard)[ok]
        bound = spread * np.exp(np.minimum(0.0, nwalks_log - gap[ok] / tau))
        assert np.all(err <= bound + 1e-12)
        errs.append(err.max())
    assert errs[0] >= errs[1] >= errs[2]
    assert errs[2] <= 1e-6


@pytest.mark.parametrize("tau", [1.0, 0.1, 0.01])
def test_free_energy_bracket(tau):
    L, k, T = 8, 2, 64
    C = oracle.code_table("1mad", L)
    s = inputs.targets(1, T, 8)[0]
    _, lz = oracle.bcjr(C, s, tau, L=L, k=k)
    estar = oracle.minsum_marginals(C, s, L=L, k=k)[0].min()
    nwalks_log = (L + k * (T - 1)) * np.log(2.0)
    f = -tau * lz
    assert estar - tau * nwalks_log - 1e-9 <= f <= estar + 1e-9


@pytest.mark.parametrize("weighted", [False, True])
def test_derivative_identity(weighted):
    L, k, T, tau = 8, 2, 20, 0.5
    C = oracle.code_table("1mad", L)
    s = inputs.targets(1, T, 21)[0]
    w = inputs.weights(1, T, 22)[0] if weighted else None
    soft, _ = oracle.bcjr(C, s, tau, w, L=L, k=k)
    h = np.float32(2.0 ** -10)
    for t in (0, 7, T - 1):
        sp = s.copy(); sp[t] += h
        sm = s.copy(); sm[t] -= h
        assert sp[t] - s[t] == h and s[t] - sm[t] == h     # exact perturbations
        _, lp = oracle.bcjr(C, sp, tau, w, L=L, k=k)
        _, lm = oracle.bcjr(C, sm, tau, w, L=L, k=k)
        fd = (-tau * lp + tau * lm) / (2.0 * float(h))
        wt = 1.0 if w is None else float(w[t])
        exact = 2.0 * wt * (float(s[t]) - soft[t])
        assert abs(fd - exact) <= 1e-4 * max(1.0, abs(exact))
