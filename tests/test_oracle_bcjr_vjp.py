"""Pins for the oracle's binary64 BCJR gradient (vector-Jacobian product).  CPU only.

Source: BCJR-QAT abstract -- the soft relaxation is exactly differentiable.  With the
Boltzmann walk distribution p ~ exp(-E / tau) of the soft codeword and E the weighted
path cost, d soft_t / d s_u = (2 w_u / tau) Cov_p(C(state_t), C(state_u)); the oracle
computes the product with an upstream gradient g by expectation messages.

Pins (none of them retypes the oracle's recursion):
* explicit enumeration of every walk at L = 6, k = 2, T <= 6, both codes, weighted;
* central differences of sum_t g_t soft_t(s) through the (separately pinned) BCJR
  oracle, unweighted and weighted, L = 8;
* T = 1 closed form: grad = (2 w / tau) g Var(C) under softmax(-e_0 / tau);
* a constant code has zero covariance, so zero gradient;
* symmetry and positive semi-definiteness of the covariance matrix built from the
  columns g = e_t (w_t J[t][u] = w_u J[u][t]);
* tau -> infinity: walks become uniform, so (tau / 2) J[t][u] -> the uniform-walk
  covariance, Var(C) on the diagonal and 0 once |t - u| >= L / k (no shared bits).
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs


def _g(T, seed):
    return np.random.default_rng(seed).standard_normal(T)


@pytest.mark.parametrize("T", [1, 2, 4, 6])
@pytest.mark.parametrize("tau", [1.0, 0.1])
def test_bruteforce_L6(T, tau):
    L, k = 6, 2
    C = oracle.code_table("1mad", L)
    for seed in range(2):
        s = inputs.targets(1, T, 500 + seed)[0]
        g = _g(T, 600 + seed)
        grad, soft = oracle.bcjr_vjp(C, s, tau, g, L=L, k=k)
        ref = oracle.brute_bcjr_vjp(C, s, tau, g, L=L, k=k)
        bsoft, _ = oracle.brute_bcjr(C, s, tau, L=L, k=k)
        scale = np.abs(ref).max() + 1e-300
        assert np.allclose(grad, ref, rtol=1e-10, atol=1e-10 * scale)
        assert np.allclose(soft, bsoft, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("T", [3, 5])
def test_bruteforce_weighted_3inst_L6(T):
    L, k = 6, 2
    C = oracle.code_table("3inst", L)
    s = inputs.targets(1, T, 27)[0]
    w = inputs.weights(1, T, 28)[0]
    g = _g(T, 29)
    grad, _ = oracle.bcjr_vjp(C, s, 0.3, g, w, L=L, k=k)
    ref = oracle.brute_bcjr_vjp(C, s, 0.3, g, w, L=L, k=k)
    assert np.allclose(grad, ref, rtol=1e-10, atol=1e-10 * np.abs(ref).max())


@pytest.mark.parametrize("weighted", [False, True])
def test_central_differences(weighted):
    L, k, T, tau = 8, 2, 20, 0.5
    C = oracle.code_table("1mad", L)
    s = inputs.targets(1, T, 31)[0]
    w = inputs.weights(1, T, 32)[0] if weighted else None
    g = _g(T, 33)
    grad, _ = oracle.bcjr_vjp(C, s, tau, g, w, L=L, k=k)
    h = np.float32(2.0 ** -12)
    for u in (0, 5, 11, T - 1):
        sp = s.copy(); sp[u] += h
        sm = s.copy(); sm[u] -= h
        assert sp[u] - s[u] == h and s[u] - sm[u] == h      # exact perturbations
        fp, _ = oracle.bcjr(C, sp, tau, w, L=L, k=k)
        fm, _ = oracle.bcjr(C, sm, tau, w, L=L, k=k)
        fd = (g @ fp - g @ fm) / (2.0 * float(h))
        assert abs(fd - grad[u]) <= 1e-5 * max(1.0, np.abs(grad).max())


def test_single_step_closed_form():
    L, tau = 8, 0.3
    C = oracle.code_table("3inst", L).astype(np.float64)
    s = inputs.targets(1, 1, 41)[0]
    w = inputs.weights(1, 1, 42)[0]
    for wt in (None, w):
        ww = 1.0 if wt is None else float(wt[0])
        e = ww * (C - float(s[0])) ** 2
        p = np.exp(-(e - e.min()) / tau)
        p /= p.sum()
        mean = p @ C
        var = p @ (C - mean) ** 2
        grad, soft = oracle.bcjr_vjp(C.astype(np.float32), s, tau, np.array([1.7]), wt, L=L)
        assert abs(soft[0] - mean) <= 1e-12
        assert abs(grad[0] - 2.0 * ww / tau * 1.7 * var) <= 1e-12 * max(1.0, abs(grad[0]))


def test_constant_code_has_zero_gradient():
    L, T = 8, 16
    ones = np.full(1 << L, 0.75, dtype=np.float32)
    s = inputs.targets(1, T, 43)[0]
    grad, soft = oracle.bcjr_vjp(ones, s, 0.2, _g(T, 44), L=L)
    assert np.allclose(soft, 0.75, atol=1e-13)
    assert np.abs(grad).max() <= 1e-12


def _jacobian(C, s, tau, w, L):
    T = s.shape[-1]
    J = np.empty((T, T))
    for t in range(T):
        g = np.zeros(T)
        g[t] = 1.0
        J[t], _ = oracle.bcjr_vjp(C, s, tau, g, w, L=L)    # row t: d soft_t / d s_u
    return J


def test_covariance_symmetric_and_psd():
    L, T, tau = 8, 14, 0.4
    C = oracle.code_table("1mad", L)
    s = inputs.targets(1, T, 45)[0]
    w = inputs.weights(1, T, 46)[0].astype(np.float64)
    J = _jacobian(C, s, tau, w.astype(np.float32), L)
    K = J * tau / (2.0 * w[None, :])                     # Cov(C_t, C_u)
    assert np.allclose(K, K.T, rtol=1e-9, atol=1e-12)
    ev = np.linalg.eigvalsh(0.5 * (K + K.T))
    assert ev.min() >= -1e-10 * ev.max()
    assert np.all(np.diag(K) > 0)


def test_high_temperature_uniform_covariance():
    L, k, T, tau = 8, 2, 20, 1e7
    C = oracle.code_table("1mad", L).astype(np.float64)
    s = inputs.targets(1, T, 47)[0]
    J = _jacobian(C.astype(np.float32), s, tau, None, L)
    K = J * tau / 2.0
    var = C.var()
    assert np.allclose(np.diag(K), var, rtol=1e-5)
    far = np.abs(np.subtract.outer(np.arange(T), np.arange(T))) >= L // k
    assert np.abs(K[far]).max() <= 1e-5 * var
    # one step apart a state shares L-k bits with the next: uniform-walk covariance of
    # C(x) and C(y) with y = (x << k | b) mod 2^L, b uniform
    N = 1 << L
    x = np.arange(N)
    mean = C.mean()
    cov1 = np.mean([(C[x] - mean) @ (C[((x << k) | b) & (N - 1)] - mean) / N
                    for b in range(1 << k)])
    assert np.allclose(np.diag(K, 1), cov1, rtol=1e-4, atol=1e-5 * var)


# ---- low temperatures: the range where the GPU gradient is compared with this oracle --
# At tau <= 0.01 the walk distribution concentrates on a few walks and the covariance is
# a small difference of large products; these pins check the expectation-message form
# there against the explicit enumeration (both codes, weighted and unweighted) and
# against differences of the separately pinned soft codeword.

@pytest.mark.parametrize("tau", [0.01, 3e-3, 1e-3])
@pytest.mark.parametrize("T", [2, 4, 6])
@pytest.mark.parametrize("code", ["1mad", "3inst"])
def test_bruteforce_L6_low_temperature(code, T, tau):
    L, k = 6, 2
    C = oracle.code_table(code, L)
    for seed in range(3):
        s = inputs.targets(1, T, 700 + seed)[0]
        g = _g(T, 710 + seed)
        grad, soft = oracle.bcjr_vjp(C, s, tau, g, L=L, k=k)
        ref = oracle.brute_bcjr_vjp(C, s, tau, g, L=L, k=k)
        bsoft, _ = oracle.brute_bcjr(C, s, tau, L=L, k=k)
        scale = np.abs(ref).max() + 1e-300
        assert np.allclose(grad, ref, rtol=1e-9, atol=1e-9 * scale), (seed, grad, ref)
        assert np.allclose(soft, bsoft, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("tau", [0.01, 3e-3, 1e-3])
def test_bruteforce_weighted_L6_low_temperature(tau):
    L, k, T = 6, 2, 5
    for code in ("1mad", "3inst"):
        C = oracle.code_table(code, L)
        s = inputs.targets(1, T, 720)[0]
        w = inputs.weights(1, T, 721)[0]
        g = _g(T, 722)
        grad, _ = oracle.bcjr_vjp(C, s, tau, g, w, L=L, k=k)
        ref = oracle.brute_bcjr_vjp(C, s, tau, g, w, L=L, k=k)
        assert np.allclose(grad, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def test_bruteforce_near_tie_low_temperature():
    """Two walks a hair apart in energy: the covariance is then carried by the pair alone
    (a two-point distribution), the case where the gradient collapses onto few entries."""
    L, k, T, tau = 6, 2, 4, 1e-3
    C = oracle.code_table("1mad", L)
    # targets halfway between two code values at every step give near-ties
    vals = np.unique(C)
    s = np.array([(vals[20] + vals[21]) / 2, vals[30], (vals[10] + vals[11]) / 2, vals[40]],
                 dtype=np.float32)
    g = _g(T, 730)
    grad, _ = oracle.bcjr_vjp(C, s, tau, g, L=L, k=k)
    ref = oracle.brute_bcjr_vjp(C, s, tau, g, L=L, k=k)
    assert np.abs(ref).max() > 0
    assert np.allclose(grad, ref, rtol=1e-9, atol=1e-9 * np.abs(ref).max())


def _richardson_fd(C, s, tau, w, g, u, h, L):
    """d(g . soft)/d s_u by central differences at h and h/2, Richardson-combined
    (error O(h^4)); every perturbed target is exact in binary32."""
    def cd(hh):
        hh = np.float32(hh)
        sp = s.copy(); sp[u] += hh
        sm = s.copy(); sm[u] -= hh
        assert sp[u] - s[u] == hh and s[u] - sm[u] == hh
        fp, _ = oracle.bcjr(C, sp, tau, w, L=L, k=2)
        fm, _ = oracle.bcjr(C, sm, tau, w, L=L, k=2)
        return (g @ fp - g @ fm) / (2.0 * float(hh))
    return (4.0 * cd(h / 2) - cd(h)) / 3.0


@pytest.mark.parametrize("weighted", [False, True])
def test_central_differences_low_temperature(weighted):
    L, T, tau = 8, 16, 0.01
    C = oracle.code_table("1mad", L)
    s = inputs.targets(1, T, 740)[0]
    w = inputs.weights(1, T, 741)[0] if weighted else None
    g = _g(T, 742)
    grad, _ = oracle.bcjr_vjp(C, s, tau, g, w, L=L, k=2)
    scale = np.abs(grad).max()
    for u in range(T):
        fd = _richardson_fd(C, s, tau, w, g, u, 2.0 ** -14, L)
        assert abs(fd - grad[u]) <= 1e-6 * scale, (u, fd, grad[u])


def test_central_differences_tau_1e3():
    """Targets at midpoints between neighbouring code values (near-ties at every step),
    so that the gradient at tau = 1e-3 is carried by competing walks, not ~0."""
    L, T, tau = 6, 10, 1e-3
    C = oracle.code_table("3inst", L)
    vals = np.unique(C.astype(np.float64))
    pick = np.random.default_rng(752).integers(0, len(vals) - 1, T)
    s = ((vals[pick] + vals[pick + 1]) / 2).astype(np.float32)
    g = _g(T, 751)
    grad, _ = oracle.bcjr_vjp(C, s, tau, g, L=L, k=2)
    scale = np.abs(grad).max()
    assert scale > 1e-3
    for u in range(T):
        fd = _richardson_fd(C, s, tau, None, g, u, 2.0 ** -18, L)
        assert abs(fd - grad[u]) <= 1e-6 * scale, (u, fd, grad[u])
