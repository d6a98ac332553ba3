"""GPU parity at the largest sizes the C ABI accepts and at odd batch shapes: sequences
of T = 4096 weights (the maximum) through the plain and tail-biting encoders, the
decoders, the BCJR soft pass and its gradient; odd batches (the encoder interleaves two
sequences per workgroup); the decode -> matvec with a 65,536-wide inner dimension;
batches just above the device's compute-unit count, where the search switches from one
sequence per workgroup to interleaved pairs.  Each against the oracle at the bar of its
own test module."""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs

from helpers import bcjr_err, dev, oracle_bcjr_par, oracle_vjp_par, say
from test_gpu_encode import check_encode
from test_gpu_tailbiting import check_tb

pytestmark = pytest.mark.gpu

TMAX = 4096


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    from trellis_coded_weight_amd import api as a
    return a


def sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("L,B,code,weighted", [(16, 3, "1mad", False), (12, 5, "3inst", True)])
def test_encode_decode_longest_sequences(api, L, B, code, weighted):
    s = inputs.targets(B, TMAX, 4242 + L)
    w = inputs.weights(B, TMAX, 4243 + L) if weighted else None
    check_encode(api, s, w, L, code)


@pytest.mark.parametrize("L,B", [(16, 2), (10, 3)])
def test_tailbiting_longest_sequences(api, L, B):
    s = inputs.targets(B, TMAX, 4343 + L)
    check_tb(api, s, None, L, "1mad")


# The search stages targets through an LDS ring of two 256-step chunks and refills a
# slot while the other is read; lengths around the chunk boundaries exercise the refill
# schedule (and the tail-biting rotation, which wraps inside a chunk).
@pytest.mark.parametrize("T", [255, 257, 511, 512, 513, 767, 768, 769, 1025])
def test_encode_ring_boundaries(api, T):
    s = inputs.targets(3, T, 4500 + T)
    w = inputs.weights(3, T, 4600 + T) if T % 2 else None
    check_encode(api, s, w, 10, "1mad")


@pytest.mark.parametrize("T", [257, 513, 768])
def test_tailbiting_ring_boundaries(api, T):
    s = inputs.targets(3, T, 4700 + T)
    check_tb(api, s, None, 10, "3inst")


def test_encode_odd_batch_L16(api):
    s = inputs.targets(7, 256, 4444)
    check_encode(api, s, None, 16, "1mad")


# The search runs one sequence per workgroup when the batch fits in one round of compute
# units, and interleaved pairs above that; the small batches above run the first form.
# These batches take the paired form at every trellis size, with sequence lengths around
# the target ring's chunk boundaries.
def n_cus():
    import torch
    return torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count


@pytest.mark.parametrize("L,T,code,weighted", [(6, 17, "1mad", False), (8, 256, "3inst", True),
                                               (10, 513, "1mad", False), (10, 1025, "xor", True),
                                               (12, 257, "1mad", True)])
def test_encode_paired_workgroups(api, L, T, code, weighted):
    B = n_cus() + 3
    s = inputs.targets(B, T, 5000 + 10 * L + T % 7)
    w = inputs.weights(B, T, 5001 + L) if weighted else None
    if code == "xor":
        code = ("xor", inputs.xor_masks(L))
    check_encode(api, s, w, L, code)


@pytest.mark.parametrize("L,T", [(6, 37), (8, 513), (12, 256)])
def test_tailbiting_paired_workgroups(api, L, T):
    B = n_cus() + 1
    check_tb(api, inputs.targets(B, T, 5100 + L), None, L, "1mad")


def test_encode_single_and_paired_agree(api):
    """The last batch of one sequence per workgroup and the first of pairs give the same
    bits for the rows they share (L = 16)."""
    import torch
    n = n_cus()
    s = dev(inputs.targets(n + 1, 256, 5200))
    b1, m1, x1 = api.encode(s[:n].contiguous(), want_states=True)
    b2, m2, x2 = api.encode(s, want_states=True)
    sync()
    assert torch.equal(b1, b2[:n]) and torch.equal(x1, x2[:n])
    assert torch.equal(m1.view(torch.int32), m2[:n].view(torch.int32))


@pytest.mark.parametrize("tau", [1.0, 0.01])
def test_bcjr_longest_sequences(api, tau):
    L, B = 8, 3
    s = inputs.targets(B, TMAX, 4545)
    say("bcjr T=%d L=%d tau=%g" % (TMAX, L, tau))
    soft, logz = api.bcjr_soft(dev(s), tau, L=L)
    sync()
    C = oracle.code_table("1mad", L)
    soft_o, logz_o = oracle_bcjr_par(C, s, tau, L=L)
    assert bcjr_err(soft.cpu().numpy(), soft_o).max() <= 1e-5
    lz = logz.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(lz - logz_o) <= 1e-5 * np.maximum(1.0, np.abs(logz_o)))


def test_bcjr_vjp_longest_sequence(api):
    L, B, tau = 8, 2, 0.1
    s = inputs.targets(B, TMAX, 4646)
    g = np.random.default_rng(4647).standard_normal((B, TMAX)).astype(np.float32)
    say("bcjr vjp T=%d L=%d" % (TMAX, L))
    grad, _, _ = api.bcjr_vjp(dev(s), tau, dev(g), L=L)
    sync()
    C = oracle.code_table("1mad", L)
    grad_o, _ = oracle_vjp_par(C, s, tau, g.astype(np.float64), L=L)
    assert bcjr_err(grad.cpu().numpy(), grad_o).max() <= 1e-5


def test_matvec_wide_inner_dimension(api):
    import torch
    M, N, L = 32, 65536, 16
    W = oracle.stream_words(L, 2, 256)
    words = np.random.default_rng(4748).integers(0, 1 << 32, size=((M // 16) * (N // 16), W),
                                                  dtype=np.uint32)
    x = inputs.targets(2, N, 4749)
    say("matvec M=%d N=%d" % (M, N))
    y = api.decode_matvec(torch.from_numpy(words.view(np.int32)).cuda(), M, N, dev(x))
    sync()
    C = oracle.code_table("1mad", L)
    y_o = oracle.decode_matvec(words, M, N, C, x, L, 2)
    _, rec = oracle.decode(words, 256, C, L, 2)
    Wm = oracle.tiles_to_matrix(rec, M, N).astype(np.float64)
    mag = np.abs(x.astype(np.float64)) @ np.abs(Wm).T
    bound = (4 * -(-N // 1024) + 23) * 2.0 ** -24 * mag
    assert np.all(np.abs(y.cpu().numpy() - y_o) <= bound)


@pytest.mark.parametrize("L", [14, 16])
@pytest.mark.parametrize("T", [1, 2, 37])
def test_bcjr_and_gradient_short_sequences_multiwave(api, L, T):
    """Multi-wave workgroups (4 waves at L = 14, 16 at L = 16) on short sequences."""
    B, tau = 2, 0.1
    s = inputs.targets(B, T, 4800 + L + T)
    g = np.random.default_rng(4900 + L + T).standard_normal((B, T)).astype(np.float32)
    say("bcjr + vjp L=%d T=%d" % (L, T))
    grad, soft, logz = api.bcjr_vjp(dev(s), tau, dev(g), L=L, want_soft=True)
    sync()
    C = oracle.code_table("1mad", L)
    grad_o, soft_o = oracle_vjp_par(C, s, tau, g.astype(np.float64), L=L)
    assert bcjr_err(soft.cpu().numpy(), soft_o).max() <= 1e-5
    assert bcjr_err(grad.cpu().numpy(), grad_o).max() <= 1e-5
