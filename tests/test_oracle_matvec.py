"""Pins for the oracle's decode -> matrix-vector product.  CPU only.

QTIP blog, "What it buys end to end": each 16x16 tile of a weight matrix is one 256-long
sequence that decodes straight into the matrix operand.  Reading: row-major tiles, and
row-major weights within a tile (t = 16 r + c).  The product is a binary64 matmul.

Pins:
* single weights, read with the pages' own window rule on the stream as one big integer
  (independent of the C decode and of the matrix assembly), for plain and tail-biting
  streams: x = e_n gives y = column n;
* layout-free: x = 1 gives sum(y) = the sum of every decoded weight;
* tile geometry: x = the indicator of tile column J gives, at row 16 I + r, the sum of
  weights t = 16 r .. 16 r + 15 of sequence (I, J) -- a transposed tile would give
  column sums instead;
* batch rows are independent products.
"""
import numpy as np
import pytest

import oracle
from trellis_coded_weight_amd import inputs


def window_value(words, t, C, L, k, nbits, cyclic):
    """The pages' decode rule: the stream as one MSB-first integer, window of bits
    [t k, t k + L) (taken modulo nbits for a cyclic stream)."""
    big = 0
    for w in words:
        big = (big << 32) | int(w)
    total = 32 * len(words)
    start = t * k
    if cyclic:
        win = 0
        for i in range(L):
            p = (start + i) % nbits
            win = (win << 1) | ((big >> (total - 1 - p)) & 1)
    else:
        win = (big >> (total - start - L)) & ((1 << L) - 1)
    return float(C[win])


def random_streams(nseq, L, k, cyclic, seed):
    """Streams of random walks: plain = free start; cyclic = wrap-consistent."""
    rng = np.random.default_rng(seed)
    T = 256
    st = np.empty((nseq, T), dtype=np.uint32)
    mask = (1 << L) - 1
    for b in range(nseq):
        s = int(rng.integers(0, 1 << L))
        for t in range(T):
            st[b, t] = s
            s = ((s << k) | int(rng.integers(0, 1 << k))) & mask
    if cyclic:
        # force the cyclic condition by rewriting the last L/k - 1 states from the start
        for b in range(nseq):
            bits = [(int(st[b, t]) >> (L - k)) for t in range(T)]      # k high bits per state
            for t in range(T):
                v = 0
                for i in range(L // k):
                    v = (v << k) | bits[(t + i) % T]
                st[b, t] = v
        return oracle.tb_pack(st, L, k), st
    return oracle.pack(st, L, k), st


@pytest.mark.parametrize("cyclic", [False, True])
@pytest.mark.parametrize("L,code", [(16, "1mad"), (12, "3inst")])
def test_columns_by_window_rule(cyclic, L, code):
    k, M, N = 2, 32, 48
    C = oracle.code_table(code, L)
    words, _ = random_streams((M // 16) * (N // 16), L, k, cyclic, 11 + L)
    nbits = 2 * 256 if cyclic else oracle.stream_bits(L, k, 256)
    rng = np.random.default_rng(3)
    for n in rng.choice(N, size=6, replace=False):
        x = np.zeros(N)
        x[n] = 1.0
        y = oracle.decode_matvec(words, M, N, C, x, L, k, tailbiting=cyclic)[0]
        J, c = divmod(int(n), 16)
        for m in range(M):
            I, r = divmod(m, 16)
            b = I * (N // 16) + J
            assert y[m] == window_value(words[b], 16 * r + c, C, L, k, nbits, cyclic)


def test_sum_of_all_weights():
    L, k, M, N = 16, 2, 64, 32
    C = oracle.code_table("1mad", L)
    words, st = random_streams((M // 16) * (N // 16), L, k, False, 5)
    y = oracle.decode_matvec(words, M, N, C, np.ones(N), L, k)[0]
    assert abs(y.sum() - C.astype(np.float64)[st].sum()) <= 1e-9


@pytest.mark.parametrize("cyclic", [False, True])
def test_tile_row_segments(cyclic):
    L, k, M, N = 16, 2, 48, 64
    C = oracle.code_table("1mad", L)
    words, _ = random_streams((M // 16) * (N // 16), L, k, cyclic, 7)
    dec = oracle.tb_decode if cyclic else oracle.decode
    _, rec = dec(words, 256, C, L, k)
    for J in range(N // 16):
        x = np.zeros(N)
        x[16 * J:16 * J + 16] = 1.0
        y = oracle.decode_matvec(words, M, N, C, x, L, k, tailbiting=cyclic)[0]
        for m in range(M):
            I, r = divmod(m, 16)
            seg = rec[I * (N // 16) + J, 16 * r:16 * r + 16].astype(np.float64)
            assert abs(y[m] - seg.sum()) <= 1e-12


def test_batch_rows_independent():
    L, k, M, N = 16, 2, 32, 32
    C = oracle.code_table("1mad", L)
    words, _ = random_streams(4, L, k, False, 9)
    x = inputs.targets(3, N, 10)
    y = oracle.decode_matvec(words, M, N, C, x, L, k)
    for i in range(3):
        # (BLAS may block a batch differently from one vector: binary64 rounding only)
        assert np.allclose(y[i], oracle.decode_matvec(words, M, N, C, x[i], L, k)[0],
                           rtol=1e-12, atol=1e-12)
