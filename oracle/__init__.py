"""CPU oracle for the bitshift-trellis hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path (``trellis_coded_weight_amd``) never does,
and this package never imports the product: the two only share the seeded input
arrays.

The arithmetic lives in ``qtcq_oracle.c`` (plain C, binary32 search, binary64 BCJR,
brute-force enumerators); this module only builds it with gcc and marshals numpy
arrays through ctypes.  See the C file's header for the sources it follows and the
readings it takes where the pages are silent.  Parity unpinned: the LCG inside 3INST.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qtcq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CODE_1MAD = 0
CODE_3INST = 1
_CODES = {"1mad": CODE_1MAD, "3inst": CODE_3INST, CODE_1MAD: CODE_1MAD, CODE_3INST: CODE_3INST}


# QTCQ_ORACLE_SANITIZE=1 builds and loads an AddressSanitizer + UndefinedBehaviorSanitizer
# build instead (liboracle_san.so; the process must preload the ASan runtime).
_SANITIZE = os.environ.get("QTCQ_ORACLE_SANITIZE") == "1"
_LIB_SAN = os.path.join(_HERE, "liboracle_san.so")


def build(force: bool = False, sanitize: bool = _SANITIZE) -> str:
    """Compile liboracle.so with gcc (no contraction, no fast-math); with sanitize, the
    ASan/UBSan build liboracle_san.so (UB reports abort the process)."""
    out = _LIB_SAN if sanitize else _LIB
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        if sanitize:
            cmd[1:1] = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        f32p = ctypes.POINTER(ctypes.c_float)
        f64p = ctypes.POINTER(ctypes.c_double)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        c_int, c_i64, c_u32, c_dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, ctypes.c_double
        sig = {
            "oracle_code_1mad": (ctypes.c_float, [c_u32]),
            "oracle_code_3inst": (ctypes.c_float, [c_u32]),
            "oracle_code_3inst_raw": (c_dbl, [c_u32]),
            "oracle_code_table": (c_int, [c_int, c_int, f32p]),
            "oracle_code_xor": (ctypes.c_float, [c_u32, u32p]),
            "oracle_code_table_xor": (c_int, [c_int, u32p, f32p]),
            "oracle_viterbi": (c_int, [f32p, f32p, f32p, c_int, c_int, c_int, u32p, f32p]),
            "oracle_viterbi_batch": (c_int, [f32p, f32p, f32p, c_i64, c_int, c_int, c_int,
                                             u32p, f32p, f32p]),
            "oracle_stream_bits": (c_i64, [c_int, c_int, c_int]),
            "oracle_stream_words": (c_i64, [c_int, c_int, c_int]),
            "oracle_pack": (c_int, [u32p, c_int, c_int, c_int, u32p]),
            "oracle_pack_batch": (c_int, [u32p, c_i64, c_int, c_int, c_int, u32p]),
            "oracle_decode": (c_int, [u32p, c_int, c_int, c_int, f32p, u32p, f32p]),
            "oracle_decode_batch": (c_int, [u32p, c_i64, c_int, c_int, c_int, f32p, u32p, f32p]),
            "oracle_path_cost": (ctypes.c_float, [f32p, f32p, f32p, c_int]),
            "oracle_bcjr": (c_int, [f32p, f32p, f32p, c_int, c_int, c_int, c_dbl, f64p, f64p]),
            "oracle_bcjr_batch": (c_int, [f32p, f32p, f32p, c_i64, c_int, c_int, c_int, c_dbl,
                                          f64p, f64p]),
            "oracle_minsum_marginals": (c_int, [f32p, f32p, f32p, c_int, c_int, c_int, f64p]),
            "oracle_brute_viterbi": (c_int, [f32p, f32p, f32p, c_int, c_int, c_int, f32p, u32p,
                                             i64p]),
            "oracle_brute_bcjr": (c_int, [f32p, f32p, f32p, c_int, c_int, c_int, c_dbl, f64p,
                                          f64p]),
            "oracle_bcjr_vjp_batch": (c_int, [f32p, f32p, f32p, c_i64, c_int, c_int, c_int, c_dbl,
                                              f64p, f64p, f64p]),
            "oracle_brute_bcjr_vjp": (c_int, [f32p, f32p, f32p, c_int, c_int, c_int, c_dbl, f64p,
                                              f64p]),
            "oracle_tb_stream_bits": (c_i64, [c_int, c_int, c_int]),
            "oracle_tb_stream_words": (c_i64, [c_int, c_int, c_int]),
            "oracle_viterbi_pinned": (c_int, [f32p, f32p, f32p, c_int, c_int, c_int, c_u32,
                                              u32p, f32p]),
            "oracle_tailbiting_exact": (c_int, [f32p, f32p, f32p, c_int, c_int, c_int, u32p,
                                                f32p]),
            "oracle_tailbiting_alg4": (c_int, [f32p, f32p, f32p, c_int, c_int, c_int, u32p, f32p,
                                               u32p]),
            "oracle_tailbiting_alg4_batch": (c_int, [f32p, f32p, f32p, c_i64, c_int, c_int, c_int,
                                                     u32p, f32p, f32p]),
            "oracle_tb_pack_batch": (c_int, [u32p, c_i64, c_int, c_int, c_int, u32p]),
            "oracle_tb_decode_batch": (c_int, [u32p, c_i64, c_int, c_int, c_int, f32p, u32p,
                                               f32p]),
            "oracle_brute_tailbiting": (c_int, [f32p, f32p, f32p, c_int, c_int, c_int, f32p,
                                                i64p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


# ---------------------------------------------------------------------------------
# codes
# ---------------------------------------------------------------------------------

def code_value(code, x: int) -> float:
    c = _CODES[code]
    fn = lib().oracle_code_1mad if c == CODE_1MAD else lib().oracle_code_3inst
    return fn(x)


def code_3inst_raw(x: int) -> float:
    return lib().oracle_code_3inst_raw(x)


def code_table(code, L: int) -> np.ndarray:
    """Code value of every L-bit state: code "1mad", "3inst", or ("xor", masks) for the
    XOR-Trellis palette code with parity masks (m0, m1, m2, m3)."""
    out = np.empty(1 << L, dtype=np.float32)
    if isinstance(code, tuple) and code[0] == "xor":
        m = np.ascontiguousarray(np.array(code[1], dtype=np.uint32))
        _check(lib().oracle_code_table_xor(L, _p(m, ctypes.c_uint32), _p(out, ctypes.c_float)),
               "code_table_xor")
        return out
    _check(lib().oracle_code_table(_CODES[code], L, _p(out, ctypes.c_float)), "code_table")
    return out


def code_xor(x: int, masks) -> float:
    m = np.ascontiguousarray(np.array(masks, dtype=np.uint32))
    return lib().oracle_code_xor(x, _p(m, ctypes.c_uint32))


# ---------------------------------------------------------------------------------
# search, pack, decode
# ---------------------------------------------------------------------------------

def viterbi(C, s, w=None, L=16, k=2):
    """Batch Viterbi.  s: [B][T] (or [T]) float32.  Returns (states u32, cost f32, mse f32)."""
    C = _f32(C)
    s = _f32(s)
    one = s.ndim == 1
    s2 = s.reshape(1, -1) if one else s
    B, T = s2.shape
    w2 = None if w is None else _f32(w).reshape(B, T)
    st = np.empty((B, T), dtype=np.uint32)
    cost = np.empty(B, dtype=np.float32)
    mse = np.empty(B, dtype=np.float32)
    _check(lib().oracle_viterbi_batch(_p(C, ctypes.c_float), _p(s2, ctypes.c_float),
                                      _p(w2, ctypes.c_float), B, T, L, k,
                                      _p(st, ctypes.c_uint32), _p(cost, ctypes.c_float),
                                      _p(mse, ctypes.c_float)), "viterbi")
    if one:
        return st[0], cost[0], mse[0]
    return st, cost, mse


def stream_bits(L, k, T) -> int:
    return lib().oracle_stream_bits(L, k, T)


def stream_words(L, k, T) -> int:
    return lib().oracle_stream_words(L, k, T)


def pack(states, L=16, k=2):
    st = np.ascontiguousarray(states, dtype=np.uint32)
    one = st.ndim == 1
    st2 = st.reshape(1, -1) if one else st
    B, T = st2.shape
    W = stream_words(L, k, T)
    words = np.empty((B, W), dtype=np.uint32)
    _check(lib().oracle_pack_batch(_p(st2, ctypes.c_uint32), B, T, L, k,
                                   _p(words, ctypes.c_uint32)), "pack")
    return words[0] if one else words


def decode(words, T, C, L=16, k=2):
    """Returns (windows u32 [B][T], recon f32 [B][T])."""
    C = _f32(C)
    wd = np.ascontiguousarray(words, dtype=np.uint32)
    one = wd.ndim == 1
    wd2 = wd.reshape(1, -1) if one else wd
    B = wd2.shape[0]
    assert wd2.shape[1] == stream_words(L, k, T)
    win = np.empty((B, T), dtype=np.uint32)
    rec = np.empty((B, T), dtype=np.float32)
    _check(lib().oracle_decode_batch(_p(wd2, ctypes.c_uint32), B, T, L, k, _p(C, ctypes.c_float),
                                     _p(win, ctypes.c_uint32), _p(rec, ctypes.c_float)), "decode")
    if one:
        return win[0], rec[0]
    return win, rec


def path_cost(recon, s, w=None) -> float:
    r = _f32(recon)
    s = _f32(s)
    w = _f32(w)
    return lib().oracle_path_cost(_p(r, ctypes.c_float), _p(s, ctypes.c_float),
                                  _p(w, ctypes.c_float), r.shape[-1])


# ---------------------------------------------------------------------------------
# BCJR and exact references
# ---------------------------------------------------------------------------------

def bcjr(C, s, tau, w=None, L=16, k=2):
    """Batch fp64 BCJR.  Returns (soft f64 [B][T], logz f64 [B])."""
    C = _f32(C)
    s = _f32(s)
    one = s.ndim == 1
    s2 = s.reshape(1, -1) if one else s
    B, T = s2.shape
    w2 = None if w is None else _f32(w).reshape(B, T)
    soft = np.empty((B, T), dtype=np.float64)
    logz = np.empty(B, dtype=np.float64)
    _check(lib().oracle_bcjr_batch(_p(C, ctypes.c_float), _p(s2, ctypes.c_float),
                                   _p(w2, ctypes.c_float), B, T, L, k, float(tau),
                                   _p(soft, ctypes.c_double), _p(logz, ctypes.c_double)), "bcjr")
    if one:
        return soft[0], logz[0]
    return soft, logz


def bcjr_vjp(C, s, tau, g, w=None, L=16, k=2):
    """Batch fp64 vector-Jacobian product of the soft codeword w.r.t. the targets.
    g: upstream gradient, shape of s.  Returns (grad f64 [B][T], soft f64 [B][T])."""
    C = _f32(C)
    s = _f32(s)
    one = s.ndim == 1
    s2 = s.reshape(1, -1) if one else s
    B, T = s2.shape
    w2 = None if w is None else _f32(w).reshape(B, T)
    g2 = np.ascontiguousarray(g, dtype=np.float64).reshape(B, T)
    grad = np.empty((B, T), dtype=np.float64)
    soft = np.empty((B, T), dtype=np.float64)
    _check(lib().oracle_bcjr_vjp_batch(_p(C, ctypes.c_float), _p(s2, ctypes.c_float),
                                       _p(w2, ctypes.c_float), B, T, L, k, float(tau),
                                       _p(g2, ctypes.c_double), _p(grad, ctypes.c_double),
                                       _p(soft, ctypes.c_double)), "bcjr_vjp")
    if one:
        return grad[0], soft[0]
    return grad, soft


def brute_bcjr_vjp(C, s, tau, g, w=None, L=6, k=2):
    C = _f32(C)
    s = _f32(s)
    w = _f32(w)
    T = s.shape[-1]
    g = np.ascontiguousarray(g, dtype=np.float64)
    grad = np.empty(T, dtype=np.float64)
    _check(lib().oracle_brute_bcjr_vjp(_p(C, ctypes.c_float), _p(s, ctypes.c_float),
                                       _p(w, ctypes.c_float), T, L, k, float(tau),
                                       _p(g, ctypes.c_double), _p(grad, ctypes.c_double)),
           "brute_bcjr_vjp")
    return grad


def minsum_marginals(C, s, w=None, L=16, k=2) -> np.ndarray:
    C = _f32(C)
    s = _f32(s)
    w = _f32(w)
    T = s.shape[-1]
    out = np.empty((T, 1 << L), dtype=np.float64)
    _check(lib().oracle_minsum_marginals(_p(C, ctypes.c_float), _p(s, ctypes.c_float),
                                         _p(w, ctypes.c_float), T, L, k,
                                         _p(out, ctypes.c_double)), "minsum")
    return out


def brute_viterbi(C, s, w=None, L=6, k=2):
    """Returns (min cost f32, reverse-lex smallest optimal path u32[T], #optimal walks)."""
    C = _f32(C)
    s = _f32(s)
    w = _f32(w)
    T = s.shape[-1]
    best = np.empty(1, dtype=np.float32)
    path = np.empty(T, dtype=np.uint32)
    n = np.empty(1, dtype=np.int64)
    _check(lib().oracle_brute_viterbi(_p(C, ctypes.c_float), _p(s, ctypes.c_float),
                                      _p(w, ctypes.c_float), T, L, k, _p(best, ctypes.c_float),
                                      _p(path, ctypes.c_uint32), _p(n, ctypes.c_int64)),
           "brute_viterbi")
    return best[0], path, int(n[0])


def brute_bcjr(C, s, tau, w=None, L=6, k=2):
    C = _f32(C)
    s = _f32(s)
    w = _f32(w)
    T = s.shape[-1]
    soft = np.empty(T, dtype=np.float64)
    logz = np.empty(1, dtype=np.float64)
    _check(lib().oracle_brute_bcjr(_p(C, ctypes.c_float), _p(s, ctypes.c_float),
                                   _p(w, ctypes.c_float), T, L, k, float(tau),
                                   _p(soft, ctypes.c_double), _p(logz, ctypes.c_double)),
           "brute_bcjr")
    return soft, logz[0]


# ---------------------------------------------------------------------------------
# tail-biting trellis
# ---------------------------------------------------------------------------------

def tb_stream_bits(L, k, T) -> int:
    return lib().oracle_tb_stream_bits(L, k, T)


def tb_stream_words(L, k, T) -> int:
    return lib().oracle_tb_stream_words(L, k, T)


def viterbi_pinned(C, s, o, w=None, L=16, k=2):
    """One sequence, both ends pinned to overlap o.  Returns (states u32 [T], cost f32)."""
    C = _f32(C)
    s = _f32(s)
    w = _f32(w)
    T = s.shape[-1]
    st = np.empty(T, dtype=np.uint32)
    cost = np.empty(1, dtype=np.float32)
    _check(lib().oracle_viterbi_pinned(_p(C, ctypes.c_float), _p(s, ctypes.c_float),
                                       _p(w, ctypes.c_float), T, L, k, int(o),
                                       _p(st, ctypes.c_uint32), _p(cost, ctypes.c_float)),
           "viterbi_pinned")
    return st, cost[0]


def tailbiting_exact(C, s, w=None, L=12, k=2):
    """Exact tail-biting optimum of one sequence (2^(L-k) pinned searches).
    Returns (states u32 [T], cost f32)."""
    C = _f32(C)
    s = _f32(s)
    w = _f32(w)
    T = s.shape[-1]
    st = np.empty(T, dtype=np.uint32)
    cost = np.empty(1, dtype=np.float32)
    _check(lib().oracle_tailbiting_exact(_p(C, ctypes.c_float), _p(s, ctypes.c_float),
                                         _p(w, ctypes.c_float), T, L, k,
                                         _p(st, ctypes.c_uint32), _p(cost, ctypes.c_float)),
           "tailbiting_exact")
    return st, cost[0]


def tailbiting_overlap(C, s, w=None, L=16, k=2) -> int:
    """The overlap the two-search encoder pins the ends to, for one sequence."""
    C = _f32(C)
    s = _f32(s)
    w = _f32(w)
    T = s.shape[-1]
    st = np.empty(T, dtype=np.uint32)
    cost = np.empty(1, dtype=np.float32)
    o = np.empty(1, dtype=np.uint32)
    _check(lib().oracle_tailbiting_alg4(_p(C, ctypes.c_float), _p(s, ctypes.c_float),
                                        _p(w, ctypes.c_float), T, L, k, _p(st, ctypes.c_uint32),
                                        _p(cost, ctypes.c_float), _p(o, ctypes.c_uint32)),
           "tailbiting_alg4")
    return int(o[0])


def tailbiting(C, s, w=None, L=16, k=2):
    """Batch two-search tail-biting encode.  Returns (states u32, cost f32, mse f32)."""
    C = _f32(C)
    s = _f32(s)
    one = s.ndim == 1
    s2 = s.reshape(1, -1) if one else s
    B, T = s2.shape
    w2 = None if w is None else _f32(w).reshape(B, T)
    st = np.empty((B, T), dtype=np.uint32)
    cost = np.empty(B, dtype=np.float32)
    mse = np.empty(B, dtype=np.float32)
    _check(lib().oracle_tailbiting_alg4_batch(_p(C, ctypes.c_float), _p(s2, ctypes.c_float),
                                              _p(w2, ctypes.c_float), B, T, L, k,
                                              _p(st, ctypes.c_uint32), _p(cost, ctypes.c_float),
                                              _p(mse, ctypes.c_float)), "tailbiting")
    if one:
        return st[0], cost[0], mse[0]
    return st, cost, mse


def tb_pack(states, L=16, k=2):
    st = np.ascontiguousarray(states, dtype=np.uint32)
    one = st.ndim == 1
    st2 = st.reshape(1, -1) if one else st
    B, T = st2.shape
    W = tb_stream_words(L, k, T)
    words = np.empty((B, W), dtype=np.uint32)
    _check(lib().oracle_tb_pack_batch(_p(st2, ctypes.c_uint32), B, T, L, k,
                                      _p(words, ctypes.c_uint32)), "tb_pack")
    return words[0] if one else words


def tb_decode(words, T, C, L=16, k=2):
    """Cyclic window decode.  Returns (windows u32 [B][T], recon f32 [B][T])."""
    C = _f32(C)
    wd = np.ascontiguousarray(words, dtype=np.uint32)
    one = wd.ndim == 1
    wd2 = wd.reshape(1, -1) if one else wd
    B = wd2.shape[0]
    assert wd2.shape[1] == tb_stream_words(L, k, T)
    win = np.empty((B, T), dtype=np.uint32)
    rec = np.empty((B, T), dtype=np.float32)
    _check(lib().oracle_tb_decode_batch(_p(wd2, ctypes.c_uint32), B, T, L, k,
                                        _p(C, ctypes.c_float), _p(win, ctypes.c_uint32),
                                        _p(rec, ctypes.c_float)), "tb_decode")
    if one:
        return win[0], rec[0]
    return win, rec


def brute_tailbiting(C, s, w=None, L=6, k=2):
    """Returns (min cost over every cyclic walk f32, #walks attaining it)."""
    C = _f32(C)
    s = _f32(s)
    w = _f32(w)
    T = s.shape[-1]
    best = np.empty(1, dtype=np.float32)
    n = np.empty(1, dtype=np.int64)
    _check(lib().oracle_brute_tailbiting(_p(C, ctypes.c_float), _p(s, ctypes.c_float),
                                         _p(w, ctypes.c_float), T, L, k, _p(best, ctypes.c_float),
                                         _p(n, ctypes.c_int64)), "brute_tailbiting")
    return best[0], int(n[0])


# ---------------------------------------------------------------------------------
# Decode -> matrix-vector product (inference side)
# ---------------------------------------------------------------------------------
# QTIP blog, "What it buys end to end": every 16x16 tile of a weight matrix is one
# 256-long sequence that decodes straight into the matrix operand.  Reading (the pages
# give no order): tiles are numbered row-major, sequence b = I * (N / 16) + J holds
# tile (I, J), and within a tile weight t = 16 r + c is W[16 I + r][16 J + c].

TILE = 16


def tiles_to_matrix(vals, M: int, N: int) -> np.ndarray:
    """Assemble the M x N matrix from per-tile sequences vals [(M/16)(N/16)][256]."""
    v = np.asarray(vals)
    assert M % TILE == 0 and N % TILE == 0 and v.shape == ((M // TILE) * (N // TILE), TILE * TILE)
    return v.reshape(M // TILE, N // TILE, TILE, TILE).transpose(0, 2, 1, 3).reshape(M, N)


def decode_matvec(words, M: int, N: int, C, x, L=16, k=2, tailbiting=False) -> np.ndarray:
    """y [Bx][M] = W x_i for every row x_i of x [Bx][N], in binary64, with W the window
    decode (plain or cyclic) of the tile streams words [(M/16)(N/16)][W]."""
    dec = tb_decode if tailbiting else decode
    _, rec = dec(words, TILE * TILE, C, L, k)
    Wm = tiles_to_matrix(rec, M, N).astype(np.float64)
    x2 = np.asarray(x, dtype=np.float64).reshape(-1, N)
    return x2 @ Wm.T
