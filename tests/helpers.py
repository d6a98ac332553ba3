"""Shared helpers for the GPU parity tests: device transfer, uint32 views, and fanning
the single-threaded oracle out over host threads (ctypes releases the GIL)."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle

N_WORKERS = max(1, min(16, os.cpu_count() or 1))


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run still shows it."""
    print("[case] " + msg, file=sys.stderr, flush=True)


def u32(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _split(n, parts):
    step = max(1, -(-n // parts))
    return [(i, min(n, i + step)) for i in range(0, n, step)]


def oracle_viterbi_par(C, s, w=None, L=16, k=2):
    """Oracle Viterbi over rows of s, fanned out over threads."""
    B, T = s.shape
    st = np.empty((B, T), dtype=np.uint32)
    cost = np.empty(B, dtype=np.float32)
    mse = np.empty(B, dtype=np.float32)

    def job(r):
        a, b = r
        o = oracle.viterbi(C, s[a:b], None if w is None else w[a:b], L=L, k=k)
        st[a:b], cost[a:b], mse[a:b] = o

    with ThreadPoolExecutor(N_WORKERS) as ex:
        list(ex.map(job, _split(B, N_WORKERS * 2)))
    return st, cost, mse


def oracle_bcjr_par(C, s, tau, w=None, L=16, k=2):
    B, T = s.shape
    soft = np.empty((B, T))
    logz = np.empty(B)

    def job(r):
        a, b = r
        so, lz = oracle.bcjr(C, s[a:b], tau, None if w is None else w[a:b], L=L, k=k)
        soft[a:b], logz[a:b] = so, lz

    with ThreadPoolExecutor(N_WORKERS) as ex:
        list(ex.map(job, _split(B, N_WORKERS)))
    return soft, logz


def oracle_vjp_par(C, s, tau, g, w=None, L=16, k=2):
    """Oracle BCJR gradient over rows of s, fanned out over threads (one row per job:
    the binary64 oracle keeps every step's messages, 3 x T x 2^L doubles per row)."""
    B, T = s.shape
    grad = np.empty((B, T))
    soft = np.empty((B, T))
    workers = N_WORKERS if L < 16 else max(1, min(N_WORKERS, 8))

    def job(b):
        gr, so = oracle.bcjr_vjp(C, s[b:b + 1], tau, g[b:b + 1], None if w is None else w[b:b + 1],
                                 L=L, k=k)
        grad[b], soft[b] = gr, so

    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(job, range(B)))
    return grad, soft


def bcjr_err(soft_gpu, soft_ref):
    """Per sequence: max_t |soft_gpu - soft_ref| / RMS_t(soft_ref)."""
    soft_gpu = np.asarray(soft_gpu, dtype=np.float64)
    rms = np.sqrt((soft_ref ** 2).mean(axis=-1))
    dmax = np.abs(soft_gpu - soft_ref).max(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(rms > 0, dmax / rms, np.where(dmax > 0, np.inf, 0.0))
