#!/usr/bin/env python3
"""Benchmark of the bitshift-trellis hot path on one MI355X.

A step = one pass of the path over one 4096x4096 weight matrix (65,536 sequences x
T = 256 i.i.d. N(0,1) float32 targets, L = 16, k = 2, 1MAD code): Viterbi encode
(forward ACS + traceback/pack) and parallel window decode with the round-trip MSE.
Inputs are resident in HBM before timing starts.  Prints ONE JSON line.

Extra objects on the line:
  roofline      -- the dominant kernel (the ACS forward pass) against the VALU peak,
                   from algorithmic ops / HIP-event-timed duration of the encode call
  cpu_baseline  -- the CPU oracle on a bounded sample, on this host's cores
  tailbiting    -- the tail-biting encode (two searches per sequence) of a 4096x4096
                   matrix
  bcjr          -- one BCJR soft-relaxation pass over 65,536 sequences (tau = 0.1)
  bcjr_vjp      -- the gradient of that soft codeword with respect to the targets
  decode        -- the decode kernels' own time and algorithmic HBM bytes
  xor           -- the XOR palette code: encode/decode of a 4096x4096 matrix, matvec
  decode_matvec -- y = W x straight from the streams (per call, batch 1 and 8 with fp32
                   VALU products; batch 1, 8 and 32 with matrix-core products)
  configs       -- the other encode configurations (16 sequences; 4096x14336 3INST;
                   weighted 4096x4096) and the BCJR pass at tau = 1, 0.1, 0.01
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published figures.  fp32 vector peak 157.3 TFLOP/s counts an FMA as two flops:
# 256 CUs x 2.4 GHz x 128 lane-instructions per CU per cycle = 78.6 T lane-ops/s.  On
# gfx950 simple 2-operand VGPR ops (v_add/v_sub/v_mul_f32, integer add/logic/right
# shifts) do issue at 2 wave64 instructions per CU cycle (128 lanes), compares, min/max,
# add-with-carry and 3-operand ops at 1; the peak counts every op at the fast rate.
PEAK_HBM_GBS = 8000.0
CUS, CLOCK_GHZ = 256, 2.4
VALU_LANES_PER_CU_CYCLE = 128
PEAK_VALU_TOPS = CUS * VALU_LANES_PER_CU_CYCLE * CLOCK_GHZ / 1000.0   # 78.64 T lane-ops/s

L, K, T = 16, 2, 256
N_STATES = 1 << L
N_GROUPS = N_STATES >> K


def acs_ops_per_sequence(T: int, weighted: bool = False) -> int:
    """Algorithmic VALU work of the Viterbi forward pass for one sequence: per step
    t = 1..T-1 every state's cost is rebuilt (sub, square[, weight], add) and every
    group takes a 4-way minimum (3 compares); the last step rebuilds all costs once more
    and takes the argmin over 2^L states (2^L - 1 compares)."""
    per_state = 4 if weighted else 3
    per_step = N_STATES * per_state + N_GROUPS * 3
    final = N_STATES * per_state + (N_STATES - 1)
    return (T - 1) * per_step + final


# v_exp_f32 / v_log_f32 issue at one wave64 instruction per two CU cycles (measured):
# a quarter of the fast rate above
PEAK_TRANSC_TOPS = PEAK_VALU_TOPS / 4.0


def bcjr_soft_ops(T: int, L: int = 16, weighted: bool = False):
    """Algorithmic work of one soft pass over one sequence, as the BCJR-QAT abstract's
    forward-backward defines it on 2^L states (N) and 2^(L-2) predecessor groups (G):
      forward, every step: the energies w (C_j - s_t)^2 / tau (3 ops per state, 4
        weighted) and la_t(j) = A_t(j >> 2) - energy (1); from step 1 on, each group's
        A_t = log-sum-exp of its 4 predecessors (16 ops: 3 max, 4 sub, 4 exp, 3 add,
        1 log, 1 add);
      backward, steps T-2..0: lb - energy per state (1) and one 4-way log-sum-exp per
        group (16);
      posterior, every step: gamma = exp(la + lb - log Z) (3 ops, 1 exp) and the sums
        sum gamma, sum gamma C (2).
    Returns (ops, transcendental ops)."""
    N, G = 1 << L, 1 << (L - 2)
    e = 4 if weighted else 3
    fwd = T * (e + 1) * N + (T - 1) * 16 * G
    bwd = (T - 1) * (N + 16 * G)
    post = T * 5 * N
    transc = (T - 1) * 10 * G + T * N
    return fwd + bwd + post, transc


def bcjr_grad_ops(T: int, L: int = 16):
    """Algorithmic work of the gradient beyond its soft pass, per sequence: the
    expectation messages Psi (steps T-2..0) and Phi (steps 1..T-1), each group taking
    4 transition weights (4 sub, 4 exp) and 4 multiply-adds of (g C + message) twice
    (16 ops per group); and at every step the covariance from the posterior (3 ops,
    1 exp), the message sum Phi + g C + Psi (2) and four weighted sums (5) per state.
    Returns (ops, transcendental ops)."""
    N, G = 1 << L, 1 << (L - 2)
    ops = (T - 1) * 2 * 16 * G + T * 10 * N
    transc = (T - 1) * 2 * 4 * G + T * N
    return ops, transc


def mix_ceiling(ops: float, transc: float) -> float:
    """Top/s at which a mix of ops, transc of them exp2/log2, issues when every other op
    runs at the fast VALU rate and the transcendentals at a quarter of it."""
    return ops / (transc / PEAK_TRANSC_TOPS + (ops - transc) / PEAK_VALU_TOPS)


def bcjr_stash_bytes(T: int, L: int = 16, grad: bool = False) -> int:
    """HBM bytes of the message stashes per sequence, 32 bits per group and step: the soft
    pass writes the forward messages once and reads them once; the gradient writes the
    forward stash (read by the soft pass's backward and both halves of the gradient
    sweep: 3 reads), the backward stash and the Phi stash (each written and read once)."""
    G = 1 << (L - 2)
    x = (T - 1) * G * 4
    if not grad:
        return 2 * x
    return 4 * x + 2 * (T * G * 4) + 2 * (T * G * 4)


def roofline_alu(ops: float, transc: float, seconds: float, nbytes: float) -> dict:
    ach = ops / seconds / 1e12
    ceil = mix_ceiling(ops, transc)
    return {"bound": "alu", "achieved": ach, "peak": PEAK_VALU_TOPS, "unit": "Top/s",
            "frac": ach / PEAK_VALU_TOPS, "mix_ceiling": ceil, "frac_of_mix": ach / ceil,
            "transcendental_share": transc / ops,
            "stash_gbs": nbytes / seconds / 1e9, "stash_frac_hbm": nbytes / seconds / 1e9 / PEAK_HBM_GBS}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, s_host) -> dict:
    """The CPU oracle as it stands (single-threaded C, one sequence per call) fanned over
    this host's threads (ctypes releases the GIL), on bounded samples of each
    configuration: the first sequences of the 4096x4096 1MAD encode (the headline's
    workload; its rate is `value`), of the 3INST 4096x14336 and weighted 4096x4096
    encodes, all 16 sequences of the small encode, and the binary64 BCJR of the first
    sequences of the BCJR workload at each temperature."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    from trellis_coded_weight_amd import inputs

    ncpu = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(16, ncpu))

    def fan(fn, n):
        parts = np.array_split(np.arange(n), min(threads, n))
        t0 = time.perf_counter()
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fn, parts))
        return time.perf_counter() - t0

    samples = {}
    for name, n in (("enc4096x4096_1mad", args.cpu_seqs), ("enc4096x14336_3inst", args.cpu_seqs // 4),
                    ("enc4096x4096_1mad_weighted", args.cpu_seqs // 4), ("enc16_1mad", 16)):
        sh, wh, cd = inputs.workload(name, B=n)
        C = oracle.code_table(cd, L)
        sec = fan(lambda ix: oracle.viterbi(C, sh[ix], None if wh is None else wh[ix], L=L, k=K), n)
        samples[name] = {"sequences": n, "seconds": sec, "weights_per_s": n * T / sec}
    nb = args.cpu_bcjr_seqs
    if nb > 0:
        sh, _, _ = inputs.workload("bcjr4096x4096_1mad", B=nb)
        C = oracle.code_table("1mad", L)
        for tau in (1.0, 0.1, 0.01):
            # one sequence per call: the binary64 oracle keeps every step's messages
            sec = fan(lambda ix: [oracle.bcjr(C, sh[i:i + 1], tau, L=L, k=K) for i in ix], nb)
            samples["bcjr4096x4096_1mad tau=%g" % tau] = {"sequences": nb, "seconds": sec,
                                                         "weights_per_s": nb * T / sec}
    head = samples["enc4096x4096_1mad"]
    total = sum(v["seconds"] for v in samples.values())
    print("[bench] cpu baseline %.1f s on %d threads" % (total, threads), file=sys.stderr, flush=True)
    return {"value": head["weights_per_s"], "unit": "weights/s", "cores": threads,
            "kind": "oracle",
            "sample": "oracle Viterbi encode of the first %d of the 65536 sequences of the "
                      "4096x4096 1MAD workload, %d host threads, %.1f s; other configurations "
                      "in 'configs'" % (head["sequences"], threads, head["seconds"]),
            "host_cpu": cpu_model(), "host_cores": os.cpu_count(), "threads": threads,
            "configs": samples}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-bcjr", action="store_true", help="skip the BCJR pass")
    ap.add_argument("--no-tb", action="store_true", help="skip the tail-biting encode")
    ap.add_argument("--no-matvec", action="store_true", help="skip the decode -> matvec")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other encode / BCJR configurations")
    ap.add_argument("--no-xor", action="store_true", help="skip the XOR palette code")
    ap.add_argument("--cpu-seqs", type=int, default=2048,
                    help="CPU baseline: sequences of the 4096x4096 encode sample")
    ap.add_argument("--cpu-bcjr-seqs", type=int, default=32,
                    help="CPU baseline: sequences of the BCJR sample per temperature")
    ap.add_argument("--seqs", type=int, default=0,
                    help="profiling only: encode the first N sequences instead of all 65536")
    ap.add_argument("--bcjr-seqs", type=int, default=0,
                    help="profiling only: run the BCJR passes on the first N sequences")
    ap.add_argument("--matvec-reps", type=int, default=200,
                    help="launches timed per decode -> matvec shape (fewer under a profiler)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for profiles)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (sequences are "
              "independent; see the design notes on sharding)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from trellis_coded_weight_amd import api, inputs

    assert torch.cuda.is_available(), "no GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    name = "enc4096x4096_1mad"
    s_host, _, code = inputs.workload(name, B=args.seqs or None)
    B = s_host.shape[0]
    seq = torch.from_numpy(s_host).to(dev)
    W = api.bitstream_words(L, K, T)
    bits = torch.empty((B, W), dtype=torch.int32, device=dev)
    mse = torch.empty(B, dtype=torch.float32, device=dev)
    recon = torch.empty((B, T), dtype=torch.float32, device=dev)
    mse_rt = torch.empty(B, dtype=torch.float32, device=dev)
    ws = api.encode_workspace(B, T, L, K, max_bytes=64 << 30)

    from trellis_coded_weight_amd import _native as nat
    sptr = stream.cuda_stream

    def encode():
        nat.qtcq_viterbi_encode(seq.data_ptr(), None, B, T, L, K, nat.QTCQ_CODE_1MAD,
                                bits.data_ptr(), mse.data_ptr(), None, ws.data_ptr(),
                                ws.numel(), sptr)

    def decode():
        nat.qtcq_decode(bits.data_ptr(), B, T, L, K, nat.QTCQ_CODE_1MAD, recon.data_ptr(),
                        seq.data_ptr(), None, mse_rt.data_ptr(), sptr)

    if args.calib_copy:
        # a plain elementwise copy of known size: 1 GiB read + 1 GiB written
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)     # an elementwise kernel, not a DMA blit
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        encode()
        decode()
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1, e2 in ev:
        e0.record(stream)
        encode()
        e1.record(stream)
        decode()
        e2.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_ms = [a.elapsed_time(b) for a, b, _ in ev]
    dec_ms = [b.elapsed_time(c) for _, b, c in ev]
    ms_per_step = wall * 1000.0 / args.steps
    print("[bench] timed %d steps: %.2f ms/step (encode %.2f ms, decode %.3f ms)"
          % (args.steps, ms_per_step, float(np.mean(enc_ms)), float(np.mean(dec_ms))),
          file=sys.stderr, flush=True)
    if not torch.equal(mse, mse_rt):
        print("[bench] WARNING: decoded MSE differs from the encoder's", file=sys.stderr)

    weights_per_step = B * T
    value = weights_per_step / (ms_per_step / 1000.0)
    enc_s = float(np.mean(enc_ms)) / 1000.0
    ops = acs_ops_per_sequence(T) * B
    achieved_tops = ops / enc_s / 1e12
    dec_s = float(np.mean(dec_ms)) / 1000.0
    # decode (one fused kernel): read 17 stream words and 256 targets, write 256
    # reconstructed weights and the MSE, per sequence
    dec_bytes = B * (W * 4 + T * 4 + T * 4 + 4)

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "viterbi_forward_traffic.json")
    if os.path.exists(tpath):
        try:
            traffic = json.load(open(tpath)).get("bytes_per_launch")
        except Exception:
            traffic = None

    out = {
        "metric": "trellis-encoded weights/s (L=16,k=2, 1 GPU); % of VALU peak; HBM GB/s",
        "value": value,
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "viterbi encode + window decode, 4096x4096 matrix = 65536 "
                               "sequences x T=256, N(0,1) seed 2, L=16 k=2, 1MAD, plain trellis",
                   "sequences": B, "T": T, "L": L, "k": K, "code": "1mad"},
        "seq_per_s": B / (ms_per_step / 1000.0),
        "encode_ms": float(np.mean(enc_ms)),
        "decode_ms": float(np.mean(dec_ms)),
        "roofline": {
            "bound": "alu",
            "kernel": "viterbi_forward<16,1MAD> (event-timed with its traceback launch)",
            "achieved": achieved_tops,
            "peak": PEAK_VALU_TOPS,
            "unit": "Top/s",
            "frac": achieved_tops / PEAK_VALU_TOPS,
            "traffic": traffic,
        },
        "decode": {"bound": "hbm", "achieved": dec_bytes / dec_s / 1e9, "peak": PEAK_HBM_GBS,
                   "unit": "GB/s", "frac": dec_bytes / dec_s / 1e9 / PEAK_HBM_GBS},
        "mse_mean": float(mse.mean().item()),
    }
    del ws

    if not args.no_matvec and B == 65536:
        # decode -> matrix-vector product straight from the streams just encoded (the
        # 4096x4096 matrix as 16x16 tiles), and from 4096x14336 (3INST) and 28672x8192
        # (1MAD) matrices of tail-biting streams (random words: every bit pattern is a
        # stream; the rate does not depend on the content).  Per launch, back to back, through
        # the C entry point with preallocated outputs (the smallest shape is near the host's
        # launch rate).
        mv = {}
        cases = [("4096x4096 1MAD plain (the encoded matrix)", bits, 4096, 4096, "1mad", False)]
        g = np.random.default_rng(13)
        tbw = api.tailbiting_words(L, K, T)
        rand_bits = torch.from_numpy(g.integers(0, 1 << 32, size=(256 * 896, tbw), dtype=np.uint32)
                                     .view(np.int32)).to(dev)
        cases.append(("4096x14336 3INST tail-biting", rand_bits, 4096, 14336, "3inst", True))
        big_bits = torch.from_numpy(g.integers(0, 1 << 32, size=(1792 * 512, tbw), dtype=np.uint32)
                                    .view(np.int32)).to(dev)
        cases.append(("28672x8192 1MAD tail-biting", big_bits, 28672, 8192, "1mad", True))
        # Each shape is timed through both entry points: the fp32 VALU product
        # (qtcq_decode_matvec) and the matrix-core product (qtcq_decode_matvec_mfma, its
        # split of x included, workspace preallocated).
        reps = max(1, args.matvec_reps)
        for label, bb, M_, N_, cd, tbf in cases:
            mws = api.matvec_mfma_workspace(N_)
            for nb in (1, 8, 32):
                xv = torch.from_numpy(g.standard_normal((nb, N_), dtype=np.float32)).to(dev)
                yv = api.decode_matvec_mfma(bb, M_, N_, xv, code=cd, tailbiting=tbf, workspace=mws)
                if nb <= 8:
                    api.decode_matvec(bb, M_, N_, xv, code=cd, tailbiting=tbf)   # checks shapes
                codei = nat.QTCQ_CODE_1MAD if cd == "1mad" else nat.QTCQ_CODE_3INST
                args_ = (bb.data_ptr(), M_, N_, L, K, codei, tbf, xv.data_ptr(), nb, yv.data_ptr())
                calls = [(", mfma", lambda: nat.qtcq_decode_matvec_mfma(
                    *args_, mws.data_ptr(), mws.numel(), sptr))]
                if nb <= 8:      # the fp32 VALU product takes at most 8 rows
                    calls.insert(0, ("", lambda: nat.qtcq_decode_matvec(*args_, sptr)))
                for kind, call in calls:
                    for _ in range(reps):      # untimed: the clocks settle under the load
                        call()
                    torch.cuda.synchronize()
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for _ in range(reps):
                        call()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    sec = e0.elapsed_time(e1) / 1000.0 / reps
                    nbytes = bb.numel() * 4 + nb * (N_ + M_) * 4
                    mv["%s, batch %d%s" % (label, nb, kind)] = {
                        "us": sec * 1e6, "weights_per_s": M_ * N_ / sec,
                        "hbm_gbs": nbytes / sec / 1e9, "hbm_frac": nbytes / sec / 1e9 / PEAK_HBM_GBS}
            del mws
        out["decode_matvec"] = mv
        print("[bench] decode matvec " + ", ".join("%.1f us" % v["us"] for v in mv.values()),
              file=sys.stderr, flush=True)
        del rand_bits, big_bits

    if not args.no_tb:
        # tail-biting encode of the same matrix: two forward searches per sequence
        tname = "tb4096x4096_1mad"
        st_host, _, _ = inputs.workload(tname, B=args.seqs or None)
        stb = torch.from_numpy(st_host).to(dev)
        Bt = stb.shape[0]
        tws = api.tailbiting_workspace(Bt, T, L, K, max_bytes=64 << 30)
        tbits = torch.empty((Bt, api.tailbiting_words(L, K, T)), dtype=torch.int32, device=dev)
        tmse = torch.empty(Bt, dtype=torch.float32, device=dev)

        def tb_encode():
            nat.qtcq_tailbiting_encode(stb.data_ptr(), None, Bt, T, L, K, nat.QTCQ_CODE_1MAD,
                                       tbits.data_ptr(), tmse.data_ptr(), None, tws.data_ptr(),
                                       tws.numel(), sptr)
        tb_encode()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 2
        e0.record(stream)
        for _ in range(reps):
            tb_encode()
        e1.record(stream)
        torch.cuda.synchronize()
        tsec = e0.elapsed_time(e1) / 1000.0 / reps
        tops = 2 * acs_ops_per_sequence(T) * Bt / tsec / 1e12
        out["tailbiting"] = {"workload": "tail-biting encode (two searches), 4096x4096 = %d "
                                         "sequences x T=256, N(0,1) seed 6, L=16, 1MAD" % Bt,
                             "ms": tsec * 1000.0, "weights_per_s": Bt * T / tsec,
                             "mse_mean": float(tmse.mean().item()),
                             "achieved": tops, "unit": "Top/s", "frac": tops / PEAK_VALU_TOPS}
        print("[bench] tail-biting %.2f ms" % (tsec * 1000.0), file=sys.stderr, flush=True)
        del tws

    if not args.no_xor and not args.seqs:
        # the XOR-Trellis palette code (the workload's four 14-bit parity masks): encode
        # and decode of a 4096x4096 matrix, targets N(0,1) times the palettes' RMS (seed
        # 8), and y = W x on a 28672x8192 tail-biting matrix of random streams (both
        # products at batch 1 and 8, the matrix-core product also at 32)
        xc = nat.qtcq_xor_code(*inputs.xor_masks(L))
        sx = torch.from_numpy(inputs.xor_targets(65536, T, 8)).to(dev)
        Bx = sx.shape[0]
        xws = api.encode_workspace(Bx, T, L, K, max_bytes=64 << 30)
        xbits = torch.empty((Bx, W), dtype=torch.int32, device=dev)
        xmse = torch.empty(Bx, dtype=torch.float32, device=dev)
        xrec = torch.empty((Bx, T), dtype=torch.float32, device=dev)
        xmse2 = torch.empty(Bx, dtype=torch.float32, device=dev)

        def x_enc():
            nat.qtcq_viterbi_encode(sx.data_ptr(), None, Bx, T, L, K, xc, xbits.data_ptr(),
                                    xmse.data_ptr(), None, xws.data_ptr(), xws.numel(), sptr)

        def x_dec():
            nat.qtcq_decode(xbits.data_ptr(), Bx, T, L, K, xc, xrec.data_ptr(), sx.data_ptr(),
                            None, xmse2.data_ptr(), sptr)

        def ev_time(fn, reps):
            for _ in range(reps):      # untimed: the clocks settle under the load
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 1000.0 / reps

        xesec = ev_time(x_enc, 2)
        xdsec = ev_time(x_dec, 20)
        xo = {"workload": "XOR palette code, 4096x4096 = %d sequences x T=256, N(0,1) x %.4f "
                          "seed 8, L=16, masks %s" % (Bx, inputs.XOR_TARGET_SCALE,
                                                      [hex(m) for m in inputs.xor_masks(L)]),
              "encode_ms": xesec * 1e3, "decode_ms": xdsec * 1e3,
              "encode_valu_frac": acs_ops_per_sequence(T) * Bx / xesec / 1e12 / PEAK_VALU_TOPS,
              "mse_mean": float(xmse.mean().item()),
              "decoded_mse_equal": bool(torch.equal(xmse, xmse2))}
        del xws, xbits, xrec, sx
        if not args.no_matvec:
            g2 = np.random.default_rng(14)
            Mx, Nx = 28672, 8192
            xb = torch.from_numpy(g2.integers(0, 1 << 32, size=((Mx // 16) * (Nx // 16), 16),
                                              dtype=np.uint32).view(np.int32)).to(dev)
            mws = api.matvec_mfma_workspace(Nx)
            for nb in (1, 8, 32):
                xv = torch.from_numpy(g2.standard_normal((nb, Nx), dtype=np.float32)).to(dev)
                yv = torch.empty((nb, Mx), dtype=torch.float32, device=dev)
                a_ = (xb.data_ptr(), Mx, Nx, L, K, xc, True, xv.data_ptr(), nb, yv.data_ptr())
                if nb <= 8:      # the fp32 VALU product takes at most 8 rows
                    t1 = ev_time(lambda: nat.qtcq_decode_matvec(*a_, sptr), max(1, args.matvec_reps))
                    xo["matvec 28672x8192 tail-biting, batch %d" % nb] = {"us": t1 * 1e6,
                                                                          "weights_per_s": Mx * Nx / t1}
                # the matrix-core product decodes this code through its LDS code table
                t2 = ev_time(lambda: nat.qtcq_decode_matvec_mfma(*a_, mws.data_ptr(), mws.numel(), sptr),
                             max(1, args.matvec_reps))
                xo["matvec 28672x8192 tail-biting, batch %d, mfma" % nb] = {"us": t2 * 1e6,
                                                                            "weights_per_s": Mx * Nx / t2}
            del xb, mws
        out["xor"] = xo
        print("[bench] xor encode %.2f ms, decode %.3f ms" % (xesec * 1e3, xdsec * 1e3),
              file=sys.stderr, flush=True)

    if not args.no_bcjr:
        bname = "bcjr4096x4096_1mad"
        sb_host, _, _ = inputs.workload(bname, B=args.bcjr_seqs or None)
        sb = torch.from_numpy(sb_host).to(dev)
        bws = api.bcjr_workspace(sb.shape[0], T, L, K)
        api.bcjr_soft(sb[:256], 0.1, workspace=bws)      # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        soft, logz = api.bcjr_soft(sb, 0.1, workspace=bws)
        e1.record(stream)
        torch.cuda.synchronize()
        bsec = e0.elapsed_time(e1) / 1000.0
        nb_ = sb.shape[0]
        sops, stransc = bcjr_soft_ops(T, L)
        out["bcjr"] = {"workload": "%d sequences x T=256, N(0,1) seed 5, L=16, 1MAD, tau=0.1"
                                   % nb_,
                       "seconds": bsec, "seq_per_s": nb_ / bsec,
                       "weights_per_s": nb_ * T / bsec,
                       "ops_per_seq": sops,
                       "roofline": roofline_alu(sops * nb_, stransc * nb_, bsec,
                                                bcjr_stash_bytes(T, L) * nb_)}
        print("[bench] bcjr %.3f s" % bsec, file=sys.stderr, flush=True)
        del bws, soft, logz

        # gradient of the soft codeword (soft pass in VJP mode + expectation messages)
        g = torch.from_numpy(np.random.default_rng(9).standard_normal(sb.shape, dtype=np.float32)).to(dev)
        vws = api.bcjr_vjp_workspace(sb.shape[0], T, L, K)
        api.bcjr_vjp(sb[:256], 0.1, g[:256], workspace=vws)      # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        grad, _, _ = api.bcjr_vjp(sb, 0.1, g, workspace=vws)
        e1.record(stream)
        torch.cuda.synchronize()
        vsec = e0.elapsed_time(e1) / 1000.0
        gops, gtransc = bcjr_grad_ops(T, L)
        vops, vtransc = sops + gops, stransc + gtransc
        out["bcjr_vjp"] = {"workload": "gradient of the soft codeword w.r.t. the targets, "
                                       "%d sequences x T=256, N(0,1) seed 5, upstream "
                                       "N(0,1) seed 9, L=16, 1MAD, tau=0.1" % nb_,
                           "seconds": vsec, "seq_per_s": nb_ / vsec,
                           "ops_per_seq": vops,
                           "roofline": roofline_alu(vops * nb_, vtransc * nb_, vsec,
                                                    bcjr_stash_bytes(T, L, True) * nb_),
                           "finite": bool(torch.isfinite(grad).all().item())}
        print("[bench] bcjr vjp %.3f s" % vsec, file=sys.stderr, flush=True)
        del vws, grad, g

    if not args.no_configs and not args.seqs:
        # the other configurations of the path, one timed call each after a warm-up:
        # encode (+ decode with the round-trip MSE) of 16 sequences, of the 4096x14336
        # matrix in 3INST and of the weighted 4096x4096 matrix; the BCJR soft pass of the
        # 4096x4096 matrix at each temperature
        cfg = {}

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            r = fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 1000.0, r

        for wname in ("enc16_1mad", "enc4096x14336_3inst", "enc4096x4096_1mad_weighted"):
            sh, wh, cd = inputs.workload(wname)
            sd = torch.from_numpy(sh).to(dev)
            wd = None if wh is None else torch.from_numpy(wh).to(dev)
            Bc = sd.shape[0]
            cws = api.encode_workspace(Bc, T, L, K)
            esec, (cb, cm, _) = timed(lambda: api.encode(sd, wd, L=L, k=K, code=cd, workspace=cws))
            dsec, (_, cm2) = timed(lambda: api.decode(cb, T, L=L, k=K, code=cd, seq=sd, weights=wd,
                                                      want_mse=True))
            ops = (acs_ops_per_sequence(T, wd is not None)) * Bc
            cfg[wname] = {"sequences": Bc, "code": cd, "weighted": wd is not None,
                          "encode_ms": esec * 1e3, "decode_ms": dsec * 1e3,
                          "weights_per_s": Bc * T / (esec + dsec),
                          "encode_valu_frac": ops / esec / 1e12 / PEAK_VALU_TOPS,
                          "mse_mean": float(cm.mean().item()),
                          "decoded_mse_equal": bool(torch.equal(cm, cm2))}
            del sd, wd, cws, cb, cm, cm2
        sh, _, _ = inputs.workload("bcjr4096x4096_1mad")
        sd = torch.from_numpy(sh).to(dev)
        bws = api.bcjr_workspace(sd.shape[0], T, L, K)
        sops, stransc = bcjr_soft_ops(T, L)
        for tau in (1.0, 0.1, 0.01):
            bsec, (bsoft, _) = timed(lambda: api.bcjr_soft(sd, tau, workspace=bws))
            cfg["bcjr4096x4096_1mad tau=%g" % tau] = {
                "sequences": sd.shape[0], "seconds": bsec, "seq_per_s": sd.shape[0] / bsec,
                "valu_frac": sops * sd.shape[0] / bsec / 1e12 / PEAK_VALU_TOPS,
                "finite": bool(torch.isfinite(bsoft).all().item())}
        del sd, bws
        out["configs"] = cfg
        print("[bench] configs " + ", ".join("%s %.3g ms" % (k, v.get("encode_ms", v.get("seconds", 0) * 1e3))
                                             for k, v in cfg.items()), file=sys.stderr, flush=True)

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(args, s_host)

    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
