"""Torch-facing convenience layer over the C ABI: allocates outputs and workspaces as
CUDA (HIP) tensors and calls the entry points on the current stream.  Only argument
marshalling happens here; every step of the path runs in the HIP kernels.
"""
from __future__ import annotations

import torch

from . import _native as nat

CODES = {"1mad": nat.QTCQ_CODE_1MAD, "3inst": nat.QTCQ_CODE_3INST}


def xor_code(masks) -> int:
    """The XOR-Trellis palette code with parity masks (m0, m1, m2, m3): m0 and m1 pick the
    palette, m2 and m3 the branch shuffle; each an (L - 2)-bit history mask."""
    code = nat.qtcq_xor_code(*masks)
    if code == nat.QTCQ_CODE_INVALID:
        raise ValueError("XOR parity masks must fit in 14 bits")
    return code


def _code(code) -> int:
    """A code name ("1mad", "3inst"), ("xor", masks), or a qtcq_code descriptor."""
    if isinstance(code, str):
        return CODES[code]
    if isinstance(code, tuple) and len(code) == 2 and code[0] == "xor":
        return xor_code(code[1])
    return int(code)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _on_current_device(x: torch.Tensor, name: str) -> None:
    # the kernels run on the current device's current stream, and workspaces and outputs
    # are allocated there
    if x.device.index is not None and x.device.index != torch.cuda.current_device():
        raise ValueError("%s is on %s, not on the current device cuda:%d"
                         % (name, x.device, torch.cuda.current_device()))


def _dev_f32(x: torch.Tensor, name: str) -> torch.Tensor:
    if not (x.is_cuda and x.dtype == torch.float32 and x.is_contiguous() and x.dim() == 2):
        raise ValueError("%s must be a contiguous 2-D float32 device tensor" % name)
    _on_current_device(x, name)
    return x


def _dev_workspace(ws, name: str = "workspace") -> int:
    """A caller-supplied device scratch tensor: contiguous and on the current device (the
    kernels write through its pointer).  Returns its size in bytes, whatever its dtype."""
    if not (isinstance(ws, torch.Tensor) and ws.is_cuda and ws.is_contiguous()):
        raise ValueError("%s must be a contiguous device tensor" % name)
    _on_current_device(ws, name)
    return ws.numel() * ws.element_size()


def _like_seq(x: torch.Tensor | None, seq: torch.Tensor, name: str) -> None:
    """An optional per-weight tensor (error weights, upstream gradient) shaped as seq."""
    if x is not None:
        _dev_f32(x, name)
        if x.shape != seq.shape:
            raise ValueError("%s must have the shape of seq" % name)


def _dev_words(bits: torch.Tensor, B: int, W: int) -> None:
    """Streams as the kernels read them: B rows of W contiguous 32-bit words."""
    if not (bits.is_cuda and bits.is_contiguous() and bits.element_size() == 4
            and bits.dtype in (torch.int32, torch.uint32) and tuple(bits.shape) == (B, W)):
        raise ValueError("bits must be a contiguous [%d][%d] 32-bit device tensor" % (B, W))
    _on_current_device(bits, "bits")


def _decode_inputs(bits, T, W, seq, weights, want_mse):
    B = bits.shape[0]
    if W < 0:
        raise ValueError("unsupported (L, k, T)")
    _dev_words(bits, B, W)
    if seq is not None:
        _dev_f32(seq, "seq")
        if tuple(seq.shape) != (B, T):
            raise ValueError("seq must be [B][T]")
        _like_seq(weights, seq, "weights")
    elif want_mse or weights is not None:
        raise ValueError("the MSE needs seq (and weights only come with seq)")
    return B


def bitstream_words(L: int = 16, k: int = 2, T: int = 256) -> int:
    return nat.qtcq_bitstream_words(L, k, T)


def code_table(code="1mad", L: int = 16) -> torch.Tensor:
    out = torch.empty(1 << L, dtype=torch.float32, device="cuda")
    nat.qtcq_code_table(_code(code), L, out.data_ptr(), _stream())
    return out


# Default workspace caps: a chunk of sequences is one launch, so the cap bounds HBM use
# while keeping each launch many workgroups deep (the 4096x4096 encode fits one chunk).
ENCODE_WS_CAP = 64 << 30
BCJR_WS_CAP = 16 << 30
VJP_WS_CAP = 32 << 30


def _chunk_bytes(B: int, per: int, max_bytes: int | None, seqs_per_wg: int = 1) -> int:
    """Workspace bytes for min(B, what max_bytes holds) sequences of `per` bytes.  A
    partial batch is rounded down to whole multiples of the device's CU count times the
    sequences one workgroup takes (two in the search once a chunk exceeds the CU count),
    so that no launch ends with a partly empty round of workgroups."""
    if max_bytes is None or B * per <= max_bytes:
        return max(1, B) * per
    n = max(1, max_bytes // per)
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    if n > cus * seqs_per_wg:
        n = n // (cus * seqs_per_wg) * (cus * seqs_per_wg)
    elif n > cus:
        n = n // cus * cus
    return n * per


def encode_workspace(B: int, T: int = 256, L: int = 16, k: int = 2,
                     max_bytes: int | None = ENCODE_WS_CAP) -> torch.Tensor:
    per = nat.qtcq_encode_workspace_bytes(1, T, L, k)
    return torch.empty(_chunk_bytes(B, per, max_bytes, 2), dtype=torch.uint8, device="cuda")


def bcjr_workspace(B: int, T: int = 256, L: int = 16, k: int = 2,
                   max_bytes: int | None = BCJR_WS_CAP) -> torch.Tensor:
    per = nat.qtcq_bcjr_workspace_bytes(1, T, L, k)
    return torch.empty(_chunk_bytes(B, per, max_bytes), dtype=torch.uint8, device="cuda")


def encode(seq: torch.Tensor, weights: torch.Tensor | None = None, L: int = 16, k: int = 2,
           code="1mad", want_states: bool = False, workspace: torch.Tensor | None = None):
    """Viterbi-encode [B][T] targets.  Returns (bits [B][W] int32 view of uint32 words,
    mse [B] float32, states [B][T] int32 view of uint32 or None)."""
    _dev_f32(seq, "seq")
    B, T = seq.shape
    _like_seq(weights, seq, "weights")
    W = nat.qtcq_bitstream_words(L, k, T)
    bits = torch.empty((B, W), dtype=torch.int32, device=seq.device)
    mse = torch.empty(B, dtype=torch.float32, device=seq.device)
    states = torch.empty((B, T), dtype=torch.int32, device=seq.device) if want_states else None
    if workspace is None:
        workspace = encode_workspace(B, T, L, k)
    ws_bytes = _dev_workspace(workspace)
    nat.qtcq_viterbi_encode(seq.data_ptr(), None if weights is None else weights.data_ptr(), B, T,
                            L, k, _code(code), bits.data_ptr(), mse.data_ptr(),
                            None if states is None else states.data_ptr(), workspace.data_ptr(),
                            ws_bytes, _stream())
    return bits, mse, states


def decode(bits: torch.Tensor, T: int, L: int = 16, k: int = 2, code="1mad",
           seq: torch.Tensor | None = None, weights: torch.Tensor | None = None,
           want_recon: bool = True, want_mse: bool = False):
    """Window-decode [B][W] streams.  Returns (recon [B][T] or None, mse [B] or None)."""
    B = _decode_inputs(bits, T, nat.qtcq_bitstream_words(L, k, T), seq, weights, want_mse)
    recon = torch.empty((B, T), dtype=torch.float32, device=bits.device) if want_recon else None
    mse = torch.empty(B, dtype=torch.float32, device=bits.device) if want_mse else None
    nat.qtcq_decode(bits.data_ptr(), B, T, L, k, _code(code),
                    None if recon is None else recon.data_ptr(),
                    None if seq is None else seq.data_ptr(),
                    None if weights is None else weights.data_ptr(),
                    None if mse is None else mse.data_ptr(), _stream())
    return recon, mse


def bcjr_soft(seq: torch.Tensor, temperature: float, weights: torch.Tensor | None = None,
              L: int = 16, k: int = 2, code="1mad", workspace: torch.Tensor | None = None):
    """BCJR soft codewords.  Returns (soft [B][T] float32, log_z [B] float32)."""
    _dev_f32(seq, "seq")
    _like_seq(weights, seq, "weights")
    B, T = seq.shape
    soft = torch.empty((B, T), dtype=torch.float32, device=seq.device)
    logz = torch.empty(B, dtype=torch.float32, device=seq.device)
    if workspace is None:
        workspace = bcjr_workspace(B, T, L, k)
    ws_bytes = _dev_workspace(workspace)
    nat.qtcq_bcjr_soft(seq.data_ptr(), None if weights is None else weights.data_ptr(), B, T, L, k,
                       _code(code), temperature, soft.data_ptr(), logz.data_ptr(),
                       workspace.data_ptr(), ws_bytes, _stream())
    return soft, logz


def bcjr_vjp_workspace(B: int, T: int = 256, L: int = 16, k: int = 2,
                       max_bytes: int | None = VJP_WS_CAP) -> torch.Tensor:
    per = nat.qtcq_bcjr_vjp_workspace_bytes(1, T, L, k)
    return torch.empty(_chunk_bytes(B, per, max_bytes), dtype=torch.uint8, device="cuda")


def bcjr_vjp(seq: torch.Tensor, temperature: float, grad_soft: torch.Tensor,
             weights: torch.Tensor | None = None, L: int = 16, k: int = 2, code="1mad",
             want_soft: bool = False, workspace: torch.Tensor | None = None):
    """Gradient of sum_t grad_soft[b][t] * soft[b][t] with respect to seq.  Returns
    (grad_seq [B][T] float32, soft [B][T] or None, log_z [B] or None)."""
    _dev_f32(seq, "seq")
    _like_seq(grad_soft, seq, "grad_soft")
    _like_seq(weights, seq, "weights")
    B, T = seq.shape
    grad = torch.empty((B, T), dtype=torch.float32, device=seq.device)
    soft = torch.empty((B, T), dtype=torch.float32, device=seq.device) if want_soft else None
    logz = torch.empty(B, dtype=torch.float32, device=seq.device) if want_soft else None
    if workspace is None:
        workspace = bcjr_vjp_workspace(B, T, L, k)
    ws_bytes = _dev_workspace(workspace)
    nat.qtcq_bcjr_vjp(seq.data_ptr(), None if weights is None else weights.data_ptr(), B, T, L, k,
                      _code(code), temperature, grad_soft.data_ptr(), grad.data_ptr(),
                      None if soft is None else soft.data_ptr(),
                      None if logz is None else logz.data_ptr(), workspace.data_ptr(),
                      ws_bytes, _stream())
    return grad, soft, logz


def tailbiting_words(L: int = 16, k: int = 2, T: int = 256) -> int:
    return nat.qtcq_tailbiting_words(L, k, T)


def tailbiting_workspace(B: int, T: int = 256, L: int = 16, k: int = 2,
                         max_bytes: int | None = ENCODE_WS_CAP) -> torch.Tensor:
    per = nat.qtcq_tailbiting_workspace_bytes(1, T, L, k)
    return torch.empty(_chunk_bytes(B, per, max_bytes, 2), dtype=torch.uint8, device="cuda")


def tailbiting_encode(seq: torch.Tensor, weights: torch.Tensor | None = None, L: int = 16,
                      k: int = 2, code="1mad", want_states: bool = False,
                      workspace: torch.Tensor | None = None):
    """Tail-biting encode (two searches per sequence) of [B][T] targets.  Returns
    (bits [B][ceil(kT/32)] int32 view of uint32 words, mse [B], states [B][T] or None)."""
    _dev_f32(seq, "seq")
    B, T = seq.shape
    _like_seq(weights, seq, "weights")
    W = nat.qtcq_tailbiting_words(L, k, T)
    if W < 0:
        raise ValueError("tail-biting needs k*T >= L")
    bits = torch.empty((B, W), dtype=torch.int32, device=seq.device)
    mse = torch.empty(B, dtype=torch.float32, device=seq.device)
    states = torch.empty((B, T), dtype=torch.int32, device=seq.device) if want_states else None
    if workspace is None:
        workspace = tailbiting_workspace(B, T, L, k)
    ws_bytes = _dev_workspace(workspace)
    nat.qtcq_tailbiting_encode(seq.data_ptr(), None if weights is None else weights.data_ptr(), B,
                               T, L, k, _code(code), bits.data_ptr(), mse.data_ptr(),
                               None if states is None else states.data_ptr(),
                               workspace.data_ptr(), ws_bytes, _stream())
    return bits, mse, states


def tailbiting_decode(bits: torch.Tensor, T: int, L: int = 16, k: int = 2, code="1mad",
                      seq: torch.Tensor | None = None, weights: torch.Tensor | None = None,
                      want_recon: bool = True, want_mse: bool = False):
    """Cyclic window decode of [B][W] tail-biting streams.  Returns (recon or None,
    mse or None)."""
    B = _decode_inputs(bits, T, nat.qtcq_tailbiting_words(L, k, T), seq, weights, want_mse)
    recon = torch.empty((B, T), dtype=torch.float32, device=bits.device) if want_recon else None
    mse = torch.empty(B, dtype=torch.float32, device=bits.device) if want_mse else None
    nat.qtcq_tailbiting_decode(bits.data_ptr(), B, T, L, k, _code(code),
                               None if recon is None else recon.data_ptr(),
                               None if seq is None else seq.data_ptr(),
                               None if weights is None else weights.data_ptr(),
                               None if mse is None else mse.data_ptr(), _stream())
    return recon, mse


def decode_matvec(bits: torch.Tensor, M: int, N: int, x: torch.Tensor, L: int = 16, k: int = 2,
                  code="1mad", tailbiting: bool = False) -> torch.Tensor:
    """y [batch][M] = W x for the M x N matrix whose row-major 16x16 tiles are the
    T = 256 streams `bits` ([(M/16)(N/16)][W]); x [batch][N] (or [N]) float32 on device."""
    one = x.dim() == 1
    x2 = x.reshape(1, -1) if one else x
    _dev_f32(x2, "x")
    if x2.shape[1] != N:
        raise ValueError("x must have N columns")
    W = tailbiting_words(L, k, 256) if tailbiting else bitstream_words(L, k, 256)
    if not (bits.is_cuda and bits.is_contiguous() and bits.element_size() == 4
            and bits.numel() == (M // 16) * (N // 16) * W):
        raise ValueError("bits must hold (M/16)*(N/16) contiguous streams of %d words" % W)
    _on_current_device(bits, "bits")
    y = torch.empty((x2.shape[0], M), dtype=torch.float32, device=x.device)
    nat.qtcq_decode_matvec(bits.data_ptr(), M, N, L, k, _code(code), tailbiting, x2.data_ptr(),
                           x2.shape[0], y.data_ptr(), _stream())
    return y[0] if one else y


def matvec_mfma_workspace(N: int) -> torch.Tensor:
    """Device scratch for decode_matvec_mfma over N columns (reusable across calls on one
    stream)."""
    n = nat.qtcq_decode_matvec_mfma_workspace_bytes(N)
    if n == 0:
        raise ValueError("N must be a multiple of 16 in [0, 2^22]")
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def decode_matvec_mfma(bits: torch.Tensor, M: int, N: int, x: torch.Tensor, L: int = 16,
                       k: int = 2, code="1mad", tailbiting: bool = False,
                       workspace: torch.Tensor | None = None) -> torch.Tensor:
    """decode_matvec with the products on the matrix cores: the code values (exact in fp16)
    times x split per 32-column block into two scaled fp16 parts.  Same arguments and
    result layout, with up to 32 rows of x; `workspace` (matvec_mfma_workspace(N)) is
    allocated when not given."""
    one = x.dim() == 1
    x2 = x.reshape(1, -1) if one else x
    _dev_f32(x2, "x")
    if x2.shape[1] != N:
        raise ValueError("x must have N columns")
    W = tailbiting_words(L, k, 256) if tailbiting else bitstream_words(L, k, 256)
    if not (bits.is_cuda and bits.is_contiguous() and bits.element_size() == 4
            and bits.numel() == (M // 16) * (N // 16) * W):
        raise ValueError("bits must hold (M/16)*(N/16) contiguous streams of %d words" % W)
    _on_current_device(bits, "bits")
    if workspace is None:
        workspace = matvec_mfma_workspace(N)
    ws_bytes = _dev_workspace(workspace)
    y = torch.empty((x2.shape[0], M), dtype=torch.float32, device=x.device)
    nat.qtcq_decode_matvec_mfma(bits.data_ptr(), M, N, L, k, _code(code), tailbiting,
                                x2.data_ptr(), x2.shape[0], y.data_ptr(), workspace.data_ptr(),
                                ws_bytes, _stream())
    return y[0] if one else y


class SplitX:
    """The split of x made by matvec_mfma_split_x: the device workspace holding it and the
    (N, batch) it was made for.  The product reads the fragments and block scales at
    offsets that depend on both, so decode_matvec_mfma_presplit checks them."""
    __slots__ = ("workspace", "N", "batch")

    def __init__(self, workspace: torch.Tensor, N: int, batch: int):
        self.workspace, self.N, self.batch = workspace, N, batch


def matvec_mfma_split_x(x: torch.Tensor, workspace: torch.Tensor | None = None) -> SplitX:
    """The split of x [batch][N] (or [N]) for decode_matvec_mfma_presplit, written into
    `workspace` (matvec_mfma_workspace(N), allocated when not given)."""
    x2 = x.reshape(1, -1) if x.dim() == 1 else x
    _dev_f32(x2, "x")
    N = x2.shape[1]
    if workspace is None:
        workspace = matvec_mfma_workspace(N)
    ws_bytes = _dev_workspace(workspace)
    nat.qtcq_matvec_mfma_split_x(x2.data_ptr(), N, x2.shape[0], workspace.data_ptr(), ws_bytes,
                                 _stream())
    return SplitX(workspace, N, x2.shape[0])


def decode_matvec_mfma_presplit(bits: torch.Tensor, M: int, N: int, split: SplitX,
                                L: int = 16, k: int = 2, code="1mad",
                                tailbiting: bool = False) -> torch.Tensor:
    """y [split.batch][M] = W x from a split made by matvec_mfma_split_x for this N (equal to
    decode_matvec_mfma bit for bit)."""
    if not isinstance(split, SplitX):
        raise ValueError("split must be the SplitX that matvec_mfma_split_x returned")
    if split.N != N:
        raise ValueError("split was made for N = %d, not %d" % (split.N, N))
    W = tailbiting_words(L, k, 256) if tailbiting else bitstream_words(L, k, 256)
    if not (bits.is_cuda and bits.is_contiguous() and bits.element_size() == 4
            and bits.numel() == (M // 16) * (N // 16) * W):
        raise ValueError("bits must hold (M/16)*(N/16) contiguous streams of %d words" % W)
    _on_current_device(bits, "bits")
    sp_bytes = _dev_workspace(split.workspace, "split")
    y = torch.empty((split.batch, M), dtype=torch.float32, device=bits.device)
    nat.qtcq_decode_matvec_mfma_presplit(bits.data_ptr(), M, N, L, k, _code(code), tailbiting,
                                         split.workspace.data_ptr(), sp_bytes, split.batch,
                                         y.data_ptr(), _stream())
    return y


def decode_matvec_mfma_noalloc(bits: torch.Tensor, M: int, N: int, x: torch.Tensor,
                               out: torch.Tensor, L: int = 16, k: int = 2, code="1mad",
                               tailbiting: bool = False) -> torch.Tensor:
    """decode_matvec_mfma with the split x in the library's per-device scratch array: no
    workspace, and nothing allocated here either -- the caller passes the output `out`
    ([batch][M] float32, or [M] for a 1-D x).  Calls that overlap on one GPU race."""
    one = x.dim() == 1
    x2 = x.reshape(1, -1) if one else x
    _dev_f32(x2, "x")
    if x2.shape[1] != N:
        raise ValueError("x must have N columns")
    W = tailbiting_words(L, k, 256) if tailbiting else bitstream_words(L, k, 256)
    if not (bits.is_cuda and bits.is_contiguous() and bits.element_size() == 4
            and bits.numel() == (M // 16) * (N // 16) * W):
        raise ValueError("bits must hold (M/16)*(N/16) contiguous streams of %d words" % W)
    _on_current_device(bits, "bits")
    o2 = out.reshape(1, -1) if one else out
    _dev_f32(o2, "out")
    if tuple(o2.shape) != (x2.shape[0], M):
        raise ValueError("out must be [batch][M]")
    nat.qtcq_decode_matvec_mfma_noalloc(bits.data_ptr(), M, N, L, k, _code(code), tailbiting,
                                        x2.data_ptr(), x2.shape[0], o2.data_ptr(), _stream())
    return out
