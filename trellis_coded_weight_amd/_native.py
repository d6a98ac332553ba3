"""ctypes binding of the C ABI in include/qtcq.h -- argument marshalling only.

Every function here has the name of the C entry point it calls and takes the same
arguments, with device pointers passed as Python ints (e.g. ``tensor.data_ptr()``)
and the stream as an int handle (``torch.cuda.current_stream().cuda_stream``) or 0.
A non-OK status raises :class:`QtcqError`.  The library must have been built
(``trellis_coded_weight_amd.build.build_native()``); if it is missing this module
raises at import time -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqtcq.so")

QTCQ_OK = 0
QTCQ_ERR_INVALID_ARG = 1
QTCQ_ERR_UNSUPPORTED = 2
QTCQ_ERR_WORKSPACE = 3
QTCQ_ERR_DEVICE = 4

QTCQ_CODE_1MAD = 0
QTCQ_CODE_3INST = 1
QTCQ_CODE_XOR = 2
QTCQ_CODE_INVALID = 0xFF


class QtcqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (where, qtcq_status_string(status), status))


if not os.path.exists(LIB_PATH):
    raise ImportError("libqtcq.so is not built (expected at %s); run "
                      "trellis_coded_weight_amd.build.build_native()" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t
_code = ctypes.c_uint64   # qtcq_code descriptor

_SIGS = {
    "qtcq_status_string": (ctypes.c_char_p, [_int]),
    "qtcq_bitstream_words": (_i64, [_int, _int, _int]),
    "qtcq_encode_workspace_bytes": (_sz, [_i64, _int, _int, _int]),
    "qtcq_bcjr_workspace_bytes": (_sz, [_i64, _int, _int, _int]),
    "qtcq_xor_code": (_code, [ctypes.c_uint32] * 4),
    "qtcq_code_table": (_int, [_code, _int, _vp, _vp]),
    "qtcq_viterbi_encode": (_int, [_vp, _vp, _i64, _int, _int, _int, _code, _vp, _vp, _vp, _vp,
                                   _sz, _vp]),
    "qtcq_decode": (_int, [_vp, _i64, _int, _int, _int, _code, _vp, _vp, _vp, _vp, _vp]),
    "qtcq_bcjr_soft": (_int, [_vp, _vp, _i64, _int, _int, _int, _code, ctypes.c_float, _vp, _vp,
                              _vp, _sz, _vp]),
    "qtcq_bcjr_vjp_workspace_bytes": (_sz, [_i64, _int, _int, _int]),
    "qtcq_bcjr_vjp": (_int, [_vp, _vp, _i64, _int, _int, _int, _code, ctypes.c_float, _vp, _vp, _vp,
                             _vp, _vp, _sz, _vp]),
    "qtcq_decode_matvec": (_int, [_vp, _int, _int, _int, _int, _code, _int, _vp, _int, _vp, _vp]),
    "qtcq_decode_matvec_mfma_workspace_bytes": (_sz, [_int]),
    "qtcq_decode_matvec_mfma": (_int, [_vp, _int, _int, _int, _int, _code, _int, _vp, _int, _vp,
                                       _vp, _sz, _vp]),
    "qtcq_matvec_mfma_split_x": (_int, [_vp, _int, _int, _vp, _sz, _vp]),
    "qtcq_decode_matvec_mfma_noalloc": (_int, [_vp, _int, _int, _int, _int, _code, _int, _vp,
                                               _int, _vp, _vp]),
    "qtcq_decode_matvec_mfma_presplit": (_int, [_vp, _int, _int, _int, _int, _code, _int, _vp,
                                                _sz, _int, _vp, _vp]),
    "qtcq_tailbiting_words": (_i64, [_int, _int, _int]),
    "qtcq_tailbiting_workspace_bytes": (_sz, [_i64, _int, _int, _int]),
    "qtcq_tailbiting_encode": (_int, [_vp, _vp, _i64, _int, _int, _int, _code, _vp, _vp, _vp,
                                      _vp, _sz, _vp]),
    "qtcq_tailbiting_decode": (_int, [_vp, _i64, _int, _int, _int, _code, _vp, _vp, _vp, _vp,
                                      _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


def _ptr(p):
    return None if (p is None or p == 0) else ctypes.c_void_p(int(p))


def _check(status: int, where: str) -> None:
    if status != QTCQ_OK:
        raise QtcqError(status, where)


def qtcq_xor_code(m0: int, m1: int, m2: int, m3: int) -> int:
    """The qtcq_code descriptor of the XOR palette code with parity masks m0..m3
    (QTCQ_CODE_INVALID if a mask exceeds 14 bits)."""
    ms = [int(m) for m in (m0, m1, m2, m3)]
    if any(m < 0 or m > 0xFFFFFFFF for m in ms):
        return QTCQ_CODE_INVALID
    return _lib.qtcq_xor_code(*ms)


def qtcq_status_string(status: int) -> str:
    return _lib.qtcq_status_string(status).decode()


def qtcq_bitstream_words(L: int, k: int, T: int) -> int:
    return _lib.qtcq_bitstream_words(L, k, T)


def qtcq_encode_workspace_bytes(B: int, T: int, L: int, k: int) -> int:
    return _lib.qtcq_encode_workspace_bytes(B, T, L, k)


def qtcq_bcjr_workspace_bytes(B: int, T: int, L: int, k: int) -> int:
    return _lib.qtcq_bcjr_workspace_bytes(B, T, L, k)


def qtcq_code_table(code: int, L: int, out: int, stream: int = 0) -> None:
    _check(_lib.qtcq_code_table(code, L, _ptr(out), _ptr(stream)), "qtcq_code_table")


def qtcq_viterbi_encode(seq: int, err_w, B: int, T: int, L: int, k: int, code: int, bits: int,
                        mse, states, workspace: int, workspace_bytes: int,
                        stream: int = 0) -> None:
    _check(_lib.qtcq_viterbi_encode(_ptr(seq), _ptr(err_w), B, T, L, k, code, _ptr(bits),
                                    _ptr(mse), _ptr(states), _ptr(workspace), workspace_bytes,
                                    _ptr(stream)), "qtcq_viterbi_encode")


def qtcq_decode(bits: int, B: int, T: int, L: int, k: int, code: int, recon, seq, err_w, mse,
                stream: int = 0) -> None:
    _check(_lib.qtcq_decode(_ptr(bits), B, T, L, k, code, _ptr(recon), _ptr(seq), _ptr(err_w),
                            _ptr(mse), _ptr(stream)), "qtcq_decode")


def qtcq_bcjr_soft(seq: int, err_w, B: int, T: int, L: int, k: int, code: int,
                   temperature: float, soft: int, log_z, workspace: int, workspace_bytes: int,
                   stream: int = 0) -> None:
    _check(_lib.qtcq_bcjr_soft(_ptr(seq), _ptr(err_w), B, T, L, k, code, float(temperature),
                               _ptr(soft), _ptr(log_z), _ptr(workspace), workspace_bytes,
                               _ptr(stream)), "qtcq_bcjr_soft")


def qtcq_bcjr_vjp_workspace_bytes(B: int, T: int, L: int, k: int) -> int:
    return _lib.qtcq_bcjr_vjp_workspace_bytes(B, T, L, k)


def qtcq_bcjr_vjp(seq: int, err_w, B: int, T: int, L: int, k: int, code: int,
                  temperature: float, grad_soft: int, grad_seq: int, soft, log_z, workspace: int,
                  workspace_bytes: int, stream: int = 0) -> None:
    _check(_lib.qtcq_bcjr_vjp(_ptr(seq), _ptr(err_w), B, T, L, k, code, float(temperature),
                              _ptr(grad_soft), _ptr(grad_seq), _ptr(soft), _ptr(log_z),
                              _ptr(workspace), workspace_bytes, _ptr(stream)), "qtcq_bcjr_vjp")


def qtcq_tailbiting_words(L: int, k: int, T: int) -> int:
    return _lib.qtcq_tailbiting_words(L, k, T)


def qtcq_tailbiting_workspace_bytes(B: int, T: int, L: int, k: int) -> int:
    return _lib.qtcq_tailbiting_workspace_bytes(B, T, L, k)


def qtcq_tailbiting_encode(seq: int, err_w, B: int, T: int, L: int, k: int, code: int,
                           bits: int, mse, states, workspace: int, workspace_bytes: int,
                           stream: int = 0) -> None:
    _check(_lib.qtcq_tailbiting_encode(_ptr(seq), _ptr(err_w), B, T, L, k, code, _ptr(bits),
                                       _ptr(mse), _ptr(states), _ptr(workspace), workspace_bytes,
                                       _ptr(stream)), "qtcq_tailbiting_encode")


def qtcq_tailbiting_decode(bits: int, B: int, T: int, L: int, k: int, code: int, recon, seq,
                           err_w, mse, stream: int = 0) -> None:
    _check(_lib.qtcq_tailbiting_decode(_ptr(bits), B, T, L, k, code, _ptr(recon), _ptr(seq),
                                       _ptr(err_w), _ptr(mse), _ptr(stream)),
           "qtcq_tailbiting_decode")


def raw_status(name: str, *args) -> int:
    """Call an entry point and return its status without raising (for argument-validation
    tests).  Pointer arguments are ints or None."""
    fn = getattr(_lib, name)
    conv = []
    for a, t in zip(args, _SIGS[name][1]):
        conv.append(_ptr(a) if t is _vp else a)
    return fn(*conv)


def qtcq_decode_matvec(bits: int, M: int, N: int, L: int, k: int, code: int, tailbiting: bool,
                       x: int, batch: int, y: int, stream: int = 0) -> None:
    _check(_lib.qtcq_decode_matvec(_ptr(bits), M, N, L, k, code, 1 if tailbiting else 0, _ptr(x),
                                   batch, _ptr(y), _ptr(stream)), "qtcq_decode_matvec")


def qtcq_decode_matvec_mfma_workspace_bytes(N: int) -> int:
    return _lib.qtcq_decode_matvec_mfma_workspace_bytes(N)


def qtcq_decode_matvec_mfma(bits: int, M: int, N: int, L: int, k: int, code: int,
                            tailbiting: bool, x: int, batch: int, y: int, workspace: int,
                            workspace_bytes: int, stream: int = 0) -> None:
    _check(_lib.qtcq_decode_matvec_mfma(_ptr(bits), M, N, L, k, code, 1 if tailbiting else 0,
                                        _ptr(x), batch, _ptr(y), _ptr(workspace),
                                        workspace_bytes, _ptr(stream)),
           "qtcq_decode_matvec_mfma")


def qtcq_matvec_mfma_split_x(x: int, N: int, batch: int, workspace: int, workspace_bytes: int,
                             stream: int = 0) -> None:
    _check(_lib.qtcq_matvec_mfma_split_x(_ptr(x), N, batch, _ptr(workspace), workspace_bytes,
                                         _ptr(stream)), "qtcq_matvec_mfma_split_x")


def qtcq_decode_matvec_mfma_presplit(bits: int, M: int, N: int, L: int, k: int, code: int,
                                     tailbiting: bool, split: int, split_bytes: int, batch: int,
                                     y: int, stream: int = 0) -> None:
    _check(_lib.qtcq_decode_matvec_mfma_presplit(_ptr(bits), M, N, L, k, code,
                                                 1 if tailbiting else 0, _ptr(split), split_bytes,
                                                 batch, _ptr(y), _ptr(stream)),
           "qtcq_decode_matvec_mfma_presplit")


NOALLOC_SCRATCH_BYTES = 8 << 20


def qtcq_decode_matvec_mfma_noalloc(bits: int, M: int, N: int, L: int, k: int, code: int,
                                    tailbiting: bool, x: int, batch: int, y: int,
                                    stream: int = 0) -> None:
    _check(_lib.qtcq_decode_matvec_mfma_noalloc(_ptr(bits), M, N, L, k, code,
                                                1 if tailbiting else 0, _ptr(x), batch, _ptr(y),
                                                _ptr(stream)),
           "qtcq_decode_matvec_mfma_noalloc")
