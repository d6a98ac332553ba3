"""The C-ABI library loads on the host, exports every entry point include/qtcq.h
declares, and rejects bad arguments before launching anything.  No GPU needed: every
call here returns from host-side validation (or is a pure size query).
"""
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def nat():
    from trellis_coded_weight_amd import _native
    return _native


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "qtcq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qtcq_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(nat):
    syms = declared_symbols()
    assert len(syms) >= 8
    for name in syms:
        assert hasattr(nat._lib, name), name
    assert set(syms) == set(nat.EXPORTED)


def test_status_strings(nat):
    for s in range(5):
        assert nat.qtcq_status_string(s)
    assert nat.qtcq_status_string(99) == "unknown status"


def test_bitstream_words(nat):
    assert nat.qtcq_bitstream_words(16, 2, 256) == 17
    assert nat.qtcq_bitstream_words(16, 2, 1) == 1
    assert nat.qtcq_bitstream_words(6, 2, 14) == 1       # 6 + 26 = 32 bits
    assert nat.qtcq_bitstream_words(6, 2, 15) == 2
    assert nat.qtcq_bitstream_words(16, 0, 256) == -1
    assert nat.qtcq_bitstream_words(16, 2, 0) == -1


def test_workspace_sizes(nat):
    per = nat.qtcq_encode_workspace_bytes(1, 256, 16, 2)
    assert per == 255 * 1024 * 4 + 8                      # 2 bits x 16384 groups x 255 steps
    assert nat.qtcq_encode_workspace_bytes(10, 256, 16, 2) == 10 * per
    assert nat.qtcq_encode_workspace_bytes(1, 256, 7, 2) == 0
    assert nat.qtcq_encode_workspace_bytes(1, 256, 16, 3) == 0
    assert nat.qtcq_encode_workspace_bytes(1, 5000, 16, 2) == 0
    bper = nat.qtcq_bcjr_workspace_bytes(1, 256, 16, 2)
    assert bper >= 255 * 16384 * 4
    assert nat.qtcq_bcjr_workspace_bytes(3, 256, 16, 2) == 3 * bper


FAKE = 1 << 20   # a non-NULL pointer value; never dereferenced by validation paths


def test_encode_validation(nat):
    st = lambda *a: nat.raw_status("qtcq_viterbi_encode", *a)
    ws = nat.qtcq_encode_workspace_bytes(1, 256, 16, 2)
    ok_args = [FAKE, None, 4, 256, 16, 2, 0, FAKE, FAKE, None, FAKE, ws, None]

    def call(**kw):
        a = list(ok_args)
        names = ["seq", "w", "B", "T", "L", "k", "code", "bits", "mse", "states", "ws", "wsb", "stream"]
        for kk, v in kw.items():
            a[names.index(kk)] = v
        return st(*a)

    assert call(B=-1) == nat.QTCQ_ERR_INVALID_ARG
    assert call(T=0) == nat.QTCQ_ERR_INVALID_ARG
    assert call(T=4097) == nat.QTCQ_ERR_INVALID_ARG
    assert call(L=7) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(L=18) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(k=1) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(code=3) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(B=0, seq=None, bits=None, ws=None) == nat.QTCQ_OK
    assert call(seq=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(bits=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(ws=None) == nat.QTCQ_ERR_WORKSPACE
    assert call(ws=FAKE + 4) == nat.QTCQ_ERR_WORKSPACE
    assert call(wsb=ws - 1) == nat.QTCQ_ERR_WORKSPACE


def test_decode_validation(nat):
    st = lambda *a: nat.raw_status("qtcq_decode", *a)
    # bits, B, T, L, k, code, recon, seq, w, mse, stream
    assert st(FAKE, 4, 256, 16, 2, 0, None, None, None, None, None) == nat.QTCQ_ERR_INVALID_ARG
    assert st(FAKE, 4, 256, 16, 2, 0, None, None, None, FAKE, None) == nat.QTCQ_ERR_INVALID_ARG
    assert st(FAKE, 4, 256, 12, 3, 0, FAKE, None, None, None, None) == nat.QTCQ_ERR_UNSUPPORTED
    assert st(FAKE, 4, 0, 16, 2, 0, FAKE, None, None, None, None) == nat.QTCQ_ERR_INVALID_ARG
    assert st(None, 4, 256, 16, 2, 0, FAKE, None, None, None, None) == nat.QTCQ_ERR_INVALID_ARG
    assert st(None, 0, 256, 16, 2, 0, FAKE, None, None, None, None) == nat.QTCQ_OK


def test_bcjr_validation(nat):
    st = lambda *a: nat.raw_status("qtcq_bcjr_soft", *a)
    ws = nat.qtcq_bcjr_workspace_bytes(1, 256, 16, 2)
    # seq, w, B, T, L, k, code, tau, soft, logz, ws, wsb, stream
    assert st(FAKE, None, 4, 256, 16, 2, 0, 0.0, FAKE, None, FAKE, ws, None) == nat.QTCQ_ERR_INVALID_ARG
    assert st(FAKE, None, 4, 256, 16, 2, 0, -1.0, FAKE, None, FAKE, ws, None) == nat.QTCQ_ERR_INVALID_ARG
    assert st(FAKE, None, 4, 256, 16, 2, 0, float("inf"), FAKE, None, FAKE, ws, None) == nat.QTCQ_ERR_INVALID_ARG
    assert st(FAKE, None, 4, 256, 16, 2, 0, float("nan"), FAKE, None, FAKE, ws, None) == nat.QTCQ_ERR_INVALID_ARG
    assert st(FAKE, None, 4, 256, 9, 2, 0, 1.0, FAKE, None, FAKE, ws, None) == nat.QTCQ_ERR_UNSUPPORTED
    assert st(FAKE, None, 4, 256, 16, 2, 0, 1.0, None, None, FAKE, ws, None) == nat.QTCQ_ERR_INVALID_ARG
    assert st(FAKE, None, 4, 256, 16, 2, 0, 1.0, FAKE, None, FAKE, ws - 1, None) == nat.QTCQ_ERR_WORKSPACE
    assert st(None, None, 0, 256, 16, 2, 0, 1.0, None, None, None, 0, None) == nat.QTCQ_OK


def test_bcjr_vjp_validation(nat):
    st = lambda *a: nat.raw_status("qtcq_bcjr_vjp", *a)
    ws = nat.qtcq_bcjr_vjp_workspace_bytes(1, 256, 16, 2)
    assert ws > nat.qtcq_bcjr_workspace_bytes(1, 256, 16, 2)
    assert nat.qtcq_bcjr_vjp_workspace_bytes(4, 256, 16, 2) == 4 * ws
    assert nat.qtcq_bcjr_vjp_workspace_bytes(1, 256, 9, 2) == 0
    # seq, w, B, T, L, k, code, tau, grad_soft, grad_seq, soft, logz, ws, wsb, stream
    ok = [FAKE, None, 4, 256, 16, 2, 0, 0.5, FAKE, FAKE, None, None, FAKE, ws, None]
    names = ["seq", "w", "B", "T", "L", "k", "code", "tau", "g", "grad", "soft", "logz", "ws",
             "wsb", "stream"]

    def call(**kw):
        a = list(ok)
        for kk, v in kw.items():
            a[names.index(kk)] = v
        return st(*a)

    assert call(tau=0.0) == nat.QTCQ_ERR_INVALID_ARG
    assert call(tau=float("nan")) == nat.QTCQ_ERR_INVALID_ARG
    # below the validated temperature floor (3e-3) the gradient is refused
    assert call(tau=2.9e-3) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(tau=1e-6) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(tau=3e-3, wsb=ws - 1) == nat.QTCQ_ERR_WORKSPACE     # the floor passes validation
    assert call(T=0) == nat.QTCQ_ERR_INVALID_ARG
    assert call(L=9) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(code=3) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(g=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(grad=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(seq=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(ws=None) == nat.QTCQ_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == nat.QTCQ_ERR_WORKSPACE
    assert call(wsb=ws - 1) == nat.QTCQ_ERR_WORKSPACE
    assert call(B=0, seq=None, g=None, grad=None, ws=None, wsb=0) == nat.QTCQ_OK


def test_decode_matvec_validation(nat):
    st = lambda *a: nat.raw_status("qtcq_decode_matvec", *a)
    # bits, M, N, L, k, code, tb, x, batch, y, stream
    ok = [FAKE, 32, 64, 16, 2, 0, 0, FAKE, 1, FAKE, None]
    names = ["bits", "M", "N", "L", "k", "code", "tb", "x", "batch", "y", "stream"]

    def call(**kw):
        a = list(ok)
        for kk, v in kw.items():
            a[names.index(kk)] = v
        return st(*a)

    assert call(M=24) == nat.QTCQ_ERR_INVALID_ARG
    assert call(N=-16) == nat.QTCQ_ERR_INVALID_ARG
    assert call(batch=-1) == nat.QTCQ_ERR_INVALID_ARG
    assert call(batch=9) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(L=7) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(code=4) == nat.QTCQ_ERR_UNSUPPORTED
    # the kernel reads through buffer descriptors: at most 2^22 columns
    assert call(N=(1 << 22) + 16) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(N=(1 << 22) + 16, M=0, bits=None, x=None, y=None) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(x=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(x=FAKE + 4) == nat.QTCQ_ERR_INVALID_ARG
    assert call(y=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(bits=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(M=0, bits=None, x=None, y=None) == nat.QTCQ_OK
    assert call(batch=0, bits=None, x=None, y=None) == nat.QTCQ_OK


def test_decode_matvec_mfma_validation(nat):
    st = lambda *a: nat.raw_status("qtcq_decode_matvec_mfma", *a)
    # bits, M, N, L, k, code, tb, x, batch, y, workspace, workspace_bytes, stream
    need = nat.qtcq_decode_matvec_mfma_workspace_bytes(64)
    ok = [FAKE, 32, 64, 16, 2, 0, 0, FAKE, 1, FAKE, FAKE, need, None]
    names = ["bits", "M", "N", "L", "k", "code", "tb", "x", "batch", "y", "ws", "wsb", "stream"]

    def call(**kw):
        a = list(ok)
        for kk, v in kw.items():
            a[names.index(kk)] = v
        return st(*a)

    # per 32 columns (a half block rounds up) and 8 rows of the largest batch (32): 1 KiB
    # of split x and 8 block scales, rounded up to 256 bytes, plus 256
    def size(nkb):
        return -(-nkb * 4 * (1024 + 32) // 256) * 256 + 256
    assert need == size(2)
    assert nat.qtcq_decode_matvec_mfma_workspace_bytes(48) == size(2)
    assert nat.qtcq_decode_matvec_mfma_workspace_bytes(8192) == size(256)
    assert nat.qtcq_decode_matvec_mfma_workspace_bytes(0) == 256
    assert nat.qtcq_decode_matvec_mfma_workspace_bytes(24) == 0
    assert nat.qtcq_decode_matvec_mfma_workspace_bytes(-16) == 0
    assert nat.qtcq_decode_matvec_mfma_workspace_bytes(1 << 22) == size(1 << 17)
    assert nat.qtcq_decode_matvec_mfma_workspace_bytes((1 << 22) + 16) == 0
    assert call(M=24) == nat.QTCQ_ERR_INVALID_ARG
    assert call(N=-16) == nat.QTCQ_ERR_INVALID_ARG
    assert call(batch=-1) == nat.QTCQ_ERR_INVALID_ARG
    assert call(batch=33) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(N=(1 << 22) + 16) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(L=7) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(code=4) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(x=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(x=FAKE + 4) == nat.QTCQ_ERR_INVALID_ARG
    assert call(y=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(bits=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(ws=None) == nat.QTCQ_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == nat.QTCQ_ERR_WORKSPACE
    assert call(wsb=need - 1) == nat.QTCQ_ERR_WORKSPACE
    assert call(M=0, bits=None, x=None, y=None, ws=None) == nat.QTCQ_OK
    assert call(batch=0, bits=None, x=None, y=None, ws=None) == nat.QTCQ_OK


def test_matvec_mfma_split_and_presplit_validation(nat):
    need = nat.qtcq_decode_matvec_mfma_workspace_bytes(64)
    sp = lambda *a: nat.raw_status("qtcq_matvec_mfma_split_x", *a)
    # x, N, batch, workspace, workspace_bytes, stream
    assert sp(FAKE, 24, 1, FAKE, need, None) == nat.QTCQ_ERR_INVALID_ARG
    assert sp(FAKE, 64, -1, FAKE, need, None) == nat.QTCQ_ERR_INVALID_ARG
    assert sp(FAKE, 64, 33, FAKE, need, None) == nat.QTCQ_ERR_UNSUPPORTED
    assert sp(FAKE, 64, 1, None, need, None) == nat.QTCQ_ERR_WORKSPACE
    assert sp(FAKE, 64, 1, FAKE, need - 1, None) == nat.QTCQ_ERR_WORKSPACE
    assert sp(None, 64, 1, FAKE, need, None) == nat.QTCQ_ERR_INVALID_ARG
    assert sp(FAKE + 4, 64, 1, FAKE, need, None) == nat.QTCQ_ERR_INVALID_ARG
    assert sp(None, 64, 0, FAKE, need, None) == nat.QTCQ_OK
    pp = lambda *a: nat.raw_status("qtcq_decode_matvec_mfma_presplit", *a)
    # bits, M, N, L, k, code, tb, split, split_bytes, batch, y, stream
    ok = [FAKE, 32, 64, 16, 2, 0, 0, FAKE, need, 1, FAKE, None]
    names = ["bits", "M", "N", "L", "k", "code", "tb", "split", "sb", "batch", "y", "stream"]

    def call(**kw):
        a = list(ok)
        for kk, v in kw.items():
            a[names.index(kk)] = v
        return pp(*a)

    assert call(M=24) == nat.QTCQ_ERR_INVALID_ARG
    assert call(batch=33) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(L=7) == nat.QTCQ_ERR_UNSUPPORTED
    assert call(split=None) == nat.QTCQ_ERR_WORKSPACE
    assert call(sb=need - 1) == nat.QTCQ_ERR_WORKSPACE
    assert call(y=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(bits=None) == nat.QTCQ_ERR_INVALID_ARG
    assert call(M=0, bits=None, y=None) == nat.QTCQ_OK


def test_tailbiting_sizes(nat):
    assert nat.qtcq_tailbiting_words(16, 2, 256) == 16     # exactly 2T bits, word-aligned
    assert nat.qtcq_tailbiting_words(16, 2, 8) == 1
    assert nat.qtcq_tailbiting_words(16, 2, 7) == -1       # 14 bits < one 16-bit window
    assert nat.qtcq_tailbiting_words(6, 2, 3) == 1
    assert nat.qtcq_tailbiting_words(16, 2, 17) == 2
    per = nat.qtcq_tailbiting_workspace_bytes(1, 256, 16, 2)
    assert per == nat.qtcq_encode_workspace_bytes(1, 256, 16, 2) + 4
    assert nat.qtcq_tailbiting_workspace_bytes(5, 256, 16, 2) == 5 * per
    assert nat.qtcq_tailbiting_workspace_bytes(1, 7, 16, 2) == 0
    assert nat.qtcq_tailbiting_workspace_bytes(1, 256, 9, 2) == 0


def test_tailbiting_validation(nat):
    enc = lambda *a: nat.raw_status("qtcq_tailbiting_encode", *a)
    ws = nat.qtcq_tailbiting_workspace_bytes(1, 256, 16, 2)
    # seq, w, B, T, L, k, code, bits, mse, states, ws, wsb, stream
    assert enc(FAKE, None, 4, 7, 16, 2, 0, FAKE, None, None, FAKE, ws, None) == nat.QTCQ_ERR_INVALID_ARG
    assert enc(FAKE, None, 4, 256, 16, 2, 7, FAKE, None, None, FAKE, ws, None) == nat.QTCQ_ERR_UNSUPPORTED
    assert enc(FAKE, None, 4, 256, 16, 2, 0, None, None, None, FAKE, ws, None) == nat.QTCQ_ERR_INVALID_ARG
    assert enc(FAKE, None, 4, 256, 16, 2, 0, FAKE, None, None, FAKE, ws - 1, None) == nat.QTCQ_ERR_WORKSPACE
    assert enc(FAKE, None, 4, 256, 16, 2, 0, FAKE, None, None, FAKE + 8, ws, None) == nat.QTCQ_ERR_WORKSPACE
    assert enc(None, None, 0, 256, 16, 2, 0, None, None, None, None, 0, None) == nat.QTCQ_OK
    dec = lambda *a: nat.raw_status("qtcq_tailbiting_decode", *a)
    # bits, B, T, L, k, code, recon, seq, w, mse, stream
    assert dec(FAKE, 4, 7, 16, 2, 0, FAKE, None, None, None, None) == nat.QTCQ_ERR_INVALID_ARG
    assert dec(FAKE, 4, 256, 16, 2, 0, None, None, None, None, None) == nat.QTCQ_ERR_INVALID_ARG
    assert dec(FAKE, 4, 256, 16, 2, 0, None, None, None, FAKE, None) == nat.QTCQ_ERR_INVALID_ARG
    assert dec(FAKE, 4, 256, 11, 2, 0, FAKE, None, None, None, None) == nat.QTCQ_ERR_UNSUPPORTED
    assert dec(None, 0, 256, 16, 2, 0, FAKE, None, None, None, None) == nat.QTCQ_OK


def test_code_table_validation(nat):
    assert nat.raw_status("qtcq_code_table", 0, 16, None, None) == nat.QTCQ_ERR_INVALID_ARG
    assert nat.raw_status("qtcq_code_table", 0, 25, FAKE, None) == nat.QTCQ_ERR_INVALID_ARG
    assert nat.raw_status("qtcq_code_table", 5, 16, FAKE, None) == nat.QTCQ_ERR_UNSUPPORTED


def test_product_does_not_import_oracle():
    # the HIP path's package never references the oracle
    pkg = os.path.join(ROOT, "trellis_coded_weight_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text and "qtcq_oracle" not in text, f


def test_header_is_plain_c_and_links(tmp_path):
    """include/qtcq.h compiles as C11 with warnings as errors, and a C program taking the
    address of every declared entry point links against the built library."""
    import subprocess
    from trellis_coded_weight_amd import _native
    syms = declared_symbols()
    src = tmp_path / "use_abi.c"
    src.write_text('#include "qtcq.h"\n#include <stdio.h>\n'
                   "typedef void (*fn)(void);\n"
                   "int main(void) {\n    fn p[] = {\n" +
                   "".join("        (fn)&%s,\n" % n for n in syms) +
                   "    };\n    printf(\"%d\\n\", (int)(sizeof p / sizeof p[0]));\n"
                   "    return qtcq_bitstream_words(16, 2, 256) == 17 ? 0 : 1;\n}\n")
    exe = tmp_path / "use_abi"
    lib = os.path.dirname(_native.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I" + os.path.join(ROOT, "include"),
           str(src), "-o", str(exe), "-L" + lib, "-l:libqtcq.so", "-Wl,-rpath," + lib,
           "-Wl,--unresolved-symbols=ignore-in-shared-libs"]
    subprocess.run(cmd, check=True, capture_output=True)
    assert exe.exists()


def test_code_descriptors(nat):
    """qtcq_code: 1MAD and 3INST are their ids; the XOR palette code carries four 14-bit
    parity masks.  Unknown ids and parameter bits on 1MAD/3INST are unsupported; XOR masks
    that reach beyond the L - 2 history bits are invalid arguments.  Each call below fails
    after the code check (workspace too small), so nothing is launched."""
    masks = (0x2D35, 0x1ACB, 0x34AE, 0x0F53)
    xc = nat.qtcq_xor_code(*masks)
    assert xc & 0xFF == nat.QTCQ_CODE_XOR
    assert [(xc >> (8 + 14 * i)) & 0x3FFF for i in range(4)] == list(masks)
    assert nat.qtcq_xor_code(1 << 14, 0, 0, 0) == nat.QTCQ_CODE_INVALID
    st = lambda *a: nat.raw_status("qtcq_viterbi_encode", *a)
    small = 16       # below one sequence's workspace: QTCQ_ERR_WORKSPACE once the code is accepted

    def enc(code, L):
        return st(FAKE, None, 4, 256, L, 2, code, FAKE, None, None, FAKE, small, None)
    assert enc(xc, 16) == nat.QTCQ_ERR_WORKSPACE
    assert enc(xc, 12) == nat.QTCQ_ERR_INVALID_ARG          # masks need 14 history bits
    low = nat.qtcq_xor_code(*[m & 0x3FF for m in masks])
    assert enc(low, 12) == nat.QTCQ_ERR_WORKSPACE
    assert enc(nat.QTCQ_CODE_XOR, 6) == nat.QTCQ_ERR_WORKSPACE   # zero masks: palette 0
    assert enc(nat.QTCQ_CODE_1MAD | (1 << 8), 16) == nat.QTCQ_ERR_UNSUPPORTED
    assert enc(nat.QTCQ_CODE_INVALID, 16) == nat.QTCQ_ERR_UNSUPPORTED
    assert enc(3, 16) == nat.QTCQ_ERR_UNSUPPORTED
    tab = lambda *a: nat.raw_status("qtcq_code_table", *a)
    assert tab(xc, 20, FAKE, None) == nat.QTCQ_ERR_INVALID_ARG    # XOR: L <= 16
    assert tab(xc, 1, FAKE, None) == nat.QTCQ_ERR_INVALID_ARG
    assert tab(3, 16, FAKE, None) == nat.QTCQ_ERR_UNSUPPORTED
