"""Register budgets of the built kernels, read on the CPU from the code objects inside
libqtcq.so (the AMDGPU metadata note of each gfx950 code object): the step loops of the
search, BCJR, gradient, decode and matvec kernels are tuned to fit their registers, and
a change that makes one spill to scratch memory (private segment) slows it several
times over without changing any result.  No GPU needed.

* every kernel keeps a private segment of 0 bytes, except the weighted soft passes in
  gradient mode at L = 16 (at most 16 bytes, every code) and the XOR-code matrix-core
  product at four B fragments with two bands per workgroup (at most 64 bytes);
* nothing anywhere exceeds 64 bytes;
* the LDS-table kernels of both products (XOR code) keep no static LDS: they read the
  table at LDS address 0, where the dynamic area then starts.
"""
import os
import re
import struct
import subprocess

import pytest
import yaml

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "trellis_coded_weight_amd", "libqtcq.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def kernels(tmp_path):
    """[(mangled name, private segment bytes, vgpr spill count, static LDS bytes)] of every
    gfx950 kernel."""
    fat = tmp_path / "fatbin.bin"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "-O", "binary", "--only-section=.hip_fatbin",
                    LIB, str(fat)], check=True)
    data = fat.read_bytes()
    out = []
    p = data.find(MAGIC)
    n_obj = 0
    while p != -1:
        n = struct.unpack_from("<Q", data, p + 24)[0]
        off = p + 32
        for _ in range(n):
            o, sz, idl = struct.unpack_from("<QQQ", data, off)
            tid = data[off + 24:off + 24 + idl].decode()
            off += 24 + idl
            if "gfx950" not in tid:
                continue
            elf = tmp_path / ("co%d.elf" % n_obj)
            n_obj += 1
            elf.write_bytes(data[p + o:p + o + sz])
            notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(elf)],
                                   check=True, capture_output=True, text=True).stdout
            doc = notes[notes.index("---"):notes.index("\n...") + 4]
            for k in yaml.safe_load(doc)["amdhsa.kernels"]:
                out.append((k[".name"], k[".private_segment_fixed_size"], k[".vgpr_spill_count"],
                            k[".group_segment_fixed_size"]))
        p = data.find(MAGIC, p + 1)
    return out


def code_of(name):
    """The CODE template argument of a kernel (0 1MAD, 1 3INST, 2 XOR), or None."""
    m = re.match(r"_ZN4qtcq\d+(\w+?)ILi(\d+)ELi(\d)E", name)
    return int(m.group(3)) if m and m.group(1) in (
        "viterbi_forward", "decode_tile", "bcjr_sweep", "bcjr_vjp_sweep", "decode_matvec",
        "decode_matvec_mfma") else None


@pytest.mark.skipif(not (os.path.exists(LIB) and os.path.exists(os.path.join(LLVM, "llvm-readelf"))),
                    reason="library or ROCm LLVM tools missing")
def test_kernels_keep_their_registers(tmp_path):
    ks = kernels(tmp_path)
    assert len(ks) > 500
    names = [k[0] for k in ks]
    for fam in ("viterbi_forward", "bcjr_sweep", "bcjr_vjp_sweep", "decode_tile", "decode_matvec",
                "decode_matvec_mfma"):
        assert any(fam in n for n in names), fam
    bad = []
    for name, priv, spill, _ in ks:
        code = code_of(name)
        allowed = 0
        if re.search(r"bcjr_sweepILi16ELi[012]ELb1ELb1E", name):
            allowed = 16        # weighted soft pass in gradient mode, L = 16
        if code == 2 and re.search(r"decode_matvec_mfmaILi\d+ELi2ELb[01]ELi4ELi2E", name):
            allowed = 64        # XOR, four fragments, two bands
        if priv > allowed:
            bad.append((name, priv, spill))
    assert not bad, "kernels spilling to scratch: %s" % bad


@pytest.mark.skipif(not (os.path.exists(LIB) and os.path.exists(os.path.join(LLVM, "llvm-readelf"))),
                    reason="library or ROCm LLVM tools missing")
def test_table_kernels_keep_no_static_lds(tmp_path):
    """The LDS-table kernels place the table at LDS address 0 (a window's address is twice
    the window), so they may hold no static LDS; and they use no scratch."""
    ks = kernels(tmp_path)
    table = [k for k in ks if re.search(r"decode_matvec_mfmaILi\d+ELi\d+ELb[01]ELi\dELi\dELb1E", k[0])]
    # XOR code only: six trellis sizes x plain / tail-biting x four fragment counts
    assert len(table) == 48
    valu = [k for k in ks if re.search(r"13decode_matvecILi\d+ELi\d+ELb[01]ELi\dELb1E", k[0])]
    # the fp32 VALU product's: six trellis sizes x plain / tail-biting x four batch widths
    assert len(valu) == 48
    for k in table + valu:
        assert code_of(k[0]) == 2, k[0]
        assert k[3] == 0, (k[0], k[3])
        assert k[1] == 0, (k[0], k[1])
