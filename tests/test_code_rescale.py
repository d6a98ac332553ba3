"""Host check of the device codes' rescale shortcut (no GPU): the GPU code evaluation
multiplies by the binary64 reciprocal of the divisor (147.8 for 1MAD, 1.244 for 3INST)
where the definition divides in binary64 and rounds once to binary32.  The shortcut is
exact iff it gives the same binary32 bits on the code's whole input domain: every byte
sum 0..1020 (1MAD; QTIP blog, "The codebook is computed") and every finite fp16 value
(3INST raw value).  Both domains are small, so this is checked exhaustively."""
import numpy as np


def test_1mad_reciprocal_exact_on_all_byte_sums():
    num = (np.arange(0, 1021, dtype=np.int64) - 510).astype(np.float64)
    want = (num / 147.8).astype(np.float32)
    got = (num * (1.0 / 147.8)).astype(np.float32)
    assert np.array_equal(want.view(np.uint32), got.view(np.uint32))


def test_3inst_reciprocal_exact_on_all_fp16_values():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    h = h[np.isfinite(h)].astype(np.float64)
    want = (h / 1.244).astype(np.float32)
    got = (h * (1.0 / 1.244)).astype(np.float32)
    assert np.array_equal(want.view(np.uint32), got.view(np.uint32))
