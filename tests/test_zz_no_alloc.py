"""The no-allocation matrix-core product, qtcq_decode_matvec_mfma_noalloc, through the C
ABI: its output equals qtcq_decode_matvec_mfma's (with a caller workspace) bit for bit,
on calls in a row where the later ones are smaller (fewer columns and rows of x), so
that anything read from the previous call's scratch contents would show; the largest
N the scratch holds runs, the next one is refused before any launch; and repeated calls
do not change the device's free memory."""
import numpy as np
import pytest

from trellis_coded_weight_amd import inputs

from helpers import dev, say
from test_gpu_matvec import random_words

pytestmark = pytest.mark.gpu

MAX_N = 63520     # the largest N whose split fits the 8 MiB scratch


@pytest.fixture(scope="module")
def nat():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    from trellis_coded_weight_amd import _native
    return _native


def sync():
    import torch
    torch.cuda.synchronize()


def both(nat, M, N, L, code, tb, batch, seed):
    """(y from the workspace entry point, y from the no-allocation entry point)."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    words = random_words(M, N, L, tb, seed)
    bd = torch.from_numpy(words.view(np.int32)).cuda()
    x = dev(inputs.targets(batch, N, seed + 1))
    ws = torch.empty(nat.qtcq_decode_matvec_mfma_workspace_bytes(N), dtype=torch.uint8, device="cuda")
    y_ref = torch.full((batch, M), float("nan"), dtype=torch.float32, device="cuda")
    y = torch.full((batch, M), float("nan"), dtype=torch.float32, device="cuda")
    say("noalloc M=%d N=%d L=%d code=%#x tb=%s batch=%d" % (M, N, L, code, tb, batch))
    nat.qtcq_decode_matvec_mfma(bd.data_ptr(), M, N, L, 2, code, tb, x.data_ptr(), batch,
                                y_ref.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    nat.qtcq_decode_matvec_mfma_noalloc(bd.data_ptr(), M, N, L, 2, code, tb, x.data_ptr(), batch,
                                        y.data_ptr(), stream)
    sync()
    return y_ref, y


def test_noalloc_equals_workspace_product_calls_in_a_row(nat):
    import torch
    xor8 = nat.qtcq_xor_code(*inputs.xor_masks(8))
    cases = [
        (4096, 8192, 16, nat.QTCQ_CODE_3INST, True, 32, 11),   # large
        (48, 1040, 16, nat.QTCQ_CODE_1MAD, False, 3, 12),      # smaller N and batch
        (16, 16, 8, xor8, True, 1, 13),                        # smaller still
    ]
    for M, N, L, code, tb, batch, seed in cases:
        y_ref, y = both(nat, M, N, L, code, tb, batch, seed)
        assert torch.isfinite(y_ref).all()
        assert torch.equal(y, y_ref), "M=%d N=%d batch=%d" % (M, N, batch)


def test_noalloc_scratch_limit(nat):
    import torch
    y_ref, y = both(nat, 16, MAX_N, 16, nat.QTCQ_CODE_1MAD, False, 32, 21)
    assert torch.equal(y, y_ref)
    assert nat.qtcq_decode_matvec_mfma_workspace_bytes(MAX_N) <= nat.NOALLOC_SCRATCH_BYTES
    assert nat.qtcq_decode_matvec_mfma_workspace_bytes(MAX_N + 16) > nat.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20    # never dereferenced: the size check comes before any launch
    st = nat.raw_status("qtcq_decode_matvec_mfma_noalloc", fake, 16, MAX_N + 16, 16, 2,
                        nat.QTCQ_CODE_1MAD, 0, fake, 1, fake, None)
    assert st == nat.QTCQ_ERR_WORKSPACE


def test_noalloc_allocates_nothing(nat):
    import torch
    M, N, L, batch = 256, 4096, 16, 8
    stream = torch.cuda.current_stream().cuda_stream
    bd = torch.from_numpy(random_words(M, N, L, False, 31).view(np.int32)).cuda()
    x = dev(inputs.targets(batch, N, 32))
    y = torch.empty((batch, M), dtype=torch.float32, device="cuda")
    call = lambda: nat.qtcq_decode_matvec_mfma_noalloc(bd.data_ptr(), M, N, L, 2, nat.QTCQ_CODE_1MAD,
                                                       False, x.data_ptr(), batch, y.data_ptr(), stream)
    say("noalloc free-memory check")
    call()
    sync()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(20):
        call()
    sync()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0
