"""The torch wrappers check every tensor against the shapes the kernels read before any
launch (the C ABI takes raw pointers): wrong shapes, dtypes or layouts raise
ValueError and leave the device untouched."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def api():
    import torch
    assert torch.cuda.is_available(), "GPU test without a GPU"
    from trellis_coded_weight_amd import api as a
    return a


def test_wrappers_reject_mismatched_tensors(api):
    import torch
    dev = "cuda"
    s = torch.zeros((4, 256), dtype=torch.float32, device=dev)
    bad_bits = torch.zeros((4, 16), dtype=torch.int32, device=dev)          # plain needs 17
    with pytest.raises(ValueError):
        api.decode(bad_bits, 256)
    with pytest.raises(ValueError):
        api.decode(torch.zeros((4, 17), dtype=torch.int32, device=dev), 256, seq=s[:, :128].contiguous(),
                   want_mse=True)
    with pytest.raises(ValueError):
        api.decode(torch.zeros((4, 17), dtype=torch.int32, device=dev), 256, want_mse=True)
    with pytest.raises(ValueError):
        api.tailbiting_decode(torch.zeros((4, 17), dtype=torch.int32, device=dev), 256)
    with pytest.raises(ValueError):
        api.encode(s, torch.ones((4, 128), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        api.encode(s.t())                                                    # not contiguous
    with pytest.raises(ValueError):
        api.bcjr_soft(s, 0.1, torch.ones((3, 256), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        api.bcjr_vjp(s, 0.1, torch.zeros((4, 255), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        api.decode_matvec(torch.zeros((3, 17), dtype=torch.int32, device=dev), 32, 32,
                          torch.zeros(32, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        api.decode_matvec(torch.zeros((4, 17), dtype=torch.int32, device=dev), 32, 32,
                          torch.zeros(48, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        api.decode_matvec_mfma(torch.zeros((3, 17), dtype=torch.int32, device=dev), 32, 32,
                               torch.zeros(32, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        api.decode_matvec_mfma(torch.zeros((4, 17), dtype=torch.int32, device=dev), 32, 32,
                               torch.zeros((2, 48), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        api.matvec_mfma_workspace(40)
    torch.cuda.synchronize()


def test_matvec_mfma_rejects_small_workspace(api):
    """A workspace below qtcq_decode_matvec_mfma_workspace_bytes(N) is refused by the C
    entry point before any launch."""
    import torch
    from trellis_coded_weight_amd import _native as nat
    dev = "cuda"
    small = torch.empty(nat.qtcq_decode_matvec_mfma_workspace_bytes(64) - 16, dtype=torch.uint8, device=dev)
    with pytest.raises(RuntimeError, match="QTCQ_ERR_WORKSPACE|workspace"):
        api.decode_matvec_mfma(torch.zeros((16, 17), dtype=torch.int32, device=dev), 64, 64,
                               torch.zeros(64, dtype=torch.float32, device=dev), workspace=small)
    torch.cuda.synchronize()
