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


def test_wrappers_reject_foreign_workspaces(api):
    """A caller-supplied workspace that is not a contiguous tensor on the current device is
    refused before any launch (a host pointer would reach the kernels), and a workspace of
    any dtype is measured in bytes."""
    import torch
    from trellis_coded_weight_amd import _native as nat
    dev = "cuda"
    s = torch.zeros((2, 256), dtype=torch.float32, device=dev)
    g = torch.zeros_like(s)
    host_ws = torch.empty(nat.qtcq_encode_workspace_bytes(2, 256, 16, 2), dtype=torch.uint8)
    strided = torch.empty((2, nat.qtcq_encode_workspace_bytes(2, 256, 16, 2)), dtype=torch.uint8,
                          device=dev)[:, ::2]
    for bad in (host_ws, strided):
        with pytest.raises(ValueError):
            api.encode(s, workspace=bad)
        with pytest.raises(ValueError):
            api.tailbiting_encode(s, workspace=bad)
        with pytest.raises(ValueError):
            api.bcjr_soft(s, 0.1, workspace=bad)
        with pytest.raises(ValueError):
            api.bcjr_vjp(s, 0.1, g, workspace=bad)
        with pytest.raises(ValueError):
            api.decode_matvec_mfma(torch.zeros((16, 17), dtype=torch.int32, device=dev), 64, 64,
                                   torch.zeros(64, dtype=torch.float32, device=dev), workspace=bad)
        with pytest.raises(ValueError):
            api.matvec_mfma_split_x(torch.zeros(64, dtype=torch.float32, device=dev), workspace=bad)
    # a float32 workspace of the right byte size is accepted for the encode: numel * 4 bytes
    n = nat.qtcq_encode_workspace_bytes(2, 256, 16, 2)
    ws32 = torch.empty((n + 3) // 4, dtype=torch.float32, device=dev)
    bits, mse, _ = api.encode(s, workspace=ws32)
    ref_bits, ref_mse, _ = api.encode(s)
    torch.cuda.synchronize()
    assert torch.equal(bits, ref_bits) and torch.equal(mse, ref_mse)


def test_presplit_checks_its_split(api):
    """The split handle carries (N, batch): a split of another N is refused, and the
    product takes the batch the split was made for."""
    import torch
    dev = "cuda"
    x = torch.ones((8, 64), dtype=torch.float32, device=dev)
    sp = api.matvec_mfma_split_x(x)
    bits = torch.zeros((4 * 4, 17), dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        api.decode_matvec_mfma_presplit(torch.zeros((4 * 2, 17), dtype=torch.int32, device=dev),
                                        64, 32, sp)
    with pytest.raises(ValueError):
        api.decode_matvec_mfma_presplit(bits, 64, 64, sp.workspace)
    y = api.decode_matvec_mfma_presplit(bits, 64, 64, sp)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (8, 64)


def test_default_workspaces_hold_whole_rounds(api):
    """A capped workspace holds whole rounds of workgroups: twice the CU count of
    sequences for the search (two per workgroup), the CU count for the soft pass."""
    import torch
    from trellis_coded_weight_amd import _native as nat
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    per = nat.qtcq_encode_workspace_bytes(1, 256, 16, 2)
    ws = api.encode_workspace(10 * cus, 256, 16, 2, max_bytes=per * (2 * cus + 5))
    assert ws.numel() == per * 2 * cus
    tper = nat.qtcq_tailbiting_workspace_bytes(1, 256, 16, 2)
    ws = api.tailbiting_workspace(10 * cus, 256, 16, 2, max_bytes=tper * (3 * cus))
    assert ws.numel() == tper * 2 * cus
    bper = nat.qtcq_bcjr_workspace_bytes(1, 256, 16, 2)
    ws = api.bcjr_workspace(10 * cus, 256, 16, 2, max_bytes=bper * (cus + 5))
    assert ws.numel() == bper * cus
    del ws
    # a cap below one round is taken as it is
    ws = api.encode_workspace(10 * cus, 256, 16, 2, max_bytes=per * 7)
    assert ws.numel() == per * 7
