"""The benchmark's plain copies and reads (cross_entropy_loss_amd/csrc/calib_copy.hip): every shape
copies every byte exactly, at sizes that leave a partial last pass, and the read shapes leave their
sink untouched. bench.py reports the fastest of them as the copy / read ceiling."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
VP = ctypes.c_void_p


@pytest.fixture(scope="module")
def calib():
    # torch's HIP runtime first: a HIP library loaded before it would bring up a runtime of its own, in
    # which torch's device pointers are not valid
    import torch
    torch.zeros(1, device="cuda")
    lib = ctypes.CDLL(os.path.join(ROOT, "cross_entropy_loss_amd", "libce_calib.so"))
    lib.ce_calib_copy_shape.argtypes = [VP, VP, ctypes.c_size_t, ctypes.c_int, VP]
    lib.ce_calib_read_shape.argtypes = [VP, ctypes.c_size_t, ctypes.c_int, VP, VP]
    return lib


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 3 * (1 << 20) + 16 * 7, 64 << 20])
def test_every_shape_copies_exactly(calib, nbytes):
    import torch
    print(f"calib copy {nbytes} B", flush=True)
    rng = np.random.default_rng(nbytes)
    host = torch.from_numpy(rng.integers(0, 2**31 - 1, size=nbytes // 4, dtype=np.int32))
    src = host.cuda()
    st = torch.cuda.current_stream()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for sh in range(calib.ce_calib_shapes()):
        dst = torch.full_like(src, -1)
        assert calib.ce_calib_copy_shape(VP(src.data_ptr()), VP(dst.data_ptr()), nbytes, sh, VP(st.cuda_stream)) == 0
        assert calib.ce_calib_read_shape(VP(src.data_ptr()), nbytes, sh, VP(sink.data_ptr()), VP(st.cuda_stream)) == 0
        torch.cuda.synchronize()
        assert torch.equal(dst.cpu(), host), f"shape {sh}"
    assert int(sink.abs().sum().item()) == 0
