"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/ce_mi355x.h declares, and rejects bad arguments before it
enqueues anything.  Every call below must fail validation -- none may reach a
kernel launch, because the pointers are fake."""
import ctypes
import os
import re

import pytest

from cross_entropy_loss_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ce_mi355x.h")

FAKE = 0x100000  # 16-byte aligned, never dereferenced
VP = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ce_[a-z_0-9]+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n)


def test_abi_version_and_strings(lib):
    assert lib.ce_abi_version() == _lib.ABI_VERSION
    for code in range(6):
        assert len(lib.ce_error_string(code)) > 0
    assert b"unknown" in lib.ce_error_string(99)


def test_workspace_bytes(lib):
    whole = lib.ce_workspace_bytes(4096, 32000, 0, _lib.CE_DTYPE_BF16)
    # a 128256-wide bf16 row fits on chip: reduced whole, chunk or not
    fits = lib.ce_workspace_bytes(8192, 128256, 65536, _lib.CE_DTYPE_BF16)
    assert 0 < whole <= 1024 + 4096 * 8 + 256  # header + one tagged loss slot per row
    assert fits == lib.ce_workspace_bytes(8192, 128256, 0, _lib.CE_DTYPE_BF16) <= 1024 + 8192 * 8 + 256
    # wider rows are cut into slabs: (max, sum) pairs and the label logit per row
    chunked = lib.ce_workspace_bytes(8192, 200000, 65536, _lib.CE_DTYPE_BF16)
    assert chunked >= 8192 * 4 * 16 + 8192 * 4
    auto = lib.ce_workspace_bytes(8, 300000, 0, _lib.CE_DTYPE_BF16)  # > on-chip row: auto-chunked
    assert auto > lib.ce_workspace_bytes(8, 30000, 0, _lib.CE_DTYPE_BF16)
    assert lib.ce_workspace_bytes(-1, 10, 0, 1) == 0
    assert lib.ce_workspace_bytes(4, 0, 0, 1) == 0
    assert lib.ce_workspace_bytes(4, 10, -1, 1) == 0
    assert lib.ce_workspace_bytes(4, 10, 0, 7) == 0
    assert lib.ce_workspace_bytes(4, 300000, 200000, 1) == 0  # chunk wider than a workgroup holds


def fused(lib, logits=FAKE, ld=100, labels=FAKE, N=4, V=100, dtype=1, ignore=-100, chunk=0, dloss=None,
          loss_mean=FAKE, loss_rows=FAKE, lse=FAKE, pcomp=FAKE, n_valid=FAKE, status=FAKE, ws=FAKE,
          ws_bytes=1 << 20):
    return lib.ce_fwd_bwd_inplace(VP(logits), ld, VP(labels), N, V, dtype, ignore, chunk, VP(dloss),
                                  VP(loss_mean), VP(loss_rows), VP(lse), VP(pcomp), VP(n_valid), VP(status),
                                  VP(ws), ws_bytes, None)


def forward(lib, **kw):
    d = dict(logits=FAKE, ld=100, labels=FAKE, N=4, V=100, dtype=1, ignore=-100, chunk=0, loss_mean=FAKE,
             loss_rows=FAKE, lse=FAKE, pcomp=FAKE, n_valid=FAKE, status=FAKE, ws=FAKE, ws_bytes=1 << 20)
    d.update(kw)
    return lib.ce_forward(VP(d["logits"]), d["ld"], VP(d["labels"]), d["N"], d["V"], d["dtype"], d["ignore"],
                          d["chunk"], VP(d["loss_mean"]), VP(d["loss_rows"]), VP(d["lse"]), VP(d["pcomp"]),
                          VP(d["n_valid"]), VP(d["status"]), VP(d["ws"]), d["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), _lib.CE_ERR_DTYPE),
    (dict(dtype=-1), _lib.CE_ERR_DTYPE),
    (dict(N=-1), _lib.CE_ERR_INVALID_ARG),
    (dict(N=1 << 31), _lib.CE_ERR_INVALID_ARG),
    (dict(V=0), _lib.CE_ERR_INVALID_ARG),
    (dict(ld=99), _lib.CE_ERR_INVALID_ARG),
    (dict(logits=0), _lib.CE_ERR_INVALID_ARG),
    (dict(labels=0), _lib.CE_ERR_INVALID_ARG),
    (dict(logits=FAKE + 1), _lib.CE_ERR_INVALID_ARG),      # not aligned to a bf16 element
    (dict(logits=FAKE + 2, dtype=0), _lib.CE_ERR_INVALID_ARG),  # not aligned to an fp32 element
    (dict(labels=FAKE + 4), _lib.CE_ERR_INVALID_ARG),
    (dict(chunk=-5), _lib.CE_ERR_INVALID_ARG),
    (dict(loss_mean=0), _lib.CE_ERR_INVALID_ARG),
    (dict(loss_rows=0), _lib.CE_ERR_INVALID_ARG),
    (dict(n_valid=0), _lib.CE_ERR_INVALID_ARG),
    (dict(ws=0), _lib.CE_ERR_WORKSPACE),
    (dict(ws_bytes=100), _lib.CE_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), _lib.CE_ERR_WORKSPACE),            # workspace must be 256-byte aligned
    (dict(V=300000, ld=300000, chunk=200000), _lib.CE_ERR_UNSUPPORTED),
    (dict(N=8192, V=128256, ld=128256, chunk=65536, ws_bytes=4096), _lib.CE_ERR_WORKSPACE),
    (dict(N=64, V=200000, ld=200000, chunk=65536, ws_bytes=1024 + 64 * 8 + 256), _lib.CE_ERR_WORKSPACE),
])
def test_fused_rejects(lib, kw, code):
    assert fused(lib, **kw) == code
    assert forward(lib, **kw) == code


def backward(lib, logits=FAKE, ld=100, labels=FAKE, lse=FAKE, pcomp=FAKE, n_valid=FAKE, dloss=None, N=4, V=100,
             dtype=1, ignore=-100, grad=FAKE, grad_ld=100):
    return lib.ce_backward(VP(logits), ld, VP(labels), VP(lse), VP(pcomp), VP(n_valid), VP(dloss), N, V, dtype,
                           ignore, VP(grad), grad_ld, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=9), _lib.CE_ERR_DTYPE),
    (dict(lse=0), _lib.CE_ERR_INVALID_ARG),
    (dict(pcomp=0), _lib.CE_ERR_INVALID_ARG),
    (dict(n_valid=0), _lib.CE_ERR_INVALID_ARG),
    (dict(grad=0), _lib.CE_ERR_INVALID_ARG),
    (dict(grad_ld=99), _lib.CE_ERR_INVALID_ARG),
    (dict(grad_ld=104), _lib.CE_ERR_INVALID_ARG),            # in place needs the same stride
    (dict(grad=FAKE + 64), _lib.CE_ERR_INVALID_ARG),         # partial overlap with the logits
    (dict(grad=FAKE + 4096 + 2, lse=0), _lib.CE_ERR_INVALID_ARG),  # another layout is served; NULL lse is not
    (dict(grad=FAKE + 4097), _lib.CE_ERR_INVALID_ARG),       # not element aligned
])
def test_backward_rejects(lib, kw, code):
    assert backward(lib, **kw) == code


def test_sync_override_rejects(lib):
    assert lib.ce_debug_sync_override(-1, 0) == _lib.CE_ERR_INVALID_ARG
    assert lib.ce_debug_sync_override(0, -1) == _lib.CE_ERR_INVALID_ARG
    assert lib.ce_debug_sync_override(0, 65) == _lib.CE_ERR_INVALID_ARG
    assert lib.ce_debug_sync_override(0, 0) == _lib.CE_OK


def test_noalloc_rejects_oversized_request(lib):
    # 2^21 rows need 16 MiB of tagged loss slots: more than the static scratch
    f = VP(FAKE)
    assert lib.ce_fwd_bwd_inplace_noalloc(f, 100, f, 1 << 21, 100, 1, -100, 0, None, f, f, f, f, f, f,
                                          None) == _lib.CE_ERR_SCRATCH
    # argument errors come first
    assert lib.ce_fwd_bwd_inplace_noalloc(f, 99, f, 4, 100, 1, -100, 0, None, f, f, f, f, f, f,
                                          None) == _lib.CE_ERR_INVALID_ARG


def test_workspace_init_rejects(lib):
    assert lib.ce_workspace_init(None, 4096, None) == _lib.CE_ERR_WORKSPACE
    assert lib.ce_workspace_init(VP(FAKE), 100, None) == _lib.CE_ERR_WORKSPACE
    assert lib.ce_workspace_init(VP(FAKE + 8), 4096, None) == _lib.CE_ERR_WORKSPACE


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "missing.so"))


def linear(lib, hidden=FAKE, ldh=64, weight=FAKE, ldw=64, labels=FAKE, N=8, H=64, V=100, dtype=1, ignore=-100,
           chunk=0, dloss=None, loss_mean=FAKE, loss_rows=FAKE, n_valid=FAKE, status=FAKE, gh=FAKE, ldgh=64,
           gw=FAKE, ldgw=64, ws=FAKE, ws_bytes=1 << 30):
    return lib.ce_linear_fwd_bwd(VP(hidden), ldh, VP(weight), ldw, VP(labels), N, H, V, dtype, ignore, chunk,
                                 VP(dloss), VP(loss_mean), VP(loss_rows), VP(n_valid), VP(status), VP(gh), ldgh,
                                 VP(gw), ldgw, VP(ws), ws_bytes, None)


def test_linear_workspace_bytes(lib):
    b = lib.ce_linear_workspace_bytes(4096, 4096, 32000, 1024, _lib.CE_DTYPE_BF16)
    # 16-bit: the batch's gradient g in the input format and two floats per row
    # and 256-column tile -- no fp32 logits, no transposed copies
    assert 4096 * 32000 * 2 + 4096 * 125 * 8 <= b < 4096 * 32000 * 2 + (8 << 20)
    assert lib.ce_linear_workspace_bytes(4096, 4096, 32000, 64, 1) == b  # chunk_rows does not enter
    f32 = lib.ce_linear_workspace_bytes(4096, 4096, 32000, 1024, _lib.CE_DTYPE_F32)
    assert 1024 * 32000 * 4 <= f32 < 1024 * 32000 * 4 + (64 << 20)  # one fp32 chunk of logits
    assert lib.ce_linear_workspace_bytes(4096, 4096, 32000, 64, _lib.CE_DTYPE_F32) < f32  # smaller chunks
    assert lib.ce_linear_workspace_bytes(-1, 64, 10, 0, 1) == 0
    assert lib.ce_linear_workspace_bytes(4, 0, 10, 0, 1) == 0
    assert lib.ce_linear_workspace_bytes(4, 64, 10, -1, 1) == 0
    assert lib.ce_linear_workspace_bytes(4, 64, 10, 0, 5) == 0
    assert lib.ce_linear_workspace_bytes(4, 64, 1 << 31, 0, 1) == 0
    # 16-bit: up to 8192 vocabulary tiles of 256 per row
    assert lib.ce_linear_workspace_bytes(4, 64, 8192 * 256, 0, 1) > 0
    assert lib.ce_linear_workspace_bytes(4, 64, 8192 * 256 + 1, 0, 1) == 0
    assert lib.ce_linear_workspace_bytes(4, 64, 8192 * 256 + 1, 0, _lib.CE_DTYPE_F32) > 0


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), _lib.CE_ERR_DTYPE),
    (dict(N=-1), _lib.CE_ERR_INVALID_ARG),
    (dict(H=0), _lib.CE_ERR_INVALID_ARG),
    (dict(V=0), _lib.CE_ERR_INVALID_ARG),
    (dict(ldh=63), _lib.CE_ERR_INVALID_ARG),
    (dict(ldw=10), _lib.CE_ERR_INVALID_ARG),
    (dict(ldgh=63), _lib.CE_ERR_INVALID_ARG),
    (dict(ldgw=1), _lib.CE_ERR_INVALID_ARG),
    (dict(hidden=0), _lib.CE_ERR_INVALID_ARG),
    (dict(weight=0), _lib.CE_ERR_INVALID_ARG),
    (dict(labels=0), _lib.CE_ERR_INVALID_ARG),
    (dict(loss_rows=0), _lib.CE_ERR_INVALID_ARG),
    (dict(loss_mean=0), _lib.CE_ERR_INVALID_ARG),
    (dict(n_valid=0), _lib.CE_ERR_INVALID_ARG),
    (dict(hidden=FAKE + 1), _lib.CE_ERR_INVALID_ARG),
    (dict(gw=FAKE + 1), _lib.CE_ERR_INVALID_ARG),
    (dict(labels=FAKE + 4), _lib.CE_ERR_INVALID_ARG),
    (dict(chunk=-1), _lib.CE_ERR_INVALID_ARG),
    (dict(ws=0), _lib.CE_ERR_WORKSPACE),
    (dict(ws_bytes=1000), _lib.CE_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), _lib.CE_ERR_WORKSPACE),
    (dict(V=1 << 31), _lib.CE_ERR_UNSUPPORTED),
    (dict(ldh=1 << 31), _lib.CE_ERR_UNSUPPORTED),
])
def test_linear_rejects(lib, kw, code):
    assert linear(lib, **kw) == code


def rms_fwd(lib, x=FAKE, ldx=64, w=FAKE, N=8, H=64, dtype=1, eps=1e-6, y=FAKE + 4096, ldy=64, rstd=FAKE):
    return lib.ce_rmsnorm_forward(VP(x), ldx, VP(w), N, H, dtype, eps, VP(y), ldy, VP(rstd), None)


def rms_bwd(lib, dy=FAKE, lddy=64, x=FAKE + 4096, ldx=64, w=FAKE, rstd=FAKE, N=8, H=64, dtype=1, dx=FAKE + 8192,
            lddx=64, dw=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return lib.ce_rmsnorm_backward(VP(dy), lddy, VP(x), ldx, VP(w), VP(rstd), N, H, dtype, VP(dx), lddx, VP(dw),
                                   VP(ws), ws_bytes, None)


def test_rmsnorm_workspace_bytes(lib):
    b = lib.ce_rmsnorm_workspace_bytes(4096, 4096, _lib.CE_DTYPE_BF16)
    assert b >= 4096 * 4 and b % 256 == 0  # at least one fp32 partial row of dweight
    assert b <= 1024 * 4096 * 4            # a bounded number of partial rows, not one per token
    assert lib.ce_rmsnorm_workspace_bytes(1, 8, 1) >= 8 * 4
    assert lib.ce_rmsnorm_workspace_bytes(0, 64, 1) >= 64 * 4  # the zero-row backward still reduces
    assert lib.ce_rmsnorm_workspace_bytes(-1, 64, 1) == 0
    assert lib.ce_rmsnorm_workspace_bytes(4, 0, 1) == 0
    assert lib.ce_rmsnorm_workspace_bytes(4, 60, 1) == 0   # not a multiple of 8 (16-bit)
    assert lib.ce_rmsnorm_workspace_bytes(4, 60, 0) > 0    # fp32: multiple of 4
    assert lib.ce_rmsnorm_workspace_bytes(4, 64, 5) == 0


def test_rmsnorm_zero_rows_forward_is_a_no_op(lib):
    # nothing is launched for an empty batch, so the fake pointers are never touched
    assert rms_fwd(lib, N=0) == _lib.CE_OK


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), _lib.CE_ERR_DTYPE),
    (dict(N=-1), _lib.CE_ERR_INVALID_ARG),
    (dict(H=0), _lib.CE_ERR_INVALID_ARG),
    (dict(ldx=63), _lib.CE_ERR_INVALID_ARG),
    (dict(ldy=8), _lib.CE_ERR_INVALID_ARG),
    (dict(eps=-1e-6), _lib.CE_ERR_INVALID_ARG),
    (dict(eps=float("nan")), _lib.CE_ERR_INVALID_ARG),
    (dict(x=0), _lib.CE_ERR_INVALID_ARG),
    (dict(w=0), _lib.CE_ERR_INVALID_ARG),
    (dict(y=0), _lib.CE_ERR_INVALID_ARG),
    (dict(rstd=0), _lib.CE_ERR_INVALID_ARG),
    (dict(y=FAKE, ldy=72), _lib.CE_ERR_INVALID_ARG),   # in place with another stride
    (dict(H=60, ldx=64, ldy=64), _lib.CE_ERR_UNSUPPORTED),
    (dict(H=16392, ldx=16392, ldy=16392), _lib.CE_ERR_UNSUPPORTED),
    (dict(dtype=0, H=8196, ldx=8196, ldy=8196), _lib.CE_ERR_UNSUPPORTED),
    (dict(x=FAKE + 2), _lib.CE_ERR_UNSUPPORTED),
    (dict(ldx=68), _lib.CE_ERR_UNSUPPORTED),            # 136-byte rows: not 16-byte aligned
])
def test_rmsnorm_forward_rejects(lib, kw, code):
    assert rms_fwd(lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), _lib.CE_ERR_DTYPE),
    (dict(N=-1), _lib.CE_ERR_INVALID_ARG),
    (dict(H=0), _lib.CE_ERR_INVALID_ARG),
    (dict(lddy=63), _lib.CE_ERR_INVALID_ARG),
    (dict(ldx=1), _lib.CE_ERR_INVALID_ARG),
    (dict(lddx=32), _lib.CE_ERR_INVALID_ARG),
    (dict(dw=0), _lib.CE_ERR_INVALID_ARG),
    (dict(w=0), _lib.CE_ERR_INVALID_ARG),
    (dict(dy=0), _lib.CE_ERR_INVALID_ARG),
    (dict(x=0), _lib.CE_ERR_INVALID_ARG),
    (dict(rstd=0), _lib.CE_ERR_INVALID_ARG),
    (dict(dx=0), _lib.CE_ERR_INVALID_ARG),
    (dict(dw=FAKE + 1), _lib.CE_ERR_INVALID_ARG),
    (dict(dx=FAKE, lddx=72), _lib.CE_ERR_INVALID_ARG),  # in place with another stride
    (dict(H=16392, lddy=16392, ldx=16392, lddx=16392), _lib.CE_ERR_UNSUPPORTED),
    (dict(dtype=0, H=8196, lddy=8196, ldx=8196, lddx=8196), _lib.CE_ERR_UNSUPPORTED),
    (dict(H=12, lddy=12, ldx=12, lddx=12), _lib.CE_ERR_UNSUPPORTED),
    (dict(x=FAKE + 8), _lib.CE_ERR_UNSUPPORTED),
    (dict(ws=0), _lib.CE_ERR_WORKSPACE),
    (dict(ws_bytes=100), _lib.CE_ERR_WORKSPACE),
    (dict(ws=FAKE + 64), _lib.CE_ERR_WORKSPACE),
])
def test_rmsnorm_backward_rejects(lib, kw, code):
    assert rms_bwd(lib, **kw) == code


def rope_call(lib, q=FAKE, qo=FAKE + 4096, ltq=32 * 128, lhq=128, hq=32, k=FAKE + 8192, ko=FAKE + 8192, ltk=8 * 128,
              lhk=128, hk=8, pos=FAKE, T=16, D=128, base=10000.0, inverse=0, dtype=1):
    return lib.ce_rope(VP(q), VP(qo), ltq, lhq, hq, VP(k), VP(ko), ltk, lhk, hk, VP(pos), T, D, base, inverse, dtype,
                       None)


def test_rope_empty_calls_are_no_ops(lib):
    # nothing is launched, so the fake pointers are never touched
    assert rope_call(lib, T=0) == _lib.CE_OK
    assert rope_call(lib, hq=0, hk=0, q=0, qo=0, k=0, ko=0) == _lib.CE_OK


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=3), _lib.CE_ERR_DTYPE),
    (dict(T=-1), _lib.CE_ERR_INVALID_ARG),
    (dict(hq=-1), _lib.CE_ERR_INVALID_ARG),
    (dict(D=0), _lib.CE_ERR_INVALID_ARG),
    (dict(D=127), _lib.CE_ERR_INVALID_ARG),
    (dict(base=0.0), _lib.CE_ERR_INVALID_ARG),
    (dict(base=-10.0), _lib.CE_ERR_INVALID_ARG),
    (dict(base=float("inf")), _lib.CE_ERR_INVALID_ARG),
    (dict(base=float("nan")), _lib.CE_ERR_INVALID_ARG),
    (dict(inverse=2), _lib.CE_ERR_INVALID_ARG),
    (dict(pos=0), _lib.CE_ERR_INVALID_ARG),
    (dict(q=0), _lib.CE_ERR_INVALID_ARG),
    (dict(qo=0), _lib.CE_ERR_INVALID_ARG),
    (dict(ko=0), _lib.CE_ERR_INVALID_ARG),
    (dict(lhq=64), _lib.CE_ERR_INVALID_ARG),            # heads overlap (stride below head_dim)
    (dict(ltq=31 * 128), _lib.CE_ERR_INVALID_ARG),      # tokens overlap
    (dict(ltk=-128), _lib.CE_ERR_INVALID_ARG),
    (dict(D=24, lhq=24, ltq=32 * 24, lhk=24, ltk=8 * 24), _lib.CE_ERR_UNSUPPORTED),  # 12 pairs: not 8-aligned
    (dict(D=272, lhq=272, ltq=32 * 272, lhk=272, ltk=8 * 272), _lib.CE_ERR_UNSUPPORTED),  # over 128 pairs
    (dict(dtype=0, D=12, lhq=12, ltq=32 * 12, lhk=12, ltk=8 * 12), _lib.CE_ERR_UNSUPPORTED),
    (dict(q=FAKE + 2), _lib.CE_ERR_UNSUPPORTED),
    (dict(lhq=132, ltq=32 * 132), _lib.CE_ERR_UNSUPPORTED),  # 264-byte head stride
    (dict(hq=1 << 20, lhq=1 << 12, ltq=(1 << 32)), _lib.CE_ERR_UNSUPPORTED),  # one token's heads over 2 GiB
])
def test_rope_rejects(lib, kw, code):
    assert rope_call(lib, **kw) == code


def test_calibration_copy_library_rejects():
    """The benchmark's plain-copy library: every shape is addressable and bad
    arguments are refused before any launch."""
    calib = ctypes.CDLL(os.path.join(ROOT, "cross_entropy_loss_amd", "libce_calib.so"))
    calib.ce_calib_copy_shape.argtypes = [VP, VP, ctypes.c_size_t, ctypes.c_int, VP]
    calib.ce_calib_read_shape.argtypes = [VP, ctypes.c_size_t, ctypes.c_int, VP, VP]
    calib.ce_calib_copy.argtypes = [VP, VP, ctypes.c_size_t, VP]
    n = calib.ce_calib_shapes()
    assert n >= 2
    for sh in (-1, n):
        assert calib.ce_calib_copy_shape(VP(FAKE), VP(FAKE), 1024, sh, None) == 1
        assert calib.ce_calib_read_shape(VP(FAKE), 1024, sh, VP(FAKE), None) == 1
    assert calib.ce_calib_copy_shape(VP(FAKE), VP(FAKE), 1000, 0, None) == 1      # not a multiple of 16
    assert calib.ce_calib_copy_shape(VP(FAKE + 8), VP(FAKE), 1024, 0, None) == 1  # misaligned
    assert calib.ce_calib_copy_shape(None, VP(FAKE), 1024, 0, None) == 1
    assert calib.ce_calib_read_shape(VP(FAKE), 1024, 0, None, None) == 1          # no sink
    assert calib.ce_calib_copy(VP(FAKE), VP(FAKE), 1000, None) == 1
    assert calib.ce_calib_copy_shape(VP(FAKE), VP(FAKE), 0, 3, None) == 0         # empty: nothing launched
