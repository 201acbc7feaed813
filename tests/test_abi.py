"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/vsa.h declares, and rejects invalid arguments before
touching the device (validation happens before any HIP call, so these calls
never launch anything)."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_cube_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")

# a 16-byte aligned non-null value; never dereferenced because every call
# below fails validation first
FAKE = ctypes.c_void_p(0x1000)
MISALIGNED = ctypes.c_void_p(0x1008)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_[a-z0-9_]+)\s*\(", text)))


def test_header_and_library_agree():
    names = declared_functions()
    assert set(names) == set(L.EXPORTS), names
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), f"libvsa.so does not export {n}"


def prob(**kw):
    base = dict(B=1, H=12, T=16, Hh=14, Ww=26, d=128, cube_t=4, cube_h=4, cube_w=4, topk=14,
                dtype=L.VSA_BF16)
    base.update(kw)
    return L.VSAProblem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), L.VSA_ERR_SHAPE), (dict(H=-1), L.VSA_ERR_SHAPE), (dict(T=0), L.VSA_ERR_SHAPE),
    (dict(Ww=0), L.VSA_ERR_SHAPE), (dict(topk=0), L.VSA_ERR_SHAPE),
    (dict(topk=113), L.VSA_ERR_SHAPE), (dict(d=96), L.VSA_ERR_UNSUPPORTED),
    (dict(cube_t=2), L.VSA_ERR_UNSUPPORTED), (dict(dtype=7), L.VSA_ERR_UNSUPPORTED),
    (dict(T=4 * 80, Hh=4 * 8, Ww=4 * 8, topk=1), L.VSA_ERR_UNSUPPORTED),   # 5120 cubes
    (dict(T=4 * 64, Hh=4 * 8, Ww=4 * 8, topk=1), L.VSA_OK),                # 4096 cubes
    (dict(), L.VSA_OK), (dict(topk=112), L.VSA_OK), (dict(T=1, Hh=1, Ww=1, topk=1), L.VSA_OK),
])
def test_problem_validation(kw, status):
    p = prob(**kw)
    assert L.lib().vsa_check_problem(ctypes.byref(p)) == status
    ws = L.lib().vsa_workspace_bytes(ctypes.byref(p), L.VSA_OP_FORWARD)
    assert (ws > 0) == (status == L.VSA_OK)


def test_null_problem():
    assert L.lib().vsa_check_problem(None) == L.VSA_ERR_NULL
    assert L.lib().vsa_workspace_bytes(None, L.VSA_OP_FORWARD) == 0
    assert L.lib().vsa_forward(None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE,
                               1 << 40, None) == L.VSA_ERR_NULL


def test_workspace_sizes():
    p = prob()
    lib = L.lib()
    fwd = lib.vsa_workspace_bytes(ctypes.byref(p), L.VSA_OP_FORWARD)
    # bf16: fp32 means of q, k, v + per-cube coarse output (q, k, v are gathered
    # from raster rows); fp32 adds cube-order copies of q, k, v
    assert fwd >= 3 * 12 * 112 * 128 * 4 + 12 * 112 * 128 * 2
    fwd32 = lib.vsa_workspace_bytes(ctypes.byref(prob(dtype=L.VSA_F32)), L.VSA_OP_FORWARD)
    assert fwd32 >= 3 * 12 * 7168 * 128 * 4 + 3 * 12 * 112 * 128 * 4 + 12 * 112 * 128 * 4
    assert lib.vsa_workspace_bytes(ctypes.byref(p), L.VSA_OP_COARSE) >= 3 * 12 * 112 * 128 * 4
    assert lib.vsa_workspace_bytes(ctypes.byref(p), L.VSA_OP_FINE) == 0
    assert lib.vsa_workspace_bytes(ctypes.byref(p), 99) == 0


def test_forward_argument_errors():
    lib = L.lib()
    p = prob()
    big = 1 << 40
    # arguments after the problem: q k v o_fine o_coarse idx lse means ws ws_bytes stream
    call = lambda *a: lib.vsa_forward(ctypes.byref(p), *a)
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, big, None)
    def with_(i, x):
        a = list(ok); a[i] = x
        return call(*a)
    assert with_(0, None) == L.VSA_ERR_NULL
    assert with_(4, None) == L.VSA_ERR_NULL
    assert with_(0, MISALIGNED) == L.VSA_ERR_ALIGN
    assert with_(6, MISALIGNED) == L.VSA_ERR_ALIGN     # lse
    assert with_(7, MISALIGNED) == L.VSA_ERR_ALIGN     # means
    assert with_(8, None) == L.VSA_ERR_NULL            # workspace
    assert with_(9, 1024) == L.VSA_ERR_WORKSPACE
    bad = prob(topk=0)
    assert lib.vsa_forward(ctypes.byref(bad), *ok) == L.VSA_ERR_SHAPE


def test_other_entry_points_validate_first():
    lib = L.lib()
    p = prob()
    big = 1 << 40
    assert lib.vsa_reorder(ctypes.byref(p), None, FAKE, 0, None) == L.VSA_ERR_NULL
    assert lib.vsa_reorder(ctypes.byref(p), FAKE, MISALIGNED, 1, None) == L.VSA_ERR_ALIGN
    assert lib.vsa_coarse(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, big,
                          None) == L.VSA_ERR_NULL
    assert lib.vsa_coarse(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 16,
                          None) == L.VSA_ERR_WORKSPACE
    assert lib.vsa_fine(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, None, None, 0,
                        None) == L.VSA_ERR_NULL
    assert lib.vsa_fine(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, None, 0,
                        None) == L.VSA_ERR_ALIGN
    bad = prob(d=80)
    assert lib.vsa_fine(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0,
                        None) == L.VSA_ERR_UNSUPPORTED
    # q k v o_fine lse idx means do_fine do_coarse dq dk dv ws ws_bytes stream
    assert lib.vsa_backward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, None,
                            FAKE, FAKE, FAKE, FAKE, big, None) == L.VSA_ERR_NULL
    assert lib.vsa_backward(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE,
                            None, FAKE, FAKE, FAKE, FAKE, big, None) == L.VSA_ERR_ALIGN


def test_reorder_direction_codes():
    lib = L.lib()
    p = prob()
    assert lib.vsa_reorder(ctypes.byref(p), FAKE, FAKE, 2, None) == L.VSA_ERR_UNSUPPORTED
    assert lib.vsa_reorder(ctypes.byref(p), FAKE, FAKE, -1, None) == L.VSA_ERR_UNSUPPORTED


def test_status_strings():
    for s in range(7):
        assert L.status_string(s).startswith("VSA_")
    assert "unknown" in L.status_string(42)


def test_fp8_entry_points_validate_before_launching():
    lib = L.lib()
    p = prob()
    # FP8: bf16 and d = 128 only
    for bad in (prob(dtype=L.VSA_F32), prob(d=64)):
        assert lib.vsa_quantize_fp8(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    None) == L.VSA_ERR_UNSUPPORTED
        assert lib.vsa_fine_fp8(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                None) == L.VSA_ERR_UNSUPPORTED
        assert lib.vsa_workspace_bytes(ctypes.byref(bad), L.VSA_OP_FORWARD_FP8) == 0
    assert lib.vsa_quantize_fp8(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                None) == L.VSA_ERR_NULL
    assert lib.vsa_fine_fp8(ctypes.byref(p), FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE, None,
                            None) == L.VSA_ERR_ALIGN
    assert lib.vsa_fine_fp8(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED,
                            None) == L.VSA_ERR_ALIGN
    ws = lib.vsa_workspace_bytes(ctypes.byref(p), L.VSA_OP_FORWARD_FP8)
    # three byte copies of q, k, v, the exponents, fp32 means and O_coarse
    assert ws >= 3 * 12 * 7168 * 128 + 3 * 12 * 112 * 4 + 3 * 12 * 112 * 128 * 4 + 12 * 112 * 128 * 2
    assert lib.vsa_forward_fp8(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                               ws - 1, None) == L.VSA_ERR_WORKSPACE
    assert lib.vsa_forward_fp8(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                               ws, None) == L.VSA_ERR_NULL
