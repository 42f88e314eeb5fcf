"""The C ABI library without a GPU: it loads, exports every declared entry
point, and rejects bad shapes and arguments on the host before any launch."""
import ctypes
import glob
import os
import re

import pytest

from variable_length_kv_amd import lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


DEBUG_HEADER = "vlkv_attn_debug.h"


def _declared(debug=False):
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        if (os.path.basename(h) == DEBUG_HEADER) != debug:
            continue
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b((?:attn|router)_[a-z_0-9]+)\s*\(", src))
    return names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    declared = _declared()
    assert declared, "no declarations found"
    assert declared == set(L.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    for name in L.DEBUG_EXPORTED:   # the counting entry is in the visit-counting build only
        assert not hasattr(lib, name), name


def test_visit_counting_build_exports_the_same_plus_its_entry():
    lib = ctypes.CDLL(L.VISITS_LIB_PATH)
    debug = _declared(debug=True)
    assert debug == set(L.DEBUG_EXPORTED)
    for name in _declared() | debug:
        assert hasattr(lib, name), name
    dbg = L.load_visits()
    # pointer and stride must agree; checked on the host before any HIP call
    assert dbg.attn_debug_visits(None, 8, None) == L.ATTN_ERR_INVALID_ARG
    assert dbg.attn_debug_visits(ctypes.c_void_p(256), 0, None) == L.ATTN_ERR_INVALID_ARG


def _shape(**kw):
    base = dict(batch=4, num_q_heads=8, num_kv_heads=1, page_size=16, num_pages=100, pt_stride=63,
                num_wgs=512)
    base.update(kw)
    return L.AttnShape(**base)


def test_valid_shape_and_workspace_size():
    s = _shape()
    L.attn_check_shape(s)
    n = L.attn_workspace_bytes(s)
    # header + plan arrays + partial slots (B*Hkv + W) * G * (D + 1) floats
    assert n >= (4 + 512) * 8 * 129 * 4
    st = _shape(mode=L.ATTN_STATIC, static_splits=3)
    assert L.attn_static_splits(st) == 3
    assert L.attn_workspace_bytes(st) >= 4 * 3 * 8 * 129 * 4


def test_default_static_splits():
    # ceil(W / (B*Hkv)) clamped to [1, ceil(pt_stride*P / T)]
    assert L.attn_static_splits(_shape(mode=L.ATTN_STATIC, num_wgs=512, batch=64, num_kv_heads=8)) == 1
    assert L.attn_static_splits(_shape(mode=L.ATTN_STATIC, num_wgs=512, batch=4, num_kv_heads=1)) == 16


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), L.ATTN_ERR_INVALID_ARG),
    (dict(num_q_heads=6, num_kv_heads=4), L.ATTN_ERR_INVALID_ARG),
    (dict(num_q_heads=64, num_kv_heads=2), L.ATTN_ERR_UNSUPPORTED),
    (dict(head_dim=64), L.ATTN_ERR_UNSUPPORTED),
    (dict(page_size=8), L.ATTN_ERR_INVALID_ARG),
    (dict(page_size=24), L.ATTN_ERR_INVALID_ARG),
    (dict(tile_tokens=32), L.ATTN_ERR_UNSUPPORTED),
    (dict(num_wgs=-1), L.ATTN_ERR_INVALID_ARG),
    (dict(num_wgs=65537), L.ATTN_ERR_INVALID_ARG),   # the plan's cuts use 32-bit products
    (dict(kv_dtype=7), L.ATTN_ERR_UNSUPPORTED),
    (dict(mode=3), L.ATTN_ERR_INVALID_ARG),
    (dict(num_pages=0), L.ATTN_ERR_INVALID_ARG),
    (dict(pt_stride=0), L.ATTN_ERR_INVALID_ARG),
])
def test_bad_shapes_are_rejected(kw, code):
    s = _shape(**kw)
    with pytest.raises(L.AttnError) as e:
        L.attn_check_shape(s)
    assert e.value.code == code
    assert L.load().attn_workspace_bytes(ctypes.byref(s.c())) == 0


def test_null_arguments_rejected_before_launch():
    lib = L.load()
    s = _shape().c()
    ws = ctypes.c_void_p(256)  # never dereferenced: rejected first
    assert lib.attn_plan(ctypes.byref(s), None, None, ws, 1 << 30, None) == L.ATTN_ERR_INVALID_ARG
    assert b"lengths" in lib.attn_last_error()
    assert lib.attn_plan(ctypes.byref(s), ctypes.c_void_p(16), None, None, 1 << 30, None) == L.ATTN_ERR_INVALID_ARG
    assert lib.attn_plan(ctypes.byref(s), ctypes.c_void_p(16), None, ctypes.c_void_p(300), 1 << 30, None) \
        == L.ATTN_ERR_INVALID_ARG  # misaligned workspace
    assert lib.attn_plan(ctypes.byref(s), ctypes.c_void_p(16), None, ws, 16, None) == L.ATTN_ERR_INVALID_ARG
    assert b"workspace" in lib.attn_last_error()
    args = [ctypes.byref(s), None, ctypes.c_void_p(16), ctypes.c_void_p(16), None, None, ctypes.c_void_p(16),
            ctypes.c_float(0.1), ws, ctypes.c_size_t(1 << 30), ctypes.c_void_p(16), None, None]
    assert lib.attn_decode(*args) == L.ATTN_ERR_INVALID_ARG
    args[7] = ctypes.c_float(float("nan"))
    args[1] = ctypes.c_void_p(16)
    assert lib.attn_decode(*args) == L.ATTN_ERR_INVALID_ARG
    s8 = _shape(kv_dtype=L.ATTN_KV_FP8_E4M3).c()
    args = [ctypes.byref(s8), ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), None, None,
            ctypes.c_void_p(16), ctypes.c_float(0.1), ws, ctypes.c_size_t(1 << 30), ctypes.c_void_p(16), None, None]
    assert lib.attn_decode(*args) == L.ATTN_ERR_INVALID_ARG
    assert b"scale" in lib.attn_last_error()
    assert lib.attn_combine(ctypes.byref(s), ws, ctypes.c_size_t(1 << 30), None, None, None) == L.ATTN_ERR_INVALID_ARG
    assert lib.attn_get_status(None, None, None) == L.ATTN_ERR_INVALID_ARG


def test_default_workgroup_count_is_the_librarys():
    # num_wgs = 0 is a valid shape (the library's default, resolved on the
    # device at call time); the binding does no plan arithmetic of its own
    s = _shape(num_wgs=0)
    L.attn_check_shape(s)
    assert not hasattr(L, "suggest_num_wgs")
    lib = L.load()
    assert lib.attn_num_wgs(ctypes.byref(_shape(num_wgs=300).c())) == 300
    assert lib.attn_num_wgs(ctypes.byref(_shape(num_wgs=-2).c())) == 0
    import torch
    if not torch.cuda.is_available():
        # without a device the default cannot be resolved: sizes are refused
        assert lib.attn_num_wgs(ctypes.byref(s.c())) == 0
        assert lib.attn_workspace_bytes(ctypes.byref(s.c())) == 0
        assert lib.attn_static_splits(ctypes.byref(_shape(num_wgs=0, mode=L.ATTN_STATIC).c())) == 0


def test_append_rejects_bad_arguments_before_launch():
    lib = L.load()
    s = _shape().c()
    nz = ctypes.c_void_p(256)       # a non-null, 16-byte aligned stand-in; never dereferenced on error paths
    args = [nz, nz, nz, nz, None, None, nz, nz, None, 0, None]
    assert lib.attn_append_kv(ctypes.byref(s), None, *args[1:]) == L.ATTN_ERR_INVALID_ARG
    assert b"non-NULL" in lib.attn_last_error()
    fp8 = _shape(kv_dtype=L.ATTN_KV_FP8_E4M3).c()
    assert lib.attn_append_kv(ctypes.byref(fp8), *args) == L.ATTN_ERR_INVALID_ARG   # scales missing
    odd = ctypes.c_void_p(258)
    assert lib.attn_append_kv(ctypes.byref(s), odd, *args[1:]) == L.ATTN_ERR_INVALID_ARG
    assert b"aligned" in lib.attn_last_error()


def test_router_shape_checks_on_the_host():
    lib = L.load()
    assert lib.router_workspace_bytes(0, 64, 16) == 0          # M < 1
    assert lib.router_workspace_bytes(4, 96, 16) == 0          # K not a multiple of 64
    assert lib.router_workspace_bytes(4, 64, 24) == 0          # E not a multiple of 16
    assert lib.router_workspace_bytes(8192, 7168, 256) == 0    # enough tiles: no split over K
    n = lib.router_workspace_bytes(16, 7168, 256)              # few tokens: K split, fp32 partials
    assert n > 0 and n % (16 * 256 * 4) == 0
    rc = lib.router_gemm(4, 96, 16, None, None, None, None, None, 0, None)
    assert rc == L.ATTN_ERR_INVALID_ARG and b"multiple of 64" in lib.attn_last_error()
    rc = lib.router_gemm(4, 64, 16, None, None, None, None, None, 0, None)
    assert rc == L.ATTN_ERR_INVALID_ARG and b"non-NULL" in lib.attn_last_error()
    rc = lib.router_gemm(16, 7168, 256, 16, 16, 16, 16, None, 0, None)   # workspace needed
    assert rc == L.ATTN_ERR_INVALID_ARG and b"workspace" in lib.attn_last_error()
    assert lib.router_split_weights(None, None, None, -1, None) == L.ATTN_ERR_INVALID_ARG
    assert lib.router_split_weights(None, None, None, 0, None) == L.ATTN_OK


def test_binding_checks_tensor_arguments():
    """The binding rejects a tensor whose dtype, element count, memory or
    layout differ from the header's before the library sees the pointer."""
    import torch
    shape = L.AttnShape(batch=2, num_q_heads=8, num_kv_heads=1, page_size=16, num_pages=4, pt_stride=2,
                        num_wgs=4)
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    cache = torch.zeros(4, 1, 16, 128, dtype=torch.bfloat16)
    pt = torch.zeros(2, 2, dtype=torch.int32)
    ws = torch.zeros(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError, match="q: dtype"):
        L.attn_decode(shape, q.float(), cache, cache, None, None, pt, 0.1, ws, q.clone())
    with pytest.raises(ValueError, match="k_cache: 4096 elements, expected 8192"):
        L.attn_decode(shape, q, cache[:2], cache, None, None, pt, 0.1, ws, q.clone())
    with pytest.raises(ValueError, match="page_table: 2 elements"):
        L.attn_decode(shape, q, cache, cache, None, None, pt[0], 0.1, ws, q.clone())
    with pytest.raises(ValueError, match="out must be contiguous"):
        L.attn_decode(shape, q, cache, cache, None, None, pt, 0.1, ws, q.transpose(0, 1).contiguous().transpose(0, 1))
    fp8 = L.AttnShape(**{**shape.__dict__, "kv_dtype": L.ATTN_KV_FP8_E4M3})
    codes = torch.zeros(4, 1, 16, 128, dtype=torch.uint8)
    with pytest.raises(ValueError, match="k_scale is required"):
        L.attn_decode(fp8, q, codes, codes, None, None, pt, 0.1, ws, q.clone())
    with pytest.raises(ValueError, match="k_cache: dtype"):
        L.attn_decode(fp8, q, cache, cache, None, None, pt, 0.1, ws, q.clone())
    with pytest.raises(ValueError, match="q must be in GPU memory"):
        L.attn_decode(shape, q, cache, cache, None, None, pt, 0.1, ws, q.clone())
    with pytest.raises(ValueError, match="lengths: 3 elements"):
        L.attn_plan(shape, torch.zeros(3, dtype=torch.int32), pt, ws)
    g = L.RouterGemm(8192, 7168, 256, "cpu")          # no workspace at this shape
    x = torch.zeros(8192, 7168, dtype=torch.bfloat16)
    w = torch.zeros(256, 7168, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="y: dtype"):
        g(x, w, w, torch.zeros(8192, 256, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="x must be in GPU memory"):
        g(x, w, w, torch.zeros(8192, 256, dtype=torch.float32))
    with pytest.raises(ValueError, match="w_hi: 9 elements"):
        L.router_split_weights(torch.zeros(10), torch.zeros(9, dtype=torch.bfloat16),
                               torch.zeros(10, dtype=torch.bfloat16))
