"""CPU reference ("oracle") for variable-length paged decode attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. The product path (the
HIP library and its binding) never imports, links or calls it, and this
package imports nothing from the product.

``decode`` is the fp64 definition of one decode-attention step (C, in
``oracle.c``); ``plan`` is the integer tile-plan specification the GPU planner
must reproduce byte for byte, and ``plan_shared`` that of the prefix-shared
plan; ``append_kv`` writes one new token per request into a paged cache
(``e4m3fn_encode`` is its fp8 rounding); ``router_split`` and ``router_gemm``
define the router GEMM with fp32 weights split into two bf16 parts
(``bf16_rne`` is their rounding); ``brute`` holds an independent NumPy
two-pass softmax used to pin ``decode`` on tiny inputs. Inputs are plain host arrays
(numpy, or CPU torch tensors), duck-typed on the attribute names of a decode
step: B, Hq, Hkv, D, P, num_pages, kv_dtype, q, k_cache, v_cache, k_scale,
v_scale, page_table, lengths, sm_scale.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

ELEN, EPAGE = -2, -3


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.oracle_decode.restype = i32
        lib.oracle_decode.argtypes = [i32] * 8 + [P] * 7 + [ctypes.c_double, P, i32, P, P, i32]
        lib.oracle_plan.restype = i32
        lib.oracle_plan.argtypes = [i32] * 9 + [P] * 8
        lib.oracle_plan_shared.restype = i32
        lib.oracle_plan_shared.argtypes = [i32] * 9 + [P] * 16
        lib.oracle_bf16_rne.restype = ctypes.c_uint16
        lib.oracle_bf16_rne.argtypes = [ctypes.c_float]
        lib.oracle_router_split.restype = None
        lib.oracle_router_split.argtypes = [P, P, P, ctypes.c_int64]
        lib.oracle_router_gemm.restype = i32
        lib.oracle_router_gemm.argtypes = [i32] * 3 + [P] * 6 + [i32]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_e4m3fn_to_f64.restype = ctypes.c_double
        lib.oracle_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3fn_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3fn_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3fn_encode_array.restype = None
        lib.oracle_e4m3fn_encode_array.argtypes = [P, P, ctypes.c_int64]
        lib.oracle_append.restype = i32
        lib.oracle_append.argtypes = [i32] * 7 + [P] * 8
        _lib = lib
    return _lib


def _np(x, dtype):
    """Host array view with the given dtype (bit reinterpretation for 16/8-bit)."""
    if hasattr(x, "detach"):  # torch tensor
        import torch
        x = x.detach().cpu().contiguous()
        if x.dtype == torch.bfloat16:
            x = x.view(torch.int16)
        elif x.dtype == getattr(torch, "float8_e4m3fn", None):
            x = x.view(torch.uint8)
        x = x.numpy()
    a = np.ascontiguousarray(x)
    if a.dtype.itemsize == np.dtype(dtype).itemsize and a.dtype.kind in "iu" and np.dtype(dtype).kind in "iu":
        return a.view(dtype)
    return np.ascontiguousarray(a, dtype=dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def bf16_to_f64(bits: int) -> float:
    return _load().oracle_bf16_to_f64(int(bits) & 0xFFFF)


def e4m3fn_to_f64(code: int) -> float:
    return _load().oracle_e4m3fn_to_f64(int(code) & 0xFF)


def e4m3fn_encode(values) -> np.ndarray:
    """e4m3fn codes (uint8) of fp32 values: nearest, ties to even, saturating."""
    y = np.ascontiguousarray(values, np.float32)
    out = np.empty(y.shape, np.uint8)
    _load().oracle_e4m3fn_encode_array(_ptr(y), _ptr(out), y.size)
    return out


def append_kv(case, k_new, v_new, positions, k_cache=None, v_cache=None, page_table=None, k_scale=None,
              v_scale=None):
    """Append one token per request into copies of the caches (see oracle.c).
    Returns (k_cache, v_cache, status) as host arrays (uint16 bits for bf16,
    uint8 codes for fp8)."""
    lib = _load()
    fp8 = case.kv_dtype == "fp8"
    kdt = np.uint8 if fp8 else np.uint16
    kc = np.array(_np(case.k_cache if k_cache is None else k_cache, kdt), copy=True)
    vc = np.array(_np(case.v_cache if v_cache is None else v_cache, kdt), copy=True)
    pt = _np(case.page_table if page_table is None else page_table, np.int32)
    kn = _np(k_new, np.uint16)
    vn = _np(v_new, np.uint16)
    pos = _np(positions, np.int32)
    ks = vs = None
    if fp8:
        ks = _np(case.k_scale if k_scale is None else k_scale, np.float32)
        vs = _np(case.v_scale if v_scale is None else v_scale, np.float32)
    st = lib.oracle_append(int(case.B), int(case.Hkv), int(case.D), int(case.P), int(case.num_pages),
                           int(pt.shape[1]), int(fp8), _ptr(kn), _ptr(vn), _ptr(pos), _ptr(pt), _ptr(ks),
                           _ptr(vs), _ptr(kc), _ptr(vc))
    return kc, vc, int(st)


def decode(case, req_ids=None, threads=0, *, lengths=None, page_table=None, sm_scale=None,
           q=None, k_cache=None, v_cache=None, k_scale=None, v_scale=None):
    """fp64 decode attention. Returns (out [n, Hq, D], lse [n, Hq]) float64 for
    the requests in ``req_ids`` (all, in order, if None). Keyword arguments
    override the corresponding attributes of ``case``."""
    lib = _load()
    lengths = _np(case.lengths if lengths is None else lengths, np.int32)
    pt = _np(case.page_table if page_table is None else page_table, np.int32)
    q = _np(case.q if q is None else q, np.uint16)
    fp8 = case.kv_dtype == "fp8"
    kdt = np.uint8 if fp8 else np.uint16
    kc = _np(case.k_cache if k_cache is None else k_cache, kdt)
    vc = _np(case.v_cache if v_cache is None else v_cache, kdt)
    ks = vs = None
    if fp8:
        ks = _np(case.k_scale if k_scale is None else k_scale, np.float32)
        vs = _np(case.v_scale if v_scale is None else v_scale, np.float32)
    B, Hq = int(case.B), int(case.Hq)
    if req_ids is None:
        ids = None
        n = B
    else:
        ids = np.ascontiguousarray(req_ids, np.int32)
        n = len(ids)
    out = np.zeros((n, Hq, case.D), np.float64)
    lse = np.zeros((n, Hq), np.float64)
    rc = lib.oracle_decode(B, Hq, case.Hkv, case.D, case.P, case.num_pages, pt.shape[1], int(fp8),
                           _ptr(q), _ptr(kc), _ptr(vc), _ptr(ks), _ptr(vs), _ptr(pt), _ptr(lengths),
                           float(case.sm_scale if sm_scale is None else sm_scale),
                           _ptr(ids), n, _ptr(out), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_decode failed with code {rc}")
    return out, lse


def plan(mode, lengths, Hkv, P, pt_stride, T, W, S=0, cus=0):
    """Integer tile plan (mode 0 dynamic, 1 static). Returns a dict of int32
    arrays. ``cus`` > 0 selects the library's default workgroup count (then
    W = 2 * cus): W when that leaves at least 32 units per workgroup, else cus."""
    lib = _load()
    lengths = _np(lengths, np.int32)
    B = len(lengths)
    out = {
        "header": np.zeros(8, np.int32),
        "len_eff": np.zeros(B, np.int32),
        "tiles_prefix": np.zeros(B + 1, np.int32),
        "seg_prefix": np.zeros(B * Hkv + 1, np.int32),
        "first_wg": np.zeros(B * Hkv, np.int32),
        "wg_begin": np.zeros(W + 1, np.int32),
        "wg_start_b": np.zeros(W, np.int32),
    }
    rc = lib.oracle_plan(int(mode), B, Hkv, P, pt_stride, T, W, int(S), int(cus), _ptr(lengths),
                         *[_ptr(out[k]) for k in ("header", "len_eff", "tiles_prefix", "seg_prefix",
                                                  "first_wg", "wg_begin", "wg_start_b")])
    if rc != 0:
        raise ValueError(f"oracle_plan failed with code {rc}")
    return out


def plan_shared(lengths, page_table, Hkv, G, P, num_pages, T, W, cus=0):
    """Integer plan with prefix-shared pages (mode 2). Returns a dict of int32
    arrays; the item arrays are cut to the number of items."""
    lib = _load()
    lengths = _np(lengths, np.int32)
    pt = np.ascontiguousarray(_np(page_table, np.int32))
    B = len(lengths)
    pt_stride = int(pt.shape[1]) if pt.ndim == 2 else 0
    if pt.ndim != 2 or pt.shape[0] != B:
        raise ValueError("page_table must be [B][pt_stride]")
    I2 = max(1, 2 * B)
    out = {
        "header": np.zeros(8, np.int32),
        "item_req": np.zeros(I2, np.int32), "item_start": np.zeros(I2, np.int32),
        "item_len": np.zeros(I2, np.int32), "item_m": np.zeros(I2, np.int32), "item_solo": np.zeros(I2, np.int32),
        "req_shared": np.zeros(B, np.int32), "req_member": np.zeros(B, np.int32), "req_own": np.zeros(B, np.int32),
        "tiles_prefix": np.zeros(I2 + 1, np.int32),
        "seg_prefix": np.zeros(I2 * Hkv + 1, np.int32),
        "first_wg": np.zeros(I2 * Hkv, np.int32),
        "wg_begin": np.zeros(W + 1, np.int32),
        "wg_start": np.zeros(W, np.int32),
    }
    keys = ("header", "item_req", "item_start", "item_len", "item_m", "item_solo", "req_shared", "req_member",
            "req_own", "tiles_prefix", "seg_prefix", "first_wg", "wg_begin", "wg_start")
    rc = lib.oracle_plan_shared(B, Hkv, G, P, pt_stride, num_pages, T, W, int(cus), _ptr(lengths), _ptr(pt),
                                *[_ptr(out[k]) for k in keys])
    if rc != 0:
        raise ValueError(f"oracle_plan_shared failed with code {rc}")
    I = int(out["header"][4])
    for k in ("item_req", "item_start", "item_len", "item_m", "item_solo"):
        out[k] = out[k][:I]
    out["tiles_prefix"] = out["tiles_prefix"][:I + 1]
    out["seg_prefix"] = out["seg_prefix"][:I * Hkv + 1]
    out["first_wg"] = out["first_wg"][:I * Hkv]
    return out


def bf16_rne(value: float) -> int:
    """fp32 -> bf16 bits by round to nearest, ties to even."""
    return int(_load().oracle_bf16_rne(ctypes.c_float(value)))


def router_split(w):
    """Split fp32 weights into bf16 (hi, lo) bit arrays: hi = bf16(w),
    lo = bf16(256 (w - hi)). Returns two uint16 arrays of w's shape."""
    w32 = np.ascontiguousarray(_np(w, np.float32))
    hi = np.empty(w32.shape, np.uint16)
    lo = np.empty(w32.shape, np.uint16)
    _load().oracle_router_split(_ptr(w32), _ptr(hi), _ptr(lo), w32.size)
    return hi, lo


def router_gemm(x_bits, w, hi=None, lo=None, threads=0):
    """fp64 y[M][E] = x[M][K] w[E][K]^T, with the exact fp32 weights and with
    hi + lo/256. x_bits: bf16 bits (uint16 array or bf16 tensor). Returns
    (y_exact, y_split)."""
    x = np.ascontiguousarray(_np(x_bits, np.uint16))
    w32 = np.ascontiguousarray(_np(w, np.float32))
    if hi is None or lo is None:
        hi, lo = router_split(w32)
    M, K = x.shape
    E = w32.shape[0]
    if w32.shape != (E, K):
        raise ValueError("w must be [E][K]")
    ye = np.zeros((M, E), np.float64)
    ys = np.zeros((M, E), np.float64)
    rc = _load().oracle_router_gemm(M, K, E, _ptr(x), _ptr(w32), _ptr(np.ascontiguousarray(hi, np.uint16)),
                                    _ptr(np.ascontiguousarray(lo, np.uint16)), _ptr(ye), _ptr(ys), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_router_gemm failed with code {rc}")
    return ye, ys
