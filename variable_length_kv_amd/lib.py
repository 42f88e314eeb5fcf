"""ctypes binding of libvlkv_attn.so (the C ABI in include/vlkv_attn.h).

Argument marshalling only: every step of the attention path runs in the HIP
library. Tensors are PyTorch device tensors (torch provides device memory and
the current stream); the functions take the same names as the C entry points.
If the library has not been built this module raises on first use: there is
no fallback implementation.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvlkv_attn.so")
# the visit-counting build of the same sources (include/vlkv_attn_debug.h)
VISITS_LIB_PATH = os.path.join(_HERE, "libvlkv_attn_visits.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_KV_BF16, ATTN_KV_FP8_E4M3 = 0, 1
ATTN_DYNAMIC, ATTN_STATIC, ATTN_SHARED = 0, 1, 2
ATTN_STATUS_BAD_LENGTH, ATTN_STATUS_BAD_PAGE, ATTN_STATUS_INTERNAL = 1, 2, 4

EXPORTED = ("attn_check_shape", "attn_workspace_bytes", "attn_static_splits", "attn_num_wgs", "attn_device_cu_count",
            "attn_plan", "attn_decode", "attn_combine", "attn_get_status", "attn_read_plan",
            "attn_workspace_init", "attn_step", "attn_step_noalloc", "attn_append_kv", "attn_read_plan_items",
            "attn_last_error",
            "router_split_weights", "router_workspace_bytes", "router_gemm")
DEBUG_EXPORTED = ("attn_debug_visits",)   # libvlkv_attn_visits.so only


class AttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class _Shape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "num_pages", "pt_stride",
        "tile_tokens", "num_wgs", "kv_dtype", "mode", "static_splits")]


@dataclass
class AttnShape:
    batch: int
    num_q_heads: int
    num_kv_heads: int
    page_size: int
    num_pages: int
    pt_stride: int
    num_wgs: int = 0   # 0: the library default (see the C header)
    head_dim: int = 128
    tile_tokens: int = 64
    kv_dtype: int = ATTN_KV_BF16
    mode: int = ATTN_DYNAMIC
    static_splits: int = 0

    def c(self) -> _Shape:
        return _Shape(self.batch, self.num_q_heads, self.num_kv_heads, self.head_dim, self.page_size,
                      self.num_pages, self.pt_stride, self.tile_tokens, self.num_wgs, self.kv_dtype,
                      self.mode, self.static_splits)


_lib = None
_visits_lib = None


def load():
    """Load libvlkv_attn.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH)
    return _lib


def _open(path, debug=False):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m variable_length_kv_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    SP = ctypes.POINTER(_Shape)
    sigs = {
        "attn_check_shape": (i32, [SP]),
        "attn_workspace_bytes": (sz, [SP]),
        "attn_static_splits": (i32, [SP]),
        "attn_num_wgs": (i32, [SP]),
        "attn_device_cu_count": (i32, [ctypes.c_int, P]),
        "attn_plan": (i32, [SP, P, P, P, sz, P]),
        "attn_decode": (i32, [SP, P, P, P, P, P, P, ctypes.c_float, P, sz, P, P, P]),
        "attn_combine": (i32, [SP, P, sz, P, P, P]),
        "attn_get_status": (i32, [P, P, P]),
        "attn_read_plan": (i32, [SP, P, P, P, P, P, P, P, P, P]),
        "attn_workspace_init": (i32, [SP, P, sz, P]),
        "attn_step": (i32, [SP, P, P, P, P, P, P, P, ctypes.c_float, P, sz, P, P, P]),
        "attn_step_noalloc": (i32, [SP, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P]),
        "attn_append_kv": (i32, [SP, P, P, P, P, P, P, P, P, P, sz, P]),
        "attn_read_plan_items": (i32, [SP, P, P, P, P, P, P, P, P, P]),
        "router_split_weights": (i32, [P, P, P, ctypes.c_int64, P]),
        "router_workspace_bytes": (sz, [i32, i32, i32]),
        "router_gemm": (i32, [i32, i32, i32, P, P, P, P, P, sz, P]),
        "attn_last_error": (ctypes.c_char_p, []),
    }
    if debug:
        sigs["attn_debug_visits"] = (i32, [P, ctypes.c_int64, P])
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load_visits():
    """Load the visit-counting build libvlkv_attn_visits.so (raises if it is not built)."""
    global _visits_lib
    if _visits_lib is None:
        _visits_lib = _open(VISITS_LIB_PATH, debug=True)
    return _visits_lib


@contextlib.contextmanager
def counting_visits(tok_counts, tok_stride, out_counts):
    """Route every call of this module through the visit-counting build while
    the block runs, with its counters set to the given int32 device tensors
    (tok_counts [B][Hkv][tok_stride], out_counts [B][Hq]; see
    include/vlkv_attn_debug.h). Workspaces made by either build serve both."""
    global _lib
    dbg = load_visits()
    saved = load()
    _on_gpu(tok_counts=tok_counts, out_counts=out_counts)
    _check_with(dbg, dbg.attn_debug_visits(_ptr(tok_counts), int(tok_stride), _ptr(out_counts)))
    _lib = dbg
    try:
        yield
    finally:
        _lib = saved
        _check_with(dbg, dbg.attn_debug_visits(None, 0, None))


def _check_with(lib, rc):
    if rc != ATTN_OK:
        raise AttnError(rc, lib.attn_last_error().decode())


def _check(rc):
    if rc != ATTN_OK:
        raise AttnError(rc, load().attn_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        if not t.is_contiguous():
            raise ValueError("tensors passed to the attention library must be contiguous")
        return ctypes.c_void_p(t.data_ptr())
    return ctypes.c_void_p(int(t))


_BF16 = (torch.bfloat16,)
_HALFWORD = (torch.bfloat16, torch.int16, torch.uint16)
_FP8 = (torch.uint8, torch.float8_e4m3fn)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _need(t, name, dtypes, numel, optional=False):
    """A tensor argument laid out as the C header says: one of `dtypes`, exactly
    `numel` elements, contiguous. Raises ValueError before anything is
    enqueued; an int (a raw device address) is passed through unchecked. Where
    the tensor lives is checked apart (_on_gpu), after every argument's
    layout."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        return
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors):
    for name, t in tensors.items():
        if isinstance(t, torch.Tensor) and t.device.type != "cuda":
            raise ValueError(f"{name} must be in GPU memory")


def _need_step(shape, q=None, k_cache=None, v_cache=None, k_scale=None, v_scale=None, page_table=None,
               lengths=None, out=None, lse=None, decode=True, plan=True):
    B, Hq, Hkv, D = shape.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    if plan:
        _need(lengths, "lengths", _I32, B)
        _need(page_table, "page_table", _I32, B * shape.pt_stride, optional=shape.mode != ATTN_SHARED)
    if decode:
        fp8 = shape.kv_dtype == ATTN_KV_FP8_E4M3
        _need(q, "q", _BF16, B * Hq * D)
        cache = shape.num_pages * Hkv * shape.page_size * D
        _need(k_cache, "k_cache", _FP8 if fp8 else _BF16, cache)
        _need(v_cache, "v_cache", _FP8 if fp8 else _BF16, cache)
        _need(k_scale, "k_scale", _F32, B * Hkv, optional=not fp8)
        _need(v_scale, "v_scale", _F32, B * Hkv, optional=not fp8)
        _need(page_table, "page_table", _I32, B * shape.pt_stride)
    if decode or out is not None:
        _need(out, "out", _BF16, B * Hq * D)
        _need(lse, "lse", _F32, B * Hq, optional=True)
    _on_gpu(q=q, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale, page_table=page_table,
            lengths=lengths, out=out, lse=lse)


def _need_append(sh, k_new, v_new, positions, page_table, k_cache, v_cache, k_scale, v_scale):
    fp8 = sh.kv_dtype == ATTN_KV_FP8_E4M3
    _need(k_new, "k_new", _BF16, sh.batch * sh.num_kv_heads * sh.head_dim)
    _need(v_new, "v_new", _BF16, sh.batch * sh.num_kv_heads * sh.head_dim)
    _need(positions, "positions", _I32, sh.batch)
    _need(page_table, "page_table", _I32, sh.batch * sh.pt_stride)
    _need(k_scale, "k_scale", _F32, sh.batch * sh.num_kv_heads, optional=not fp8)
    _need(v_scale, "v_scale", _F32, sh.batch * sh.num_kv_heads, optional=not fp8)
    cache = sh.num_pages * sh.num_kv_heads * sh.page_size * sh.head_dim
    _need(k_cache, "k_cache", _FP8 if fp8 else _BF16, cache)
    _need(v_cache, "v_cache", _FP8 if fp8 else _BF16, cache)
    _on_gpu(k_new=k_new, v_new=v_new, positions=positions, page_table=page_table, k_cache=k_cache,
            v_cache=v_cache, k_scale=k_scale, v_scale=v_scale)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _shape(shape):
    if isinstance(shape, AttnShape):
        shape = shape.c()
    return ctypes.byref(shape)


def attn_check_shape(shape) -> None:
    _check(load().attn_check_shape(_shape(shape)))


def attn_workspace_bytes(shape) -> int:
    n = load().attn_workspace_bytes(_shape(shape))
    if n == 0:
        attn_check_shape(shape)
    return int(n)


def attn_static_splits(shape) -> int:
    return int(load().attn_static_splits(_shape(shape)))


def attn_num_wgs(shape) -> int:
    """Workgroups of the decode launch (resolves num_wgs = 0 on the current device)."""
    n = int(load().attn_num_wgs(_shape(shape)))
    if n == 0:
        attn_check_shape(shape)
        raise AttnError(ATTN_ERR_INVALID_ARG, load().attn_last_error().decode())
    return n


def attn_device_cu_count(device: int = 0) -> int:
    out = ctypes.c_int32()
    _check(load().attn_device_cu_count(int(device), ctypes.byref(out)))
    return int(out.value)


def attn_plan(shape, lengths, page_table, workspace, stream=None) -> None:
    _need_step(shape, lengths=lengths, page_table=page_table, decode=False)
    _check(load().attn_plan(_shape(shape), _ptr(lengths), _ptr(page_table), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)))


def attn_decode(shape, q, k_cache, v_cache, k_scale, v_scale, page_table, sm_scale, workspace, out,
                lse=None, stream=None) -> None:
    _need_step(shape, q, k_cache, v_cache, k_scale, v_scale, page_table, out=out, lse=lse, plan=False)
    _check(load().attn_decode(_shape(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                              _ptr(v_scale), _ptr(page_table), float(sm_scale), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse),
                              _stream(stream)))


def attn_combine(shape, workspace, out, lse=None, stream=None) -> None:
    _need_step(shape, out=out, lse=lse, decode=False, plan=False)
    _check(load().attn_combine(_shape(shape), _ptr(workspace), workspace.numel() * workspace.element_size(),
                               _ptr(out), _ptr(lse), _stream(stream)))


def attn_workspace_init(shape, workspace, stream=None) -> None:
    _check(load().attn_workspace_init(_shape(shape), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))


def attn_step(shape, q, k_cache, v_cache, k_scale, v_scale, page_table, lengths, sm_scale, workspace, out,
              lse=None, stream=None) -> None:
    _need_step(shape, q, k_cache, v_cache, k_scale, v_scale, page_table, lengths, out, lse)
    _check(load().attn_step(_shape(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                            _ptr(page_table), _ptr(lengths), float(sm_scale), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))


def attn_step_noalloc(shape, q, k_cache, v_cache, k_scale, v_scale, page_table, lengths, sm_scale, out,
                      lse=None, status=None, stream=None) -> None:
    """attn_step without a workspace (the library's per-GPU scratch; see the C
    header). ``status``: optional int32 device tensor of one element that
    receives the step's status bits."""
    _need_step(shape, q, k_cache, v_cache, k_scale, v_scale, page_table, lengths, out, lse)
    _need(status, "status", _I32, 1, optional=True)
    _on_gpu(status=status)
    _check(load().attn_step_noalloc(_shape(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                    _ptr(v_scale), _ptr(page_table), _ptr(lengths), float(sm_scale), _ptr(out),
                                    _ptr(lse), _ptr(status), _stream(stream)))


def attn_append_kv(shape, k_new, v_new, positions, page_table, k_cache, v_cache, k_scale=None, v_scale=None,
                   workspace=None, stream=None) -> None:
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _need_append(shape, k_new, v_new, positions, page_table, k_cache, v_cache, k_scale, v_scale)
    _check(load().attn_append_kv(_shape(shape), _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(page_table),
                                 _ptr(k_scale), _ptr(v_scale), _ptr(k_cache), _ptr(v_cache), _ptr(workspace),
                                 nbytes, _stream(stream)))


def attn_get_status(workspace, stream=None) -> int:
    out = ctypes.c_uint32()
    _check(load().attn_get_status(_ptr(workspace), ctypes.byref(out), _stream(stream)))
    return int(out.value)


def attn_read_plan(shape, workspace, stream=None) -> dict:
    """The plan arrays of the workspace. ATTN_SHARED: over items (cut to the
    header's item count), plus the item description."""
    import numpy as np
    B, Hkv, W = shape.batch, shape.num_kv_heads, attn_num_wgs(shape)
    n = 2 * B if shape.mode == ATTN_SHARED else B
    out = {
        "header": np.zeros(8, np.int32), "len_eff": np.zeros(n, np.int32),
        "tiles_prefix": np.zeros(n + 1, np.int32), "seg_prefix": np.zeros(n * Hkv + 1, np.int32),
        "first_wg": np.zeros(n * Hkv, np.int32), "wg_begin": np.zeros(W + 1, np.int32),
        "wg_start_b": np.zeros(W, np.int32),
    }
    keys = ("header", "len_eff", "tiles_prefix", "seg_prefix", "first_wg", "wg_begin", "wg_start_b")
    _check(load().attn_read_plan(_shape(shape), _ptr(workspace),
                                 *[ctypes.c_void_p(out[k].ctypes.data) for k in keys], _stream(stream)))
    if shape.mode != ATTN_SHARED:
        return out
    items = {k: np.zeros(n, np.int32) for k in ("item_req", "item_start", "item_m", "item_solo")}
    items.update({k: np.zeros(B, np.int32) for k in ("req_shared", "req_member", "req_own")})
    ikeys = ("item_req", "item_start", "item_m", "item_solo", "req_shared", "req_member", "req_own")
    _check(load().attn_read_plan_items(_shape(shape), _ptr(workspace),
                                       *[ctypes.c_void_p(items[k].ctypes.data) for k in ikeys], _stream(stream)))
    I = int(out["header"][4])
    out.update(items)
    for k in ("len_eff", "item_req", "item_start", "item_m", "item_solo"):
        out[k] = out[k][:I]
    out["tiles_prefix"] = out["tiles_prefix"][:I + 1]
    out["seg_prefix"] = out["seg_prefix"][:I * Hkv + 1]
    out["first_wg"] = out["first_wg"][:I * Hkv]
    return out


class Attention:
    """One decode-attention configuration with its own workspace.

    ``step`` enqueues attn_plan, attn_decode and attn_combine on the current
    stream; ``fused_step`` enqueues the single-launch attn_step. The workspace
    is a torch uint8 tensor (device memory only), prepared by
    attn_workspace_init when the object is made.
    """

    def __init__(self, shape: AttnShape, device="cuda", stream=None):
        self.shape = shape
        n = attn_workspace_bytes(shape)
        self.workspace = torch.empty(n + 256, dtype=torch.uint8, device=device)
        off = (-self.workspace.data_ptr()) % 256
        self.workspace = self.workspace[off:off + n]
        attn_workspace_init(shape, self.workspace, stream)
        # per-call arguments that do not change (the shape is not to be edited
        # after construction): the C shape and the workspace
        self._cshape = ctypes.byref(shape.c())
        self._ws = (ctypes.c_void_p(self.workspace.data_ptr()), n)

    def fused_step(self, q, k_cache, v_cache, page_table, lengths, sm_scale, out, lse=None, k_scale=None,
                   v_scale=None, stream=None):
        _need_step(self.shape, q, k_cache, v_cache, k_scale, v_scale, page_table, lengths, out, lse)
        _check(load().attn_step(self._cshape, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                _ptr(v_scale), _ptr(page_table), _ptr(lengths), float(sm_scale), self._ws[0],
                                self._ws[1], _ptr(out), _ptr(lse), _stream(stream)))

    def plan(self, lengths, page_table, stream=None):
        attn_plan(self.shape, lengths, page_table, self.workspace, stream)

    def decode(self, q, k_cache, v_cache, page_table, sm_scale, out, lse=None, k_scale=None,
               v_scale=None, stream=None):
        attn_decode(self.shape, q, k_cache, v_cache, k_scale, v_scale, page_table, sm_scale,
                    self.workspace, out, lse, stream)

    def combine(self, out, lse=None, stream=None):
        attn_combine(self.shape, self.workspace, out, lse, stream)

    def step(self, q, k_cache, v_cache, page_table, lengths, sm_scale, out, lse=None, k_scale=None,
             v_scale=None, stream=None):
        self.plan(lengths, page_table, stream)
        self.decode(q, k_cache, v_cache, page_table, sm_scale, out, lse, k_scale, v_scale, stream)
        self.combine(out, lse, stream)

    def append_kv(self, k_new, v_new, positions, page_table, k_cache, v_cache, k_scale=None, v_scale=None,
                  stream=None):
        _need_append(self.shape, k_new, v_new, positions, page_table, k_cache, v_cache, k_scale, v_scale)
        _check(load().attn_append_kv(self._cshape, _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(page_table),
                                     _ptr(k_scale), _ptr(v_scale), _ptr(k_cache), _ptr(v_cache), self._ws[0],
                                     self._ws[1], _stream(stream)))

    def status(self, stream=None) -> int:
        return attn_get_status(self.workspace, stream)

    def read_plan(self, stream=None) -> dict:
        return attn_read_plan(self.shape, self.workspace, stream)


# ---------------------------------------------------------------- router GEMM --

def router_split_weights(w, w_hi, w_lo, stream=None):
    """w_hi = bf16(w), w_lo = bf16(256 (w - w_hi)) on the device (tensors: w
    fp32, w_hi / w_lo bf16 or int16 of w's size)."""
    _need(w, "w", _F32, w.numel())
    _need(w_hi, "w_hi", _HALFWORD, w.numel())
    _need(w_lo, "w_lo", _HALFWORD, w.numel())
    _on_gpu(w=w, w_hi=w_hi, w_lo=w_lo)
    _check(load().router_split_weights(_ptr(w), _ptr(w_hi), _ptr(w_lo), ctypes.c_int64(w.numel()),
                                       _stream(stream)))


def router_workspace_bytes(M, K, E) -> int:
    return int(load().router_workspace_bytes(int(M), int(K), int(E)))


class RouterGemm:
    """y = x w^T with split bf16 weights for one (M, K, E); owns its workspace."""

    def __init__(self, M, K, E, device="cuda"):
        self.M, self.K, self.E = int(M), int(K), int(E)
        n = router_workspace_bytes(self.M, self.K, self.E)   # 0 also for an invalid shape: router_gemm says which
        self.workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=device) if n else None
        self._ws = (_ptr(self.workspace), ctypes.c_size_t(n)) if n else (None, ctypes.c_size_t(0))

    def __call__(self, x, w_hi, w_lo, y, stream=None):
        _need(x, "x", _BF16, self.M * self.K)
        _need(w_hi, "w_hi", _HALFWORD, self.E * self.K)
        _need(w_lo, "w_lo", _HALFWORD, self.E * self.K)
        _need(y, "y", _F32, self.M * self.E)
        _on_gpu(x=x, w_hi=w_hi, w_lo=w_lo, y=y)
        _check(load().router_gemm(self.M, self.K, self.E, _ptr(x), _ptr(w_hi), _ptr(w_lo), _ptr(y), self._ws[0],
                                  self._ws[1], _stream(stream)))
