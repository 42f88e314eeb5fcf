"""Variable-length paged decode attention for MI355X (gfx950).

The compute path is the HIP library libvlkv_attn.so (C ABI in
include/vlkv_attn.h); ``lib`` is its ctypes binding and ``workloads`` holds
the seeded synthetic inputs. Build with ``python -m variable_length_kv_amd.build``.
"""
from .lib import (  # noqa: F401
    ATTN_DYNAMIC, ATTN_KV_BF16, ATTN_KV_FP8_E4M3, ATTN_STATIC, Attention, AttnError, AttnShape,
    attn_append_kv, attn_check_shape, attn_combine, attn_decode, attn_device_cu_count, attn_get_status, attn_plan,
    attn_read_plan, attn_static_splits, attn_workspace_bytes,
)
