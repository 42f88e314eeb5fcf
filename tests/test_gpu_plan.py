"""The device planner reproduces the CPU plan specification byte for byte.

The plan is the per-step mapping of uniform KV tiles to workgroups that the
source article says is rebuilt as request lengths change [Tencent HPC lands in
SGLang, challenging default inference kernels, sec. "Why Tencent HPC matters
for online model serving"]; the CPU reference defines it exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from variable_length_kv_amd import lib as L
from variable_length_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _device_plan(lengths, Hkv, P, pt_stride, T, W, mode, S=0):
    shape = L.AttnShape(batch=len(lengths), num_q_heads=Hkv, num_kv_heads=Hkv, page_size=P,
                        num_pages=1, pt_stride=pt_stride, num_wgs=W, tile_tokens=T, mode=mode,
                        static_splits=S)
    att = L.Attention(shape, "cuda:0")
    ln = torch.tensor(np.asarray(lengths, np.int64), dtype=torch.int32, device="cuda:0")
    pt = torch.zeros(len(lengths), pt_stride, dtype=torch.int32, device="cuda:0")
    att.plan(ln, pt)
    got = att.read_plan()
    return got, L.attn_static_splits(shape) if mode == L.ATTN_STATIC else 0


def _compare(lengths, Hkv, P, pt_stride, T, W, mode, S=0):
    got, S_eff = _device_plan(lengths, Hkv, P, pt_stride, T, W, mode, S)
    if W == 0:   # the library default: two per compute unit, or one on small steps
        cus = L.attn_device_cu_count(0)
        ref = oracle.plan(mode, lengths, Hkv, P, pt_stride, T, 2 * cus, S_eff, cus=cus if mode == 0 else 0)
    else:
        ref = oracle.plan(mode, lengths, Hkv, P, pt_stride, T, W, S_eff)
    keys = ["header", "len_eff", "tiles_prefix", "seg_prefix", "first_wg"]
    if mode == L.ATTN_DYNAMIC:
        keys += ["wg_begin", "wg_start_b"]
    for k in keys:
        assert np.array_equal(got[k], ref[k]), (k, got[k][:20], ref[k][:20])


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4])
@pytest.mark.parametrize("mode", [L.ATTN_DYNAMIC, L.ATTN_STATIC])
def test_workload_plans(cid, mode):
    lengths = wl.config_lengths(cid)
    Hkv, P = (1, 16) if cid == 0 else (8, 64)
    stride = int(-(-lengths.max() // P)) + 1
    for W in (0, 1, 256, 512, 2048):
        _compare(lengths, Hkv, P, stride, 64, W, mode)


def test_trace_plans_every_step():
    Ls, _ = wl.trace_lengths()
    stride = int(-(-Ls.max() // 64)) + 1
    for s in range(0, 256, 5):
        _compare(Ls[s], 8, 64, stride, 64, 512, L.ATTN_DYNAMIC)


def test_random_plans():
    rng = np.random.default_rng(0)
    for it in range(80):
        B = int(rng.integers(1, 3000))
        P = int(rng.choice([16, 64, 128]))
        T = int(rng.choice([64, 128, 256]))
        stride = int(rng.integers(1, 300))
        lengths = rng.integers(-3, stride * P + 20, B) * (rng.random(B) < 0.9)
        Hkv = int(rng.choice([1, 2, 8]))
        W = int(rng.choice([0, 1, 3, 512, 4096]))
        mode = int(rng.integers(2))
        _compare(lengths, Hkv, P, stride, T, W, mode, int(rng.integers(0, 5)))
