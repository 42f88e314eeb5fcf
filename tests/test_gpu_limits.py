"""GPU parity at the limits of the interface (include/vlkv_attn.h).

The variable-length decode step [Tencent HPC lands in SGLang, challenging
default inference kernels, sec. "Why Tencent HPC matters for online model
serving"] at the edges of what the library accepts: the largest batch the
planners take (8192 requests, whose tile prefix the single launch keeps in
LDS), the largest query-head group (16 per kv head), a prefix-shared batch
with more plan items than that (the shared planner's tile prefix no longer
fits its LDS copy), pages far larger than a tile, tiles of 16 blocks, and more
workgroups than units. Each case is checked against the fp64 CPU reference
(every request, or sampled requests plus every empty one), plans against the
CPU plan specification byte for byte, and the single launch against the
three-launch step bit for bit.
"""
import numpy as np
import pytest

import oracle
from variable_length_kv_amd import lib as L
from variable_length_kv_amd import workloads as wl

from gpu_helpers import check_against_oracle, device_inputs, run, shape_for

pytestmark = pytest.mark.gpu

MAX_BATCH = 8192


def _max_batch_case(kv):
    rng = np.random.default_rng(11)
    lengths = rng.integers(1, 160, MAX_BATCH)
    lengths[rng.random(MAX_BATCH) < 0.1] = 0
    lengths[:4] = [0, 1, 159, 16]
    return wl.make_case("max_batch", lengths, Hq=16, Hkv=1, P=16, kv_dtype=kv, seed=11)


def _sampled_and_empty(c, n=48, seed=0):
    rng = np.random.default_rng(seed)
    ids = set(rng.choice(c.B, n, replace=False).tolist()) | {0, 1, 2, 3, c.B - 1}
    return sorted(ids)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_max_batch_max_group(kv):
    """8192 requests (one in ten empty), 16 query heads on one kv head."""
    c = _max_batch_case(kv)
    t = device_inputs(c)
    W = 512
    out, lse, att = run(c, t=t, W=W)
    got = att.read_plan()
    ref = oracle.plan(L.ATTN_DYNAMIC, c.lengths, c.Hkv, c.P, c.pt_stride, 64, W)
    for k in ("header", "len_eff", "tiles_prefix", "seg_prefix", "first_wg", "wg_begin", "wg_start_b"):
        assert np.array_equal(got[k], ref[k]), k
    empty = np.flatnonzero(c.lengths == 0)
    assert np.all(out[empty] == 0) and np.all(lse[empty] == -np.inf)
    check_against_oracle(c, out, lse, req_ids=_sampled_and_empty(c), what=f"B=8192 {kv}")
    fo, fl, fatt = run(c, t=t, W=W, fused=True)
    assert np.array_equal(fo, out) and np.array_equal(fl, lse)
    assert att.status() == 0 and fatt.status() == 0


def test_max_batch_static():
    c = _max_batch_case("bf16")
    out, lse, _ = run(c, mode=L.ATTN_STATIC, W=512, S=2)
    check_against_oracle(c, out, lse, req_ids=_sampled_and_empty(c, seed=1), what="B=8192 static")


def test_max_batch_shared_items_beyond_lds():
    """8192 requests in groups of 4 sharing a 64-token prefix (4 pages, one
    tile): the shared plan has more items than the planner's LDS copy of the
    tile prefix holds, so it reads the prefix back from memory."""
    rng = np.random.default_rng(12)
    lengths = rng.integers(65, 140, MAX_BATCH)
    groups = [(4 * i, 4, 4) for i in range(MAX_BATCH // 4)]
    G = 4
    c = wl.make_shared_case("max_batch_shared", lengths, groups, Hq=G, Hkv=1, P=16, seed=12)
    W = 512
    p = oracle.plan_shared(c.lengths, c.page_table, c.Hkv, G, c.P, c.num_pages, 64, W)
    assert len(p["item_req"]) > MAX_BATCH
    out, lse, att = run(c, mode=L.ATTN_SHARED, W=W)
    got = att.read_plan()
    for k in ("header", "tiles_prefix", "seg_prefix", "first_wg", "wg_begin", "item_req", "item_start", "item_m",
              "item_solo", "req_shared", "req_member", "req_own"):
        assert got[k].tolist() == p[k].tolist(), k
    check_against_oracle(c, out, lse, req_ids=_sampled_and_empty(c, seed=2), what="B=8192 shared")
    assert att.status() == 0


@pytest.mark.parametrize("T", [64, 256])
def test_pages_larger_than_tiles(T):
    """1024-token pages: a tile is a slice of one page; lengths end before,
    at and after page and tile edges."""
    lengths = [1, 63, 64, 65, 1023, 1024, 1025, 3000, 5000, 0, 2048]
    c = wl.make_case("big_pages", lengths, Hq=8, Hkv=2, P=1024, seed=13)
    t = device_inputs(c)
    for W in (3, 64, 1024):
        out, lse, _ = run(c, t=t, T=T, W=W)
        check_against_oracle(c, out, lse, what=f"P=1024 T={T} W={W}")
        fo, fl, _ = run(c, t=t, T=T, W=W, fused=True)
        assert np.array_equal(fo, out) and np.array_equal(fl, lse)


def test_tiles_of_sixteen_blocks():
    """T = 1024 tokens per tile (16 blocks of 64): one unit spans many blocks,
    and a request's last tile is short."""
    lengths = [1024, 1025, 2047, 4100, 7, 0, 3333]
    c = wl.make_case("big_tiles", lengths, Hq=16, Hkv=2, P=32, seed=14)
    t = device_inputs(c)
    for W in (1, 5, 100):
        out, lse, _ = run(c, t=t, T=1024, W=W)
        check_against_oracle(c, out, lse, what=f"T=1024 W={W}")
        fo, fl, _ = run(c, t=t, T=1024, W=W, fused=True)
        assert np.array_equal(fo, out) and np.array_equal(fl, lse)


def test_more_workgroups_than_units():
    """65536 workgroups for a batch of a few dozen units: the plan caps the
    effective count at the unit count and the rest exit at once."""
    lengths = [5, 300, 129, 0, 64]
    c = wl.make_case("few_units", lengths, Hq=8, Hkv=1, P=16, seed=15)
    t = device_inputs(c)
    W = 1 << 16
    out, lse, att = run(c, t=t, W=W)
    check_against_oracle(c, out, lse, what="W=65536")
    got = att.read_plan()
    ref = oracle.plan(L.ATTN_DYNAMIC, c.lengths, c.Hkv, c.P, c.pt_stride, 64, W)
    assert np.array_equal(got["wg_begin"], ref["wg_begin"])
    fo, fl, _ = run(c, t=t, W=W, fused=True)
    assert np.array_equal(fo, out) and np.array_equal(fl, lse)
    L.attn_check_shape(shape_for(c, W=W))
