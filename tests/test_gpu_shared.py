"""GPU parity of the prefix-shared plan and decode (mode ATTN_SHARED).

Requests whose page tables begin with the same physical pages (prefix caching,
which the source article lists among the situations the kernels must handle
[Tencent HPC lands in SGLang, challenging default inference kernels, sec. "Why
Tencent HPC matters for online model serving"]) read that prefix once, as one
item whose query rows are several requests' heads. The device plan must equal
the CPU specification (oracle.plan_shared) array for array; the attention
result must match the fp64 CPU reference per request, whatever the grouping.
"""
import json

import numpy as np
import pytest
import torch

import oracle
from variable_length_kv_amd import lib as L
from variable_length_kv_amd import workloads as wl

from gpu_helpers import check_against_oracle, dev, device_inputs, run
from test_plan_shared_pins import GOLDEN, _planted

pytestmark = pytest.mark.gpu

ITEM_KEYS = ("item_req", "item_start", "item_m", "item_solo", "req_shared", "req_member", "req_own")
PLAN_KEYS = ("header", "tiles_prefix", "seg_prefix", "first_wg", "wg_begin")


def _device_plan(lengths, pt, Hkv, G, P, num_pages, T, W):
    B, stride = pt.shape
    shape = L.AttnShape(batch=B, num_q_heads=G * Hkv, num_kv_heads=Hkv, page_size=P, num_pages=num_pages,
                        pt_stride=stride, num_wgs=W, tile_tokens=T, mode=L.ATTN_SHARED)
    att = L.Attention(shape, dev())
    ln = torch.from_numpy(np.asarray(lengths, np.int32)).to(dev())
    ptd = torch.from_numpy(np.ascontiguousarray(pt, np.int32)).to(dev())
    att.plan(ln, ptd)
    return att.read_plan()


def _compare_plan(got, ref):
    for k in PLAN_KEYS + ITEM_KEYS:
        assert got[k].tolist() == ref[k].tolist(), k
    assert got["len_eff"].tolist() == ref["item_len"].tolist()
    assert got["wg_start_b"].tolist() == ref["wg_start"].tolist()


@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda e: e["name"])
def test_device_plan_hand_worked(ex):
    pt = np.array(ex["page_table"], np.int32)
    got = _device_plan(ex["lengths"], pt, ex["Hkv"], ex["G"], ex["P"], ex["num_pages"], ex["T"], ex["W"])
    ref = oracle.plan_shared(ex["lengths"], pt, ex["Hkv"], ex["G"], ex["P"], ex["num_pages"], ex["T"], ex["W"])
    _compare_plan(got, ref)


@pytest.mark.parametrize("seed", range(40))
def test_device_plan_matches_spec(seed):
    rng = np.random.default_rng(seed)
    lengths, pt, Hkv, G, P, num_pages, T, W = _planted(rng)
    got = _device_plan(lengths, pt, Hkv, G, P, num_pages, T, W)
    ref = oracle.plan_shared(lengths, pt, Hkv, G, P, num_pages, T, W)
    _compare_plan(got, ref)


def test_device_plan_long_prefixes_and_large_batch():
    """Many requests, prefixes of hundreds of pages: the page-slot comparison
    runs over several 256-slot steps."""
    lengths, groups = wl.shared_prefix_lengths(40, 5, 24576, 1, 3000, 64, seed=3)
    pt, num_pages = wl.shared_page_table(lengths, groups, 64, 7)
    for G in (1, 4, 8, 16):
        got = _device_plan(lengths, pt, 8, G, 64, num_pages, 64, 512)
        ref = oracle.plan_shared(lengths, pt, 8, G, 64, num_pages, 64, 512)
        _compare_plan(got, ref)


@pytest.mark.parametrize("run", [255, 256, 257, 511, 512, 513])
def test_device_plan_shared_runs_at_step_boundaries(run):
    """Common runs of page ids that end just before, at and just after the
    planner's 256-slot comparison steps (one and two steps), for a group of
    four requests after a request that shares nothing, one member ending a
    page inside the run."""
    P, stride = 16, 600
    rng = np.random.default_rng(run)
    num_pages = 5 * stride + 10
    perm = rng.permutation(num_pages).astype(np.int32)
    pt = perm[:5 * stride].reshape(5, stride).copy()
    for b in (2, 3, 4):
        pt[b, :run] = pt[1, :run]                   # requests 1-4 share their first `run` pages
    # (request 2 runs past the shared pages, so its comparison with request 1
    # goes on into a further step whose first slot already differs)
    lengths = np.array([stride * P, stride * P, stride * P, (run - 1) * P + 3, stride * P], np.int64)
    for G in (1, 8):
        for W in (1, 37):
            got = _device_plan(lengths, pt, 2, G, P, num_pages, 64, W)
            ref = oracle.plan_shared(lengths, pt, 2, G, P, num_pages, 64, W)
            _compare_plan(got, ref)


def _shared(lengths, groups, G, Hkv=2, P=16, kv="bf16", seed=0):
    return wl.make_shared_case("s", lengths, groups, Hq=G * Hkv, Hkv=Hkv, P=P, kv_dtype=kv, seed=seed)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_parity_with_shared_prefixes(G, kv):
    """Groups of several sizes (some beyond a pass's requests, so cut into
    several shared items), prefixes of several lengths, a lone request, and
    suffixes from one token to several tiles."""
    lengths = [300, 290, 310, 700, 75, 64 * 5 + 1, 64 * 5 + 200, 1000, 999, 1001, 1002, 1003, 1100, 130]
    groups = [(0, 3, 16), (5, 2, 20), (7, 6, 48)]
    c = _shared(lengths, groups, G, kv=kv, seed=G)
    p = oracle.plan_shared(c.lengths, c.page_table, c.Hkv, G, c.P, c.num_pages, 64, 37)
    assert (p["item_m"] > 1).any() or G == 16
    for W in (5, 37, 2 * 256):
        out, lse, att = run(c, mode=L.ATTN_SHARED, W=W)
        check_against_oracle(c, out, lse, what=f"G={G} {kv} W={W}")
        assert att.status() == 0


def test_no_sharing_is_bitwise_the_dynamic_mode():
    """Distinct pages everywhere: every item is a whole request, and the result
    is the dynamic mode's bit for bit."""
    c = wl.make_case("t", [1000, 3, 250, 4000, 0, 777], Hq=16, Hkv=2, P=32, seed=10)
    t = device_inputs(c)
    for W in (7, 64):
        a = run(c, t=t, W=W)
        b = run(c, t=t, W=W, mode=L.ATTN_SHARED)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_step_entry_equals_three_calls(kv):
    lengths, groups = wl.shared_prefix_lengths(3, 3, 512, 1, 300, 16, seed=4)
    c = _shared(lengths, groups, 8, kv=kv, seed=4)
    t = device_inputs(c)
    a = run(c, t=t, W=29, mode=L.ATTN_SHARED)
    b = run(c, t=t, W=29, mode=L.ATTN_SHARED, fused=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    check_against_oracle(c, a[0], a[1], what=kv)


def test_members_ending_inside_or_at_the_end_of_the_prefix():
    """Some members are shorter than the aliased pages (sharing is capped by
    the shorter length, whole tiles only), one ends exactly where the prefix
    does (its own item is empty), one is empty. Slack rows are not poisoned
    here: the shared pages hold other members' valid rows."""
    lengths = [512, 512, 200, 130, 512, 600, 0, 64]
    groups = [(0, 6, 32)]
    for G in (4, 8):
        c = _shared(lengths, groups, G, seed=5)
        p = oracle.plan_shared(c.lengths, c.page_table, c.Hkv, G, c.P, c.num_pages, 64, 9)
        # at G = 8 (groups of 4) the second group's first member ends exactly at its prefix
        assert (p["item_len"][p["item_solo"] == 0] == 0).any() or G == 4
        out, lse, _ = run(c, mode=L.ATTN_SHARED, W=9, poison=False)
        check_against_oracle(c, out, lse, what=f"G={G}")


def test_bad_page_inside_a_shared_prefix():
    """An invalid page id stops the sharing at that slot; the rows of that
    page are skipped (status bit). Skipping a whole page equals attending over
    the request without it (the softmax sum does not depend on token order),
    so the reference is the CPU decode with that page slot removed."""
    lengths = [400, 400, 400]
    c = _shared(lengths, [(0, 3, 20)], 8, seed=6)
    pt = c.page_table.copy()
    pt[:, 9] = c.num_pages + 5      # slot 9 of all three (aliased) rows
    bad = wl.Case(c.name, c.B, c.Hq, c.Hkv, c.D, c.P, c.lengths, pt, c.num_pages, c.kv_dtype, c.q, c.k_cache,
                  c.v_cache, c.k_scale, c.v_scale, c.sm_scale)
    p = oracle.plan_shared(bad.lengths, pt, bad.Hkv, 8, bad.P, bad.num_pages, 64, 11)
    assert p["item_len"][0] == 128 and p["item_m"][0] == 3   # slots 0-8 shared, whole tiles; one group
    out, lse, att = run(bad, mode=L.ATTN_SHARED, W=11)
    assert att.status() & L.ATTN_STATUS_BAD_PAGE
    without = np.concatenate([pt[:, :9], pt[:, 10:], np.full((3, 1), -1, np.int32)], axis=1)
    ref = wl.Case(c.name, c.B, c.Hq, c.Hkv, c.D, c.P, c.lengths - c.P, without, c.num_pages, c.kv_dtype, c.q,
                  c.k_cache, c.v_cache, c.k_scale, c.v_scale, c.sm_scale)
    check_against_oracle(ref, out, lse, what="bad page skipped")


def test_run_to_run_determinism():
    lengths, groups = wl.shared_prefix_lengths(4, 4, 1024, 1, 500, 16, seed=8)
    c = _shared(lengths, groups, 4, seed=8)
    t = device_inputs(c)
    a = run(c, t=t, W=41, mode=L.ATTN_SHARED)
    b = run(c, t=t, W=41, mode=L.ATTN_SHARED)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_bench_scale_sampled():
    """The benchmark's prefix-caching batch at full size (64 requests, 8192-token
    shared prompts, 8 kv heads, page 64): sampled requests against the CPU
    reference, in the launch configuration the benchmark times."""
    lengths, groups = wl.shared_prefix_lengths(16, 4, 8192, 64, 2048, 64, seed=0)
    for hq in (64, 32):
        c = wl.make_shared_case("shared", lengths, groups, Hq=hq, Hkv=8, P=64, seed=0)
        out, lse, att = run(c, mode=L.ATTN_SHARED, W=0, fused=True)   # the library's default count
        p = att.read_plan()
        R = max(1, (32 if c.G >= 8 else 16) // c.G)
        assert (np.asarray(p["item_m"]) > 1).sum() == 16 * -(-4 // R)   # groups of 4 cut into passes of R
        ids = [0, 1, 2, 3, 17, 30, 45, 63]
        check_against_oracle(c, out, lse, req_ids=ids, what=f"hq={hq}")
        assert att.status() == 0
