"""Pins for the integer tile-plan specification in the CPU reference (no GPU).

The source article describes the scheduler only in prose: each request's KV
work is cut into uniform tiles that are handed to CTAs by current load, and the
mapping is rebuilt as lengths change during decode; a static split-k policy is
the comparison point, and it either idles units or launches empty chunks for
short requests [Tencent HPC lands in SGLang, challenging default inference
kernels, sec. "Why Tencent HPC matters for online model serving"]. These tests
check ``oracle.plan`` against hand-worked examples (tests/golden) and against
brute-force enumeration of every unit on small random inputs.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_examples.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("ex", _golden()["dynamic"], ids=lambda e: str(e["lengths"]))
def test_dynamic_hand_worked(ex):
    p = oracle.plan(0, ex["lengths"], ex["Hkv"], ex["P"], ex["pt_stride"], ex["T"], ex["W"])
    for k in ("header", "len_eff", "tiles_prefix", "seg_prefix", "first_wg", "wg_begin", "wg_start_b"):
        assert p[k].tolist() == ex[k], k


@pytest.mark.parametrize("ex", _golden()["static"], ids=lambda e: str(e["lengths"]))
def test_static_hand_worked(ex):
    p = oracle.plan(1, ex["lengths"], ex["Hkv"], ex["P"], ex["pt_stride"], ex["T"], 1, ex["S"])
    for k in ("header", "len_eff", "tiles_prefix", "seg_prefix", "first_wg"):
        assert p[k].tolist() == ex[k], k


def _brute_units(lengths, Hkv, T, limit):
    units = []
    for b, L in enumerate(lengths):
        Le = L if 0 <= L <= limit else 0
        n = -(-Le // T)
        for g in range(Hkv):
            for t in range(n):
                units.append((b, g, t))
    return units


def _random_inputs(rng):
    B = int(rng.integers(1, 40))
    P = int(rng.choice([16, 32, 64]))
    T = int(rng.choice([16, 64, 128]))
    pt_stride = int(rng.integers(1, 40))
    kind = rng.integers(4)
    if kind == 0:
        lengths = rng.integers(0, pt_stride * P + 1, B)
    elif kind == 1:  # one long, many short
        lengths = np.full(B, int(rng.integers(1, 40)))
        lengths[int(rng.integers(B))] = pt_stride * P
    elif kind == 2:  # with invalid entries
        lengths = rng.integers(-5, pt_stride * P + 50, B)
    else:  # many empties
        lengths = rng.integers(0, 3, B) * rng.integers(0, pt_stride * P + 1, B)
    Hkv = int(rng.choice([1, 2, 8]))
    W = int(rng.choice([1, 2, 3, 7, 64, 256, 1000]))
    return B, P, T, pt_stride, lengths.astype(np.int64), Hkv, W


@pytest.mark.parametrize("seed", range(60))
def test_dynamic_plan_against_enumeration(seed):
    rng = np.random.default_rng(seed)
    B, P, T, pt_stride, lengths, Hkv, W = _random_inputs(rng)
    limit = pt_stride * P
    p = oracle.plan(0, lengths, Hkv, P, pt_stride, T, W)
    units = _brute_units(lengths.tolist(), Hkv, T, limit)
    N = len(units)
    status, hN, We = p["header"][:3]
    assert hN == N and We == min(W, N)
    assert status == (1 if np.any((lengths < 0) | (lengths > limit)) else 0)
    assert p["len_eff"].tolist() == [int(L) if 0 <= L <= limit else 0 for L in lengths]
    # every unit owned by exactly one workgroup, ranges contiguous and in order
    owner = {}
    for w in range(We):
        lo, hi = p["wg_begin"][w], p["wg_begin"][w + 1]
        assert lo < hi
        for u in range(lo, hi):
            assert u not in owner
            owner[u] = w
    assert sorted(owner) == list(range(N))
    assert all(p["wg_begin"][w] == N for w in range(We, W + 1))
    # balance: sizes differ by at most one
    if We:
        sizes = np.diff(p["wg_begin"][:We + 1])
        assert sizes.max() - sizes.min() <= 1
        assert sizes.sum() == N
    # segments: maximal runs of one (b, g) inside one workgroup
    segs = {}
    first = {}
    for u, (b, g, t) in enumerate(units):
        key = (b * Hkv + g, owner[u])
        segs.setdefault(b * Hkv + g, set()).add(owner[u])
        first.setdefault(b * Hkv + g, owner[u])
    expect_prefix = [0]
    for bg in range(B * Hkv):
        expect_prefix.append(expect_prefix[-1] + len(segs.get(bg, ())))
        assert p["first_wg"][bg] == first.get(bg, -1)
        ws = sorted(segs.get(bg, ()))
        assert ws == list(range(ws[0], ws[-1] + 1)) if ws else True  # one run per workgroup span
    assert p["seg_prefix"].tolist() == expect_prefix
    # a workgroup shares at most two pairs with other workgroups: those of its
    # first and last units (the single launch's merge list holds two entries)
    for w in range(We):
        split = {bg for bg, ws in segs.items() if len(ws) > 1 and w in ws}
        lo, hi = p["wg_begin"][w], p["wg_begin"][w + 1]
        ends = {units[lo][0] * Hkv + units[lo][1], units[hi - 1][0] * Hkv + units[hi - 1][1]}
        assert split <= ends
    for w in range(W):
        if w < We:
            assert units[p["wg_begin"][w]][0] == p["wg_start_b"][w]
        else:
            assert p["wg_start_b"][w] == B
    # the plan is a pure function of its inputs
    p2 = oracle.plan(0, lengths, Hkv, P, pt_stride, T, W)
    assert all(np.array_equal(p[k], p2[k]) for k in p)


@pytest.mark.parametrize("seed", range(40))
def test_static_plan_against_enumeration(seed):
    rng = np.random.default_rng(1000 + seed)
    B, P, T, pt_stride, lengths, Hkv, _ = _random_inputs(rng)
    S = int(rng.integers(1, 9))
    limit = pt_stride * P
    p = oracle.plan(1, lengths, Hkv, P, pt_stride, T, 1, S)
    Le = [int(L) if 0 <= L <= limit else 0 for L in lengths]
    maxle = max(Le) if Le else 0
    C = p["header"][4]
    gran = P * T // math.gcd(P, T)
    assert p["header"][3] == maxle and p["header"][5] == S
    assert p["header"][1] == p["header"][2] == B * Hkv * S
    if maxle == 0:
        assert C == 0
    else:
        assert C % gran == 0 and C * S >= maxle and (C - gran) * S < maxle
    for b, L in enumerate(Le):
        covered = []
        for s in range(S):
            covered.extend(range(s * C, min((s + 1) * C, L)))
        assert covered == list(range(L))
    assert p["seg_prefix"].tolist() == [bg * S for bg in range(B * Hkv + 1)]


def test_plan_refuses_bad_arguments():
    with pytest.raises(ValueError):
        oracle.plan(0, [1, 2], 0, 16, 4, 64, 8)
    with pytest.raises(ValueError):
        oracle.plan(1, [1, 2], 1, 16, 4, 64, 8, 0)


def test_workload_plan_sizes():
    """Unit counts N at T = 64 for the four single-step workloads, by enumeration."""
    from variable_length_kv_amd import workloads as wl
    for cid, hkv in ((0, 1), (1, 8), (2, 8), (3, 8)):
        L = wl.config_lengths(cid)
        p = oracle.plan(0, L, hkv, 16 if cid == 0 else 64, 2048, 64, 512)
        assert p["header"][1] == len(_brute_units(L.tolist(), hkv, 64, 2048 * 64))


@pytest.mark.parametrize("tiles,w_eff", [(255, 4), (256, 8), (1, 1), (3, 3), (4, 4), (5, 4), (4000, 8)])
def test_default_workgroup_count_hand_worked(tiles, w_eff):
    """The library default (num_wgs = 0) on a device of 4 compute units: W = 8
    workgroups when that leaves at least 32 units each (N >= 256), else one per
    compute unit (4), and never more than N. One request of `tiles` 64-token
    tiles on one kv head has N = tiles units."""
    p = oracle.plan(0, [64 * tiles], 1, 64, tiles, 64, 8, cus=4)
    assert p["header"][1] == tiles and p["header"][2] == w_eff
    assert p["wg_begin"].tolist() == [w * tiles // w_eff if w <= w_eff else tiles for w in range(9)]
    with pytest.raises(ValueError):   # the default spans two workgroups per compute unit
        oracle.plan(0, [64], 1, 64, 1, 64, 7, cus=4)


@pytest.mark.parametrize("seed", range(20))
def test_default_workgroup_count_equals_explicit(seed):
    """With the default count the plan is the explicit plan for the count the
    rule picks, with the arrays padded to 2 * cus workgroups."""
    rng = np.random.default_rng(500 + seed)
    B, P, T, pt_stride, lengths, Hkv, _ = _random_inputs(rng)
    cus = int(rng.choice([1, 3, 8, 256]))
    p = oracle.plan(0, lengths, Hkv, P, pt_stride, T, 2 * cus, cus=cus)
    N = len(_brute_units(lengths.tolist(), Hkv, T, pt_stride * P))
    W = 2 * cus if N >= 64 * cus else cus
    q = oracle.plan(0, lengths, Hkv, P, pt_stride, T, W)
    assert p["header"].tolist() == q["header"].tolist()
    for k in ("len_eff", "tiles_prefix", "seg_prefix", "first_wg"):
        assert np.array_equal(p[k], q[k]), k
    assert p["wg_begin"][:W + 1].tolist() == q["wg_begin"].tolist()
    assert all(x == N for x in p["wg_begin"][W + 1:])
    assert p["wg_start_b"][:W].tolist() == q["wg_start_b"].tolist()
    assert all(x == B for x in p["wg_start_b"][W:])
