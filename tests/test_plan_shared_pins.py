"""Pins for the prefix-shared plan specification in the CPU reference (no GPU).

The source article lists prefix caching among the situations the kernels must
handle [Tencent HPC lands in SGLang, challenging default inference kernels,
sec. "Why Tencent HPC matters for online model serving"]: requests whose page
tables begin with the same physical pages read the same cached rows there.
``oracle.plan_shared`` decomposes each step into items (a group's shared prefix
once, then each request's own rest) and partitions (item, kv head, tile) units
like the dynamic plan. These tests pin it against hand-worked examples
(tests/golden/plan_shared_examples.json), against the already pinned dynamic
plan when nothing is shared, and against a token-level brute force of what
"shared" means on random page tables with planted prefixes.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "plan_shared_examples.json")
KEYS = ("header", "item_req", "item_start", "item_len", "item_m", "item_solo", "req_shared", "req_member", "req_own",
        "tiles_prefix", "seg_prefix", "first_wg", "wg_begin", "wg_start")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_hand_worked(ex):
    p = oracle.plan_shared(ex["lengths"], np.array(ex["page_table"], np.int32), ex["Hkv"], ex["G"], ex["P"],
                           ex["num_pages"], ex["T"], ex["W"])
    for k in KEYS:
        assert p[k].tolist() == ex[k], k


def _brute_share(pt, Le, P, T, num_pages):
    """Tokens request b shares with b-1, by checking every token: the largest
    multiple of T such that all earlier tokens exist in both requests and sit
    in the same valid physical page."""
    B = len(Le)
    share = [0] * B
    for b in range(1, B):
        t = 0
        while t < min(Le[b], Le[b - 1]):
            j = t // P
            x, y = int(pt[b, j]), int(pt[b - 1, j])
            if x != y or not 0 <= x < num_pages:
                break
            t += 1
        share[b] = t // T * T
    return share


def _expected_items(Le, share, R):
    """Items from the definition: runs of share > 0 cut into groups of R."""
    items, req_shared, req_member, req_own = [], [], [], []
    b = 0
    B = len(Le)
    groups = []
    while b < B:
        e = b + 1
        while e < B and share[e] > 0:
            e += 1
        for g0 in range(b, e, R):
            groups.append(list(range(g0, min(g0 + R, e))))
        b = e
    for grp in groups:
        Ls = min(share[k] for k in grp[1:]) if len(grp) > 1 else 0
        if len(grp) > 1:
            si = len(items)
            items.append((grp[0], 0, Ls, len(grp), 0))
        for k, r in enumerate(grp):
            req_shared.append(si if len(grp) > 1 else -1)
            req_member.append(k if len(grp) > 1 else 0)
            req_own.append(len(items))
            items.append((r, Ls, Le[r] - Ls, 1, 0) if len(grp) > 1 else (r, 0, Le[r], 1, 1))
    return items, req_shared, req_member, req_own


def _planted(rng):
    B = int(rng.integers(1, 30))
    P = int(rng.choice([16, 32, 64]))
    T = int(rng.choice([64, 128]))
    pt_stride = int(rng.integers(1, 24))
    limit = pt_stride * P
    lengths = rng.integers(0, limit + 1, B)
    if rng.random() < 0.3:
        lengths[rng.integers(B)] = limit + 7          # invalid
    if rng.random() < 0.3:
        lengths[rng.integers(B)] = 0
    num_pages = B * pt_stride + 5
    pt = rng.permutation(num_pages)[:B * pt_stride].reshape(B, pt_stride).astype(np.int32)
    for b in range(1, B):
        if rng.random() < 0.6:
            k = int(rng.integers(0, pt_stride + 1))
            pt[b, :k] = pt[b - 1, :k]
    if rng.random() < 0.3:                            # an invalid id somewhere, possibly inside a shared prefix
        b = int(rng.integers(B))
        pt[b:, int(rng.integers(pt_stride))] = -1 if rng.random() < 0.5 else num_pages + 3
    Hkv = int(rng.choice([1, 2, 8]))
    G = int(rng.choice([1, 2, 4, 8, 16]))
    W = int(rng.choice([1, 3, 7, 64, 512]))
    return lengths.astype(np.int64), pt, Hkv, G, P, num_pages, T, W


@pytest.mark.parametrize("seed", range(80))
def test_random_against_token_brute_force(seed):
    rng = np.random.default_rng(seed)
    lengths, pt, Hkv, G, P, num_pages, T, W = _planted(rng)
    B, pt_stride = pt.shape
    limit = pt_stride * P
    Le = [int(L) if 0 <= L <= limit else 0 for L in lengths]
    R = max(1, (32 if G >= 8 else 16) // G)
    p = oracle.plan_shared(lengths, pt, Hkv, G, P, num_pages, T, W)
    share = _brute_share(pt, Le, P, T, num_pages)
    items, req_shared, req_member, req_own = _expected_items(Le, share, R)
    got = list(zip(*(p[k].tolist() for k in ("item_req", "item_start", "item_len", "item_m", "item_solo"))))
    assert got == items
    assert p["req_shared"].tolist() == req_shared
    assert p["req_member"].tolist() == req_member
    assert p["req_own"].tolist() == req_own
    # what sharing must guarantee: every member reads the leader's valid pages on [0, Ls)
    for (r, s, n, m, solo) in items:
        if m > 1:
            assert n > 0 and n % T == 0 and m <= R
            for k in range(m):
                assert Le[r + k] >= n
                for j in range(0, n, P):
                    assert pt[r + k, j // P] == pt[r, j // P] and 0 <= pt[r, j // P] < num_pages
    # every request's tokens covered exactly once by its items
    for b in range(B):
        cov = []
        if req_shared[b] >= 0:
            _, s, n, _, _ = items[req_shared[b]]
            cov += list(range(s, s + n))
        _, s, n, _, _ = items[req_own[b]]
        cov += list(range(s, s + n))
        assert cov == list(range(Le[b]))
    # units over items: the uniform partition and its segments
    units = [(i, g, t) for i, it in enumerate(items) for g in range(Hkv) for t in range(-(-it[2] // T))]
    N = len(units)
    status, hN, We, maxle, hI, hR, total, hT = p["header"].tolist()
    assert (hN, We, hI, hR, hT) == (N, min(W, N), len(items), R, T)
    assert status == (1 if any(not 0 <= L <= limit for L in lengths) else 0)
    assert maxle == max(Le, default=0)
    owner = {}
    for w in range(We):
        for u in range(p["wg_begin"][w], p["wg_begin"][w + 1]):
            owner[u] = w
    assert sorted(owner) == list(range(N))
    segs, first = {}, {}
    for u, (i, g, t) in enumerate(units):
        segs.setdefault(i * Hkv + g, set()).add(owner[u])
        first.setdefault(i * Hkv + g, owner[u])
    pref = [0]
    for ig in range(len(items) * Hkv):
        pref.append(pref[-1] + len(segs.get(ig, ())))
        assert p["first_wg"][ig] == first.get(ig, -1)
    assert p["seg_prefix"].tolist() == pref
    for w in range(W):
        assert p["wg_start"][w] == (units[p["wg_begin"][w]][0] if w < We else len(items))


@pytest.mark.parametrize("seed", range(20))
def test_without_sharing_the_plan_is_the_dynamic_plan(seed):
    """Distinct page ids everywhere: one solo item per request, and the unit
    partition is exactly the (separately pinned) dynamic plan's."""
    rng = np.random.default_rng(500 + seed)
    lengths, pt, Hkv, G, P, num_pages, T, W = _planted(rng)
    B, pt_stride = pt.shape
    pt = rng.permutation(num_pages)[:B * pt_stride].reshape(B, pt_stride).astype(np.int32)
    p = oracle.plan_shared(lengths, pt, Hkv, G, P, num_pages, T, W)
    d = oracle.plan(0, lengths, Hkv, P, pt_stride, T, W)
    assert p["item_req"].tolist() == list(range(B))
    assert p["item_start"].tolist() == [0] * B and p["item_m"].tolist() == [1] * B
    assert p["item_solo"].tolist() == [1] * B and p["req_shared"].tolist() == [-1] * B
    assert p["item_len"].tolist() == d["len_eff"].tolist()
    for a, b in (("tiles_prefix", "tiles_prefix"), ("seg_prefix", "seg_prefix"), ("first_wg", "first_wg"),
                 ("wg_begin", "wg_begin"), ("wg_start", "wg_start_b")):
        assert p[a].tolist() == d[b].tolist(), a
    h, hd = p["header"].tolist(), d["header"].tolist()
    assert h[:4] == hd[:4] and h[4] == B and h[6:] == hd[6:]


def test_refuses_bad_arguments():
    pt = np.zeros((2, 2), np.int32)
    with pytest.raises(ValueError):
        oracle.plan_shared([1, 2], pt, 0, 8, 16, 4, 64, 8)
    with pytest.raises(ValueError):
        oracle.plan_shared([1, 2], pt, 1, 0, 16, 4, 64, 8)
    with pytest.raises(ValueError):
        oracle.plan_shared([1, 2], pt, 1, 8, 16, 0, 64, 8)
