"""The seeded input recipes (no GPU): determinism and realized sizes."""
import numpy as np
import torch

from variable_length_kv_amd import workloads as wl


def test_realized_lengths_at_seed_0():
    sums = [int(wl.config_lengths(c).sum()) for c in range(5)]
    assert sums == [1281, 284965, 79000, 512126, 1648574]
    L3 = wl.config_lengths(3)
    assert L3.min() >= 128 and L3.max() <= 131072
    L1 = wl.config_lengths(1)
    assert L1.min() >= 1000 and L1.max() <= 16000


def test_trace_lengths_follow_the_rules():
    L, ev = wl.trace_lengths()
    assert L.shape == (256, 96)
    for s in range(255):
        grown = L[s] + 1
        changed = {slot for slot, _ in ev[s]}
        for b in range(96):
            if b in changed:
                assert 256 <= L[s + 1, b] <= 4096
            else:
                assert L[s + 1, b] == grown[b]


def test_generation_is_deterministic_and_thread_count_free():
    a = wl.normal_f32(5, (1,), 3 * wl.CHUNK + 17)
    old = wl._workers
    try:
        wl._workers = lambda: 1
        b = wl.normal_f32(5, (1,), 3 * wl.CHUNK + 17)
    finally:
        wl._workers = old
    assert np.array_equal(a, b)
    c1 = wl.make_case("x", [5, 40], Hq=4, Hkv=2, P=16, seed=3)
    c2 = wl.make_case("x", [5, 40], Hq=4, Hkv=2, P=16, seed=3)
    assert torch.equal(c1.k_cache, c2.k_cache) and np.array_equal(c1.page_table, c2.page_table)


def test_page_table_is_a_permutation():
    c = wl.config_case(0)
    used = np.concatenate([c.page_table[b, :-(-int(L) // c.P)] for b, L in enumerate(c.lengths)])
    assert sorted(used.tolist()) == list(range(c.num_pages))


def test_fp8_codes_saturate_and_scale():
    c = wl.make_case("x", [20, 1], Hq=4, Hkv=2, P=16, kv_dtype="fp8", seed=4)
    k = c.k_cache.view(torch.float8_e4m3fn).float()
    assert torch.isfinite(k).all() and k.abs().max() <= 448
    assert c.k_scale.shape == (2, 2) and (c.k_scale > 0).all()


def _small_trace():
    return wl.Trace(steps=40, slots=6, Hq=8, Hkv=2, P=16, seed=1, p_finish=0.15, new_lo=5, new_hi=70,
                    init_lo=10, init_hi=120)


def test_trace_host_state_is_consistent():
    tr = _small_trace()
    while tr.step < tr.steps - 1:
        tr.advance()
        P = tr.P
        used = []
        for b in range(tr.slots):
            n = -(-int(tr.lengths[b]) // P)
            assert (tr.page_table[b, :n] >= 0).all() and (tr.page_table[b, n:] == -1).all()
            used += tr.page_table[b, :n].tolist()
        # no page is owned twice, and owned pages are never on the free list
        assert len(used) == len(set(used))
        assert not (set(used) & set(tr.free))
        assert len(used) + len(tr.free) == tr.num_pages


def test_device_mirror_tracks_the_host_trace():
    from variable_length_kv_amd.trace import DeviceTrace
    tr = _small_trace()
    dt = DeviceTrace(tr, "cpu", poison=False)   # an exact copy (poisoning: test_trace_poison.py)
    assert dt.k.data_ptr() != tr.k_cache.data_ptr()
    for _ in range(tr.steps - 1):
        dt.advance()
        assert torch.equal(dt.k, tr.k_cache) and torch.equal(dt.v, tr.v_cache)
        assert torch.equal(dt.ks, tr.k_scale) and torch.equal(dt.vs, tr.v_scale)
        assert np.array_equal(dt.pt.numpy(), tr.page_table)
        assert np.array_equal(dt.len.numpy(), tr.lengths)
        assert torch.equal(dt.q, tr.q)


def test_sub_case_keeps_the_requests_step():
    """A sub-batch of a step (its requests' pages renumbered and copied) gives
    the CPU reference the same result for those requests as the whole step,
    bit for bit, for a bf16 and an fp8 cache."""
    import oracle
    for kv in ("bf16", "fp8"):
        c = wl.make_case("full", [33, 0, 500, 64, 130], Hq=8, Hkv=2, P=16, kv_dtype=kv, seed=4)
        ids = [4, 0, 2, 1]
        sub = wl.sub_case(c, ids)
        assert sub.B == 4 and sub.num_pages == sum(-(-int(c.lengths[i]) // 16) for i in ids)
        o1, l1 = oracle.decode(c, ids)
        o2, l2 = oracle.decode(sub)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
