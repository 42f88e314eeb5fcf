"""Work-list checks with the visit-counting build (libvlkv_attn_visits.so).

The dynamic schedule cuts every request's KV cache into uniform tiles and
hands them to workgroups by load, rebuilding the hand-out each step as lengths
change and requests end [Tencent HPC lands in SGLang, challenging default
inference kernels, sec. "Why Tencent HPC matters for online model serving";
sec. "What the 48.8% TPOT claim does not prove", on continuous batching and
cancellation]. A hand-out that dropped or repeated work could still give
outputs within tolerance (a repeated tile only re-weights a softmax), so these
tests count instead: the visit-counting build adds 1 per cached row that the
attention math consumes, per (request, kv head), and 1 per write of a final
output row. Every row below a request's valid length must be consumed exactly
once, no other row ever, and every output row written exactly once, in every
mode and launch form; the outputs must equal the uninstrumented library's bit
for bit (the counting changes no arithmetic).
"""
import numpy as np
import pytest
import torch

from variable_length_kv_amd import lib as L
from variable_length_kv_amd import workloads as wl
from variable_length_kv_amd.trace import DeviceTrace

from gpu_helpers import dev, device_inputs, run, shape_for
from test_gpu_random_shapes import draw

pytestmark = pytest.mark.gpu


def _counters(B, Hq, Hkv, stride):
    tok = torch.zeros(B * Hkv * stride, dtype=torch.int32, device=dev())
    out = torch.zeros(B * Hq, dtype=torch.int32, device=dev())
    return tok, out


def _expected_rows(lengths, Hkv, stride, valid_limit, dead_rows=()):
    """1 for each row j < L_b of every kv head of request b (lengths outside
    [0, valid_limit] count as 0), 0 elsewhere; ``dead_rows``: (b, j0, j1) row
    ranges that must not be read (an invalid page)."""
    B = len(lengths)
    e = np.zeros((B, Hkv, stride), np.int32)
    for b, Lb in enumerate(np.asarray(lengths, np.int64)):
        if 0 <= Lb <= valid_limit:
            e[b, :, :Lb] = 1
    for b, j0, j1 in dead_rows:
        e[b, :, j0:j1] = 0
    return e


def _check_counts(tok, outc, expected, B, Hq, what):
    got = tok.view(expected.shape).cpu().numpy()
    bad = np.argwhere(got != expected)
    assert bad.size == 0, (f"{what}: {len(bad)} rows consumed a wrong number of times; first "
                           f"(b, g, row) = {tuple(bad[0])}: {got[tuple(bad[0])]} visits, expected "
                           f"{expected[tuple(bad[0])]}")
    o = outc.view(B, Hq).cpu().numpy()
    assert (o == 1).all(), f"{what}: output rows written {np.unique(o).tolist()} times (expected once)"


def _counted_run(case, mode, fused, W, S=0, T=64, t=None, dead_rows=()):
    """One step through the visit-counting build, checked; returns its outputs."""
    stride = case.pt_stride * case.P
    tok, outc = _counters(case.B, case.Hq, case.Hkv, stride)
    torch.cuda.synchronize()
    with L.counting_visits(tok, stride, outc):
        o, l, att = run(case, mode, T, W, S, t=t, fused=fused)
        status = att.status()
    expected = _expected_rows(case.lengths, case.Hkv, stride, stride, dead_rows)
    what = f"{case.name} mode {mode} {'attn_step' if fused else 'three launches'} W {W} S {S} T {T}"
    _check_counts(tok, outc, expected, case.B, case.Hq, what)
    return o, l, status


def _plain_run(case, mode, fused, W, S=0, T=64, t=None):
    o, l, att = run(case, mode, T, W, S, t=t, fused=fused)
    return o, l, att.status()


def _same(a, b, what):
    (o1, l1, s1), (o2, l2, s2) = a, b
    assert s1 == s2, f"{what}: status {s1} vs {s2}"
    assert np.array_equal(o1, o2), f"{what}: the counting build's output differs"
    assert np.array_equal(l1, l2), f"{what}: the counting build's lse differs"


RAGGED = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 200, 1000, 0, 4097, 2500]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("fused", [False, True], ids=["three", "step"])
@pytest.mark.parametrize("W", [1, 7, None], ids=["W1", "W7", "W2cu"])
def test_dynamic_every_row_once(kv, fused, W):
    case = wl.make_case("ragged", RAGGED, Hq=16, Hkv=2, P=16, kv_dtype=kv, seed=5)
    t = device_inputs(case)
    got = _counted_run(case, L.ATTN_DYNAMIC, fused, W, t=t)
    _same(got, _plain_run(case, L.ATTN_DYNAMIC, fused, W, t=t), "dynamic")


@pytest.mark.parametrize("T", [64, 128, 320])
def test_dynamic_tile_sizes(T):
    case = wl.make_case("ragged-T", RAGGED + [777, 3, 9000], Hq=8, Hkv=1, P=32, seed=6)
    t = device_inputs(case)
    for fused in (False, True):
        got = _counted_run(case, L.ATTN_DYNAMIC, fused, 29, T=T, t=t)
        _same(got, _plain_run(case, L.ATTN_DYNAMIC, fused, 29, T=T, t=t), f"T {T}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("S", [0, 1, 3, 40])
def test_static_every_row_once(kv, S):
    case = wl.make_case("ragged-static", RAGGED, Hq=8, Hkv=2, P=16, kv_dtype=kv, seed=7)
    t = device_inputs(case)
    for fused in (False, True):
        got = _counted_run(case, L.ATTN_STATIC, fused, 64, S=S, t=t)
        _same(got, _plain_run(case, L.ATTN_STATIC, fused, 64, S=S, t=t), f"static S {S}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_shared_prefix_rows_once_per_request(kv, G):
    """A shared prefix row is read once but serves each request of its group:
    it counts once for each."""
    lengths, groups = wl.shared_prefix_lengths(3, 5, 640, 1, 300, 16, seed=G)
    lengths = np.concatenate([lengths, np.array([0, 33, 1500], np.int32)])
    case = wl.make_shared_case(f"shared-G{G}", lengths, groups, Hq=2 * G, Hkv=2, P=16, kv_dtype=kv, seed=G)
    t = device_inputs(case)
    for W in (5, None):
        got = _counted_run(case, L.ATTN_SHARED, False, W, t=t)
        _same(got, _plain_run(case, L.ATTN_SHARED, False, W, t=t), f"shared G {G} W {W}")


def test_invalid_page_and_length_rows_are_not_read():
    """Rows on a page id outside [0, num_pages) and a length beyond the page
    table are skipped (status bits set), never read; every output row is
    still written once."""
    lengths = [300, 150, 90, 40]
    case = wl.make_case("bad", lengths, Hq=8, Hkv=1, P=16, seed=8)
    case.page_table = case.page_table.copy()
    case.page_table[1, 2] = case.num_pages + 5   # rows 32..47 of request 1
    limit = case.pt_stride * case.P
    case.lengths = np.array([300, 150, limit + 1, 40], np.int32)
    t = device_inputs(case, poison=False)
    for fused in (False, True):
        stride = limit
        tok, outc = _counters(case.B, case.Hq, case.Hkv, stride)
        torch.cuda.synchronize()
        with L.counting_visits(tok, stride, outc):
            _, _, att = run(case, L.ATTN_DYNAMIC, 64, 11, 0, t=t, fused=fused)
            status = att.status()
        assert status == L.ATTN_STATUS_BAD_LENGTH | L.ATTN_STATUS_BAD_PAGE
        expected = _expected_rows(case.lengths, case.Hkv, stride, limit, dead_rows=[(1, 32, 48)])
        _check_counts(tok, outc, expected, case.B, case.Hq, f"invalid inputs fused={fused}")


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_full_size_workloads_in_the_benchmark_launch(cid):
    """Workloads 1-3 at full size, as the benchmark runs them: the single
    launch with the library's default workgroup count, and the three launches."""
    case = wl.config_case(cid)
    t = device_inputs(case)
    for fused in (True, False):
        got = _counted_run(case, L.ATTN_DYNAMIC, fused, 0, t=t)
        _same(got, _plain_run(case, L.ATTN_DYNAMIC, fused, 0, t=t), f"workload {cid}")


def test_full_size_fp8_copy_of_workload_1():
    lengths = wl.config_lengths(1)
    case = wl.make_case("uniform_mixed_fp8", lengths, Hq=64, Hkv=8, P=64, kv_dtype="fp8")
    t = device_inputs(case)
    got = _counted_run(case, L.ATTN_DYNAMIC, True, 0, t=t)
    _same(got, _plain_run(case, L.ATTN_DYNAMIC, True, 0, t=t), "fp8 workload 1")


def test_trace_every_step():
    """A continuous-batching trace with an fp8 cache: lengths grow, requests
    end and are replaced; at every step both launch forms consume each live
    row exactly once."""
    tr = wl.Trace(steps=48, slots=24, Hq=32, Hkv=4, P=64, seed=11, p_finish=0.08, new_lo=1, new_hi=3000,
                  init_lo=1, init_hi=9000)
    dt = DeviceTrace(tr)
    shape = L.AttnShape(batch=tr.slots, num_q_heads=tr.Hq, num_kv_heads=tr.Hkv, page_size=tr.P,
                        num_pages=tr.num_pages, pt_stride=tr.pt_stride, num_wgs=0,
                        kv_dtype=L.ATTN_KV_FP8_E4M3)
    stride = tr.pt_stride * tr.P
    tok, outc = _counters(tr.slots, tr.Hq, tr.Hkv, stride)
    out = torch.empty_like(dt.q)
    lse = torch.empty(tr.slots, tr.Hq, dtype=torch.float32, device=dev())
    att = L.Attention(shape, dev())
    with L.counting_visits(tok, stride, outc):
        while True:
            s = dt.step
            expected = _expected_rows(tr.lengths, tr.Hkv, stride, stride)
            for name, step in (("three launches", att.step), ("attn_step", att.fused_step)):
                tok.zero_()
                outc.zero_()
                step(dt.q, dt.k, dt.v, dt.pt, dt.len, 1.0 / np.sqrt(tr.D), out, lse, k_scale=dt.ks,
                     v_scale=dt.vs)
                torch.cuda.synchronize()
                assert att.status() == 0, f"step {s} {name}"
                _check_counts(tok, outc, expected, tr.slots, tr.Hq, f"trace step {s} {name}")
            if s == tr.steps - 1:
                break
            dt.advance()


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes_every_row_once(seed):
    """The random shapes of the parity test (head groupings 1-16, 1-8 kv heads,
    pages of 16-256 tokens, tiles of 64-256, 1-1500 workgroups, all three
    modes, both cache types, empty and page-boundary lengths): both launch
    forms consume every live row exactly once."""
    c, mode, T, W, S = draw(seed)
    t = device_inputs(c)
    for fused in (False, True):
        got = _counted_run(c, mode, fused, W, S=S, T=T, t=t)
        _same(got, _plain_run(c, mode, fused, W, S=S, T=T, t=t), f"random shape {seed}")


def test_allocation_free_step_every_row_once():
    """attn_step_noalloc (the library's per-GPU scratch instead of a
    workspace) on a large batch, then a smaller one of another shape, then the
    large one again: the scratch keeps the last call's contents, and each call
    must still consume every live row exactly once."""
    rng = np.random.default_rng(9)
    big = wl.make_case("na-big", rng.integers(1, 9000, 40).astype(np.int32), Hq=64, Hkv=8, P=64, seed=1)
    small = wl.make_case("na-small", np.array([0, 5, 700, 64, 17, 300], np.int32), Hq=16, Hkv=2, P=16,
                         kv_dtype="fp8", seed=2)
    for case, W in ((big, None), (small, 29), (big, None)):
        t = device_inputs(case)
        sh = shape_for(case, L.ATTN_DYNAMIC, W=W)
        stride = case.pt_stride * case.P
        tok, outc = _counters(case.B, case.Hq, case.Hkv, stride)
        out = torch.empty_like(t["q"])
        lse = torch.empty((case.B, case.Hq), dtype=torch.float32, device=dev())
        status = torch.zeros(1, dtype=torch.int32, device=dev())
        torch.cuda.synchronize()
        with L.counting_visits(tok, stride, outc):
            L.attn_step_noalloc(sh, t["q"], t["k"], t["v"], t["ks"], t["vs"], t["pt"], t["len"], case.sm_scale,
                                out, lse, status)
            torch.cuda.synchronize()
        assert int(status.item()) == 0
        _check_counts(tok, outc, _expected_rows(case.lengths, case.Hkv, stride, stride), case.B, case.Hq,
                      f"attn_step_noalloc {case.name}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_limits_every_row_once(kv):
    """The largest shapes: 8192 requests (one in ten empty) with 16 query heads
    on one kv head, dynamic and static, both launch forms; 1024-token pages
    under 256-token tiles; tiles of 1024 tokens; 65536 workgroups for a few
    dozen units."""
    rng = np.random.default_rng(11)
    lengths = rng.integers(1, 160, 8192)
    lengths[rng.random(8192) < 0.1] = 0
    c = wl.make_case("max_batch", lengths, Hq=16, Hkv=1, P=16, kv_dtype=kv, seed=11)
    t = device_inputs(c)
    for fused in (False, True):
        _counted_run(c, L.ATTN_DYNAMIC, fused, 512, t=t)
        _counted_run(c, L.ATTN_STATIC, fused, 512, S=2, t=t)
    big = wl.make_case("big_pages", [1, 63, 64, 65, 1023, 1024, 1025, 3000, 5000, 0, 2048], Hq=8, Hkv=2, P=1024,
                       kv_dtype=kv, seed=13)
    tiles = wl.make_case("big_tiles", [1024, 1025, 2047, 4100, 7, 0, 3333], Hq=16, Hkv=2, P=32, kv_dtype=kv, seed=14)
    few = wl.make_case("few_units", [5, 300, 129, 0, 64], Hq=8, Hkv=1, P=16, kv_dtype=kv, seed=15)
    for case, T, W in ((big, 256, 64), (tiles, 1024, 5), (few, 64, 1 << 16)):
        tc = device_inputs(case)
        for fused in (False, True):
            _counted_run(case, L.ATTN_DYNAMIC, fused, W, T=T, t=tc)


def test_limits_shared_items_beyond_lds():
    """8192 requests in groups of 4 sharing a 64-token prefix: more plan items
    than the shared planner's LDS copy of the tile prefix holds."""
    rng = np.random.default_rng(12)
    lengths = rng.integers(65, 140, 8192)
    groups = [(4 * i, 4, 4) for i in range(8192 // 4)]
    c = wl.make_shared_case("max_batch_shared", lengths, groups, Hq=4, Hkv=1, P=16, seed=12)
    t = device_inputs(c)
    _counted_run(c, L.ATTN_SHARED, False, 512, t=t)
