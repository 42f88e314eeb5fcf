"""GPU parity of the single-launch step (attn_step).

attn_step computes the same plan, split-KV decode and log-sum-exp merge as
attn_plan + attn_decode + attn_combine, inside one kernel: each workgroup
derives its unit range from the lengths and the last workgroup to finish a
split (request, kv head) pair merges the pair's partials. The partials and the
merge order are the same as the three-launch path's, so the outputs must be
bitwise equal to it, and within the oracle tolerances of the CPU reference.
The per-step rebuild of the tile mapping is the article's [Tencent HPC lands in
SGLang, challenging default inference kernels, sec. "Why Tencent HPC matters
for online model serving"].
"""
import numpy as np
import pytest
import torch

from variable_length_kv_amd import lib as L
from variable_length_kv_amd import workloads as wl
from variable_length_kv_amd.trace import DeviceTrace

from gpu_helpers import FP8_TOL, check_against_oracle, check_close, device_inputs, num_cus, run, shape_for

import oracle

pytestmark = pytest.mark.gpu


def _case(lengths, **kw):
    kw.setdefault("Hq", 8)
    kw.setdefault("Hkv", 1)
    kw.setdefault("P", 16)
    return wl.make_case("t", lengths, **kw)


def _both(c, **kw):
    t = device_inputs(c)
    o3, l3, _ = run(c, t=t, **kw)
    of, lf, att = run(c, t=t, fused=True, **kw)
    check_against_oracle(c, of, lf, what=f"fused {kw}")
    assert np.array_equal(of, o3) and np.array_equal(lf, l3), f"fused != three-launch {kw}"
    return of, lf, att


CASES = [
    ("tiny", lambda: wl.config_case(0)),
    ("bounds", lambda: _case([1, 15, 16, 17, 63, 64, 65, 1023, 1024, 1025], Hq=16, Hkv=2, P=16, seed=31)),
    ("groups", lambda: _case([5, 70, 200], Hq=12, Hkv=4, P=64, seed=32)),
    ("empties", lambda: _case([0, 17, 0, 0, 40, 0], Hq=8, Hkv=2, P=16, seed=33)),
    ("skew", lambda: _case([4000] + [60] * 20, Hq=16, Hkv=2, P=32, seed=34)),
    ("fp8", lambda: _case([1, 17, 64, 200, 1000, 0], Hq=16, Hkv=2, P=16, kv_dtype="fp8", seed=35)),
]


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("W", [1, 3, 7, 64, 512])
def test_fused_dynamic_matches(name, make, W):
    _both(make(), W=W)


@pytest.mark.parametrize("name,make", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("S", [0, 1, 2, 5])
def test_fused_static_matches(name, make, S):
    _both(make(), mode=L.ATTN_STATIC, S=S, W=16)


@pytest.mark.parametrize("T", [128, 256])
def test_fused_tile_sizes(T):
    _both(_case([1, 63, 64, 65, 300, 513], Hq=16, Hkv=2, P=32, seed=36), T=T, W=9)


def test_random_batches_fused():
    rng = np.random.default_rng(17)
    for it in range(8):
        B = int(rng.integers(1, 40))
        P = int(rng.choice([16, 32, 64]))
        lengths = rng.integers(0, 900, B) * (rng.random(B) < 0.85)
        lengths[int(rng.integers(B))] = int(rng.integers(1, 4000))
        c = _case(lengths, Hq=8, Hkv=2, P=P, seed=40 + it)
        _both(c, W=int(rng.choice([1, 5, 13, 100, 512, 2048])))


def test_repeated_steps_reuse_the_workspace():
    """Arrival counters return to zero after every step: repeated steps on one
    workspace, with different lengths in between, stay correct and identical."""
    c = _case([3000, 10, 700, 1], Hq=8, Hkv=2, P=16, seed=50)
    t = device_inputs(c)
    first = run(c, t=t, fused=True, W=37)
    att = first[2]
    for _ in range(3):
        o, l, _ = run(c, t=t, fused=True, att=att)
        assert np.array_equal(o, first[0]) and np.array_equal(l, first[1])
    short = t["len"].clone()
    short[0] = 900
    o, l, _ = run(c, t=t, fused=True, att=att, lengths=short)
    ref_case = wl.Case(c.name, c.B, c.Hq, c.Hkv, c.D, c.P, short.cpu().numpy(), c.page_table, c.num_pages,
                       c.kv_dtype, c.q, c.k_cache, c.v_cache, None, None, c.sm_scale)
    check_against_oracle(ref_case, o, l, what="shorter lengths on a reused workspace")
    o, l, _ = run(c, t=t, fused=True, att=att)
    assert np.array_equal(o, first[0]) and np.array_equal(l, first[1])


def test_fused_status_bits():
    c = _case([40, 40, 40], Hq=8, Hkv=1, P=16, seed=51)
    t = device_inputs(c)
    t["len"][1] = 10 ** 6
    t["pt"][2, 1] = c.num_pages + 5
    o, l, att = run(c, t=t, fused=True, W=4)
    st = att.status()
    assert st & L.ATTN_STATUS_BAD_LENGTH and st & L.ATTN_STATUS_BAD_PAGE
    assert np.all(o[1] == 0) and np.all(l[1] == -np.inf)
    check_against_oracle(c, o, l, req_ids=[0], what="valid request")


def test_fused_small_trace_every_step():
    tr = wl.Trace(steps=48, slots=12, Hq=16, Hkv=2, P=16, seed=4, p_finish=0.1, new_lo=1, new_hi=300,
                  init_lo=1, init_hi=1500)
    dt = DeviceTrace(tr)
    shape = L.AttnShape(batch=tr.slots, num_q_heads=tr.Hq, num_kv_heads=tr.Hkv, page_size=tr.P,
                        num_pages=tr.num_pages, pt_stride=tr.pt_stride, num_wgs=29,
                        kv_dtype=L.ATTN_KV_FP8_E4M3)
    att = L.Attention(shape, "cuda:0")
    out = torch.empty_like(dt.q)
    lse = torch.empty(tr.slots, tr.Hq, dtype=torch.float32, device="cuda:0")
    while True:
        out.fill_(float("nan"))
        att.fused_step(dt.q, dt.k, dt.v, dt.pt, dt.len, 1.0 / np.sqrt(tr.D), out, lse, k_scale=dt.ks,
                       v_scale=dt.vs)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.decode(tr.case())
        check_close(out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l, FP8_TOL,
                    what=f"fused trace step {tr.step}")
        if tr.step == tr.steps - 1:
            break
        dt.advance()
    assert att.status() == 0


def _sample(lengths, n=6):
    L_ = np.asarray(lengths)
    idx = {int(np.argmax(L_)), int(np.argmin(L_)), 0, len(L_) - 1}
    rng = np.random.default_rng(1)
    idx |= set(rng.choice(len(L_), size=min(n, len(L_)), replace=False).tolist())
    return sorted(idx)


@pytest.mark.parametrize("cid", [1, 2, 3])
def test_fused_full_size_workloads(cid):
    c = wl.config_case(cid)
    t = device_inputs(c)
    for mode in (L.ATTN_DYNAMIC, L.ATTN_STATIC):
        o3, l3, _ = run(c, mode=mode, t=t)
        of, lf, att = run(c, mode=mode, t=t, fused=True)
        assert att.status() == 0
        assert np.array_equal(of, o3) and np.array_equal(lf, l3), f"c{cid} mode={mode}"
        check_against_oracle(c, of, lf, req_ids=_sample(c.lengths), what=f"c{cid} fused mode={mode}")
