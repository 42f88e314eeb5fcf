"""attn_step_noalloc, the single-launch step for callers that cannot allocate
device memory (its scratch is a per-GPU array inside the library), against
attn_step on a caller workspace: the same kernel over the same plan, so the
outputs and lse must be equal bit for bit, call after call, on inputs that
shrink between calls; and within tolerance of the CPU reference."""
import numpy as np
import pytest
import torch

from gpu_helpers import check_against_oracle, dev, device_inputs, num_cus, shape_for
from variable_length_kv_amd import lib as L
from variable_length_kv_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _step_both(case, mode=L.ATTN_DYNAMIC, W=None, S=0):
    t = device_inputs(case)
    sh = shape_for(case, mode, W=W, S=S)
    att = L.Attention(sh, dev())
    outs = []
    for noalloc in (False, True):
        out = torch.full_like(t["q"], float("nan"))
        lse = torch.full((case.B, case.Hq), float("nan"), dtype=torch.float32, device=dev())
        status = torch.zeros(1, dtype=torch.int32, device=dev())
        if noalloc:
            L.attn_step_noalloc(sh, t["q"], t["k"], t["v"], t["ks"], t["vs"], t["pt"], t["len"], case.sm_scale,
                                out, lse, status)
        else:
            att.fused_step(t["q"], t["k"], t["v"], t["pt"], t["len"], case.sm_scale, out, lse,
                           k_scale=t["ks"], v_scale=t["vs"])
        torch.cuda.synchronize()
        outs.append((out, lse, int(status.item())))
    (o1, l1, _), (o2, l2, st2) = outs
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"{case.name}: outputs differ"
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), f"{case.name}: lse differs"
    assert st2 == 0 and att.status() == 0
    check_against_oracle(case, o2.double().cpu().numpy(), l2.double().cpu().numpy(), what=case.name)


def _lengths(seed, B, hi, empty=True):
    L_ = np.random.default_rng(seed).integers(1, hi, B, endpoint=True).astype(np.int32)
    if empty:
        L_[B // 3] = 0
    return L_


def test_noalloc_equals_attn_step_on_shrinking_inputs():
    # a large batch, then a smaller one of another shape, then the large one
    # again: the shared scratch keeps the last call's contents, and every step
    # must leave its arrival counters at zero for the next
    big = wl.make_case("noalloc-big", _lengths(1, 40, 9000), Hq=64, Hkv=8, P=64, seed=1)
    small = wl.make_case("noalloc-small", _lengths(2, 6, 700), Hq=16, Hkv=2, P=16, kv_dtype="fp8", seed=2)
    _step_both(big, W=2 * num_cus())
    _step_both(small, W=29)
    _step_both(big, W=2 * num_cus())


def test_noalloc_static_split():
    c = wl.make_case("noalloc-static", _lengths(3, 12, 3000), Hq=32, Hkv=4, P=32, seed=3)
    _step_both(c, mode=L.ATTN_STATIC, S=5)


def test_noalloc_limits_are_checked_on_the_host():
    c = wl.make_case("noalloc-limits", [100, 200], Hq=16, Hkv=1, P=16, seed=4)
    t = device_inputs(c)
    out = torch.empty_like(t["q"])
    # 2 * num_wgs slots of 16 rows x 129 floats: 4096 workgroups need 67.6 MB
    too_many = shape_for(c, W=4096)
    with pytest.raises(L.AttnError) as e:
        L.attn_step_noalloc(too_many, t["q"], t["k"], t["v"], None, None, t["pt"], t["len"], c.sm_scale, out)
    assert e.value.code == L.ATTN_ERR_INVALID_ARG
    shared = shape_for(c, mode=L.ATTN_SHARED)
    with pytest.raises(L.AttnError) as e:
        L.attn_step_noalloc(shared, t["q"], t["k"], t["v"], None, None, t["pt"], t["len"], c.sm_scale, out)
    assert e.value.code == L.ATTN_ERR_UNSUPPORTED
