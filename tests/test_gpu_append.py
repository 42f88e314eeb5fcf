"""GPU parity of the per-step KV append (attn_append_kv).

Decode grows every context by one token per step [Tencent HPC lands in SGLang,
challenging default inference kernels, sec. "Why Tencent HPC matters for online
model serving"]; attn_append_kv writes each request's new key/value row into its
page, storing bf16 bits or the e4m3fn code of x / scale for an fp8 cache [same
page, sec. "What the 48.8% TPOT claim does not prove"]. Byte output, so the
check against the CPU reference is bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from variable_length_kv_amd import lib as L
from variable_length_kv_amd import workloads as wl
from variable_length_kv_amd.trace import DeviceTrace

from gpu_helpers import FP8_TOL, check_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _shape(c, W=8):
    return L.AttnShape(batch=c.B, num_q_heads=c.Hq, num_kv_heads=c.Hkv, page_size=c.P, num_pages=c.num_pages,
                       pt_stride=c.pt_stride, num_wgs=W,
                       kv_dtype=L.ATTN_KV_FP8_E4M3 if c.kv_dtype == "fp8" else L.ATTN_KV_BF16)


def _run_append(c, k_new, v_new, positions, page_table=None, with_workspace=True):
    pt = c.page_table if page_table is None else page_table
    d = {"k": c.k_cache.to(DEV), "v": c.v_cache.to(DEV)}
    att = L.Attention(_shape(c), DEV)
    att.shape.pt_stride = pt.shape[1]
    ks = c.k_scale.to(DEV) if c.k_scale is not None else None
    vs = c.v_scale.to(DEV) if c.v_scale is not None else None
    L.attn_append_kv(att.shape, k_new.to(DEV), v_new.to(DEV), torch.from_numpy(np.asarray(positions, np.int32)).to(DEV),
                     torch.from_numpy(np.ascontiguousarray(pt)).to(DEV), d["k"], d["v"], ks, vs,
                     att.workspace if with_workspace else None)
    torch.cuda.synchronize()
    return d["k"].cpu(), d["v"].cpu(), att.status() if with_workspace else 0


def _bits(t):
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _every_bf16_pattern(B, Hkv, D):
    """All finite bf16 bit patterns (and both zeros), in a [B, Hkv, D] tensor."""
    bits = np.arange(65536, dtype=np.uint32)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]                      # no inf / NaN
    out = np.zeros(B * Hkv * D, np.uint16)
    out[:len(bits)] = bits[:B * Hkv * D]
    return torch.from_numpy(out.view(np.int16).reshape(B, Hkv, D)).view(torch.bfloat16), len(bits)


@pytest.mark.parametrize("scale", [1.0, 1.0 / 3.0, 0.0173, 2.0 ** -8, 7.5, 300.0])
def test_fp8_append_encodes_every_bf16_input_bit_exactly(scale):
    B, Hkv, D, P = 64, 8, 128, 16
    c = wl.make_case("t", [1] * B, Hq=Hkv, Hkv=Hkv, P=P, kv_dtype="fp8", seed=1)
    c.k_scale = torch.full((B, Hkv), scale, dtype=torch.float32)
    c.v_scale = torch.full((B, Hkv), scale * 0.5, dtype=torch.float32)
    k_new, n = _every_bf16_pattern(B, Hkv, D)
    assert n <= B * Hkv * D
    v_new = -k_new
    pos = np.zeros(B, np.int32)
    gk, gv, st = _run_append(c, k_new, v_new, pos)
    rk, rv, rst = oracle.append_kv(c, k_new, v_new, pos)
    assert st == rst == 0
    assert np.array_equal(gk.numpy(), rk) and np.array_equal(gv.numpy(), rv)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_random_rows_and_positions(kv):
    rng = np.random.default_rng(5)
    lengths = rng.integers(0, 200, 24)
    c = wl.make_case("t", lengths, Hq=16, Hkv=4, P=16, kv_dtype=kv, seed=6, extra_pages=32)
    # give every request room for one more token: a free page where the next row starts a page
    pt = np.full((c.B, c.pt_stride + 1), -1, np.int32)
    pt[:, :c.pt_stride] = c.page_table
    used = {int(x) for x in c.page_table.ravel() if x >= 0}
    free = iter(sorted(set(range(c.num_pages)) - used))
    for b, Lb in enumerate(lengths):
        if Lb % c.P == 0:
            pt[b, Lb // c.P] = next(free)
    c2 = wl.Case(c.name, c.B, c.Hq, c.Hkv, c.D, c.P, c.lengths, pt, c.num_pages, kv, c.q, c.k_cache, c.v_cache,
                 c.k_scale, c.v_scale, c.sm_scale)
    k_new = torch.from_numpy(rng.normal(0, 2, (c.B, c.Hkv, c.D)).astype(np.float32)).to(torch.bfloat16)
    v_new = torch.from_numpy(rng.normal(0, 2, (c.B, c.Hkv, c.D)).astype(np.float32)).to(torch.bfloat16)
    pos = lengths.astype(np.int32)
    pos[3] = -1                                  # no append for this request
    gk, gv, st = _run_append(c2, k_new, v_new, pos)
    rk, rv, rst = oracle.append_kv(c2, k_new, v_new, pos)
    assert st == rst == 0
    assert np.array_equal(_bits(gk), rk) and np.array_equal(_bits(gv), rv)


def test_append_status_and_skips():
    c = wl.make_case("t", [10, 20, 30], Hq=8, Hkv=2, P=16, kv_dtype="fp8", seed=7)
    rng = np.random.default_rng(8)
    k_new = torch.from_numpy(rng.normal(0, 1, (c.B, c.Hkv, c.D)).astype(np.float32)).to(torch.bfloat16)
    v_new = k_new.clone()
    pt = c.page_table.copy()
    pt[2, 1] = c.num_pages + 3                   # bad page id for request 2's position 17
    pos = np.array([c.pt_stride * c.P, 5, 17], np.int32)   # request 0 past the page table
    gk, gv, st = _run_append(c, k_new, v_new, pos, page_table=pt)
    c2 = wl.Case(c.name, c.B, c.Hq, c.Hkv, c.D, c.P, c.lengths, pt, c.num_pages, "fp8", c.q, c.k_cache, c.v_cache,
                 c.k_scale, c.v_scale, c.sm_scale)
    rk, rv, rst = oracle.append_kv(c2, k_new, v_new, pos)
    assert rst == 3 and st & L.ATTN_STATUS_BAD_LENGTH and st & L.ATTN_STATUS_BAD_PAGE
    assert np.array_equal(gk.numpy(), rk) and np.array_equal(gv.numpy(), rv)
    # without a workspace the same skips happen, silently
    gk2, gv2, _ = _run_append(c, k_new, v_new, pos, page_table=pt, with_workspace=False)
    assert np.array_equal(gk2.numpy(), rk)


def test_trace_with_device_append_matches_host_model():
    """The continuous-batching trace with every appended token written on the
    device: the live rows of the device cache equal the host model's codes bit
    for bit at every step, and decode on the device cache matches the CPU
    reference."""
    tr = wl.Trace(steps=40, slots=12, Hq=16, Hkv=2, P=16, seed=9, p_finish=0.1, new_lo=1, new_hi=300,
                  init_lo=1, init_hi=1200)
    shape = L.AttnShape(batch=tr.slots, num_q_heads=tr.Hq, num_kv_heads=tr.Hkv, page_size=tr.P,
                        num_pages=tr.num_pages, pt_stride=tr.pt_stride, num_wgs=29, kv_dtype=L.ATTN_KV_FP8_E4M3)
    att = L.Attention(shape, DEV)
    dt = DeviceTrace(tr, DEV, append=att.append_kv)
    out = torch.empty_like(dt.q)
    lse = torch.empty(tr.slots, tr.Hq, dtype=torch.float32, device=DEV)
    while True:
        torch.cuda.synchronize()
        kd, vd = dt.k.cpu(), dt.v.cpu()
        for b in range(tr.slots):
            Lb = int(tr.lengths[b])
            j = np.arange(Lb)
            pages = torch.from_numpy(tr.page_table[b, j // tr.P].astype(np.int64))
            rows = torch.from_numpy(j % tr.P)
            assert torch.equal(kd[pages, :, rows], tr.k_cache[pages, :, rows]), f"step {tr.step} slot {b}"
            assert torch.equal(vd[pages, :, rows], tr.v_cache[pages, :, rows]), f"step {tr.step} slot {b}"
        att.fused_step(dt.q, dt.k, dt.v, dt.pt, dt.len, 1.0 / np.sqrt(tr.D), out, lse, k_scale=dt.ks, v_scale=dt.vs)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.decode(tr.case())
        check_close(out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l, FP8_TOL,
                    what=f"step {tr.step}")
        if tr.step == tr.steps - 1:
            break
        dt.advance()
    assert att.status() == 0
