"""HIP graph capture of a whole decode step.

A serving loop issues the same step every decode iteration while the context
of every request grows by one token [Tencent HPC lands in SGLang, challenging
default inference kernels, sec. "Why Tencent HPC matters for online model
serving"]. The step here is attn_append_kv (the new K/V row of each request
written into its page) followed by the attention step: attn_step in one
launch, or attn_plan + attn_decode + attn_combine. None of these calls
allocates, synchronises or writes memory from the host, and the single
launch returns its arrival counters to zero, so the step can be captured once
in a graph and replayed with new contents in the same buffers.

Each test captures the step on one copy of the state and runs it eagerly on
an identical second copy. Before every replay the host writes new queries,
new K/V rows, positions and lengths into both copies in place. Eager work and
synchronisations fall between replays. Every replay must equal the eager step
bit for bit (outputs, lse and the appended cache rows), and the last replay
is checked against the CPU reference as well.
"""
import numpy as np
import pytest
import torch

import oracle
from variable_length_kv_amd import lib as L
from variable_length_kv_amd import workloads as wl

from gpu_helpers import BF16_TOL, FP8_TOL, check_close, num_cus

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 4


def _state(c, lengths):
    """Device copies of one decode state (caches, page table, lengths and the
    per-step inputs and outputs)."""
    d = torch.device(DEV)
    B, Hq, Hkv, D = c.B, c.Hq, c.Hkv, c.D
    return {
        "k": c.k_cache.to(d, copy=True), "v": c.v_cache.to(d, copy=True),
        "ks": None if c.k_scale is None else c.k_scale.to(d, copy=True),
        "vs": None if c.v_scale is None else c.v_scale.to(d, copy=True),
        "pt": torch.from_numpy(np.ascontiguousarray(c.page_table)).to(d),
        "len": torch.from_numpy(np.asarray(lengths, np.int32)).to(d),
        "pos": torch.zeros(B, dtype=torch.int32, device=d),
        "q": torch.zeros(B, Hq, D, dtype=torch.bfloat16, device=d),
        "kn": torch.zeros(B, Hkv, D, dtype=torch.bfloat16, device=d),
        "vn": torch.zeros(B, Hkv, D, dtype=torch.bfloat16, device=d),
        "out": torch.zeros(B, Hq, D, dtype=torch.bfloat16, device=d),
        "lse": torch.zeros(B, Hq, dtype=torch.float32, device=d),
    }


def _step(att, s, sm_scale, fused):
    att.append_kv(s["kn"], s["vn"], s["pos"], s["pt"], s["k"], s["v"], s["ks"], s["vs"])
    run = att.fused_step if fused else att.step
    run(s["q"], s["k"], s["v"], s["pt"], s["len"], sm_scale, s["out"], s["lse"], s["ks"], s["vs"])


def _bitwise(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _case(kind, kv_dtype):
    """Lengths for the last replay decide the pages; the state starts REPLAYS
    tokens shorter, so every replay appends into an allocated page."""
    rng = np.random.default_rng(7)
    if kind == "shared":
        final, groups = wl.shared_prefix_lengths(3, 3, 128, 20, 300, 16, seed=3)
        final = final + REPLAYS
        c = wl.make_shared_case("graph-shared", final, groups, Hq=16, Hkv=2, P=16, kv_dtype=kv_dtype, seed=3)
    else:
        final = np.concatenate([rng.integers(REPLAYS + 1, 400, 10), [1500, REPLAYS + 1]]).astype(np.int32)
        c = wl.make_case("graph", final, Hq=16, Hkv=2, P=16, kv_dtype=kv_dtype, seed=5)
    return c, np.asarray(c.lengths, np.int32) - REPLAYS


@pytest.mark.parametrize("kind,kv_dtype,mode,fused", [
    ("dynamic", "bf16", L.ATTN_DYNAMIC, True),
    ("dynamic", "bf16", L.ATTN_DYNAMIC, False),
    ("static", "bf16", L.ATTN_STATIC, True),
    ("dynamic", "fp8", L.ATTN_DYNAMIC, True),
    ("shared", "bf16", L.ATTN_SHARED, True),
], ids=["single-launch", "three-launch", "static-single-launch", "fp8-single-launch", "prefix-shared"])
def test_graph_replays_equal_eager_steps(kind, kv_dtype, mode, fused):
    c, start = _case(kind, kv_dtype)
    shape = L.AttnShape(batch=c.B, num_q_heads=c.Hq, num_kv_heads=c.Hkv, page_size=c.P, num_pages=c.num_pages,
                        pt_stride=c.pt_stride, num_wgs=min(2 * num_cus(), 40),
                        kv_dtype=L.ATTN_KV_FP8_E4M3 if kv_dtype == "fp8" else L.ATTN_KV_BF16, mode=mode)
    print(f"graph case {kind} {kv_dtype} mode {mode} fused {fused}: B {c.B}, lengths {start.min()}..{start.max()}",
          flush=True)
    A, E = _state(c, start), _state(c, start)
    att_a, att_e = L.Attention(shape, DEV), L.Attention(shape, DEV)

    # capture on a side stream (the binding launches on the current stream)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        _step(att_a, A, c.sm_scale, fused)
    torch.cuda.synchronize()

    gen = torch.Generator().manual_seed(11)
    lengths = start.copy()
    for r in range(REPLAYS):
        q = torch.randn(c.B, c.Hq, c.D, generator=gen).to(torch.bfloat16)
        kn = torch.randn(c.B, c.Hkv, c.D, generator=gen).to(torch.bfloat16)
        vn = torch.randn(c.B, c.Hkv, c.D, generator=gen).to(torch.bfloat16)
        pos = torch.from_numpy(lengths.copy())
        lengths = lengths + 1
        new_len = torch.from_numpy(lengths.copy())
        for s in (A, E):
            s["q"].copy_(q)
            s["kn"].copy_(kn)
            s["vn"].copy_(vn)
            s["pos"].copy_(pos)
            s["len"].copy_(new_len)
            s["out"].fill_(float("nan"))
            s["lse"].fill_(float("nan"))
        g.replay()
        _step(att_e, E, c.sm_scale, fused)
        torch.cuda.synchronize()
        for name in ("out", "lse", "k", "v"):
            assert _bitwise(A[name], E[name]), f"replay {r}: {name} differs from the eager step"
        # eager work of the program between replays
        assert torch.isfinite(A["out"].float()).all()
    assert att_a.status() == 0 and att_e.status() == 0

    # the last replay against the CPU reference, on the state it left
    ref = wl.Case(c.name, c.B, c.Hq, c.Hkv, c.D, c.P, lengths.astype(np.int32), c.page_table, c.num_pages,
                  c.kv_dtype, q, A["k"].cpu(), A["v"].cpu(), c.k_scale, c.v_scale, c.sm_scale, c.meta)
    ro, rl = oracle.decode(ref)
    check_close(A["out"].double().cpu().numpy(), A["lse"].double().cpu().numpy(), ro, rl,
                FP8_TOL if kv_dtype == "fp8" else BF16_TOL, what=f"{kind} {kv_dtype} last replay")
