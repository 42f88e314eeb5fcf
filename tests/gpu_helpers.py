"""Shared helpers of the GPU tests: run a decode step through the C ABI and
compare it with the CPU reference."""
import numpy as np
import torch

import oracle
from variable_length_kv_amd import lib as L

BF16_TOL = (1e-2, 1e-2, 2e-2)   # atol, rtol, per-(b, h) relative L2
FP8_TOL = (5e-2, 5e-2, 6e-2)
LSE_ATOL = 1e-3


def dev():
    return torch.device("cuda:0")


def num_cus():
    return L.attn_device_cu_count(0)


def device_inputs(case, poison=True):
    d = dev()
    t = {
        "q": case.q.to(d),
        "k": case.k_cache.to(d),
        "v": case.v_cache.to(d),
        "pt": torch.from_numpy(np.ascontiguousarray(case.page_table)).to(d),
        "len": torch.from_numpy(np.ascontiguousarray(case.lengths, np.int32)).to(d),
        "ks": case.k_scale.to(d) if case.k_scale is not None else None,
        "vs": case.v_scale.to(d) if case.v_scale is not None else None,
    }
    if poison:
        poison_slack(case, t["k"], t["v"])
    return t


def poison_slack(case, k, v):
    """Fill cache rows past each request's length in its last page with NaN."""
    nan = 0x7F if case.kv_dtype == "fp8" else None
    for b, Lb in enumerate(np.asarray(case.lengths)):
        Lb = int(Lb)
        if Lb <= 0 or Lb % case.P == 0:
            continue
        last = int(case.page_table[b, (Lb - 1) // case.P])
        if nan is None:
            k[last, :, Lb % case.P:] = float("nan")
            v[last, :, Lb % case.P:] = float("nan")
        else:
            k[last, :, Lb % case.P:] = nan
            v[last, :, Lb % case.P:] = nan


def shape_for(case, mode=L.ATTN_DYNAMIC, T=64, W=None, S=0):
    return L.AttnShape(batch=case.B, num_q_heads=case.Hq, num_kv_heads=case.Hkv, page_size=case.P,
                       num_pages=case.num_pages, pt_stride=case.pt_stride,
                       num_wgs=W if W is not None else 2 * num_cus(), tile_tokens=T,
                       kv_dtype=L.ATTN_KV_FP8_E4M3 if case.kv_dtype == "fp8" else L.ATTN_KV_BF16,
                       mode=mode, static_splits=S)


def run(case, mode=L.ATTN_DYNAMIC, T=64, W=None, S=0, t=None, poison=True, lengths=None,
        page_table=None, fused=False, att=None):
    """One decode step: attn_plan + attn_decode + attn_combine, or the
    single-launch attn_step if ``fused``. Returns (out float64 [B,Hq,D],
    lse float64 [B,Hq], att)."""
    if t is None:
        t = device_inputs(case, poison)
    if att is None:
        att = L.Attention(shape_for(case, mode, T, W, S), dev())
    out = torch.full_like(t["q"], float("nan"))
    lse = torch.full((case.B, case.Hq), float("nan"), dtype=torch.float32, device=dev())
    step = att.fused_step if fused else att.step
    step(t["q"], t["k"], t["v"], t["pt"] if page_table is None else page_table,
         t["len"] if lengths is None else lengths, case.sm_scale, out, lse,
         k_scale=t["ks"], v_scale=t["vs"])
    torch.cuda.synchronize()
    return out.double().cpu().numpy(), lse.double().cpu().numpy(), att


def check_close(out, lse, ref_o, ref_l, tol=BF16_TOL, what=""):
    atol, rtol, l2 = tol
    assert out.shape == ref_o.shape
    assert np.isfinite(out).all(), f"{what}: non-finite outputs"
    err = np.abs(out - ref_o)
    bound = atol + rtol * np.abs(ref_o)
    worst = float((err / bound).max()) if err.size else 0.0
    assert (err <= bound).all(), f"{what}: max err {err.max():.3e}, worst err/bound {worst:.3f}"
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs"
    assert np.all(lse[~fin] == -np.inf)
    if fin.any():
        lerr = np.abs(lse[fin] - ref_l[fin]).max()
        assert lerr <= LSE_ATOL, f"{what}: lse err {lerr:.3e}"
    num = np.linalg.norm((out - ref_o).reshape(-1, out.shape[-1]), axis=1)
    den = np.linalg.norm(ref_o.reshape(-1, out.shape[-1]), axis=1)
    nz = den > 0
    if nz.any():
        rel = (num[nz] / den[nz]).max()
        assert rel <= l2, f"{what}: per-head relative L2 {rel:.3e}"
    return worst


def check_against_oracle(case, out, lse, req_ids=None, tol=None, what=""):
    if tol is None:
        tol = FP8_TOL if case.kv_dtype == "fp8" else BF16_TOL
    ref_o, ref_l = oracle.decode(case, req_ids)
    if req_ids is not None:
        out, lse = out[req_ids], lse[req_ids]
    return check_close(out, lse, ref_o, ref_l, tol, what)
