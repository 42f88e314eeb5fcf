"""Independent NumPy two-pass softmax attention, for tiny inputs only.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``). It gathers each request's
K/V rows through the page table with NumPy fancy indexing, forms the score
vector with a matrix product and normalises with a second pass, so it shares
no loop structure with ``oracle.c``; it pins that library on small cases.
fp8 codes are decoded through ``torch.float8_e4m3fn``'s own conversion.
"""
import numpy as np


def _widen(cache, fp8):
    import torch
    if fp8:
        t = torch.as_tensor(np.ascontiguousarray(cache)).view(torch.float8_e4m3fn)
        return t.to(torch.float64).numpy()
    t = torch.as_tensor(cache)
    if t.dtype != torch.bfloat16:
        t = t.view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def decode(case):
    """Returns (out [B, Hq, D], lse [B, Hq]) in float64."""
    import torch
    fp8 = case.kv_dtype == "fp8"
    K = _widen(case.k_cache, fp8)
    V = _widen(case.v_cache, fp8)
    q = torch.as_tensor(case.q).to(torch.float64).numpy()
    pt = np.asarray(case.page_table)
    B, Hq, D, P, Hkv = case.B, case.Hq, case.D, case.P, case.Hkv
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        L = int(case.lengths[b])
        if L == 0:
            continue
        j = np.arange(L)
        pages = pt[b, j // P]
        for g in range(Hkv):
            Kb = K[pages, g, j % P, :]
            Vb = V[pages, g, j % P, :]
            if fp8:
                Kb = Kb * float(np.asarray(case.k_scale)[b, g])
                Vb = Vb * float(np.asarray(case.v_scale)[b, g])
            Q = q[b, g * G:(g + 1) * G, :]
            S = (Q @ Kb.T) * case.sm_scale          # [G, L]
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            l = E.sum(axis=1, keepdims=True)
            out[b, g * G:(g + 1) * G] = (E @ Vb) / l
            lse[b, g * G:(g + 1) * G] = (m + np.log(l))[:, 0]
    return out, lse
