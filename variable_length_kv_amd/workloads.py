"""Seeded synthetic inputs for variable-length paged decode attention.

This module holds input recipes only: per-request context lengths, paged KV
page tables, query/key/value values, the fp8 codes and per-(request, kv-head)
scales of a quantised cache, and the continuous-batching event trace. It holds
none of the attention arithmetic. The CPU reference under ``oracle/`` and the
HIP path both consume what it produces; neither is imported here.

Workload shapes follow the one concrete example the source article gives (one
request at 16,000 tokens of context next to others that have just started at
1,000) and its description of serving traffic, where requests arrive
continuously, contexts grow at different rates and users stop at unpredictable
times [Tencent HPC lands in SGLang, challenging default inference kernels,
sec. "Why Tencent HPC matters for online model serving"]. Cache precision is
named there as a benchmark dimension [same page, sec. "What the 48.8% TPOT
claim does not prove"], hence the fp8 trace.

Random streams. A base seed ``s`` gives three independent streams: lengths and
trace events from ``numpy.random.default_rng(3*s)``, page placement from
``default_rng(3*s + 1)``, and values from child streams of
``SeedSequence(3*s + 2)`` (one child per 4 Mi-element chunk of each tensor,
keyed by a tensor tag), so that bulk values can be drawn on many threads and
still be identical for every thread count. Values are float32
``standard_normal`` rounded to bfloat16 (round to nearest even).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

FP8_E4M3_MAX = 448.0
CHUNK = 1 << 22  # elements per value-stream chunk
HEAD_DIM = 128

# tensor tags for the value streams
TAG_Q, TAG_K, TAG_V = 0, 1, 2


def _workers() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_f32(data_seed: int, tag: tuple, n: int) -> np.ndarray:
    """n float32 N(0,1) draws from the chunked value stream (data_seed, tag)."""
    out = np.empty(n, np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(i):
        ss = np.random.SeedSequence(entropy=data_seed, spawn_key=tuple(tag) + (i,))
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        np.random.default_rng(ss).standard_normal(out=out[lo:hi], dtype=np.float32)

    if nchunks <= 1:
        for i in range(nchunks):
            fill(i)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def to_bf16(x: np.ndarray, shape) -> torch.Tensor:
    """float32 -> bfloat16 with round-to-nearest-even (torch's cast)."""
    return torch.from_numpy(x).reshape(shape).to(torch.bfloat16)


def fp8_codes(x: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """OCP e4m3fn codes (uint8) of x/scale, saturated to +-448, RNE.

    ``scale`` broadcasts against ``x``. This is how the synthetic fp8 cache is
    written; the method itself only ever reads codes and scales.
    """
    y = (x.float() / scale).clamp_(-FP8_E4M3_MAX, FP8_E4M3_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


@dataclass
class Case:
    """One decode step's inputs, all host (CPU) tensors.

    Layouts: q [B, Hq, D] bf16; k_cache, v_cache [num_pages, Hkv, P, D]
    (bf16, or uint8 e4m3fn codes); k_scale, v_scale [B, Hkv] float32 (fp8
    only); page_table [B, pt_stride] int32, -1 past each request's last page;
    lengths [B] int32.
    """

    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    P: int
    lengths: np.ndarray
    page_table: np.ndarray
    num_pages: int
    kv_dtype: str
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_scale: Optional[torch.Tensor]
    v_scale: Optional[torch.Tensor]
    sm_scale: float
    meta: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def pt_stride(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def elem_bytes(self) -> int:
        return 1 if self.kv_dtype == "fp8" else 2

    @property
    def total_tokens(self) -> int:
        return int(np.asarray(self.lengths, np.int64).sum())

    @property
    def kv_bytes(self) -> int:
        """Algorithmic KV bytes of one step: every cached K and V row once."""
        return 2 * self.Hkv * self.D * self.elem_bytes * self.total_tokens


def make_page_table(lengths, P, rng_pages, pt_stride=None, extra_pages=0):
    """Random physical placement: a permutation of all pages, dealt out in order."""
    lengths = np.asarray(lengths, np.int64)
    n = (lengths + P - 1) // P
    total = int(n.sum())
    num_pages = max(1, total + int(extra_pages))
    perm = rng_pages.permutation(num_pages).astype(np.int32)
    stride = int(pt_stride) if pt_stride is not None else max(1, int(n.max()) if len(n) else 1)
    if stride < (int(n.max()) if len(n) else 0):
        raise ValueError("pt_stride smaller than the longest request's page count")
    pt = np.full((len(lengths), stride), -1, np.int32)
    off = 0
    for b, nb in enumerate(n):
        pt[b, :nb] = perm[off:off + nb]
        off += int(nb)
    return pt, num_pages


def _fill_cache_bf16(data_seed, tag, num_pages, Hkv, P, D):
    return to_bf16(normal_f32(data_seed, tag, num_pages * Hkv * P * D), (num_pages, Hkv, P, D))


def _request_scale(pages_f: torch.Tensor, L: int) -> torch.Tensor:
    """amax/448 per kv-head over the first L tokens of a request's pages
    [npg, Hkv, P, D]; 1.0 where that amax is 0."""
    npg, Hkv, P, D = pages_f.shape
    x = pages_f.transpose(0, 1).reshape(Hkv, npg * P, D)[:, :L]
    amax = x.abs().amax(dim=(1, 2)).float()
    return torch.where(amax > 0, amax / FP8_E4M3_MAX, torch.ones_like(amax))


def _owner_scales(cache_f: torch.Tensor, lengths, page_table, P):
    """Per-(request, kv-head) scales of the requests that own the pages."""
    B = len(lengths)
    scale = torch.ones(B, cache_f.shape[1], dtype=torch.float32)
    for b in range(B):
        L = int(lengths[b])
        if L:
            npg = (L + P - 1) // P
            pages = torch.from_numpy(page_table[b, :npg].astype(np.int64))
            scale[b] = _request_scale(cache_f[pages], L)
    return scale


def _quantize_owned(cache_f: torch.Tensor, scale, lengths, page_table, P):
    """Codes for every page: owned pages with the owner's scale, spare pages with 1."""
    num_pages, Hkv = cache_f.shape[0], cache_f.shape[1]
    page_scale = torch.ones(num_pages, Hkv, dtype=torch.float32)
    for b in range(len(lengths)):
        npg = (int(lengths[b]) + P - 1) // P
        if npg:
            pages = torch.from_numpy(page_table[b, :npg].astype(np.int64))
            page_scale[pages] = scale[b]
    return fp8_codes(cache_f, page_scale[:, :, None, None])


def make_case(name, lengths, *, Hq=8, Hkv=1, P=16, D=HEAD_DIM, kv_dtype="bf16",
              seed=0, pt_stride=None, extra_pages=0, sm_scale=None, page_table=None, num_pages=None) -> Case:
    """Build a decode step with the given lengths; all randomness from ``seed``.
    A given ``page_table`` / ``num_pages`` replaces the random placement."""
    lengths = np.asarray(lengths, np.int32)
    B = len(lengths)
    rng_pages = np.random.default_rng(3 * seed + 1)
    data_seed = 3 * seed + 2
    if page_table is None:
        pt, num_pages = make_page_table(lengths, P, rng_pages, pt_stride, extra_pages)
    else:
        pt, num_pages = np.ascontiguousarray(page_table, np.int32), int(num_pages)
    q = to_bf16(normal_f32(data_seed, (TAG_Q,), B * Hq * D), (B, Hq, D))
    k = _fill_cache_bf16(data_seed, (TAG_K,), num_pages, Hkv, P, D)
    v = _fill_cache_bf16(data_seed, (TAG_V,), num_pages, Hkv, P, D)
    ks = vs = None
    if kv_dtype == "fp8":
        ks = _owner_scales(k, lengths, pt, P)
        vs = _owner_scales(v, lengths, pt, P)
        k = _quantize_owned(k, ks, lengths, pt, P)
        v = _quantize_owned(v, vs, lengths, pt, P)
    elif kv_dtype != "bf16":
        raise ValueError(kv_dtype)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    return Case(name, B, Hq, Hkv, D, P, lengths, pt, num_pages, kv_dtype, q, k, v, ks, vs,
                float(sm_scale), {"seed": seed})


def sub_case(case: Case, ids) -> Case:
    """The requests ``ids`` of a decode step as a batch of their own, with
    only their pages (renumbered in order of first use) and their scales: a
    compact host copy of part of a step, e.g. one of a trace whose caches
    change afterwards. Pure input bookkeeping."""
    ids = [int(i) for i in ids]
    P = case.P
    lengths = np.asarray(case.lengths, np.int64)[ids]
    n = (np.maximum(lengths, 0) + P - 1) // P
    stride = max(1, int(n.max()) if len(n) else 1)
    pt = np.full((len(ids), stride), -1, np.int32)
    pages, index = [], {}
    for r, b in enumerate(ids):
        for j in range(int(n[r])):
            p = int(case.page_table[b, j])
            if p not in index:
                index[p] = len(pages)
                pages.append(p)
            pt[r, j] = index[p]
    sel = torch.tensor(pages if pages else [0], dtype=torch.int64)
    ks = case.k_scale[ids].clone() if case.k_scale is not None else None
    vs = case.v_scale[ids].clone() if case.v_scale is not None else None
    return Case(f"{case.name}[{len(ids)}]", len(ids), case.Hq, case.Hkv, case.D, P, lengths.astype(np.int32), pt,
                max(1, len(pages)), case.kv_dtype, case.q[ids].clone(), case.k_cache[sel].clone(),
                case.v_cache[sel].clone(), ks, vs, case.sm_scale, dict(case.meta, ids=ids))


def shared_page_table(lengths, groups, P, seed):
    """Page table with prefix caching: ``groups`` lists (first, count,
    prefix_pages); requests first+1 .. first+count-1 read request first's
    pages in their first prefix_pages slots, every other slot gets a page of
    its own. Physical placement is a seeded random permutation. Returns
    (page_table, num_pages)."""
    lengths = np.asarray(lengths, np.int64)
    B = len(lengths)
    n = (lengths + P - 1) // P
    alias = {}   # (b, slot) -> (leader, slot)
    for first, count, npg in groups:
        for b in range(first + 1, first + count):
            for j in range(min(int(npg), int(n[b]), int(n[first]))):
                alias[(b, j)] = (first, j)
    own = [(b, j) for b in range(B) for j in range(int(n[b])) if (b, j) not in alias]
    perm = np.random.default_rng(seed).permutation(len(own)).astype(np.int32)
    pt = np.full((B, max(1, int(n.max()) if B else 1)), -1, np.int32)
    for (b, j), pid in zip(own, perm):
        pt[b, j] = pid
    for (b, j), (f, jj) in alias.items():
        pt[b, j] = pt[f, jj]
    return pt, max(1, len(own))


def make_shared_case(name, lengths, groups, *, Hq=8, Hkv=1, P=16, kv_dtype="bf16", seed=0) -> Case:
    """A decode step whose requests share prefix pages (see shared_page_table)."""
    pt, num_pages = shared_page_table(lengths, groups, P, 3 * seed + 1)
    c = make_case(name, lengths, Hq=Hq, Hkv=Hkv, P=P, kv_dtype=kv_dtype, seed=seed, page_table=pt,
                  num_pages=num_pages)
    c.meta["groups"] = [tuple(int(x) for x in g) for g in groups]
    return c


def shared_prefix_lengths(n_groups, group_size, prefix_tokens, suffix_lo, suffix_hi, P, seed=0):
    """Agentic batch: n_groups groups of group_size requests that share a
    prefix_tokens-long prompt (its whole pages are shared), each with its own
    suffix of U[suffix_lo, suffix_hi] tokens. Returns (lengths, groups) for
    make_shared_case."""
    rng = np.random.default_rng(3 * seed)
    suffix = rng.integers(suffix_lo, suffix_hi, n_groups * group_size, endpoint=True)
    lengths = (prefix_tokens + suffix).astype(np.int32)
    return lengths, [(g * group_size, group_size, prefix_tokens // P) for g in range(n_groups)]


# --------------------------------------------------------------------------
# The five workloads (0-based ids)
# --------------------------------------------------------------------------

CONFIG_NAMES = {
    0: "tiny: 4 requests {17,64,200,1000}, Hq/Hkv 8/1, P 16, bf16",
    1: "uniform-mixed: 32 requests U[1000,16000], Hq/Hkv 64/8, P 64, bf16",
    2: "skewed: 1x16000 + 63x1000, Hq/Hkv 64/8, P 64, bf16",
    3: "long-tail: 128 requests lognormal(median 2048, sigma 1.2) clipped [128,131072], Hq/Hkv 64/8, P 64, bf16",
    4: "continuous-batching trace: 96 slots, init U[512,32768], +1/step, 2%/step replaced by U[256,4096], fp8 e4m3 KV, 256 steps",
}


def config_lengths(cid: int, seed: int = 0) -> np.ndarray:
    rng_len = np.random.default_rng(3 * seed)
    if cid == 0:
        return np.array([17, 64, 200, 1000], np.int32)
    if cid == 1:
        return rng_len.integers(1000, 16000, 32, endpoint=True).astype(np.int32)
    if cid == 2:
        return np.array([16000] + [1000] * 63, np.int32)
    if cid == 3:
        x = np.exp(rng_len.normal(math.log(2048.0), 1.2, 128))
        return np.clip(np.rint(x), 128, 131072).astype(np.int32)
    if cid == 4:
        return rng_len.integers(512, 32768, 96, endpoint=True).astype(np.int32)
    raise ValueError(cid)


def config_case(cid: int, seed: int = 0, long_last: bool = False) -> Case:
    """Workloads 0-3 as one decode step. ``long_last`` moves workload 2's long
    request from index 0 to the last index."""
    lengths = config_lengths(cid, seed)
    if cid == 0:
        return make_case("c0", lengths, Hq=8, Hkv=1, P=16, seed=seed)
    if cid in (1, 2, 3):
        if cid == 2 and long_last:
            lengths = lengths[::-1].copy()
        return make_case(f"c{cid}", lengths, Hq=64, Hkv=8, P=64, seed=seed)
    raise ValueError("workload 4 is a trace: use Trace")


# --------------------------------------------------------------------------
# Workload 4: continuous-batching trace with an fp8 cache
# --------------------------------------------------------------------------

def trace_lengths(steps=256, slots=96, seed=0, p_finish=0.02, new_lo=256, new_hi=4096,
                  init_lo=512, init_hi=32768):
    """Per-step lengths and replacement events of the trace (integers only).

    Step 0 uses the initial lengths. Between step s and s+1 every request grows
    by one token; then each slot finishes with probability p_finish and is
    replaced, in slot order, by a new request of uniform length.
    Returns (lengths [steps, slots], events: list per transition of slot ids).
    """
    rng_len = np.random.default_rng(3 * seed)
    L = rng_len.integers(init_lo, init_hi, slots, endpoint=True).astype(np.int64)
    out = np.empty((steps, slots), np.int64)
    events = []
    for s in range(steps):
        out[s] = L
        if s == steps - 1:
            break
        L = L + 1
        fin = np.nonzero(rng_len.random(slots) < p_finish)[0]
        newL = rng_len.integers(new_lo, new_hi, len(fin), endpoint=True)
        L[fin] = newL
        events.append(list(zip(fin.tolist(), newL.tolist())))
    return out.astype(np.int32), events


class Trace:
    """Host model of the continuous-batching trace with an fp8 paged cache.

    Owns the host copy of the caches (uint8 codes), the page pool and its free
    list, the page table and the per-(slot, kv-head) scales. ``advance()``
    applies one transition and returns what changed so a device copy can be
    patched: appended token rows and freshly written pages.
    """

    def __init__(self, steps=256, slots=96, Hq=64, Hkv=8, P=64, D=HEAD_DIM, seed=0, **kw):
        self.steps, self.slots, self.Hq, self.Hkv, self.P, self.D = steps, slots, Hq, Hkv, P, D
        self.seed = seed
        self.lengths_all, self.events = trace_lengths(steps, slots, seed, **kw)
        self.rng_pages = np.random.default_rng(3 * seed + 1)
        self.data_seed = 3 * seed + 2
        # page budget: replay the page counts of the allocation order below
        npg = (self.lengths_all.astype(np.int64) + P - 1) // P
        peak = int(npg[0].sum())
        for s in range(steps - 1):
            cur = npg[s].copy()
            grown = (self.lengths_all[s].astype(np.int64) + 1 + P - 1) // P
            in_use = int(grown.sum())
            peak = max(peak, in_use)
            for slot, newL in self.events[s]:
                in_use += -int(grown[slot]) + (newL + P - 1) // P
                peak = max(peak, in_use)
            del cur
        self.num_pages = peak + slots
        self.pt_stride = int(npg.max()) + 1
        self.step = 0
        L0 = self.lengths_all[0]
        self.lengths = L0.copy()
        perm = self.rng_pages.permutation(self.num_pages).astype(np.int32)
        n0 = (L0.astype(np.int64) + P - 1) // P
        self.page_table = np.full((slots, self.pt_stride), -1, np.int32)
        off = 0
        for b in range(slots):
            self.page_table[b, :n0[b]] = perm[off:off + n0[b]]
            off += int(n0[b])
        self.free = list(perm[off:].tolist())
        # initial cache values: whole pool, then per-request scales and codes
        shape = (self.num_pages, Hkv, P, D)
        kf = _fill_cache_bf16(self.data_seed, (TAG_K,), *shape)
        self.k_scale = _owner_scales(kf, L0, self.page_table, P)
        self.k_cache = _quantize_owned(kf, self.k_scale, L0, self.page_table, P)
        del kf
        vf = _fill_cache_bf16(self.data_seed, (TAG_V,), *shape)
        self.v_scale = _owner_scales(vf, L0, self.page_table, P)
        self.v_cache = _quantize_owned(vf, self.v_scale, L0, self.page_table, P)
        del vf
        self.q = self._draw_q(0)

    def _draw_q(self, s):
        n = self.slots * self.Hq * self.D
        return to_bf16(normal_f32(self.data_seed, (100 + s, TAG_Q), n), (self.slots, self.Hq, self.D))

    def _pop_page(self):
        i = int(self.rng_pages.integers(len(self.free)))
        p = self.free[i]
        self.free[i] = self.free[-1]
        self.free.pop()
        return p

    def case(self) -> Case:
        return Case(f"c4@{self.step}", self.slots, self.Hq, self.Hkv, self.D, self.P,
                    self.lengths.copy(), self.page_table.copy(), self.num_pages, "fp8",
                    self.q, self.k_cache, self.v_cache, self.k_scale, self.v_scale,
                    1.0 / math.sqrt(self.D), {"step": self.step})

    def advance(self):
        """Apply the transition step -> step+1. Returns a dict of patches:
        rows: (pages, slots_in_page) int64 tensors of appended token rows;
        pages: int64 tensor of pages rewritten whole; slots: slots whose scales changed
        (replaced requests); new_k, new_v: the appended bf16 rows [slots, Hkv, D]."""
        s = self.step
        if s >= self.steps - 1:
            raise StopIteration
        P, Hkv, D = self.P, self.Hkv, self.D
        # 1) every request appends one token (K/V quantised with its own scales)
        nb = self.slots
        kn = torch.from_numpy(normal_f32(self.data_seed, (100 + s, 10), nb * Hkv * D)).reshape(nb, Hkv, D)
        vn = torch.from_numpy(normal_f32(self.data_seed, (100 + s, 11), nb * Hkv * D)).reshape(nb, Hkv, D)
        kn = kn.to(torch.bfloat16)
        vn = vn.to(torch.bfloat16)
        row_pages, row_slots = [], []
        for b in range(nb):
            j = int(self.lengths[b])
            if j % P == 0:
                self.page_table[b, j // P] = self._pop_page()
            pg = int(self.page_table[b, j // P])
            self.k_cache[pg, :, j % P, :] = fp8_codes(kn[b], self.k_scale[b][:, None])
            self.v_cache[pg, :, j % P, :] = fp8_codes(vn[b], self.v_scale[b][:, None])
            row_pages.append(pg)
            row_slots.append(j % P)
            self.lengths[b] = j + 1
        # 2) finished requests free their pages and are replaced
        new_pages = []
        for slot, newL in self.events[s]:
            npg_old = (int(self.lengths[slot]) + P - 1) // P
            self.free.extend(self.page_table[slot, :npg_old].tolist())
            self.page_table[slot, :] = -1
            npg = (newL + P - 1) // P
            pages = [self._pop_page() for _ in range(npg)]
            self.page_table[slot, :npg] = pages
            self.lengths[slot] = newL
            n = npg * Hkv * P * D
            kf = to_bf16(normal_f32(self.data_seed, (100 + s, 20, slot), n), (npg, Hkv, P, D))
            vf = to_bf16(normal_f32(self.data_seed, (100 + s, 21, slot), n), (npg, Hkv, P, D))
            self.k_scale[slot] = _request_scale(kf, newL)
            self.v_scale[slot] = _request_scale(vf, newL)
            idx = torch.tensor(pages, dtype=torch.int64)
            self.k_cache[idx] = fp8_codes(kf, self.k_scale[slot][None, :, None, None])
            self.v_cache[idx] = fp8_codes(vf, self.v_scale[slot][None, :, None, None])
            new_pages.extend(pages)
        self.step = s + 1
        assert np.array_equal(self.lengths, self.lengths_all[self.step])
        self.q = self._draw_q(self.step)
        return {
            "rows": (torch.tensor(row_pages, dtype=torch.int64), torch.tensor(row_slots, dtype=torch.int64)),
            "pages": torch.tensor(sorted(set(new_pages)), dtype=torch.int64),
            "slots": [slot for slot, _ in self.events[s]],
            "new_k": kn, "new_v": vn,
        }
