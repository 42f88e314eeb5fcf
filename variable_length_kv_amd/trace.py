"""Device mirror of the continuous-batching trace (``workloads.Trace``).

The host trace owns the fp8 page pool, the page table, the lengths and the
per-(slot, kv-head) scales; after each ``advance()`` this class patches the
device copies with exactly what changed (the appended token rows, the pages
written for replacement requests) and re-uploads the small arrays (lengths,
page table, scales, queries). Copies are plain host-to-device transfers made
between steps, outside any timed region. With ``append`` given, the appended
rows are instead written on the device by that call (the library's
attn_append_kv) from the bf16 rows, positions and scales; the host model's
own codes then serve to check it. No attention arithmetic lives here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import workloads as wl


class DeviceTrace:
    def __init__(self, trace: wl.Trace, device="cuda:0", append=None):
        self.tr = trace
        self.dev = torch.device(device)
        self.append = append
        def up(t):
            return t.to(self.dev, copy=True)
        self.k = up(trace.k_cache)
        self.v = up(trace.v_cache)
        self.ks = up(trace.k_scale)
        self.vs = up(trace.v_scale)
        self.pt = up(torch.from_numpy(np.ascontiguousarray(trace.page_table)))
        self.len = up(torch.from_numpy(np.ascontiguousarray(trace.lengths, np.int32)))
        self.q = up(trace.q)

    @property
    def step(self) -> int:
        return self.tr.step

    def advance(self):
        """Host transition step -> step+1, then patch the device copies."""
        tr = self.tr
        old_len = np.asarray(tr.lengths, np.int32).copy()
        patch = tr.advance()
        up = lambda t: t.to(self.dev, non_blocking=False)
        self.ks.copy_(tr.k_scale)
        self.vs.copy_(tr.v_scale)
        self.pt.copy_(torch.from_numpy(np.ascontiguousarray(tr.page_table)))
        if self.append is not None:
            # appended rows written on the device; replaced slots get fresh pages below
            pos = old_len.copy()
            pos[patch["slots"]] = -1
            self.append(up(patch["new_k"].contiguous()), up(patch["new_v"].contiguous()), up(torch.from_numpy(pos)),
                        self.pt, self.k, self.v, self.ks, self.vs)
        else:
            pages, slots = patch["rows"]
            if len(pages):
                dp, ds = pages.to(self.dev), slots.to(self.dev)
                self.k[dp, :, ds] = tr.k_cache[pages, :, slots].to(self.dev)
                self.v[dp, :, ds] = tr.v_cache[pages, :, slots].to(self.dev)
        whole = patch["pages"]
        if len(whole):
            dw = whole.to(self.dev)
            self.k[dw] = tr.k_cache[whole].to(self.dev)
            self.v[dw] = tr.v_cache[whole].to(self.dev)
        self.len.copy_(torch.from_numpy(np.ascontiguousarray(tr.lengths, np.int32)))
        self.q.copy_(tr.q)
        return patch
