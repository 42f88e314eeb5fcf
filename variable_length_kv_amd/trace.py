"""Device mirror of the continuous-batching trace (``workloads.Trace``).

The host trace owns the fp8 page pool, the page table, the lengths and the
per-(slot, kv-head) scales; after each ``advance()`` this class patches the
device copies with exactly what changed (the appended token rows, the pages
written for replacement requests) and re-uploads the small arrays (lengths,
page table, scales, queries). Copies are plain host-to-device transfers made
between steps, outside any timed region. With ``append`` given, the appended
rows are instead written on the device by that call (the library's
attn_append_kv) from the bf16 rows, positions and scales; the host model's
own codes then serve to check it. With ``poison`` (the default), every cache
row that no request may read holds the e4m3fn NaN code 0x7F on the device:
the free pages of the pool, pages freed when a request finishes, and the rows
past each request's length in its last page, so that a read outside the
live rows turns into NaN outputs. No attention arithmetic lives here.
"""
from __future__ import annotations

import numpy as np
import torch

from . import workloads as wl


NAN_E4M3FN = 0x7F


class DeviceTrace:
    def __init__(self, trace: wl.Trace, device="cuda:0", append=None, poison=True):
        self.tr = trace
        self.dev = torch.device(device)
        self.append = append
        self.poison = poison
        def up(t):
            return t.to(self.dev, copy=True)
        self.k = up(trace.k_cache)
        self.v = up(trace.v_cache)
        self.ks = up(trace.k_scale)
        self.vs = up(trace.v_scale)
        self.pt = up(torch.from_numpy(np.ascontiguousarray(trace.page_table)))
        self.len = up(torch.from_numpy(np.ascontiguousarray(trace.lengths, np.int32)))
        self.q = up(trace.q)
        if poison:
            self._poison_pages(trace.free)
            self._poison_slack(range(trace.slots))

    def _poison_pages(self, pages):
        if len(pages):
            idx = torch.as_tensor(np.asarray(pages, np.int64), device=self.dev)
            self.k[idx] = NAN_E4M3FN
            self.v[idx] = NAN_E4M3FN

    def _poison_slack(self, slots):
        """Rows past the length of each given slot, in its last page."""
        tr = self.tr
        for b in slots:
            Lb = int(tr.lengths[b])
            if Lb > 0 and Lb % tr.P:
                last = int(tr.page_table[b, (Lb - 1) // tr.P])
                self.k[last, :, Lb % tr.P:] = NAN_E4M3FN
                self.v[last, :, Lb % tr.P:] = NAN_E4M3FN

    @property
    def step(self) -> int:
        return self.tr.step

    def advance(self):
        """Host transition step -> step+1, then patch the device copies."""
        tr = self.tr
        old_len = np.asarray(tr.lengths, np.int32).copy()
        old_free = set(tr.free)
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
        if self.poison:
            # pages that finished requests gave back and no replacement took,
            # with the rows appended to them this step (also a free page that
            # a finished request took for its last token and gave back);
            # reused pages are written whole below
            free_now = set(tr.free)
            appended = set(patch["rows"][0].tolist())
            self._poison_pages(sorted((free_now - old_free) | (appended & free_now)))
        whole = patch["pages"]
        if len(whole):
            dw = whole.to(self.dev)
            self.k[dw] = tr.k_cache[whole].to(self.dev)
            self.v[dw] = tr.v_cache[whole].to(self.dev)
            if self.poison:
                self._poison_slack(patch["slots"])
        self.len.copy_(torch.from_numpy(np.ascontiguousarray(tr.lengths, np.int32)))
        self.q.copy_(tr.q)
        return patch
