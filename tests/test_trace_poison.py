"""The device mirror of the continuous-batching trace, run on CPU tensors: after
every transition the live cache rows equal the host model's codes and every
other row (free pages of the pool, pages of finished requests, rows past a
request's length in its last page) holds the e4m3fn NaN code, so that a decode
that reads outside the live rows produces NaN. Finishing requests is what the
source article's serving traffic does (users stop at unpredictable times)
[Tencent HPC lands in SGLang, challenging default inference kernels, sec. "Why
Tencent HPC matters for online model serving"]."""
import pytest
import torch

from variable_length_kv_amd import workloads as wl
from variable_length_kv_amd.trace import NAN_E4M3FN, DeviceTrace


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_dead_rows_are_nan_live_rows_exact(seed):
    tr = wl.Trace(steps=60, slots=10, Hq=8, Hkv=2, P=16, seed=seed, p_finish=0.15, new_lo=1, new_hi=200,
                  init_lo=1, init_hi=400)
    dt = DeviceTrace(tr, device="cpu")
    replaced = 0
    for s in range(tr.steps):
        live = torch.zeros(tr.num_pages, tr.P, dtype=torch.bool)
        for b in range(tr.slots):
            for j in range(int(tr.lengths[b])):
                live[int(tr.page_table[b, j // tr.P]), j % tr.P] = True
        for dev, host in ((dt.k, tr.k_cache), (dt.v, tr.v_cache)):
            d, h = dev.permute(0, 2, 1, 3), host.permute(0, 2, 1, 3)
            assert torch.equal(d[live], h[live]), f"step {s}: live rows differ"
            assert bool((d[~live] == NAN_E4M3FN).all()), f"step {s}: a dead row is not NaN"
        if s == tr.steps - 1:
            break
        replaced += len(dt.advance()["slots"])
    assert replaced > 20
