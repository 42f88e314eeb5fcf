"""Benchmark: variable-length paged decode attention on one MI355X, through the
C ABI of libvlkv_attn.so.

Headline workload: 32 requests with context lengths uniform in [1000, 16000],
64 query / 8 kv heads, head dim 128, bf16 paged cache with 64-token pages and a
random page table. A step is one decode step over the whole batch: the tile
plan for the current lengths, the split-KV decode and the log-sum-exp merge,
all in one launch (attn_step); the three-launch form (attn_plan + attn_decode +
attn_combine) is timed too. After --settle-s seconds of untimed steps (GPU
clocks out of idle) and W warm-up steps, K steps are timed one at a time with
HIP events, each after a 1 GiB read sweep that evicts the 256 MB Infinity Cache
(the sweep is outside the timed region); the median is the step time. The
figure of merit is effective KV bandwidth: every cached K and V row of the
batch once (2 * Hkv * D * 2 bytes per token) divided by the step time. The
same steps back to back are reported beside it.

Also reported (field "extra"): the tiny batch (4 requests, launch-bound), the
skewed batch (1 x 16000 + 63 x 1000 tokens) under the dynamic plan and under
the in-library static split-K at its default split count and a split sweep,
the long-tail batch, the 256-step continuous-batching trace over an fp8 e4m3
cache (plan rebuilt every step; the single-launch step also captured once in a
HIP graph and replayed), prefix caching, and the router GEMM, each timed per
step after a cache sweep. Every leg keeps a host copy of the outputs it timed;
the CPU reference leg ("cpu_baseline": the oracle timed on the host as a
reported baseline) also checks each of them against the oracle ("parity"),
and the process exits with status 1 if any is out of bounds.

Prints ONE JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
Profile summaries: --kernel-stats DIR OUT_JSON [BENCH_OUTPUT], --traffic-summary
FETCH_DIR WRITE_DIR PROBE_OUTPUT OUT_JSON (rocprofv3 output directories, see
profiles/).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/step and effective KV GB/s (% of HBM peak), mixed lengths"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic_uniform_mixed.json")
KERNEL_STATS_FILE = os.path.join(ROOT, "profiles", "decode_kernel_trace_uniform_mixed.json")
FUSED_KERNEL = "decode_kernel<2, 0>"     # single launch, dynamic plan, bf16 cache
THREE_KERNEL = "decode_kernel<0, 0>"     # decode launch of the three-launch step
# parity bounds against the CPU reference: |o - ref| <= atol + rtol |ref|,
# per-(request, head) relative L2, and lse within LSE_ATOL
TOL = {"bf16": (1e-2, 1e-2, 2e-2), "fp8": (5e-2, 5e-2, 6e-2)}
LSE_ATOL = 1e-3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_hash():
    """Hash of the device code inside the built library (its .hip_fatbin
    section, every kernel of it): a committed profile counts for the kernels
    only while the library carries the code it was taken on. Comments and
    host-side edits leave it unchanged; the section records the build
    directory too, so it is compared on the tree that built it."""
    import struct
    path = os.path.join(ROOT, "variable_length_kv_amd", "libvlkv_attn.so")
    if not os.path.exists(path):
        return None
    with open(path, "rb") as f:
        b = f.read()
    shoff = struct.unpack_from("<Q", b, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)
    secs = [struct.unpack_from("<IIQQQQ", b, shoff + i * shentsize) for i in range(shnum)]
    names = secs[shstrndx][4]
    for name, _typ, _flags, _addr, off, size in secs:
        if b[names + name:b.index(b"\0", names + name)] == b".hip_fatbin":
            return hashlib.sha256(b[off:off + size]).hexdigest()[:16]
    return None


def us(x_ms):
    return round(float(x_ms) * 1e3, 2)


class Runner:
    """Device copies of one decode step and Attention objects for it (W = 0:
    the library's default workgroup count)."""

    def __init__(self, case, torch, L, W=0):
        self.c, self.torch, self.L = case, torch, L
        d = torch.device("cuda:0")
        self.q = case.q.to(d)
        self.k = case.k_cache.to(d)
        self.v = case.v_cache.to(d)
        self.ks = case.k_scale.to(d) if case.k_scale is not None else None
        self.vs = case.v_scale.to(d) if case.v_scale is not None else None
        self.pt = torch.from_numpy(np.ascontiguousarray(case.page_table)).to(d)
        self.len = torch.from_numpy(np.ascontiguousarray(case.lengths, np.int32)).to(d)
        self.out = torch.empty_like(self.q)
        self.lse = torch.empty(case.B, case.Hq, dtype=torch.float32, device=d)
        self.W = W

    def attention(self, mode, S=0):
        c, L = self.c, self.L
        shape = L.AttnShape(batch=c.B, num_q_heads=c.Hq, num_kv_heads=c.Hkv, page_size=c.P,
                            num_pages=c.num_pages, pt_stride=c.pt_stride, num_wgs=self.W,
                            kv_dtype=L.ATTN_KV_FP8_E4M3 if c.kv_dtype == "fp8" else L.ATTN_KV_BF16,
                            mode=mode, static_splits=S)
        return L.Attention(shape, "cuda:0")

    def plan(self, att):
        att.plan(self.len, self.pt)

    def decode(self, att):
        att.decode(self.q, self.k, self.v, self.pt, self.c.sm_scale, self.out, self.lse, self.ks, self.vs)

    def combine(self, att):
        att.combine(self.out, self.lse)

    def three(self, att):
        self.plan(att)
        self.decode(att)
        self.combine(att)

    def fused(self, att):
        att.fused_step(self.q, self.k, self.v, self.pt, self.len, self.c.sm_scale, self.out, self.lse,
                       self.ks, self.vs)

    def step(self, att, fused):
        (self.fused if fused else self.three)(att)

    def w_eff(self, att):
        """Workgroups the dynamic plan of this step uses (from attn_plan's header)."""
        self.plan(att)
        self.torch.cuda.synchronize()
        return int(att.read_plan()["header"][2])


# Host copies of the outputs the legs timed, checked against the CPU reference
# by the cpu_baseline leg (the only part of this file that runs the oracle).
CAPTURES = []


def capture(name, case, out, lse):
    """Keep (a host copy of) the bf16 outputs and lse of `case` for the parity
    check."""
    CAPTURES.append({"name": name, "case": case, "out": out.detach().cpu().clone(),
                     "lse": lse.detach().cpu().clone()})


def capture_sample(name, case, out, lse, ids):
    """As capture, for the requests `ids` only (a compact copy of their pages)."""
    from variable_length_kv_amd import workloads as wl
    ids = sorted(int(i) for i in ids)
    CAPTURES.append({"name": name, "case": wl.sub_case(case, ids), "out": out.detach().cpu()[ids].clone(),
                     "lse": lse.detach().cpu()[ids].clone()})


def compare(out, lse, ref_o, ref_l, kv_dtype):
    """Errors of GPU outputs against the CPU reference, and whether they are
    within the parity bounds."""
    atol, rtol, l2tol = TOL[kv_dtype]
    o = out.double().numpy()
    ls = lse.double().numpy()
    err = np.abs(o - ref_o)
    bound = atol + rtol * np.abs(ref_o)
    finite = bool(np.isfinite(o).all())
    worst = float((err / bound).max()) if err.size else 0.0
    fin = np.isfinite(ref_l)
    lse_shape_ok = bool(np.array_equal(np.isfinite(ls), fin) and np.all(ls[~fin] == -np.inf))
    lerr = float(np.abs(ls[fin] - ref_l[fin]).max()) if fin.any() else 0.0
    num = np.linalg.norm((o - ref_o).reshape(-1, o.shape[-1]), axis=1)
    den = np.linalg.norm(ref_o.reshape(-1, o.shape[-1]), axis=1)
    rel = float((num[den > 0] / den[den > 0]).max()) if (den > 0).any() else 0.0
    ok = finite and worst <= 1.0 and lse_shape_ok and lerr <= LSE_ATOL and rel <= l2tol
    return {"ok": bool(ok), "max_abs_err": float(err.max()) if err.size else 0.0, "worst_err_over_bound": round(worst, 4),
            "max_lse_err": lerr, "max_rel_l2": round(rel, 5), "requests": int(o.shape[0]),
            "bound": f"|o-ref| <= {atol:g} + {rtol:g}|ref|, rel L2 <= {l2tol:g}, |lse-ref| <= {LSE_ATOL:g}"}


def ev(torch):
    return torch.cuda.Event(enable_timing=True)


def bracketed(fn, steps, torch):
    """ms per step of `steps` back-to-back calls of fn, from one pair of events
    around all of them (no event between steps)."""
    start, end = ev(torch), ev(torch)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def bracketed_ahead(fn, steps, torch, spin_cycles=4_000_000):
    """As bracketed, but behind a spin kernel of about a millisecond, so that
    the host has queued every call before the first one starts: the events
    then see the GPU's time for short calls, not the host's time to issue
    them."""
    fn()
    start, end = ev(torch), ev(torch)
    torch.cuda.synchronize()
    torch.cuda._sleep(spin_cycles)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def timed_three(run, att, steps, warmup, torch):
    """Three-launch steps back to back. Returns (ms per step from events around
    all K steps, per-launch ms [K, 3] from a second pass with HIP events around
    each launch on the stream the library launches on)."""
    for _ in range(warmup):
        run.three(att)
    ms = bracketed(lambda: run.three(att), steps, torch)
    evs = [[ev(torch) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        run.plan(att)
        evs[i][1].record()
        run.decode(att)
        evs[i][2].record()
        run.combine(att)
        evs[i][3].record()
    torch.cuda.synchronize()
    per = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in evs])
    return ms, per


def settle(run, att, torch, seconds):
    """Untimed single-launch and three-launch steps for `seconds` of wall time
    before anything is measured, so that the GPU clocks have left their idle
    state: with only the W warm-up steps (a few ms) the first measurement of a
    process reads a few per cent slow."""
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(25):
            run.fused(att)
            run.three(att)
        torch.cuda.synchronize()
        n += 25
    return n


def timed_fused(run, att, steps, warmup, torch):
    """Single-launch steps back to back. Returns (ms per step from events
    around all K steps, per-launch ms [K] from a second pass with events
    directly around each launch)."""
    for _ in range(warmup):
        run.fused(att)
    ms = bracketed(lambda: run.fused(att), steps, torch)
    evs = [[ev(torch), ev(torch)] for _ in range(steps)]
    for i in range(steps):
        evs[i][0].record()
        run.fused(att)
        evs[i][1].record()
    torch.cuda.synchronize()
    per = np.array([e[0].elapsed_time(e[1]) for e in evs])
    return ms, per


def per_step_flushed(run, att, steps, warmup, torch, flush, fused):
    """Steps timed one at a time (events around the step), each after a cache
    flush. Returns per-step ms."""
    for _ in range(warmup):
        run.step(att, fused)
    ts = []
    for _ in range(steps):
        flush.sum()  # read-only sweep: evicts the step's data, leaves no dirty lines
        a, b = ev(torch), ev(torch)
        a.record()
        run.step(att, fused)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b))
    return np.array(ts)


def cpu_baseline(case, budget_s=10.0, captures=()):
    """The CPU reference (fp64 C, OpenMP over (request, kv head)) on the same
    workload: whole passes over all requests, repeated until budget_s seconds
    have been spent (at least one pass). Then, untimed, the reference for each
    captured GPU output and its errors against the parity bounds. Returns
    (baseline, parity)."""
    import oracle
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    passes, t_total = 0, 0.0
    ref = None
    while passes == 0 or t_total < budget_s:
        t0 = time.perf_counter()
        ref = oracle.decode(case, threads=threads)
        t_total += time.perf_counter() - t0
        passes += 1
    nbytes = case.kv_bytes * passes
    # one thread, on the first eighth of the requests (a bounded sample of the same workload)
    ids = list(range(max(1, case.B // 8)))
    sub_bytes = 2 * case.Hkv * case.D * case.elem_bytes * int(np.asarray(case.lengths)[ids].sum())
    t0 = time.perf_counter()
    oracle.decode(case, req_ids=ids, threads=1)
    t1 = time.perf_counter() - t0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    base = {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} whole passes over the headline workload ({case.B} requests, "
                      f"{case.total_tokens} tokens, {case.kv_bytes / 1e6:.1f} MB of KV each) in "
                      f"{t_total:.1f} s; fp64 C, OpenMP over (request, kv head)",
            "value_1_thread": round(sub_bytes / t1 / 1e9, 4),
            "sample_1_thread": f"requests 0..{len(ids) - 1} of the same workload ({sub_bytes / 1e6:.1f} MB of KV) "
                               f"in {t1:.1f} s on one thread",
            "cpu_model": model}
    parity = {}
    for cap in captures:
        c = cap["case"]
        ro, rl = ref if c is case else oracle.decode(c, threads=threads)
        parity[cap["name"]] = compare(cap["out"], cap["lse"], ro, rl, c.kv_dtype)
    return base, parity


def stats(ts_ms, kv_bytes):
    med = float(np.median(ts_ms))
    return {"us_median": us(med), "us_p10": us(np.percentile(ts_ms, 10)), "us_p90": us(np.percentile(ts_ms, 90)),
            "pct_hbm": round(100 * kv_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}


def pick_wgs(args, cus):
    """Workgroups of the launch: --wgs-per-cu if given, else 0 (the library's
    default: two per compute unit, of which the plan uses one per compute unit
    on steps too small to give each workgroup 32 tiles)."""
    return args.wgs_per_cu * cus if args.wgs_per_cu > 0 else 0


def batch_leg(cid, torch, L, wl, W_of, flush, static_sweep=False):
    c = wl.config_case(cid)
    W = W_of(c.lengths, c.Hkv)
    r = Runner(c, torch, L, W)
    name = {2: "skewed", 3: "long_tail"}[cid]
    entry = {"kv_gb": round(c.kv_bytes / 1e9, 4), "tokens": c.total_tokens}
    a = r.attention(L.ATTN_DYNAMIC)
    entry["num_wgs"] = r.w_eff(a)
    entry["dynamic"] = stats(per_step_flushed(r, a, 30, 5, torch, flush, True), c.kv_bytes)
    capture(f"{name}.dynamic", c, r.out, r.lse)
    entry["dynamic_three_launch"] = stats(per_step_flushed(r, a, 30, 5, torch, flush, False), c.kv_bytes)
    ms_b2b, _ = timed_fused(r, a, 30, 5, torch)
    entry["dynamic_us_back_to_back"] = us(ms_b2b)
    del a
    if static_sweep:
        sweep, sweep3 = {}, {}
        for S in (0, 1, 2, 4, 8, 16, 32, 64):
            a = r.attention(L.ATTN_STATIC, S)
            t = per_step_flushed(r, a, 20, 3, torch, flush, True)
            t3 = per_step_flushed(r, a, 20, 3, torch, flush, False)
            if S == 0:
                capture(f"{name}.static_default", c, r.out, r.lse)
                entry["static_default_splits"] = L.attn_static_splits(a.shape)
                entry["static_default"] = stats(t, c.kv_bytes)
                entry["static_default_three_launch"] = stats(t3, c.kv_bytes)
            else:
                sweep[str(S)] = us(np.median(t))
                sweep3[str(S)] = us(np.median(t3))
            del a
        entry["static_sweep_us_median"] = sweep
        entry["static_sweep_three_launch_us_median"] = sweep3
        dyn = entry["dynamic"]["us_median"]
        entry["speedup_vs_static_default"] = round(entry["static_default"]["us_median"] / dyn, 3)
        entry["speedup_vs_best_static"] = round(min(sweep.values()) / dyn, 3)
        d3 = entry["dynamic_three_launch"]["us_median"]
        entry["three_launch_speedup_vs_static_default"] = round(
            entry["static_default_three_launch"]["us_median"] / d3, 3)
        entry["three_launch_speedup_vs_best_static"] = round(min(sweep3.values()) / d3, 3)
    if cid == 2:
        # the long request last instead of first: static's worse case
        cl = wl.config_case(2, long_last=True)
        rl = Runner(cl, torch, L, W)
        a = rl.attention(L.ATTN_DYNAMIC)
        t = per_step_flushed(rl, a, 20, 3, torch, flush, True)
        capture(f"{name}.long_request_last.dynamic", cl, rl.out, rl.lse)
        del a
        a = rl.attention(L.ATTN_STATIC)
        ts = per_step_flushed(rl, a, 20, 3, torch, flush, True)
        del a, rl
        entry["long_request_last"] = {"dynamic": stats(t, cl.kv_bytes), "static_default": stats(ts, cl.kv_bytes),
                                      "speedup_vs_static_default": round(float(np.median(ts) / np.median(t)), 3)}
    del r
    torch.cuda.empty_cache()
    return entry


def tiny_leg(torch, L, wl, W_of, steps=200):
    """Workload 0: 4 requests of {17, 64, 200, 1000} tokens, 8 query heads on
    one kv head, 16-token pages. It moves 0.66 MB of KV, so a step is bound by
    launch latency, not by HBM. Steps are queued behind a spin kernel so that
    the events see the GPU's time per step rather than the host's time to issue
    it."""
    c = wl.config_case(0)
    W = W_of(c.lengths, c.Hkv)
    r = Runner(c, torch, L, W)
    a = r.attention(L.ATTN_DYNAMIC)
    fused = bracketed_ahead(lambda: r.fused(a), steps, torch)
    capture("tiny", c, r.out, r.lse)
    three = bracketed_ahead(lambda: r.three(a), steps, torch)
    W_eff = r.w_eff(a)
    del a, r
    return {"kv_mb": round(c.kv_bytes / 1e6, 3), "tokens": c.total_tokens, "num_wgs": W_eff,
            "single_launch_us_per_step": us(fused), "three_launch_us_per_step": us(three),
            "single_launch_gbs": round(c.kv_bytes / (fused * 1e-3) / 1e9, 1)}


def shared_leg(torch, L, wl, W_of, flush, Hq):
    """Workload 5: prefix caching. 16 groups of 4 requests share an 8192-token
    prompt (its 128 pages aliased in their page tables), each request with its
    own suffix of U[64, 2048] tokens; 8 kv heads, page 64, bf16. The dynamic
    plan (single launch) reads every request's prefix; the shared plan
    (ATTN_SHARED, three launches) reads a group's prefix once per 32/G
    requests at G >= 8, 16/G below. Logical bytes count every request's rows; read bytes count the
    rows the shared plan's items read."""
    lengths, groups = wl.shared_prefix_lengths(16, 4, 8192, 64, 2048, 64, seed=0)
    c = wl.make_shared_case("shared", lengths, groups, Hq=Hq, Hkv=8, P=64, seed=0)
    W = W_of(c.lengths, c.Hkv)
    r = Runner(c, torch, L, W)
    per_tok = 2 * c.Hkv * c.D * c.elem_bytes
    entry = {"requests": c.B, "q_heads": Hq, "kv_heads": c.Hkv, "requests_per_shared_pass": max(1, (32 if c.G >= 8 else 16) // c.G),
             "logical_gb": round(c.kv_bytes / 1e9, 4)}
    a = r.attention(L.ATTN_DYNAMIC)
    t_dyn = per_step_flushed(r, a, 30, 5, torch, flush, True)
    entry["dynamic"] = stats(t_dyn, c.kv_bytes)
    capture_sample(f"shared_prefix_hq{Hq}.dynamic", c, r.out, r.lse, [0, 1, 5, 30, 63])
    del a
    a = r.attention(L.ATTN_SHARED)
    r.plan(a)
    torch.cuda.synchronize()
    p = a.read_plan()
    entry["num_wgs"] = int(p["header"][2])
    read = int(np.asarray(p["len_eff"], np.int64).sum()) * per_tok
    entry["shared_items"] = int((np.asarray(p["item_m"]) > 1).sum())
    entry["read_gb"] = round(read / 1e9, 4)
    t_sh = per_step_flushed(r, a, 30, 5, torch, flush, True)
    capture_sample(f"shared_prefix_hq{Hq}.shared", c, r.out, r.lse, [0, 1, 2, 3, 17, 30, 45, 63])
    med = float(np.median(t_sh))
    entry["shared"] = {"us_median": us(med), "us_p10": us(np.percentile(t_sh, 10)),
                       "us_p90": us(np.percentile(t_sh, 90)),
                       "logical_gbs": round(c.kv_bytes / (med * 1e-3) / 1e9, 1),
                       "pct_hbm_on_read_bytes": round(100 * read / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
    entry["speedup_vs_dynamic"] = round(entry["dynamic"]["us_median"] / us(med), 3)
    del a, r
    torch.cuda.empty_cache()
    return entry


ROUTER_SHAPES = ((16, 7168, 256), (512, 7168, 256), (8192, 7168, 256), (4096, 4096, 128))
MFMA_BF16_PEAK_TFS = 2500.0


def router_leg(torch, L, reps=30):
    """Router GEMM (y = x w^T, fp32 weights split into two bf16 parts) at
    decode, mid and prefill token counts: the split-bf16 MFMA kernel against
    torch's fp32 product of the same operands and its bf16 product with the
    weights rounded to bf16. fp32-GEMM flops = 2 M K E; the kernel runs twice
    that on the matrix cores. Each figure is the mean over `reps` calls queued
    behind a spin kernel (one warm-up call first)."""
    d = "cuda:0"
    out = {}
    for M, K, E in ROUTER_SHAPES:
        g = torch.Generator(device=d).manual_seed(M + K + E)
        x = torch.randn(M, K, generator=g, device=d).to(torch.bfloat16)
        w = torch.randn(E, K, generator=g, device=d) * 0.02
        hi = torch.empty(E, K, dtype=torch.bfloat16, device=d)
        lo = torch.empty_like(hi)
        L.router_split_weights(w, hi, lo)
        y = torch.empty(M, E, dtype=torch.float32, device=d)
        gemm = L.RouterGemm(M, K, E, d)
        xf = x.float()
        split_ms = bracketed_ahead(lambda: gemm(x, hi, lo, y), reps, torch)
        fp32_ms = bracketed_ahead(lambda: torch.matmul(xf, w.t()), reps, torch)
        hic = hi.contiguous()
        bf16_ms = bracketed_ahead(lambda: torch.matmul(x, hic.t()), reps, torch)
        flops = 2.0 * M * K * E
        key = f"{M}x{K}x{E}"
        out[key] = {"split_us": us(split_ms), "torch_fp32_us": us(fp32_ms), "torch_bf16_weights_us": us(bf16_ms),
                    "split_fp32_equiv_tflops": round(flops / (split_ms * 1e-3) / 1e12, 2),
                    "mfma_tflops": round(2 * flops / (split_ms * 1e-3) / 1e12, 2),
                    "mfma_pct_of_bf16_peak": round(100 * 2 * flops / (split_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 2),
                    "weight_gb_s": round(4.0 * E * K / (split_ms * 1e-3) / 1e9, 1),
                    "speedup_vs_torch_fp32": round(fp32_ms / split_ms, 3),
                    "k_split_workspace_bytes": L.router_workspace_bytes(M, K, E)}
        del x, w, hi, lo, y, gemm, xf, hic
    torch.cuda.empty_cache()
    return out


def trace_leg(torch, L, W_of, flush, steps=256):
    """Workload 4: the continuous-batching trace with an fp8 cache. Each step is
    timed alone after a cache flush: the single-launch step (its plan is built
    inside the kernel) and the three-launch step (attn_plan included). Between
    steps the host draws the new tokens and requests and uploads the small
    arrays; each step's appended K/V rows are written on the device by
    attn_append_kv, timed on its own and also reported added to the step."""
    from variable_length_kv_amd import workloads as wl
    from variable_length_kv_amd.trace import DeviceTrace
    t0 = time.perf_counter()
    tr = wl.Trace(steps=steps)
    W = W_of(tr.lengths, tr.Hkv)
    shape = L.AttnShape(batch=tr.slots, num_q_heads=tr.Hq, num_kv_heads=tr.Hkv, page_size=tr.P,
                        num_pages=tr.num_pages, pt_stride=tr.pt_stride, num_wgs=W,
                        kv_dtype=L.ATTN_KV_FP8_E4M3)
    att = L.Attention(shape, "cuda:0")
    append_ev, append_host = [], []

    def timed_append(*args):
        # The step's new rows written on the device (attn_append_kv), timed
        # alone: queued behind the cache sweep so that the events see the kernel
        # and not the host's time to issue it (which is recorded apart).
        flush.sum()
        e0, e1 = ev(torch), ev(torch)
        e0.record()
        h0 = time.perf_counter()
        att.append_kv(*args)
        append_host.append(time.perf_counter() - h0)
        e1.record()
        append_ev.append((e0, e1))

    dt = DeviceTrace(tr, append=timed_append)
    log(f"bench: trace generated in {time.perf_counter() - t0:.1f} s ({tr.num_pages} pages)")
    out = torch.empty_like(dt.q)
    lse = torch.empty(tr.slots, tr.Hq, dtype=torch.float32, device="cuda:0")
    sm = 1.0 / math.sqrt(tr.D)

    def fused():
        att.fused_step(dt.q, dt.k, dt.v, dt.pt, dt.len, sm, out, lse, dt.ks, dt.vs)

    def three(evs):
        evs[0].record()
        att.plan(dt.len, dt.pt)
        evs[1].record()
        att.decode(dt.q, dt.k, dt.v, dt.pt, sm, out, lse, dt.ks, dt.vs)
        evs[2].record()
        att.combine(out, lse)
        evs[3].record()

    for _ in range(5):
        fused()
        three([ev(torch) for _ in range(4)])
    torch.cuda.synchronize()
    # the single-launch step captured once in a HIP graph; every step's inputs
    # are written in place into the same buffers, so one graph serves them all
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fused()
    torch.cuda.synchronize()
    tf, t3, tg, kvb, host_eager, host_graph, weff = [], [], [], [], [], [], []
    check_at = {0, steps // 2, steps - 1}
    rng = np.random.default_rng(0)
    while True:
        flush.sum()
        a, b = ev(torch), ev(torch)
        a.record()
        h0 = time.perf_counter()
        fused()
        host_eager.append(time.perf_counter() - h0)
        b.record()
        torch.cuda.synchronize()
        tf.append(a.elapsed_time(b))
        if dt.step in check_at:
            # sampled requests (the longest, those just replaced, and random ones)
            ids = set(rng.choice(tr.slots, 8, replace=False).tolist()) | {int(np.argmax(tr.lengths))}
            if dt.step > 0:
                ids |= {slot for slot, _ in tr.events[dt.step - 1]}
            capture_sample(f"trace_fp8.step{dt.step}", tr.case(), out, lse, ids)
        flush.sum()
        a, b = ev(torch), ev(torch)
        a.record()
        h0 = time.perf_counter()
        graph.replay()
        host_graph.append(time.perf_counter() - h0)
        b.record()
        torch.cuda.synchronize()
        tg.append(a.elapsed_time(b))
        flush.sum()
        evs = [ev(torch) for _ in range(4)]
        three(evs)
        torch.cuda.synchronize()
        t3.append([evs[j].elapsed_time(evs[j + 1]) for j in range(3)])
        weff.append(int(att.read_plan()["header"][2]))
        kvb.append(2 * tr.Hkv * tr.D * int(np.asarray(tr.lengths, np.int64).sum()))
        if dt.step == steps - 1:
            break
        dt.advance()
    torch.cuda.synchronize()
    ta = np.array([a.elapsed_time(b) for a, b in append_ev]) * 1e3   # us, steps 1..
    tf = np.array(tf) * 1e3   # us
    tg = np.array(tg) * 1e3
    t3 = np.array(t3) * 1e3
    t3s = t3.sum(axis=1)
    kvb = np.array(kvb, np.float64)

    def summary(t):
        gbs = kvb.sum() / (t.sum() * 1e-6) / 1e9
        return {"us_per_step_median": round(float(np.median(t)), 2),
                "us_per_step_p10": round(float(np.percentile(t, 10)), 2),
                "us_per_step_p90": round(float(np.percentile(t, 90)), 2),
                "us_per_step_p99": round(float(np.percentile(t, 99)), 2),
                "us_per_step_mean": round(float(t.mean()), 2),
                "effective_gbs": round(gbs, 2), "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 2)}

    out_d = {"steps": steps, "num_wgs": {"min": min(weff), "max": max(weff)},
             "kv_gb_mean": round(float(kvb.mean()) / 1e9, 4),
             "single_launch": summary(tf),
             "single_launch_graph_replay": summary(tg),
             "host_issue_us_median": {"single_launch_eager": round(float(np.median(host_eager)) * 1e6, 2),
                                      "graph_replay": round(float(np.median(host_graph)) * 1e6, 2)},
             "three_launch": summary(t3s)}
    with_append = tf[1:] + ta
    out_d["append_us_median"] = round(float(np.median(ta)), 2)
    out_d["append_host_issue_us_median"] = round(float(np.median(append_host)) * 1e6, 2)
    out_d["single_launch_with_append"] = {"us_per_step_median": round(float(np.median(with_append)), 2),
                                          "us_per_step_p99": round(float(np.percentile(with_append, 99)), 2)}
    out_d["three_launch"].update({"plan_us_median": round(float(np.median(t3[:, 0])), 2),
                                  "decode_us_median": round(float(np.median(t3[:, 1])), 2),
                                  "combine_us_median": round(float(np.median(t3[:, 2])), 2)})
    return out_d


def traffic_probe(torch, L, W, reps=3):
    """Launches for rocprofv3 --pmc runs: a plain 1 GiB device copy (the
    counter scale), then the headline step, single-launch and three-launch,
    each `reps` times, then the single launch on an fp8 e4m3 copy of the same
    batch `reps` times, with a cache flush before each launch."""
    from variable_length_kv_amd import workloads as wl
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        flush.sum()
        dst.copy_(src)
    torch.cuda.synchronize()
    c1 = wl.config_case(1)
    r = Runner(c1, torch, L, W)
    att = r.attention(L.ATTN_DYNAMIC)
    for fused in (True, False):
        for _ in range(reps):
            flush.sum()
            r.step(att, fused)
    torch.cuda.synchronize()
    del att, r
    c8 = wl.make_case("uniform_mixed_fp8", c1.lengths, Hq=c1.Hq, Hkv=c1.Hkv, P=c1.P, kv_dtype="fp8")
    r8 = Runner(c8, torch, L, W)
    att8 = r8.attention(L.ATTN_DYNAMIC)
    for _ in range(reps):
        flush.sum()
        r8.step(att8, True)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "decode_kv_bytes": c1.kv_bytes,
                      "decode_kv_bytes_fp8": c8.kv_bytes, "reps": reps, "code_hash": code_hash()}), flush=True)


def router_probe(torch, L, reps=3):
    """Launches for rocprofv3 runs of the router GEMM: a plain 1 GiB device
    copy (the counter scale), then for each router shape in order the weight
    split once and `reps` GEMM calls, each after a cache flush."""
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        flush.sum()
        dst.copy_(src)
    d = "cuda:0"
    for M, K, E in ROUTER_SHAPES:
        g = torch.Generator(device=d).manual_seed(M + K + E)
        x = torch.randn(M, K, generator=g, device=d).to(torch.bfloat16)
        w = torch.randn(E, K, generator=g, device=d) * 0.02
        hi = torch.empty(E, K, dtype=torch.bfloat16, device=d)
        lo = torch.empty_like(hi)
        L.router_split_weights(w, hi, lo)
        y = torch.empty(M, E, dtype=torch.float32, device=d)
        gemm = L.RouterGemm(M, K, E, d)
        for _ in range(reps):
            flush.sum()
            gemm(x, hi, lo, y)
        torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": src.numel() * 4, "router_shapes": ROUTER_SHAPES, "reps": reps}), flush=True)


def traffic_entry(kernel):
    """HBM bytes per launch of `kernel` from committed rocprofv3 counters, only
    if they were taken on the library's current device code."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("code_hash") is None or t.get("code_hash") != code_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def kernel_stats_entry(kernel):
    """Average duration (ns) of `kernel` in the committed rocprofv3 kernel
    trace of the headline command, only if taken on the library's current device code."""
    if not os.path.exists(KERNEL_STATS_FILE):
        return None
    with open(KERNEL_STATS_FILE) as f:
        t = json.load(f)
    if t.get("code_hash") is None or t.get("code_hash") != code_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k.get("avg_ns")


def _short_name(name):
    """'vlkv::(anonymous namespace)::decode_kernel<2, 0>(vlkv::DecodeArgs)' -> 'decode_kernel<2, 0>'."""
    n = name.split("(")[0] if "(anonymous" not in name else name.replace("(anonymous namespace)", "")
    n = n.split("(")[0]
    return n.split("::")[-1].strip()


def write_kernel_stats(d, out_json, bench_output=None):
    """Summarise a rocprofv3 kernel trace. ``bench_output``: the profiled
    bench run's output, whose JSON line names the device code it ran (else the
    library here is taken to be that code)."""
    import csv
    import glob
    h = code_hash()
    if bench_output:
        with open(bench_output) as f:
            line = [l for l in f.read().splitlines() if l.startswith("{")][-1]
        h = json.loads(line)["roofline"]["code_hash"]
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    kernels = {}
    for row in csv.DictReader(open(files[0])):
        kernels[_short_name(row["Name"])] = {"calls": int(row["Calls"]), "avg_ns": float(row["AverageNs"]),
                                             "min_ns": float(row["MinNs"]), "max_ns": float(row["MaxNs"])}
    res = {"code_hash": h, "stats_file": os.path.basename(files[0]), "kernels": kernels}
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def write_traffic_summary(fetch_dir, write_dir, probe_output, out_json):
    """HBM bytes per launch from the FETCH_SIZE and WRITE_SIZE counters (KiB
    per dispatch), each scaled by what it reads for the plain 1 GiB copy that
    --traffic-probe runs first."""
    import csv
    import glob
    from collections import defaultdict

    def per_dispatch(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals, names = defaultdict(float), {}
        for fn in files:
            for row in csv.DictReader(open(fn)):
                if row["Counter_Name"] != counter:
                    continue
                key = (fn, int(row["Dispatch_Id"]))
                vals[key] += float(row["Counter_Value"])
                names[key] = _short_name(row["Kernel_Name"])
        out = defaultdict(list)
        for k in sorted(vals, key=lambda kk: kk[1]):
            out[names[k]].append(vals[k])
        return out

    def pick(d, sub):
        ks = [k for k in d if sub in k]
        if len(ks) != 1:
            raise SystemExit(f"kernel {sub!r}: found {ks}")
        return d[ks[0]]

    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")
    probe = json.loads([ln for ln in open(probe_output) if ln.startswith("{")][-1])
    copy_bytes = probe["copy_bytes"]
    big = lambda v: [x for x in v if x > copy_bytes / 1024 / 4]   # the 1 GiB copies only
    cf = float(np.mean(big(pick(fetch, "copyBuffer"))))
    cw = float(np.mean(big(pick(write, "copyBuffer"))))
    fs, ws = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    alg = probe["decode_kv_bytes"]
    res = {"workload": "uniform-mixed, 32 requests, 284965 tokens (headline step)",
           "code_hash": probe["code_hash"], "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
           "fetch_scale": round(fs, 5), "write_scale": round(ws, 5), "algorithmic_bytes_per_launch": alg,
           "kernels": {}}
    for k in (FUSED_KERNEL, THREE_KERNEL, "plan_kernel", "combine_kernel"):
        f, w = pick(fetch, k), pick(write, k)
        fk, wk = float(np.mean(f)), float(np.mean(w))
        rb, wb = round(fk * 1024 * fs), round(wk * 1024 * ws)
        res["kernels"][k] = {"launches": len(f), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                             "hbm_read_bytes_per_launch": rb, "hbm_write_bytes_per_launch": wb,
                             "hbm_bytes_per_launch": rb + wb, "read_over_algorithmic": round(rb / alg, 4),
                             "spread_fetch_kib": [round(min(f), 1), round(max(f), 1)]}
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--wgs-per-cu", type=int, default=0,
                    help="workgroups per CU of the launches (0: the library's default)")
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--extra-legs", default="tiny,skewed,long_tail,trace,shared,router",
                    help="comma list of the extra workloads to run (tiny, skewed, long_tail, trace, shared, router)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of untimed steps before the first measurement (GPU clocks leave idle)")
    ap.add_argument("--trace-steps", type=int, default=256)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only the launches that the rocprofv3 --pmc runs measure")
    ap.add_argument("--router-probe", action="store_true",
                    help="only the router GEMM launches that its rocprofv3 runs measure")
    ap.add_argument("--kernel-stats", nargs="+", metavar="ARG",
                    help="ROCPROF_DIR OUT_JSON [BENCH_OUTPUT]: summarise a rocprofv3 --kernel-trace --stats "
                         "run of this bench (no GPU work)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "PROBE_OUTPUT", "OUT_JSON"),
                    help="summarise the FETCH_SIZE and WRITE_SIZE rocprofv3 --pmc runs of --traffic-probe")
    args = ap.parse_args()
    if args.kernel_stats:
        if len(args.kernel_stats) not in (2, 3):
            ap.error("--kernel-stats takes ROCPROF_DIR OUT_JSON [BENCH_OUTPUT]")
        write_kernel_stats(*args.kernel_stats)
        return
    if args.traffic_summary:
        write_traffic_summary(*args.traffic_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU would run its own "
              "requests' plan independently); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from variable_length_kv_amd import lib as L
    from variable_length_kv_amd import workloads as wl
    L.load()
    cus = L.attn_device_cu_count(0)

    def W_of(lengths, Hkv):
        return pick_wgs(args, cus)

    if args.traffic_probe:
        traffic_probe(torch, L, W_of(wl.config_lengths(1), 8))
        return
    if args.router_probe:
        router_probe(torch, L)
        return

    # ---- headline: uniform-mixed batch, dynamic plan ------------------------
    t0 = time.perf_counter()
    c1 = wl.config_case(1)
    log(f"bench: workload 1 generated in {time.perf_counter() - t0:.1f} s "
        f"({c1.kv_bytes / 1e9:.3f} GB of KV, {c1.total_tokens} tokens)")
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")   # 1 GiB read sweep
    W = W_of(c1.lengths, c1.Hkv)
    r1 = Runner(c1, torch, L, W)
    att = r1.attention(L.ATTN_DYNAMIC)
    n_settle = settle(r1, att, torch, args.settle_s)
    log(f"bench: {n_settle} untimed settling steps of each form ({args.settle_s} s)")
    ms_b2b, _ = timed_fused(r1, att, args.steps, args.warmup, torch)
    ms3, per3 = timed_three(r1, att, args.steps, args.warmup, torch)
    # the headline: exactly K steps, each timed alone after the sweep
    ts = per_step_flushed(r1, att, args.steps, args.warmup, torch, flush, True)
    capture("uniform_mixed", c1, r1.out, r1.lse)
    ms = float(np.median(ts))
    launch_ms = float(ts.mean())
    W_eff = r1.w_eff(att)
    plan_ms, dec_ms, comb_ms = per3.mean(axis=0)
    log(f"bench: headline single launch {ms * 1e3:.1f} us/step flushed (mean {launch_ms * 1e3:.1f}), "
        f"{ms_b2b * 1e3:.1f} back to back; three launches {ms3 * 1e3:.1f} us/step back to back (plan "
        f"{plan_ms * 1e3:.1f}, decode {dec_ms * 1e3:.1f}, combine {comb_ms * 1e3:.1f})")
    kv = c1.kv_bytes
    value = kv / (ms * 1e-3) / 1e9
    achieved = kv / (launch_ms * 1e-3) / 1e9
    rp = kernel_stats_entry(FUSED_KERNEL)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "uniform-mixed: 32 requests, lengths U[1000,16000] (seed 0, 284965 tokens), "
                               "64 q / 8 kv heads, head_dim 128, bf16 KV, page 64, random page table",
                   "global_batch": c1.B, "seq_len": int(c1.lengths.max()), "parallelism": "single GPU",
                   "step": "attn_step: tile plan + split-KV decode + LSE merge in one launch",
                   "timing": "median of K steps, each between HIP events after a 1 GiB read sweep",
                   "tile_tokens": 64, "num_wgs": W_eff, "settle_s": args.settle_s, "us_per_step": us(ms),
                   "us_per_step_p10": us(np.percentile(ts, 10)), "us_per_step_p90": us(np.percentile(ts, 90)),
                   "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "us_per_step_back_to_back": us(ms_b2b),
                   "pct_hbm_peak_back_to_back": round(100 * kv / (ms_b2b * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                   "three_launch": {"us_per_step_back_to_back": us(ms3),
                                    "pct_hbm_peak": round(100 * kv / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                                    "plan_us": us(plan_ms), "decode_us": us(dec_ms), "combine_us": us(comb_ms),
                                    "decode_kernel_pct_hbm": round(100 * kv / (dec_ms * 1e-3) / 1e9
                                                                   / HBM_PEAK_GBS, 2)}},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_entry(FUSED_KERNEL),
                     "kernel": FUSED_KERNEL + " (single launch, dynamic plan, bf16 KV)",
                     "algorithmic_bytes_per_launch": kv, "launch_avg_us": us(launch_ms),
                     "launch_timing": "HIP events around each launch on the library's stream, after a 1 GiB "
                                      "sweep (dispatch included)",
                     "code_hash": code_hash(),
                     "rocprof": None if rp is None else {
                         "avg_us": round(rp / 1e3, 2),
                         "frac": round(kv / (rp * 1e-9) / 1e9 / HBM_PEAK_GBS, 4),
                         "source": os.path.relpath(KERNEL_STATS_FILE, ROOT)}},
    }
    del att, r1
    torch.cuda.empty_cache()

    # ---- extra workloads ------------------------------------------------------
    if not args.no_extra:
        extra = {}
        legs = set(args.extra_legs.split(","))
        if "tiny" in legs:
            extra["tiny"] = tiny_leg(torch, L, wl, W_of)
            log(f"bench: tiny: {json.dumps(extra['tiny'])}")
        if "skewed" in legs:
            extra["skewed"] = batch_leg(2, torch, L, wl, W_of, flush, static_sweep=True)
            log(f"bench: skewed: {json.dumps(extra['skewed'])}")
        if "long_tail" in legs:
            extra["long_tail"] = batch_leg(3, torch, L, wl, W_of, flush)
            log(f"bench: long_tail: {json.dumps(extra['long_tail'])}")
        if "trace" in legs:
            extra["trace_fp8"] = trace_leg(torch, L, W_of, flush, args.trace_steps)
            log(f"bench: trace_fp8: {json.dumps(extra['trace_fp8'])}")
        if "shared" in legs:
            for hq in (64, 32):
                key = f"shared_prefix_hq{hq}"
                extra[key] = shared_leg(torch, L, wl, W_of, flush, hq)
                log(f"bench: {key}: {json.dumps(extra[key])}")
        if "router" in legs:
            extra["router_gemm"] = router_leg(torch, L)
            log(f"bench: router_gemm: {json.dumps(extra['router_gemm'])}")
        result["extra"] = extra
    del flush
    torch.cuda.empty_cache()

    # ---- CPU baseline (the oracle on the headline workload) and parity --------
    ok = True
    if args.cpu_budget > 0:
        result["cpu_baseline"], parity = cpu_baseline(c1, args.cpu_budget, CAPTURES)
        ok = all(v["ok"] for v in parity.values())
        result["parity"] = {"ok": ok, "reference": "CPU fp64 oracle", "checks": parity}
        log(f"bench: cpu baseline {result['cpu_baseline']}")
        log(f"bench: parity {'ok' if ok else 'FAILED'}: " + ", ".join(
            f"{k} {v['worst_err_over_bound']}" for k, v in parity.items()))
    print(json.dumps(result), flush=True)
    if not ok:
        sys.exit(1)


if __name__ == "__main__":
    main()
