"""Host logic of bench.py (no GPU): the one-GPU refusal, the settling loop and
the committed traffic counters' source check."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


class _CountingRun:
    def __init__(self):
        self.fused_calls = self.three_calls = 0

    def fused(self, att):
        self.fused_calls += 1

    def three(self, att):
        self.three_calls += 1


class _Torch:
    class cuda:
        @staticmethod
        def synchronize():
            pass


def test_settle_runs_both_forms_and_stops():
    run = _CountingRun()
    assert bench.settle(run, None, _Torch, 0.0) == 0
    n = bench.settle(run, None, _Torch, 0.01)
    assert n > 0 and n % 25 == 0
    assert run.fused_calls == run.three_calls == n


def test_traffic_counters_follow_the_device_code():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    entry = bench.traffic_entry(bench.FUSED_KERNEL)
    if t["code_hash"] == bench.code_hash():
        assert entry == t["kernels"][bench.FUSED_KERNEL]["hbm_bytes_per_launch"]
        # every K/V byte fetched once, plus a little (q, page table, partials)
        assert 1.0 <= t["kernels"][bench.FUSED_KERNEL]["read_over_algorithmic"] < 1.05
    else:
        assert entry is None


def test_compare_flags_out_of_bound_outputs():
    import numpy as np
    import torch
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((3, 4, 128)) * 0.05
    ref_l = rng.standard_normal((3, 4))
    ref_l[1] = -np.inf                       # an empty request
    out = torch.tensor(ref).to(torch.bfloat16)
    lse = torch.tensor(ref_l, dtype=torch.float32)
    good = bench.compare(out, lse, ref, ref_l, "bf16")
    assert good["ok"] and good["worst_err_over_bound"] < 0.1
    bad = out.clone()
    bad[2, 1, 7] += 0.5                      # one element off by far more than the bound
    assert not bench.compare(bad, lse, ref, ref_l, "bf16")["ok"]
    nan = out.clone()
    nan[0, 0, 0] = float("nan")
    assert not bench.compare(nan, lse, ref, ref_l, "bf16")["ok"]
    lbad = lse.clone()
    lbad[0, 0] += 0.01
    assert not bench.compare(out, lbad, ref, ref_l, "bf16")["ok"]
    lfin = lse.clone()
    lfin[1, 0] = 0.0                         # a finite lse where the reference has none
    assert not bench.compare(out, lfin, ref, ref_l, "bf16")["ok"]


def test_code_hash_reads_the_device_code_section(tmp_path, monkeypatch):
    """The hash covers the library's .hip_fatbin section and nothing else: a
    minimal ELF with that section hashes its bytes; changing another section
    leaves the hash alone, changing the section changes it."""
    import hashlib
    import struct

    def elf(fatbin, other):
        names = b"\0.shstrtab\0.hip_fatbin\0.text\0"
        data = names + fatbin + other
        shoff = 64 + len(data)
        secs = [(0, 0, 0, 0, 0, 0),
                (1, 3, 0, 0, 64, len(names)),                                  # .shstrtab
                (11, 1, 2, 0, 64 + len(names), len(fatbin)),                   # .hip_fatbin
                (23, 1, 6, 0, 64 + len(names) + len(fatbin), len(other))]      # .text
        head = bytearray(64)
        head[:4] = b"\x7fELF"
        struct.pack_into("<Q", head, 0x28, shoff)
        struct.pack_into("<HHH", head, 0x3A, 64, len(secs), 1)
        body = b"".join(struct.pack("<IIQQQQ", *sec) + bytes(24) for sec in secs)
        return bytes(head) + data + body

    lib_dir = tmp_path / "variable_length_kv_amd"
    lib_dir.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (lib_dir / "libvlkv_attn.so").write_bytes(elf(b"DEVICE-CODE-1", b"host code A"))
    h1 = bench.code_hash()
    assert h1 == hashlib.sha256(b"DEVICE-CODE-1").hexdigest()[:16]
    (lib_dir / "libvlkv_attn.so").write_bytes(elf(b"DEVICE-CODE-1", b"host code B, longer"))
    assert bench.code_hash() == h1
    (lib_dir / "libvlkv_attn.so").write_bytes(elf(b"DEVICE-CODE-2", b"host code A"))
    assert bench.code_hash() != h1


def test_profile_kernel_names():
    assert bench._short_name("vlkv::(anonymous namespace)::decode_kernel<2, 0>(vlkv::DecodeArgs)") == \
        "decode_kernel<2, 0>"
    assert bench._short_name("vlkv::(anonymous namespace)::plan_kernel(vlkv::PlanArgs)") == "plan_kernel"
    assert bench._short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_kernel_stats_follow_the_device_code():
    if not os.path.exists(bench.KERNEL_STATS_FILE):
        return
    with open(bench.KERNEL_STATS_FILE) as f:
        t = json.load(f)
    avg = bench.kernel_stats_entry(bench.FUSED_KERNEL)
    if t["code_hash"] == bench.code_hash():
        assert avg == t["kernels"][bench.FUSED_KERNEL]["avg_ns"]
    else:
        assert avg is None
