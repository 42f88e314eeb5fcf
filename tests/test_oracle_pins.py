"""Pins for the CPU reference's decode attention (no GPU).

Every test here checks ``oracle.decode`` against something other than itself:
an independent NumPy brute force, a closed form, an exact special case, an
invariance the definition implies, or a library conversion routine. The
definition being pinned is the plain softmax attention of one decode query per
head over its request's cached rows; splitting the KV work (the "split-k" of
the source article [Tencent HPC lands in SGLang, challenging default inference
kernels, sec. "Why Tencent HPC matters for online model serving"]) must not
change it.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.brute as brute
from variable_length_kv_amd import workloads as wl


def _case(lengths, **kw):
    kw.setdefault("Hq", 8)
    kw.setdefault("Hkv", 2)
    kw.setdefault("P", 16)
    return wl.make_case("t", lengths, **kw)


# ----------------------------------------------------------- brute force --

@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_numpy_brute_force(kv, seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 4))
    lengths = rng.integers(0, 41, B)
    lengths[0] = max(lengths[0], 1)
    c = _case(lengths, kv_dtype=kv, seed=seed, Hq=4 * (1 + seed % 2), Hkv=1 + seed % 2, P=8)
    o, l = oracle.decode(c)
    bo, bl = brute.decode(c)
    assert np.allclose(o, bo, rtol=1e-12, atol=1e-14)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(l))
    assert np.allclose(l[fin], bl[fin], rtol=1e-12, atol=1e-13)
    assert np.all(l[~fin] == -np.inf)


def test_matches_numpy_brute_force_small_head_dim():
    c = _case([3, 40, 1], Hq=4, Hkv=2, P=8, D=4, seed=7)
    o, l = oracle.decode(c)
    bo, bl = brute.decode(c)
    assert np.allclose(o, bo, rtol=1e-12, atol=1e-15)
    assert np.allclose(l, bl, rtol=1e-12, atol=1e-15)


def test_tiny_workload_matches_brute_force():
    c = wl.config_case(0)
    o, l = oracle.decode(c)
    bo, bl = brute.decode(c)
    assert np.max(np.abs(o - bo)) <= 1e-12 * max(1.0, np.abs(bo).max())
    assert np.max(np.abs(l - bl)) <= 1e-12 * np.abs(bl).max()


# --------------------------------------------------------- closed forms --

def _rows(c, b, g, which):
    cache = c.k_cache if which == "k" else c.v_cache
    x = cache.float().double() if c.kv_dtype == "bf16" else None
    L = int(c.lengths[b])
    j = np.arange(L)
    pages = torch.from_numpy(c.page_table[b, j // c.P].astype(np.int64))
    return x[pages, g, torch.from_numpy(j % c.P), :].numpy()


def test_single_token_returns_v_exactly():
    c = _case([1, 1, 1], Hq=8, Hkv=2, seed=4)
    o, l = oracle.decode(c)
    for b in range(3):
        for h in range(8):
            g = h // 4
            v = _rows(c, b, g, "v")[0]
            k = _rows(c, b, g, "k")[0]
            assert np.array_equal(o[b, h], v)
            s = c.sm_scale * float(np.dot(c.q[b, h].double().numpy(), k))
            assert l[b, h] == pytest.approx(s, rel=1e-15, abs=1e-15)


def test_identical_value_rows_return_that_row():
    c = _case([37, 64, 5], Hq=8, Hkv=2, seed=5)
    v = c.v_cache.clone()
    row = v[0, 0, 0].clone()
    v[:] = row
    o, _ = oracle.decode(c, v_cache=v)
    ref = row.double().numpy()
    assert np.max(np.abs(o - ref[None, None, :])) <= 1e-15 * np.abs(ref).max() * 4


def test_zero_query_gives_mean_and_log_length():
    c = _case([1, 9, 50], Hq=4, Hkv=2, seed=6)
    q0 = torch.zeros_like(c.q)
    o, l = oracle.decode(c, q=q0)
    for b in range(3):
        L = int(c.lengths[b])
        for h in range(4):
            mean = _rows(c, b, h // 2, "v").mean(axis=0)
            assert np.allclose(o[b, h], mean, rtol=1e-13, atol=1e-15)
            assert l[b, h] == pytest.approx(math.log(L), rel=1e-15, abs=1e-15)


def test_two_tokens_sigmoid_form():
    c = _case([2], Hq=2, Hkv=1, seed=8)
    o, l = oracle.decode(c)
    K = _rows(c, 0, 0, "k")
    V = _rows(c, 0, 0, "v")
    for h in range(2):
        qh = c.q[0, h].double().numpy()
        s0 = c.sm_scale * math.fsum(qh * K[0])
        s1 = c.sm_scale * math.fsum(qh * K[1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        assert np.allclose(o[0, h], w0 * V[0] + w1 * V[1], rtol=1e-13, atol=1e-15)
        assert l[0, h] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), rel=1e-14)


@pytest.mark.parametrize("jstar", [0, 31, 47, 199])
def test_peaked_query_selects_one_row(jstar):
    """q proportional to K_j* with a large factor puts all weight on row j*,
    wherever j* falls (first, middle or last tile)."""
    c = _case([200], Hq=1, Hkv=1, seed=9)
    K = _rows(c, 0, 0, "k")
    V = _rows(c, 0, 0, "v")
    # make row j* the unique maximiser: keys on the unit sphere, query along K_j*
    Kn = K / np.linalg.norm(K, axis=1, keepdims=True)
    kc = c.k_cache.clone().float()
    pages = c.page_table[0, np.arange(200) // c.P]
    for j in range(200):
        kc[int(pages[j]), 0, j % c.P] = torch.from_numpy(Kn[j]).float()
    kc = kc.to(torch.bfloat16)
    Kb = kc.double()[torch.from_numpy(pages.astype(np.int64)), 0, torch.from_numpy(np.arange(200) % c.P)].numpy()
    q = torch.from_numpy(Kb[jstar] * 4000.0).to(torch.bfloat16).reshape(1, 1, -1)
    o, _ = oracle.decode(c, q=q, k_cache=kc)
    assert np.allclose(o[0, 0], V[jstar], rtol=0, atol=1e-9)


def test_empty_request():
    c = _case([0, 5], Hq=4, Hkv=2, seed=10)
    o, l = oracle.decode(c)
    assert np.all(o[0] == 0) and np.all(l[0] == -np.inf)
    assert np.all(np.isfinite(l[1]))


# ----------------------------------------------------------- invariances --

def test_page_permutation_is_bitwise_invariant():
    c = _case([30, 64, 129, 7], Hq=8, Hkv=2, seed=11)
    perm = np.random.default_rng(5).permutation(c.num_pages)  # new id of old page p is perm[p]
    inv = torch.from_numpy(np.argsort(perm).astype(np.int64))
    k2 = c.k_cache[inv]
    v2 = c.v_cache[inv]
    pt2 = np.where(c.page_table >= 0, perm[np.maximum(c.page_table, 0)], -1).astype(np.int32)
    o1, l1 = oracle.decode(c)
    o2, l2 = oracle.decode(c, k_cache=k2, v_cache=v2, page_table=pt2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("cut_pages", [1, 3, 7])
def test_split_and_merge_equals_whole(cut_pages):
    """Attend to the first part and the rest of one request separately (as two
    requests sharing its pages), merge by log-sum-exp weights: same result."""
    c = _case([150], Hq=4, Hkv=1, P=16, seed=12)
    L = 150
    pt = c.page_table[0]
    npg = (L + 15) // 16
    a_len = cut_pages * 16
    stride = npg
    pt2 = np.full((2, stride), -1, np.int32)
    pt2[0, :cut_pages] = pt[:cut_pages]
    pt2[1, :npg - cut_pages] = pt[cut_pages:npg]
    q2 = torch.cat([c.q, c.q], 0)
    two = wl.Case("split", 2, c.Hq, c.Hkv, c.D, c.P, np.array([a_len, L - a_len], np.int32), pt2,
                  c.num_pages, "bf16", q2, c.k_cache, c.v_cache, None, None, c.sm_scale)
    o2, l2 = oracle.decode(two)
    o, l = oracle.decode(c)
    M = np.maximum(l2[0], l2[1])
    w0, w1 = np.exp(l2[0] - M), np.exp(l2[1] - M)
    merged = (w0[:, None] * o2[0] + w1[:, None] * o2[1]) / (w0 + w1)[:, None]
    assert np.allclose(merged, o[0], rtol=1e-12, atol=1e-15)
    assert np.allclose(M + np.log(w0 + w1), l[0], rtol=1e-13, atol=1e-14)


def test_query_head_permutation_within_group():
    c = _case([77, 20], Hq=8, Hkv=2, seed=13)
    perm = np.array([2, 0, 3, 1, 7, 6, 5, 4])  # stays inside each group of 4
    o, l = oracle.decode(c)
    o2, l2 = oracle.decode(c, q=c.q[:, perm])
    assert np.array_equal(o2, o[:, perm]) and np.array_equal(l2, l[:, perm])


def test_fp8_scale_algebra():
    c = _case([40, 3], Hq=4, Hkv=2, kv_dtype="fp8", seed=14)
    o, l = oracle.decode(c)
    o2, l2 = oracle.decode(c, v_scale=c.v_scale * 2)
    assert np.array_equal(o2, 2 * o) and np.array_equal(l2, l)
    o3, l3 = oracle.decode(c, k_scale=c.k_scale * 2)
    o4, l4 = oracle.decode(c, sm_scale=c.sm_scale * 2)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)


def test_result_does_not_read_slack_slots():
    c = _case([17, 33], Hq=4, Hkv=1, seed=15)
    k = c.k_cache.clone()
    v = c.v_cache.clone()
    for b in range(2):
        L = int(c.lengths[b])
        last = int(c.page_table[b, (L - 1) // c.P])
        k[last, :, L % c.P:] = float("nan")
        v[last, :, L % c.P:] = float("nan")
    o, l = oracle.decode(c)
    o2, l2 = oracle.decode(c, k_cache=k, v_cache=v)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_invalid_inputs_are_refused():
    c = _case([20], Hq=4, Hkv=1, seed=16)
    with pytest.raises(ValueError):
        oracle.decode(c, lengths=np.array([10 ** 6], np.int32))
    pt = c.page_table.copy()
    pt[0, 1] = c.num_pages
    with pytest.raises(ValueError):
        oracle.decode(c, page_table=pt)


# ------------------------------------------------------- value decoders --

def test_e4m3fn_decoder_against_library_and_spec_points():
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = np.array([oracle.e4m3fn_to_f64(c) for c in range(256)])
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan) and nan.sum() == 2
    assert np.array_equal(ours[~nan], lib[~nan])
    assert oracle.e4m3fn_to_f64(0x7E) == 448.0       # largest finite
    assert oracle.e4m3fn_to_f64(0x01) == 2.0 ** -9    # smallest subnormal
    assert oracle.e4m3fn_to_f64(0x08) == 2.0 ** -6    # smallest normal
    assert oracle.e4m3fn_to_f64(0x38) == 1.0
    assert oracle.e4m3fn_to_f64(0xB8) == -1.0


def test_bf16_decoder_against_library():
    bits = np.random.default_rng(0).integers(0, 1 << 16, 4000).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite patterns
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    ours = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    assert np.array_equal(ours, lib)


# ------------------------------------------------ planted-mistake check --

def test_pins_catch_a_dropped_last_row(tmp_path):
    """Build a copy of the oracle with one plausible mistake (the last cached
    row of each request skipped in the value pass) and check that the
    brute-force pin rejects it. The mistake is planted in a CPU copy only."""
    import ctypes
    import subprocess
    src = open(oracle.__file__.replace("__init__.py", "oracle.c")).read()
    bad = src.replace("/* pass 3: weighted sum of value rows */\n        memset(o, 0, sizeof(double) * (size_t)G * D);\n        for (int64_t j = 0; j < L; ++j) {",
                      "/* pass 3: weighted sum of value rows */\n        memset(o, 0, sizeof(double) * (size_t)G * D);\n        for (int64_t j = 0; j < L - 1; ++j) {")
    assert bad != src
    cfile = tmp_path / "bad.c"
    cfile.write_text(bad)
    so = tmp_path / "libbad.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(cfile), "-lm"], check=True)
    good_lib = oracle._lib
    try:
        oracle._lib = None
        lib = ctypes.CDLL(str(so))
        oracle._load()  # set signatures on the real library, then copy them
        for name in ("oracle_decode",):
            getattr(lib, name).restype = getattr(oracle._lib, name).restype
            getattr(lib, name).argtypes = getattr(oracle._lib, name).argtypes
        oracle._lib = lib
        c = _case([9, 30], Hq=4, Hkv=1, seed=17)
        o, _ = oracle.decode(c)
        bo, _ = brute.decode(c)
        assert not np.allclose(o, bo, rtol=1e-6, atol=1e-6)
    finally:
        oracle._lib = good_lib


# ------------------------------------------------------------ KV append --

def _torch_e4m3fn(y):
    """Library reference: torch's own float -> float8_e4m3fn conversion, after
    saturating to the format's largest finite value."""
    t = torch.from_numpy(np.ascontiguousarray(y, np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3fn_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = np.array([oracle.e4m3fn_to_f64(int(c)) for c in codes], np.float32)
    assert np.array_equal(oracle.e4m3fn_encode(vals), codes)


def test_e4m3fn_encoder_matches_library_on_ties_and_a_dense_sweep():
    finite = np.array(sorted({oracle.e4m3fn_to_f64(c) for c in range(0x7F)}))   # non-negative values
    mids = (finite[:-1] + finite[1:]) / 2                                      # exact ties
    f32 = mids.astype(np.float32)
    near = np.concatenate([f32, np.nextafter(f32, np.float32(np.inf)), np.nextafter(f32, np.float32(-np.inf))])
    rng = np.random.default_rng(0)
    dense = np.concatenate([
        rng.uniform(0, 2.0 ** -6, 20000), rng.uniform(0, 1, 20000), rng.uniform(0, 500, 20000),
        np.exp(rng.uniform(np.log(1e-6), np.log(1e6), 20000)), finite, [0.0, 448.0, 449.0, 464.0, 480.0, 1e30],
    ]).astype(np.float32)
    y = np.concatenate([near, dense])
    y = np.concatenate([y, -y])
    assert np.array_equal(oracle.e4m3fn_encode(y), _torch_e4m3fn(y))
    assert oracle.e4m3fn_encode(np.array([np.nan], np.float32))[0] == 0x7F


def _append_expected(c, k_new, v_new, positions):
    """Independent construction of the appended caches with torch indexing and
    torch's conversions (no loop shared with the C reference)."""
    kc, vc = c.k_cache.clone(), c.v_cache.clone()
    for b, pos in enumerate(positions):
        if pos < 0 or pos >= c.pt_stride * c.P:
            continue
        page = int(c.page_table[b, pos // c.P])
        if page < 0 or page >= c.num_pages:
            continue
        if c.kv_dtype == "fp8":
            kq = torch.from_numpy(_torch_e4m3fn((k_new[b].float() / c.k_scale[b][:, None]).numpy()))
            vq = torch.from_numpy(_torch_e4m3fn((v_new[b].float() / c.v_scale[b][:, None]).numpy()))
            kc[page, :, pos % c.P] = kq
            vc[page, :, pos % c.P] = vq
        else:
            kc[page, :, pos % c.P] = k_new[b]
            vc[page, :, pos % c.P] = v_new[b]
    return kc, vc


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_reference_against_independent_construction(kv):
    c = _case([5, 16, 31, 0], Hq=4, Hkv=2, P=16, kv_dtype=kv, seed=21, pt_stride=3, extra_pages=2)
    rng = np.random.default_rng(3)
    k_new = torch.from_numpy(rng.normal(0, 3, (c.B, c.Hkv, c.D)).astype(np.float32)).to(torch.bfloat16)
    v_new = torch.from_numpy(rng.normal(0, 3, (c.B, c.Hkv, c.D)).astype(np.float32)).to(torch.bfloat16)
    pos = np.array([5, 16, 31, 0], np.int32)             # new pages at 16 (page 1) need a page id
    pt = c.page_table.copy()
    pt[1, 1] = c.num_pages - 1
    pt[3, 0] = c.num_pages - 2
    c2 = wl.Case(c.name, c.B, c.Hq, c.Hkv, c.D, c.P, c.lengths, pt, c.num_pages, c.kv_dtype, c.q, c.k_cache,
                 c.v_cache, c.k_scale, c.v_scale, c.sm_scale)
    kc, vc, st = oracle.append_kv(c2, k_new, v_new, pos)
    ek, ev = _append_expected(c2, k_new, v_new, pos)
    view = torch.uint8 if kv == "fp8" else torch.int16
    assert st == 0
    assert np.array_equal(kc.view(ek.view(view).numpy().dtype), ek.view(view).numpy())
    assert np.array_equal(vc.view(ev.view(view).numpy().dtype), ev.view(view).numpy())
    # skips: no append (-1), a position past the page table (bit 1), a bad page id (bit 2)
    pt[2, 1] = c.num_pages + 7
    c3 = wl.Case(c.name, c.B, c.Hq, c.Hkv, c.D, c.P, c.lengths, pt, c.num_pages, c.kv_dtype, c.q, c.k_cache,
                 c.v_cache, c.k_scale, c.v_scale, c.sm_scale)
    kc, vc, st = oracle.append_kv(c3, k_new, v_new, np.array([-1, 48, 17, 0], np.int32))
    assert st == 3
    ek, ev = _append_expected(c3, k_new, v_new, [-1, -1, -1, 0])
    assert np.array_equal(kc.view(ek.view(view).numpy().dtype), ek.view(view).numpy())
