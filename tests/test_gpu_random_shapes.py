"""GPU parity over randomly drawn problem shapes.

Each case draws a batch size, a head grouping (1 to 16 query heads per kv
head, 1 to 8 kv heads), a page size, a tile size, a workgroup count, a cache
type and a length mix with empty, single-token and page-boundary requests next
to one long request: the uneven contexts the dynamic schedule exists for
[Tencent HPC lands in SGLang, challenging default inference kernels, sec. "Why
Tencent HPC matters for online model serving"]. Every case runs the
three-launch step and the single launch in its mode (dynamic, static split-K
or prefix-shared). Both are compared with the CPU reference, and with each
other bit for bit (prefix-shared: attn_step enqueues the same three launches,
so it must equal them too). Rows past each length are NaN, so a read beyond a
request's last token would show.
"""
import numpy as np
import pytest

from variable_length_kv_amd import lib as L
from variable_length_kv_amd import workloads as wl

from gpu_helpers import check_against_oracle, device_inputs, run

pytestmark = pytest.mark.gpu

N_CASES = 48


def draw(seed):
    """One random case: (case, mode, T, W, S)."""
    rng = np.random.default_rng(1000 + seed)
    Hkv = int(rng.choice([1, 2, 3, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
    P = int(rng.choice([16, 32, 48, 64, 128, 256]))
    T = int(rng.choice([64, 128, 192, 256]))
    mode = int(rng.choice([L.ATTN_DYNAMIC, L.ATTN_DYNAMIC, L.ATTN_STATIC, L.ATTN_SHARED]))
    kv = "fp8" if rng.random() < 0.3 else "bf16"
    W = int(rng.choice([1, 2, 7, 33, 96, 256, 512, 1500]))
    S = int(rng.choice([0, 0, 1, 2, 3, 7]))
    if mode == L.ATTN_SHARED:
        n_groups, size = int(rng.integers(1, 4)), int(rng.integers(2, 5))
        prefix = P * int(rng.integers(1, 6))
        lengths, groups = wl.shared_prefix_lengths(n_groups, size, prefix, 0, 300, P, seed=seed)
        # a few requests outside any group, one of them empty
        lengths = np.concatenate([lengths, rng.integers(0, 400, 3), [0]]).astype(np.int32)
        c = wl.make_shared_case(f"rand{seed}", lengths, groups, Hq=G * Hkv, Hkv=Hkv, P=P, kv_dtype=kv, seed=seed)
    else:
        B = int(rng.integers(1, 28))
        lengths = rng.integers(0, 600, B)
        lengths[rng.random(B) < 0.15] = 0
        special = [1, P - 1, P, P + 1, T, T + 1, 2 * T - 1]
        for i in range(min(B, 3)):
            lengths[int(rng.integers(B))] = int(rng.choice(special))
        lengths[int(rng.integers(B))] = int(rng.integers(1, 5000))
        c = wl.make_case(f"rand{seed}", lengths.astype(np.int32), Hq=G * Hkv, Hkv=Hkv, P=P, kv_dtype=kv, seed=seed)
    return c, mode, T, W, S


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    c, mode, T, W, S = draw(seed)
    what = (f"seed {seed}: B {c.B}, Hq {c.Hq}, Hkv {c.Hkv}, P {c.P}, T {T}, W {W}, mode {mode}, S {S}, "
            f"{c.kv_dtype}, lengths {int(np.min(c.lengths))}..{int(np.max(c.lengths))}")
    print(what, flush=True)
    t = device_inputs(c)
    o3, l3, att = run(c, mode=mode, T=T, W=W, S=S, t=t)
    assert att.status() == 0, what
    check_against_oracle(c, o3, l3, what="three launches, " + what)
    of, lf, att = run(c, mode=mode, T=T, W=W, S=S, t=t, fused=True)
    assert att.status() == 0, what
    assert np.array_equal(of, o3) and np.array_equal(lf, l3), "single launch != three launches, " + what
