"""min_p (the pages' exercise: keep p_i >= min_p * p_max on the full
temperature-scaled distribution, intersected with the top-k / top-p set),
through the C ABI, against the fp64 oracle on every row."""
import numpy as np
import pytest
import torch

import decode_step_token_amd as dst
import workloads as wl
from tests.parity import compare, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

MIN_P_VALUES = [0.0, -1.0, 0.01, 0.05, 0.2, 0.5, 1.0, 1.5]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    dst.load()
    yield
    torch.cuda.synchronize()


def _check(w, **kw):
    log(f"case {w.name} B={w.B} V={w.V} dtype={w.dtype} "
        f"{'exact path' if kw.get('force_exact') else ''}")
    gpu = run_gpu(w, **kw)
    stats = compare(w, gpu, run_oracle(w))
    log(f"  ok {stats}")
    return gpu


@pytest.mark.parametrize("V,dtype,seed", [(64, "f32", 1), (1000, "bf16", 2), (5000, "f32", 3),
                                          (33000, "bf16", 4), (151936, "f32", 5)])
def test_tiny_batches(V, dtype, seed):
    rng = np.random.default_rng(seed)
    w = wl.with_min_p(wl.tiny(rng, 48, V, dtype), MIN_P_VALUES, seed)
    _check(w)


@pytest.mark.parametrize("V,dtype,seed", [(1000, "f32", 6), (33000, "bf16", 7)])
def test_exact_path(V, dtype, seed):
    rng = np.random.default_rng(seed)
    w = wl.with_min_p(wl.tiny(rng, 32, V, dtype), MIN_P_VALUES, seed)
    _check(w, force_exact=True)


def test_c3_with_min_p():
    """c3's parameter mix with min_p from {0, 0.02, 0.05, 0.1}: the kept set
    is mostly min_p's own (a few tokens), listed from the candidates."""
    w = wl.with_min_p(wl.c3(), [0.0, 0.02, 0.05, 0.1], 8)
    _check(w)


def test_flat_rows_min_p_only():
    """c3 logits at T = 1.5 with min_p alone: small min_p keeps thousands of
    tokens (finished from the row), larger ones a few (listed)."""
    w = wl.c3()
    B = 64
    w = wl.Workload("c3_T1.5_min_p", w.dtype, w.logits[:B].copy(),
                    np.full(B, 1.5, np.float32), None, None, w.uid[:B].copy(), 3,
                    w.pool[:B].copy(), np.arange(B, dtype=np.int64), w.cols[:B].copy())
    w = wl.with_min_p(w, [0.001, 0.01, 0.1, 0.5], 9)
    _check(w)


def test_min_p_zero_changes_nothing():
    rng = np.random.default_rng(10)
    w = wl.tiny(rng, 64, 20000, "f32")
    log(f"case min_p all zero on {w.name}")
    a = run_gpu(w, debug=False)
    b = run_gpu(wl.with_min_p(w, [0.0], 0), debug=False)
    assert np.array_equal(a["tokens"], b["tokens"])


@pytest.mark.parametrize("B,V,dtype,seed", [(500, 2000, "bf16", 11), (512, 3000, "f32", 13),
                                          (777, 1000, "bf16", 14), (1500, 700, "f32", 12)])
def test_more_rows_than_compute_units(B, V, dtype, seed):
    """More rows than blocks resident at once: up to 512 rows the long rows
    (sampled, top-k off, top-p or min_p on) are started first, larger batches
    keep index order; every row still lands in its own outputs, checked on
    every row against the oracle."""
    rng = np.random.default_rng(seed)
    w = wl.with_min_p(wl.tiny(rng, B, V, dtype), [0.0, 0.0, 0.0, 0.05, 0.3], seed)
    _check(w)


@pytest.mark.parametrize("case", ["scattered", "all_long", "none_long"])
def test_long_rows_first_edges(case):
    """Reordered batches (257 <= B <= 512) with the long rows at the very end
    and scattered, with every row long, and with none: each row's token
    still equals the oracle's."""
    B, V = 300, 1500
    rng = np.random.default_rng({"scattered": 21, "all_long": 22, "none_long": 23}[case])
    w = wl.tiny(rng, B, V, "f32")
    T = np.full(B, 0.8, np.float32)
    k = np.full(B, 20, np.int64)
    p = np.full(B, 0.9, np.float64)
    if case == "scattered":
        T[::7] = 0.0                               # greedy rows are never long
        for r in (B - 1, 150, 3, 0):
            T[r], k[r], p[r] = 1.1, -1, 0.85       # top-p without top-k
    elif case == "all_long":
        k[:] = -1
    w.temperature[:] = T
    w.top_k[:] = k.astype(w.top_k.dtype)
    w.top_p[:] = p.astype(w.top_p.dtype)
    _check(w)
