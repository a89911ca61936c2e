"""Both row kernels on the same workloads: the one-workgroup-per-row kernel
and the split-row kernel (many workgroups per row) are each forced through
the debug flags, whatever the batch size would pick, and each must match the
fp64 oracle on every row."""
import numpy as np
import pytest
import torch

import decode_step_token_amd as dst
import workloads as wl
from tests.parity import compare, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    dst.load()
    yield
    torch.cuda.synchronize()


def _check(w, path, probs_rows=None):
    log(f"case {w.name} B={w.B} V={w.V} dtype={w.dtype} step={w.step} path={path}")
    gpu = run_gpu(w, path=path)
    stats = compare(w, gpu, run_oracle(w), check_probs_rows=probs_rows)
    log(f"  ok {stats}")
    return gpu


def _flat(w, T=1.5, p=(0.95, 0.99)):
    w.temperature[:] = np.float32(T)
    w.top_k[:] = -1
    w.top_p[:] = np.where(np.arange(w.B) % 2 == 0, p[0], p[1]).astype(np.float32)
    return w


@pytest.mark.parametrize("path", ["stream", "split"])
@pytest.mark.parametrize("V,dtype", [(1000, "f32"), (5000, "bf16"), (33000, "f32"), (151936, "bf16")])
def test_tiny_mixed(path, V, dtype):
    _check(wl.tiny(np.random.default_rng(V + 5), 48, V, dtype), path)


@pytest.mark.parametrize("path", ["stream", "split"])
def test_c0_c1(path):
    _check(wl.c0(), path)
    _check(wl.c1(), path)


def test_c3_split():
    _check(wl.c3(), "split", probs_rows=set(range(0, 256, 19)))


def test_c2_split():
    _check(wl.c2(), "split", probs_rows=set(range(0, 256, 23)))


def test_c4_split():
    _check(wl.c4(0), "split", probs_rows=set(range(0, 512, 67)))


@pytest.mark.parametrize("path", ["stream", "split"])
def test_flat_top_p_rows(path):
    """Top-p only at T = 1.5: nuclei of thousands of tokens (the split kernel
    cuts them through the row's weight histogram)."""
    _check(_flat(wl.c3()), path, probs_rows=set(range(0, 256, 17)))


@pytest.mark.parametrize("path", ["stream", "split"])
def test_flat_bf16_rows_with_ties(path):
    """bf16 rows at T = 1.5: the boundary bin holds long runs of equal values,
    cut in token order."""
    w = wl.tiny(np.random.default_rng(21), 32, 152064, "bf16", scale=2.5)
    _check(_flat(w, p=(0.9, 0.95)), path, probs_rows={0, 7, 31})


@pytest.mark.parametrize("path", ["stream", "split"])
def test_flat_bf16_rows_late_spike(path):
    """bf16 rows at T = 1.5 that the first tiles show to be flat, so the
    per-row kernel builds their weight histogram while it streams.  A value
    beyond the first tiles by far more than 2^30 in weight makes that row
    build the histogram again after the stream (the nucleus is then that one
    token); a value 3 above the maximum lands in the top bin; the other rows
    are plain flat rows."""
    rng = np.random.default_rng(23)
    w = wl.tiny(rng, 24, 152064, "bf16", scale=2.5)
    x = wl.bf16_bits_to_f32(w.logits)
    for b in range(w.B):
        j = int(rng.integers(60000, w.V))
        x[b, j] = x[b].max() + (40.0, 3.0, 0.0)[b % 3]
    w.logits = wl.to_bf16_bits(x)
    _check(_flat(w, p=(0.9, 0.95)), path, probs_rows={0, 1, 2, 23})


@pytest.mark.parametrize("path", ["stream", "split"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_flat_rows_crowded_boundary_bin(path, dtype):
    """Top-p rows at T = 1.5 with a block of one repeated value (2,000 to
    100,000 copies at random positions).  The larger blocks hold enough of the
    mass for the nucleus to end inside them, so the boundary bin holds tens of
    thousands of equal entries, cut in token order; that many entries do not
    fit the per-wave regions, and the row is finished from the row itself.
    The smaller blocks fit."""
    rng = np.random.default_rng(31)
    w = wl.tiny(rng, 16, 152064, dtype, scale=2.5)
    x = wl.bf16_bits_to_f32(w.logits) if dtype == "bf16" else w.logits
    for b in range(w.B):
        n = (2000, 5000, 20000, 100000)[b % 4]
        x[b, rng.choice(w.V, n, replace=False)] = 0.0
    w.logits = wl.to_bf16_bits(x) if dtype == "bf16" else x
    _check(_flat(w, p=(0.9, 0.95)), path, probs_rows={0, 3, 6, 15})


@pytest.mark.parametrize("path", ["stream", "split"])
def test_min_p_mix(path):
    w = wl.with_min_p(wl.tiny(np.random.default_rng(22), 48, 40000, "f32"),
                      [0.0, 0.01, 0.05, 0.2, 0.5], 22)
    _check(w, path)
    w = wl.with_min_p(_flat(wl.tiny(np.random.default_rng(23), 32, 33000, "bf16")),
                      [0.0, 0.001, 0.02, 0.3], 23)
    _check(w, path)
