"""Seeded random batches through the library's default path against the
oracle: vocabulary sizes from 17 to 200,000, both dtypes, logit shapes the
configured workloads do not have (heavy Gumbel heads, values quantised into
ties, a block of large values anywhere in the row, flat rows at high
temperature) and min_p on some batches."""
import numpy as np
import pytest
import torch

import decode_step_token_amd as dst
import workloads as wl
from tests.parity import compare, log, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

VOCABS = [17, 1000, 4097, 32000, 50257, 128256, 151936, 152064, 200000]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    dst.load()
    yield
    torch.cuda.synchronize()


def random_batch(seed: int) -> wl.Workload:
    rng = np.random.default_rng([7100, seed])
    V = int(rng.choice(VOCABS))
    B = int(rng.integers(1, max(2, min(300, 3_000_000 // V))))
    dtype = str(rng.choice(["f32", "bf16"]))
    w = wl.tiny(rng, B, V, dtype, scale=float(rng.choice([0.5, 1.0, 2.5, 4.0])))
    x = wl.bf16_bits_to_f32(w.logits) if dtype == "bf16" else w.logits.astype(np.float32)
    kind = int(rng.integers(5))
    if kind == 1:                         # heavy head
        x = (rng.gumbel(0.0, 1.0, (B, V)) * 2.0).astype(np.float32)
    elif kind == 2:                       # ties
        x = (np.round(x * 2.0) / 2.0).astype(np.float32)
    elif kind == 3:                       # a block of large values anywhere
        for b in range(B):
            n = int(rng.integers(1, min(V, 3000) + 1))
            j0 = int(rng.integers(0, V - n + 1))
            x[b, j0:j0 + n] += np.float32(rng.uniform(2.0, 8.0))
    elif kind == 4:                       # flat rows
        w.temperature[:] = np.float32(rng.uniform(1.0, 2.0))
        w.top_k[:] = -1
    w.logits = wl.to_bf16_bits(x) if dtype == "bf16" else x
    w.name = f"random_{seed}_{B}x{V}_{dtype}_kind{kind}"
    if rng.random() < 0.3:
        w = wl.with_min_p(w, [0.0, 0.01, 0.1], seed)
    return w


@pytest.mark.parametrize("block", range(4))
def test_random_batches(block):
    for seed in range(block * 25, (block + 1) * 25):
        w = random_batch(seed)
        log(f"case {w.name}")
        stats = compare(w, run_gpu(w), run_oracle(w))
        log(f"  ok {stats}")
