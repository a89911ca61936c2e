"""sample_batch_static, the entry point that allocates nothing, against
sample_batch (the handle's entry point, forced onto the same split-row
kernel) on the same inputs: two calls in a row on the shared static
workspace, the second with fewer rows and a shorter bf16 vocabulary."""
import numpy as np
import pytest
import torch

import decode_step_token_amd as dst
import workloads as wl
from tests.parity import compare, log, opt, run_gpu, run_oracle, to_device_logits

pytestmark = pytest.mark.gpu


def _static(w):
    logits = to_device_logits(w)
    toks = dst.sample_batch_static(
        logits, w.V, w.dtype, w.seed, temperature=opt(w.temperature, torch.float32),
        top_k=opt(w.top_k, torch.int32), top_p=opt(w.top_p, torch.float32),
        uid=opt(w.uid, torch.int64), step=w.step, min_p=opt(w.min_p, torch.float32))
    torch.cuda.synchronize()
    return toks.cpu().numpy()


def test_static_entry_matches_sample_batch():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    dst.load()
    cases = [wl.with_min_p(wl.tiny(np.random.default_rng(31), 48, 151936, "f32"), [0.0, 0.0, 0.05], 31),
             wl.tiny(np.random.default_rng(32), 20, 50000, "bf16", scale=2.5)]
    for w in cases:
        log(f"case static entry {w.name} B={w.B} V={w.V}")
        got = _static(w)
        ref = run_gpu(w, debug=False, path="split")["tokens"]
        diff = np.flatnonzero(got != ref)
        if diff.size:
            # only rows whose draw or cut the oracle flags as ambiguous may differ,
            # and then both tokens must be acceptable there
            compare(w, {"tokens": got}, run_oracle(w))
            compare(w, {"tokens": ref}, run_oracle(w))
            res = run_oracle(w, rows=list(diff))
            for r, b in zip(res, diff):
                assert r.draw_ambiguous or r.cutoff_ambiguous, \
                    f"{w.name} row {b}: static {got[b]} != sample_batch {ref[b]}"
        log(f"  ok, {diff.size} ambiguous rows differ")


def test_static_entry_rejects_sizes_beyond_its_workspace():
    dst.load()
    w = wl.tiny(np.random.default_rng(33), 65, 1000, "f32")
    with pytest.raises(dst.SamplerError, match="B outside"):
        _static(w)
    x = torch.zeros((2, 163841), dtype=torch.float32, device="cuda")
    with pytest.raises(dst.SamplerError, match="vocab_size beyond"):
        dst.sample_batch_static(x, 163841, "f32", 1)
