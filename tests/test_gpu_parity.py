"""Parity of the HIP sampler with the fp64 oracle, through the C ABI.

Every case prints its name before touching the GPU.  Small cases compare
every row and every probability; the full-size workloads compare every row's
token, kept length, top-k list and Philox word, and the probabilities of a
sample of rows.
"""
import numpy as np
import pytest
import scipy.stats
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


def _check(w, **kw):
    log(f"case {w.name} B={w.B} V={w.V} dtype={w.dtype} step={w.step} "
        f"{'exact path' if kw.get('force_exact') else ''}{kw.get('path') or ''}")
    gpu = run_gpu(w, **{k: v for k, v in kw.items() if k in ("pad", "debug", "force_exact", "path")})
    ref = run_oracle(w)
    stats = compare(w, gpu, ref, check_probs_rows=kw.get("probs_rows"))
    log(f"  ok {stats}")
    return gpu, ref


def test_c0_mixed_batch():
    gpu, ref = _check(wl.c0())
    assert [r.greedy for r in ref] == [True, True, False, False]


def test_c0_permuted():
    a, _ = _check(wl.c0())
    b, _ = _check(wl.c0_permuted())
    perm = [2, 0, 3, 1]
    assert list(b["tokens"]) == [a["tokens"][i] for i in perm]


def test_c1_all_greedy_with_ties():
    w = wl.c1()
    gpu, ref = _check(w)
    for b, i_star, j in w.meta["ties"]:
        assert gpu["tokens"][b] == min(i_star, j)
    assert np.array_equal(gpu["tokens"], np.argmax(w.logits, axis=1))


@pytest.mark.parametrize("V,dtype,pad", [
    (1, "f32", 0), (2, "bf16", 0), (63, "f32", 1), (64, "bf16", 0), (1000, "f32", 0),
    (1023, "bf16", 3), (4097, "f32", 1), (5000, "bf16", 0), (33000, "f32", 0),
])
def test_tiny_mixed_batches(V, dtype, pad):
    rng = np.random.default_rng(V * 7 + pad)
    w = wl.tiny(rng, 48, V, dtype)
    _check(w, pad=pad)


def test_all_equal_and_signed_zero_rows():
    rng = np.random.default_rng(11)
    w = wl.tiny(rng, 16, 300, "f32")
    w.logits[0:4] = 0.0
    w.logits[2, ::2] = -0.0
    w.logits[4:8] = 1.5
    w.logits[8, 100:] = w.logits[8].max()
    w.temperature[:8] = np.float32(0.9)
    w.top_k[:8] = np.array([-1, 5, 150, 1, -1, 20, 299, 0], dtype=np.int32)
    w.top_p[:8] = np.array([0.5, 1.0, 0.3, 0.9, 0.95, 0.5, 0.999, 1.0], dtype=np.float32)
    _check(w)


def test_extreme_temperatures_and_parameters():
    rng = np.random.default_rng(12)
    w = wl.tiny(rng, 32, 2000, "f32", scale=6.0)
    w.temperature[:] = np.array([1.1e-6, 2e-6, 1e-5, 1e-3, 0.05, 20.0, 1e4, float("nan")] * 4,
                                dtype=np.float32)
    w.top_p[::3] = np.float32(float("nan"))
    w.top_k[::5] = np.int32(-(2 ** 31))
    _check(w)


def test_late_maximum_weight_reference():
    """Top-p rows whose maximum lies beyond the first tiles: with a small gap
    the weights stay relative to the first tiles' maximum, with a large gap
    (relative to the temperature) they switch to the row maximum; both must
    match the oracle, and so must top-k rows with the same rows."""
    rng = np.random.default_rng(17)
    B, V = 24, 40000
    w = wl.tiny(rng, B, V, "f32")
    for b in range(B):
        top = float(w.logits[b].max())
        j = int(rng.integers(20000, V))
        w.logits[b, j] = np.float32(top + (8.0 if b % 3 == 0 else 1.5 if b % 3 == 1 else 0.0))
    w.temperature[:] = np.array([0.05, 0.5, 1.0] * 8, dtype=np.float32)
    w.top_k[:] = -1
    w.top_k[18:] = np.array([20, 50, 64, 65, 500, 3], dtype=np.int32)
    w.top_p[:] = np.array([0.9, 0.5, 0.99, 0.8, 0.95, 0.3] * 4, dtype=np.float32)
    _check(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_clustered_candidates(dtype):
    """Rows whose large values sit in one contiguous block past the first
    tiles: every value of the block clears the threshold the first tiles
    give, so the wave that reads those tiles collects far more candidates
    than it can hold (staged loads for top-p and small top-k, per-element
    entries for top-k above 128), and the row must still match the oracle
    (it finishes from the row itself).  Rows with a smaller block stay within
    the candidate regions."""
    rng = np.random.default_rng(29)
    B, V = 16, 151936
    w = wl.tiny(rng, B, V, dtype)
    x = w.logits.astype(np.float32) if dtype == "f32" else wl.bf16_bits_to_f32(w.logits)
    for b in range(B):
        n = (3000, 400, 100)[b % 3]
        j0 = int(rng.integers(40000, V - n))
        x[b, j0:j0 + n] = 7.0 + rng.standard_normal(n).astype(np.float32) * 0.5
    w.logits = x if dtype == "f32" else wl.to_bf16_bits(x)
    w.temperature[:] = np.float32(0.8)
    w.top_k[:] = np.array([-1, 20, 64, 200, 1000, -1, 50, -1] * 2, dtype=np.int32)
    w.top_p[:] = np.array([0.9, 1.0, 0.95, 1.0, 0.9, 0.5, 0.8, 0.99] * 2, dtype=np.float32)
    _check(w, probs_rows={0, 1, 5})


@pytest.mark.parametrize("f_first", [0.5, 1.6])
def test_unrepresentative_first_tiles(f_first):
    """c2-like rows (bf16, N(0, 3), half greedy, T = 0.7 with top-p 0.9) whose
    first 16,384 logits have another spread than the rest.  The threshold
    comes from the first tiles, so it lands too low (narrower start: far more
    candidates than the regions hold) or too high (wider start: nuclei reach
    below it); either way the rows must still match the oracle."""
    rng = np.random.default_rng(1002 + int(f_first * 10))
    B, V = 32, 128256
    x = rng.standard_normal((B, V), dtype=np.float32) * np.float32(3.0)
    x[:, :16384] *= np.float32(f_first)
    w = wl.tiny(rng, B, V, "bf16")
    w.logits = wl.to_bf16_bits(x)
    greedy = np.arange(B) % 2 == 0
    w.temperature = np.where(greedy, 0.0, 0.7).astype(np.float32)
    w.top_k = None
    w.top_p = np.where(greedy, 1.0, 0.9).astype(np.float32)
    _check(w, probs_rows={1, 3, 31})


def test_greedy_batch_without_temperature_bf16():
    rng = np.random.default_rng(13)
    w = wl.tiny(rng, 100, 7000, "bf16")
    w.temperature = None
    _check(w)


@pytest.mark.parametrize("B,V,dtype", [(256, 5000, "bf16"), (300, 20000, "f32"), (255, 3001, "f32")])
def test_all_greedy_batches_both_kernels(B, V, dtype):
    """No temperature array: batches below 256 rows split rows across
    workgroups, larger ones take one workgroup per row; both must give the
    lowest-index maximum, including injected ties."""
    rng = np.random.default_rng(B * 31 + V)
    w = wl.tiny(rng, B, V, dtype)
    w.temperature = None
    for b in range(0, B, 7):            # exact ties with the row maximum
        i = int(np.argmax(w.logits[b]))
        j = int(rng.integers(0, V))
        w.logits[b, j] = w.logits[b, i]
    gpu, _ = _check(w)
    want = np.argmax(oracle_widen(w), axis=1)
    assert np.array_equal(gpu["tokens"], want)


def oracle_widen(w):
    import oracle
    return oracle.widen_logits(w.logits, w.dtype)


@pytest.mark.parametrize("V,dtype", [(1000, "f32"), (5000, "bf16"), (33000, "f32")])
def test_tiny_mixed_batches_exact_path(V, dtype):
    w = wl.tiny(np.random.default_rng(V * 11), 48, V, dtype)
    _check(w, force_exact=True)


def test_c3_exact_path():
    _check(wl.c3(), probs_rows=set(range(0, 256, 29)), force_exact=True)


def test_c3_without_debug_outputs():
    """The production launch (no debug buffers) gives the same tokens."""
    w = wl.c3()
    log("case c3 without debug outputs")
    a = run_gpu(w, debug=False)
    b = run_gpu(w, debug=True)
    assert np.array_equal(a["tokens"], b["tokens"])
    assert np.array_equal(a["pool"], b["pool"])


def test_flat_rows_fall_back_to_exact():
    """Very flat rows with top-p only: the nucleus is far larger than the
    candidate buffer, so the single-pass kernel must hand them to the exact
    path and still match the oracle."""
    rng = np.random.default_rng(16)
    w = wl.tiny(rng, 8, 40000, "bf16", scale=0.5)
    w.temperature[:] = np.float32(2.0)
    w.top_k[:] = -1
    w.top_p[:] = np.array([0.9, 0.5, 0.99, 0.999, 0.7, 0.95, 0.3, 0.8], dtype=np.float32)
    _check(w)


def test_c3_flat_top_p_rows():
    """c3 logits with a high temperature and top-p only: the nucleus of many
    rows reaches below the candidate threshold, so they take the two-pass
    flat-row path (depth histogram, then the boundary bin in LDS)."""
    w = wl.c3()
    w.temperature[:] = np.float32(1.5)
    w.top_k[:] = -1
    w.top_p[:] = np.where(np.arange(w.B) % 2 == 0, 0.95, 0.99).astype(np.float32)
    _check(w, probs_rows=set(range(0, 256, 17)))


def test_large_top_k_rows():
    """Top-k above the list size at full vocabulary: the threshold aims at a
    bounded candidate count (k = 3000 keeps thousands), the pass-driven
    descent finishes the rows; with and without top-p."""
    w = wl.c3()
    sel = np.arange(32)
    w = wl.Workload("c3_large_k", w.dtype, w.logits[sel].copy(), w.temperature[sel].copy(),
                    np.array([100, 500, 1000, 3000] * 8, dtype=np.int32),
                    np.array([1.0] * 16 + [0.9] * 16, dtype=np.float32),
                    w.uid[sel].copy(), w.step, w.pool[sel].copy(), np.arange(32, dtype=np.int64),
                    w.cols[sel].copy())
    _check(w, probs_rows={0, 5, 30})


def test_c2_full():
    _check(wl.c2(), probs_rows=set(range(0, 256, 17)))


def test_c3_full():
    _check(wl.c3(), probs_rows=set(range(0, 256, 13)))


@pytest.mark.parametrize("step,half_greedy", [(0, False), (1, False), (63, False), (0, True), (31, True),
                                               (63, True)])
def test_c4_decode_steps(step, half_greedy):
    _check(wl.c4(step, half_greedy), probs_rows=set(range(0, 512, 61)))


def test_repeat_and_recreate_are_identical():
    w = wl.tiny(np.random.default_rng(14), 64, 5000, "f32")
    log("case repeat/recreate")
    a = run_gpu(w, debug=False)
    b = run_gpu(w, debug=False)
    s = dst.Sampler(0, 64, 5000, "f32", w.seed)
    c = run_gpu(w, sampler=s, debug=False)
    d = run_gpu(w, sampler=s, debug=False)
    s.close()
    for o in (b, c, d):
        assert np.array_equal(a["tokens"], o["tokens"])


def test_draw_distribution_chi_square():
    """Many independent draws (distinct uids) from one row match r."""
    rng = np.random.default_rng(15)
    V, B = 1024, 4096
    x = rng.normal(0, 2, V).astype(np.float32)
    w = wl.Workload("chi2", "f32", np.tile(x, (B, 1)), np.full(B, 0.7, np.float32),
                    np.full(B, 50, np.int32), np.full(B, 0.9, np.float32),
                    np.arange(B, dtype=np.int64) * 7919, 3, np.zeros((B, 2), np.int32),
                    np.arange(B, dtype=np.int64), np.zeros(B, np.int64))
    log("case chi-square")
    gpu = run_gpu(w, debug=False)
    r = run_oracle(w, rows=[0])[0].r
    support = np.flatnonzero(r > 0)
    counts = np.bincount(gpu["tokens"], minlength=V)
    assert counts[r == 0].sum() == 0
    expected = r[support] * B
    big = expected >= 5
    obs = np.append(counts[support][big], counts[support][~big].sum())
    exp = np.append(expected[big], expected[~big].sum())
    keep = exp > 0
    stat, pval = scipy.stats.chisquare(obs[keep], exp[keep] * obs[keep].sum() / exp[keep].sum())
    log(f"  chi2={stat:.1f} p={pval:.3g} support={len(support)}")
    assert pval > 1e-4


def test_write_tokens_errors_and_tickets():
    log("case write_tokens errors")
    s = dst.Sampler(0, 8, 100, "f32")
    pool = torch.zeros((4, 10), dtype=torch.int32, device="cuda")
    toks = torch.arange(3, dtype=torch.int32, device="cuda") + 5
    rows = torch.tensor([0, 1, 2], dtype=torch.int64, device="cuda")
    cols = torch.tensor([-1, 3, 9], dtype=torch.int64, device="cuda")
    host = torch.zeros(3, dtype=torch.int32).pin_memory()
    t = s.write(pool, rows, cols, toks, host)
    s.wait(t)
    assert pool[0, 9].item() == 5 and pool[1, 3].item() == 6 and pool[2, 9].item() == 7
    assert host.tolist() == [5, 6, 7]
    assert s.query(t)
    # out of range: skipped, reported by wait and check
    bad_cols = torch.tensor([10, -2, 0], dtype=torch.int64, device="cuda")
    before = pool.clone()
    t2 = s.write(pool, rows, bad_cols, toks)
    with pytest.raises(dst.SamplerError) as e:
        s.wait(t2)
    assert e.value.code == -5
    with pytest.raises(dst.SamplerError):
        s.check()
    s.check()  # cleared
    assert torch.equal(pool[:, 1:], before[:, 1:]) and pool[2, 0].item() == 7
    # pageable host memory is refused before anything is enqueued
    with pytest.raises(dst.SamplerError) as e:
        s.write(pool, rows, cols, toks, torch.zeros(3, dtype=torch.int32))
    assert e.value.code == -4
    with pytest.raises(dst.SamplerError) as e:
        s.wait(10 ** 6)
    assert e.value.code == -6
    # debug check: two requests on one pool row (cols -1 do not count)
    s.set_checks(dst.SAMPLER_CHECK_DUPLICATE_ROWS)
    t3 = s.write(pool, torch.tensor([0, 1, 1], dtype=torch.int64, device="cuda"),
                 torch.tensor([2, -1, 4], dtype=torch.int64, device="cuda"), toks)
    s.wait(t3)
    t4 = s.write(pool, torch.tensor([3, 1, 3], dtype=torch.int64, device="cuda"),
                 torch.tensor([2, 5, 4], dtype=torch.int64, device="cuda"), toks)
    with pytest.raises(dst.SamplerError, match="same pool row") as e:
        s.wait(t4)
    assert e.value.code == -5
    with pytest.raises(dst.SamplerError):
        s.check()
    s.check()  # cleared
    s.set_checks(0)
    t5 = s.write(pool, torch.tensor([3, 1, 3], dtype=torch.int64, device="cuda"),
                 torch.tensor([2, 5, 4], dtype=torch.int64, device="cuda"), toks)
    s.wait(t5)                                        # unchecked: no flag
    with pytest.raises(dst.SamplerError):
        s.set_checks(8)
    s.close()


def test_argument_errors():
    log("case argument errors")
    s = dst.Sampler(0, 4, 100, "f32")
    x = torch.zeros((5, 100), device="cuda")
    with pytest.raises(ValueError, match="max_batch"):
        s.sample(x)                                   # B > max_batch: the binding refuses it
    # ... and so does the library itself, called through the C ABI directly
    import ctypes
    code = dst.load().sample_batch(s.handle, None, ctypes.c_void_p(x.data_ptr()), 100, 5,
                                   None, None, None, None, None, 0,
                                   ctypes.c_void_p(torch.empty(5, dtype=torch.int32, device="cuda").data_ptr()),
                                   None)
    assert code == -1
    y = torch.zeros((2, 100), device="cuda")
    with pytest.raises(dst.SamplerError):
        s.sample(y, temperature=torch.ones(2, device="cuda"))   # uid missing
    with pytest.raises(ValueError, match="row_stride"):
        s.sample(y, row_stride=50)
    code = dst.load().sample_batch(s.handle, None, ctypes.c_void_p(y.data_ptr()), 50, 2,
                                   None, None, None, None, None, 0,
                                   ctypes.c_void_p(torch.empty(2, dtype=torch.int32, device="cuda").data_ptr()),
                                   None)
    assert code == -1
    out = s.sample(y[:0])                             # B == 0 is a no-op
    assert out.numel() == 0
    s.close()
