"""sampler_prepare (the engine's Sampler.prepare inside the library), through
the C ABI: the device tensors it fills equal the oracle's ``prepare`` bit for
bit, None where the pages pass None, and sampling from them equals sampling
from the raw parameters."""
import ctypes

import numpy as np
import pytest
import torch

import decode_step_token_amd as dst
import oracle
import workloads as wl
from tests.parity import compare, log, run_gpu, run_oracle, to_device_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    dst.load()
    yield
    torch.cuda.synchronize()


def _params(rng, B, V):
    T = rng.choice(np.array([0.0, -1.0, np.nan, 1e-9, 1e-6, 0.3, 0.7, 1.5], np.float32), B)
    k = rng.choice(np.array([-3, 0, 1, 2, 50, V - 1, V, V + 4], np.int32), B)
    p = rng.choice(np.array([1e-12, 1e-6, 0.5, 0.9, 1.0, 2.0], np.float32), B)
    mp = rng.choice(np.array([0.0, 0.0, -0.5, 0.05, 0.3, 1.0, 3.0], np.float32), B)
    uid = rng.integers(-(1 << 40), 1 << 40, B).astype(np.int64)
    return T, k, p, mp, uid


def _same(got, want, name):
    if want is None:
        assert got is None, f"{name}: expected None"
        return
    assert got is not None, f"{name}: expected a tensor"
    g = got.cpu().numpy()
    assert g.dtype == want.dtype and g.shape == want.shape, name
    if g.dtype.kind == "f":
        assert np.array_equal(np.isnan(g), np.isnan(want)), name
        m = ~np.isnan(want)
        assert np.array_equal(g[m].view(np.uint32), want[m].view(np.uint32)), name
    else:
        assert np.array_equal(g, want), name


@pytest.mark.parametrize("B,V,seed", [(1, 10, 0), (300, 1000, 1), (4096, 151936, 2)])
def test_prepare_matches_oracle(B, V, seed):
    log(f"case prepare B={B} V={V}")
    rng = np.random.default_rng(seed)
    T, k, p, mp, uid = _params(rng, B, V)
    T[0] = 0.5                                 # at least one sampled request
    with dst.Sampler(0, B, V) as s:
        got = s.prepare(B, T, k, p, uid, min_p=mp)
        nomp = s.prepare(B, T, k, p, uid)
        torch.cuda.synchronize()
        ts, ks, ps, ms = oracle.prepare(V, T, k, p, mp)
        _same(got["temperature"], ts, "temperature")
        _same(got["top_k"], ks, "top_k")
        _same(got["top_p"], ps, "top_p")
        _same(got["min_p"], ms, "min_p")
        assert np.array_equal(got["uid"].cpu().numpy(), uid)
        assert nomp["min_p"] is None


def test_prepare_none_rules_and_errors():
    log("case prepare None rules and errors")
    V = 64
    with dst.Sampler(0, 8, V) as s:
        g = s.prepare(3, np.array([0.0, -1.0, 0.0], np.float32), None, None, None)
        assert all(g[n] is None for n in ("temperature", "top_k", "top_p", "uid"))
        g = s.prepare(2, None, np.array([3, 4], np.int32), None, None)
        assert g["temperature"] is None
        T = np.array([0.0, 0.9], np.float32)
        uid = np.array([7, 8], np.int64)
        g = s.prepare(2, T, np.array([-1, V], np.int32), np.array([1.0, 1.5], np.float32), uid)
        assert g["temperature"] is not None and g["top_k"] is None and g["top_p"] is None
        g = s.prepare(0, None, None, None, None)
        assert g["temperature"] is None
        lib = dst.load()
        out = dst.SamplerArgs()
        blk = torch.zeros(64, dtype=torch.uint8, device="cuda")
        Th = torch.from_numpy(T)
        uh = torch.from_numpy(uid)
        vp = lambda t: ctypes.c_void_p(t.data_ptr())
        # B above max_batch, uid missing, block too small, misaligned block
        assert lib.sampler_prepare(s.handle, None, 9, None, None, None, None, None, vp(blk), 64,
                                   ctypes.byref(out)) == -1
        assert lib.sampler_prepare(s.handle, None, 2, vp(Th), None, None, None, None, vp(blk),
                                   64, ctypes.byref(out)) == -1
        assert lib.sampler_prepare(s.handle, None, 2, vp(Th), None, None, None, vp(uh), vp(blk),
                                   47, ctypes.byref(out)) == -1
        assert lib.sampler_prepare(s.handle, None, 2, vp(Th), None, None, None, vp(uh),
                                   ctypes.c_void_p(blk.data_ptr() + 4), 60,
                                   ctypes.byref(out)) == -1
        assert lib.sampler_prepare(s.handle, None, 2, vp(Th), None, None, None, vp(uh), vp(blk),
                                   48, None) == -1
        s.check()


def test_prepared_sampling_equals_raw_and_oracle():
    rng = np.random.default_rng(7)
    w = wl.tiny(rng, 96, 5000, "bf16", greedy_frac=0.3)
    log(f"case prepare then sample {w.name}")
    with dst.Sampler(0, w.B, w.V, w.dtype, w.seed) as s:
        logits = to_device_logits(w)
        g = s.prepare(w.B, w.temperature, w.top_k, w.top_p, w.uid)
        toks = s.sample(logits, step=w.step, **g)
        raw = run_gpu(w, sampler=s, debug=False)
        assert np.array_equal(toks.cpu().numpy(), raw["tokens"])
    gpu = dict(raw)
    compare(w, gpu, run_oracle(w))


def test_prepare_staging_rotation_under_load():
    """Three times as many prepares as staging buffers, enqueued behind a
    busy stream with no host synchronisation: every block holds its own
    parameters, and every sample used them."""
    B, V = 256, 2048
    n = 3 * dst._binding.PREP_SLOTS
    log(f"case prepare staging rotation, {n} calls")
    rng = np.random.default_rng(11)
    sets = [_params(rng, B, V) for _ in range(n)]
    for T, *_ in sets:
        T[0] = 0.8
    logits = torch.from_numpy(rng.standard_normal((B, V)).astype(np.float32)).cuda()
    with dst.Sampler(0, B, V) as s:
        blocks = [torch.empty(dst._binding.PREP_BYTES_PER_REQUEST * B, dtype=torch.uint8,
                              device="cuda") for _ in range(n)]
        toks = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(n)]
        got = []
        torch.cuda._sleep(int(2e6))            # keep the stream busy while calls pile up
        for i, (T, k, p, mp, uid) in enumerate(sets):
            g = s.prepare(B, T, k, p, uid, dev_block=blocks[i], min_p=mp)
            s.sample(logits, step=i, tokens_out=toks[i], **g)
            got.append(g)
        torch.cuda.synchronize()
        for i, (T, k, p, mp, uid) in enumerate(sets):
            ts, ks, ps, ms = oracle.prepare(V, T, k, p, mp)
            _same(got[i]["temperature"], ts, f"call {i} temperature")
            _same(got[i]["top_k"], ks, f"call {i} top_k")
            _same(got[i]["top_p"], ps, f"call {i} top_p")
            _same(got[i]["min_p"], ms, f"call {i} min_p")
            ref = s.sample(logits, step=i, temperature=torch.from_numpy(ts).cuda(),
                           top_k=None if ks is None else torch.from_numpy(ks).cuda(),
                           top_p=None if ps is None else torch.from_numpy(ps).cuda(),
                           min_p=None if ms is None else torch.from_numpy(ms).cuda(),
                           uid=torch.from_numpy(uid).cuda())
            assert torch.equal(ref, toks[i]), f"call {i}: tokens"
        s.check()
