"""Input gather and the overlapped decode loop, through the C ABI.

The scheduler's step ("The scheduler skeleton and the offline interface",
sections "Preparing a batch" and "_forward") gathers the input ids from the
token pool at (row, position), runs the model, samples, and writes the
tokens back at (row, device_len); its overlap loop waits for step N-1's host
copy only after step N is enqueued; the sampling parameters are prepared from
host arrays every step ("The engine and the sampler", section "The
sampler").  The gather is compared bit for bit with
the oracle's ``token_pool[rows, positions]``; the loops compare every step's
gathered ids, tokens, host copies and the final pool.
"""
import ctypes

import numpy as np
import pytest
import torch

import decode_step_token_amd as dst
import oracle
import workloads as wl
from tests.parity import compare, log, run_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    dst.load()
    yield
    torch.cuda.synchronize()


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t if dtype is None else t.to(dtype)


@pytest.mark.parametrize("n", [1, 63, 255, 256, 257, 256 * 7 + 37, 100_000])
def test_gather_random_entries(n):
    log(f"case gather random n={n}")
    pool, _, _, _ = wl.mixed_input_batch(20 + n)
    rng = np.random.default_rng(n)
    rows = rng.integers(0, pool.shape[0], n).astype(np.int64)
    pos = rng.integers(0, pool.shape[1], n).astype(np.int64)
    want, bad = oracle.gather_tokens(pool, rows, pos)
    assert not bad
    with dst.Sampler(0, 1, 8) as s:
        out = torch.full((n,), -7, dtype=torch.int32, device="cuda")
        s.gather(_dev(pool), _dev(rows), _dev(pos), ids_out=out)
        s.check()
        assert np.array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_gather_mixed_prefill_and_decode(seed):
    pool, table_idx, cached, device_len = wl.mixed_input_batch(seed)
    lens = device_len - cached
    rows = np.repeat(table_idx, lens)
    pos = np.concatenate([np.arange(c, d) for c, d in zip(cached, device_len)]).astype(np.int64)
    o_rows, o_pos = oracle.input_tuple(table_idx, cached, device_len)
    assert np.array_equal(rows, o_rows) and np.array_equal(pos, o_pos)
    log(f"case gather mixed batch seed={seed} n={len(rows)} longest span={lens.max()}")
    want, bad = oracle.gather_tokens(pool, o_rows, o_pos)
    assert not bad
    with dst.Sampler(0, 1, 8) as s:
        got = s.gather(_dev(pool), _dev(rows), _dev(pos))
        s.check()
        assert np.array_equal(got.cpu().numpy(), want)


def test_gather_out_of_range_and_empty():
    log("case gather errors")
    pool = np.arange(40, dtype=np.int32).reshape(4, 10) + 100
    rows = np.array([0, 4, 1, -1, 3, 2, 0], dtype=np.int64)
    pos = np.array([9, 0, -1, 0, 10, 5, 1 << 40], dtype=np.int64)
    want, bad = oracle.gather_tokens(pool, rows, pos)
    assert bad
    s = dst.Sampler(0, 1, 8)
    try:
        got = s.gather(_dev(pool), _dev(rows), _dev(pos))
        with pytest.raises(dst.SamplerError) as e:
            s.check()
        assert e.value.code == -5
        s.check()                                   # cleared
        assert np.array_equal(got.cpu().numpy(), want)
        # n == 0 enqueues nothing and succeeds
        empty = torch.zeros(0, dtype=torch.int64, device="cuda")
        assert s.gather(_dev(pool), empty, empty).numel() == 0
        # host-visible argument errors are synchronous
        lib = dst.load()
        code = lib.gather_tokens(s.handle, None, ctypes.c_void_p(0), 4, 10, None, None, -1, None)
        assert code == -1
        code = lib.gather_tokens(s.handle, None, ctypes.c_void_p(0), 4, 10, None, None, 3, None)
        assert code == -1
        d = _dev(pool)
        code = lib.gather_tokens(s.handle, None, ctypes.c_void_p(d.data_ptr()), 0, 10, None,
                                 None, 0, None)
        assert code == -1
        with pytest.raises(ValueError):
            s.gather(d, _dev(rows), _dev(pos[:3]))
        s.check()
    finally:
        s.close()


def test_gather_sees_write_on_same_stream():
    log("case write then gather, one stream, no host sync")
    R, C, B = 32, 100, 32
    rng = np.random.default_rng(5)
    pool0 = rng.integers(0, 1000, (R, C)).astype(np.int32)
    rows = rng.permutation(R).astype(np.int64)
    cols = rng.integers(0, C, B).astype(np.int64)
    cols[::7] = -1
    toks = rng.integers(5000, 6000, B).astype(np.int32)
    new, _, _ = oracle.write_tokens(pool0, rows, cols, toks)
    want, _ = oracle.gather_tokens(new, rows, np.where(cols == -1, C - 1, cols))
    with dst.Sampler(0, B, 8) as s:
        pool = _dev(pool0)
        s.write(pool, _dev(rows), _dev(cols), _dev(toks))
        got = s.gather(pool, _dev(rows), _dev(np.where(cols == -1, C - 1, cols)))
        s.check()
        assert np.array_equal(got.cpu().numpy(), want)
        assert np.array_equal(got.cpu().numpy(), toks)


def _overlap_loop(s, w0, logits_dev, steps, debug):
    """Enqueue prepare -> gather -> sample -> write for every step; wait for
    step N-1's ticket only after step N is enqueued, reading its pinned ring
    slot."""
    B = w0.B
    pool = _dev(w0.pool.copy())
    rows = _dev(w0.rows)
    pos0 = w0.meta["pos0"]
    in_pos = [_dev(pos0 + st - 1) for st in range(steps)]
    out_pos = [_dev(pos0 + st) for st in range(steps)]
    # the parameters are prepared every step from host arrays, as the
    # scheduler does; two device blocks alternate
    blocks = [torch.empty(dst._binding.PREP_BYTES_PER_REQUEST * B, dtype=torch.uint8,
                          device="cuda") for _ in range(2)]
    ring = [torch.full((B,), -7, dtype=torch.int32).pin_memory() for _ in range(2)]
    ids = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(steps)]
    toks = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(steps)]
    dbg = [({"kept_out": torch.full((B,), -7, dtype=torch.int32, device="cuda"),
             "rand_out": torch.full((B,), -7, dtype=torch.int64, device="cuda")}
            if debug else None) for _ in range(steps)]
    host = []
    prev = None
    for st in range(steps):
        args = s.prepare(B, w0.temperature, w0.top_k, w0.top_p, w0.uid,
                         dev_block=blocks[st % 2])
        s.gather(pool, rows, in_pos[st], ids_out=ids[st])
        s.sample(logits_dev[st], step=st, tokens_out=toks[st], debug=dbg[st], **args)
        t = s.write(pool, rows, out_pos[st], toks[st], ring[st % 2])
        if prev is not None:
            s.wait(prev)
            host.append(ring[(st - 1) % 2].numpy().copy())
        prev = t
    s.wait(prev)
    host.append(ring[(steps - 1) % 2].numpy().copy())
    s.check()
    out = {"pool": pool.cpu().numpy(), "ids": [x.cpu().numpy() for x in ids],
           "tokens": [x.cpu().numpy() for x in toks], "host": host}
    if debug:
        out["debug"] = [{n: t.cpu().numpy() for n, t in d.items()} for d in dbg]
    return out


def _check_chain(w0, res, steps):
    """Bit-exact chain: each step's input ids are the previous step's tokens
    (step 0: the pool's initial contents), each host copy equals the device
    tokens, and the final pool is the oracle's sequence of writes."""
    pool = w0.pool.copy()
    pos0 = w0.meta["pos0"]
    for st in range(steps):
        want_ids, bad = oracle.gather_tokens(pool, w0.rows, pos0 + st - 1)
        assert not bad
        assert np.array_equal(res["ids"][st], want_ids), f"step {st}: gathered ids"
        if st:
            assert np.array_equal(res["ids"][st], res["tokens"][st - 1]), f"step {st}: chain"
        assert np.array_equal(res["host"][st], res["tokens"][st]), f"step {st}: host copy"
        pool, _, bad = oracle.write_tokens(pool, w0.rows, pos0 + st, res["tokens"][st])
        assert not bad
    assert np.array_equal(res["pool"], pool), "final pool"


def test_small_decode_loop_every_row():
    steps = 12
    w0 = wl.loop_small(0)
    log(f"case overlap decode loop B={w0.B} V={w0.V} bf16 steps={steps}")
    logits = [torch.from_numpy(wl.loop_small_logits(st).view(np.int16)).cuda()
              .view(torch.bfloat16) for st in range(steps)]
    with dst.Sampler(0, w0.B, w0.V, "bf16", w0.seed) as s:
        res = _overlap_loop(s, w0, logits, steps, debug=True)
    _check_chain(w0, res, steps)
    amb = 0
    for st in range(steps):
        w = wl.loop_small(st)
        gpu = {"tokens": res["tokens"][st], **res["debug"][st]}
        stats = compare(w, gpu, run_oracle(w))
        amb += stats["draw_ambiguous"] + stats["cutoff_ambiguous"]
    log(f"  ok, ambiguous rows over all steps: {amb}")


def test_c4_overlap_loop_full_size():
    steps = 8
    w0 = wl.c4(0)
    log(f"case overlap decode loop c4 B={w0.B} V={w0.V} bf16 steps={steps}")
    logits = []
    for st in range(steps):
        logits.append(torch.from_numpy(wl.c4_logits(st).view(np.int16)).cuda()
                      .view(torch.bfloat16))
        log(f"  logits of step {st} resident")
    with dst.Sampler(0, w0.B, w0.V, "bf16", w0.seed) as s:
        res = _overlap_loop(s, w0, logits, steps, debug=False)
    _check_chain(w0, res, steps)
    sel = list(range(3, w0.B, 64))
    for st in (0, steps - 1):
        w = wl.c4(st)
        compare(w, {"tokens": res["tokens"][st]}, run_oracle(w, rows=sel), rows=sel)
        log(f"  step {st}: oracle rows {sel} ok")
