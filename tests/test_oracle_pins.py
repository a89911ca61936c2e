"""Pins of the fp64 oracle against things other than itself.

Each test checks the oracle against a value the pages print, a closed form,
a library routine with a documented tie rule, exact dyadic arithmetic, or a
brute-force sweep.  None of these re-types the oracle's own formula.
"""
import heapq
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
import oracle.sampler_ref as sr
from oracle import (filter_sorted, inverse_cdf, philox4x64, request_uniform, request_word,
                    row_params, sample_batch, sample_row, widen_logits, write_tokens)
from oracle import (PagePool, gather_tokens, input_tuple, min_p_count, page_to_token, paged_info,
                    prepare, write_page_table)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
M64 = (1 << 64) - 1


# ---------------------------------------------------------------- Philox --

def _numpy_block(counter, key):
    """First block of numpy.random.Philox (Philox-4x64-10) for `counter`.

    NumPy increments its 256-bit counter before producing a block, so the
    generator is started one below the counter we want."""
    c = sum(int(w) << (64 * i) for i, w in enumerate(counter))
    c = (c - 1) % (1 << 256)
    words = np.array([(c >> (64 * i)) & M64 for i in range(4)], dtype=np.uint64)
    bg = np.random.Philox(counter=words, key=np.array(key, dtype=np.uint64))
    return tuple(int(v) for v in bg.random_raw(4))


@pytest.mark.parametrize("counter,key", [
    ((0, 0, 0, 0), (0, 0)),
    ((1, 0, 0, 0), (42, 0)),
    ((0, 1, 0, 0), (42, 0)),          # borrow across words when starting NumPy one below
    ((7, 1999, 0, 0), (42, 0)),
    ((M64, M64, M64, M64), (M64, M64)),
    ((0x243F6A8885A308D3, 0x13198A2E03707344, 0xA4093822299F31D0, 0x082EFA98EC4E6C89),
     (0x452821E638D01377, 0xBE5466CF34E90C6C)),
])
def test_philox_matches_numpy(counter, key):
    assert philox4x64(counter, key) == _numpy_block(counter, key)


def test_request_word_keys_and_twos_complement():
    # uid -1 is the all-ones counter word (the engine's dummy request has uid -1)
    assert request_word(42, -1, 3) == _numpy_block((M64, 3, 0, 0), (42, 0))[0]
    assert request_word(42, 5, 9) == _numpy_block((5, 9, 0, 0), (42, 0))[0]
    assert request_word(7, 5, 9) != request_word(42, 5, 9)


def test_uniform_is_24bit_dyadic_and_uniform():
    us = np.array([request_uniform(42, uid, 0) for uid in range(20000)])
    assert np.all(us >= 0.0) and np.all(us < 1.0)
    assert np.all(us * 2 ** 24 == np.floor(us * 2 ** 24))
    assert scipy.stats.kstest(us, "uniform").pvalue > 1e-3


# -------------------------------------------------- the pages' example --

def _golden():
    with open(os.path.join(GOLDEN, "pages_worked_example.json")) as f:
        return json.load(f)


def test_pages_example_supports_and_closed_form():
    g = _golden()
    x = np.array(g["logits"], dtype=np.float64)
    V = g["vocab_size"]
    for req in g["requests"]:
        prm = row_params(V, req["temperature"], req["top_k"], req["top_p"])
        res = sample_row(x, prm, 0.5)
        assert sorted(np.flatnonzero(res.r > 0).tolist()) == req["support"]
        for u in np.linspace(0, 1 - 2 ** -24, 257):
            assert sample_row(x, prm, float(u)).token in req["support"]
    # request 0: top-k 2 renormalises to e^5/(e^5+e^4) and e^4/(e^5+e^4)
    prm = row_params(V, 1.0, 2, 1.0)
    r = sample_row(x, prm, 0.0).r
    e = math.e
    np.testing.assert_allclose(r, [e / (1 + e), 1 / (1 + e), 0, 0, 0, 0], rtol=0, atol=1e-15)


def test_pages_example_all_greedy_batch():
    g = _golden()
    assert g["all_greedy_batch_has_no_temperature"]
    x = np.array([g["logits"]] * 2, dtype=np.float32)
    res = sample_batch(x, "f32", None, None, None, np.arange(2), 0, 42)
    assert [r.token for r in res] == [0, 0] and all(r.greedy for r in res)


def test_pages_example_draw_frequency():
    g = _golden()
    x = np.array(g["logits"], dtype=np.float64)
    prm = row_params(g["vocab_size"], 1.0, 2, 1.0)
    toks = [sample_row(x, prm, request_uniform(42, 0, s)).token for s in range(g["draws"])]
    f0 = toks.count(0) / len(toks)
    assert abs(f0 - g["freq_token0_request0"]) < g["freq_tolerance"]
    assert set(toks) == {0, 1}


# ------------------------------------------------------ argmax identities --

def _rows_with_ties(rng, n, V):
    X = rng.normal(0, 2, (n, V))
    for b in range(0, n, 2):          # every other row: the maximum appears twice
        X[b, int(rng.integers(0, V))] = X[b].max()
    return X.astype(np.float32).astype(np.float64)


def test_greedy_is_numpy_first_argmax():
    rng = np.random.default_rng(1)
    X = _rows_with_ties(rng, 40, 300)
    X[3, :] = 1.25  # all equal: index 0
    for x in X:
        for T in (None, 0.0, 1e-6, float(np.float32(1e-6)), -3.0, float("nan")):
            prm = row_params(len(x), T, 50, 0.9)
            assert prm.greedy
            assert sample_row(x, prm, 0.3).token == int(np.argmax(x))


def test_topk1_is_argmax_for_every_u():
    rng = np.random.default_rng(2)
    X = _rows_with_ties(rng, 20, 200)
    for x in X:
        prm = row_params(len(x), float(rng.uniform(0.2, 2)), 1, float(rng.uniform(0.1, 1)))
        for u in (0.0, 2 ** -24, 0.5, 1 - 2 ** -24):
            assert sample_row(x, prm, u).token == int(np.argmax(x))


def test_tiny_temperature_gives_argmax():
    """A temperature just above the greedy cut (1e-4) through the sampling
    path collapses to the argmax on rows whose maximum is unique."""
    rng = np.random.default_rng(3)
    for _ in range(20):
        x = rng.normal(0, 2, 500)
        top = np.argsort(-x)
        x[top[0]] = x[top[1]] + 0.05
        prm = row_params(500, 1e-4, -1, 1.0)
        assert not prm.greedy
        for u in (1e-12, 0.25, 0.5, 1 - 2 ** -24):
            assert sample_row(x, prm, u).token == int(top[0])


# ------------------------------------------------ softmax identities ----

def test_full_softmax_matches_scipy():
    rng = np.random.default_rng(4)
    for T in (0.3, 0.7, 1.0, 1.5, 3.0):
        x = rng.normal(0, 3, 2000)
        prm = row_params(2000, T, -1, 1.0)
        r = sample_row(x, prm, 0.5).r
        want = scipy.special.softmax(x / float(np.float32(T)))
        np.testing.assert_allclose(r, want, rtol=1e-12, atol=1e-15)


def test_two_token_closed_form():
    for a, b, T in ((1.0, 0.0, 0.5), (2.0, 3.5, 1.5), (-1.0, -1.25, 0.3)):
        prm = row_params(2, T, -1, 1.0)
        r = sample_row(np.array([a, b]), prm, 0.5).r
        t = float(np.float32(T))
        assert abs(r[0] - 1.0 / (1.0 + math.exp((b - a) / t))) < 1e-15


# ---------------------------------------------------------- top-k set ---

def test_topk_set_matches_heapq_with_index_ties():
    rng = np.random.default_rng(5)
    for trial in range(30):
        V = int(rng.integers(2, 400))
        x = np.round(rng.normal(0, 1.5, V), 1)          # many exact ties
        if trial % 5 == 0:
            x[: V // 2] = 0.0
            x[V // 2] = -0.0
        k = int(rng.integers(1, V + 1))
        prm = row_params(V, 0.9, k, 1.0)
        res = sample_row(x, prm, 0.5)
        want = heapq.nsmallest(min(k, V), range(V), key=lambda i: (-x[i] + 0.0, i))
        assert res.kept == min(k, V)
        assert res.order_prefix.tolist() == want[:min(k, 64)]
        assert sorted(np.flatnonzero(res.r > 0)) == sorted(want)


def test_bf16_rows_widen_exactly():
    bits = np.array([[0x3F80, 0xC000, 0x8000, 0x0000, 0x4049, 0x7F7F]], dtype=np.uint16)
    x = widen_logits(bits, "bf16")[0]
    assert x[0] == 1.0 and x[1] == -2.0 and x[2] == 0.0 and math.copysign(1, x[2]) == -1
    assert x[4] == 3.140625 and x[5] == float(np.float32(3.3895313892515355e38))


# --------------------------------------------------- top-p, exact cases --

@pytest.mark.parametrize("q,k,p,n", [
    # exclusive prefixes 0, 1/2, 3/4, 7/8; strict "<" drops rank 2 at p = 3/4
    ((0.5, 0.25, 0.125, 0.125), 4, 0.75, 2),
    ((0.5, 0.25, 0.125, 0.125), 4, 0.75 + 2 ** -20, 3),
    ((0.5, 0.25, 0.125, 0.125), 4, 0.5, 1),
    ((0.5, 0.25, 0.125, 0.125), 4, 2 ** -30, 1),        # rank 0's prefix is empty: it survives any p
    ((0.5, 0.25, 0.125, 0.125), 4, 1.0, 4),
    # top-k 2 renormalises (1/2, 1/4) to (2/3, 1/3): prefix 2/3 >= 0.6 drops rank 1
    ((0.5, 0.25, 0.125, 0.125), 2, 0.6, 1),
    ((0.5, 0.25, 0.125, 0.125), 2, 0.6875, 2),
    # the order example: (0.4, 0.3, 0.2, 0.1), k=3, p=0.42
    ((0.4, 0.3, 0.2, 0.1), 3, 0.42, 1),
])
def test_top_p_cutoffs_exact(q, k, p, n):
    assert filter_sorted(np.array(q), k, p) == n


def test_filter_order_matters():
    q = np.array([0.4, 0.3, 0.2, 0.1])
    assert filter_sorted(q, 3, 0.42, "k_then_p") == 1
    assert filter_sorted(q, 3, 0.42, "p_then_k") == 2


def test_filter_order_brute_force():
    """On every small grid case, top-k-then-top-p keeps a prefix no longer than
    the reverse order, both are prefixes of the descending order, the kept
    prefix is the shortest one whose renormalised mass reaches p, and some
    cases differ."""
    grid = [0.0, 0.5, 1.0, 2.0]
    differ = 0
    for V in (3, 4, 5):
        for xs in itertools.product(grid, repeat=V):
            x = np.array(xs)
            if len(set(xs)) == 1:
                continue
            pi = np.argsort(-x, kind="stable")
            for k in range(1, V + 1):
                for p in (0.05, 0.25, 0.45, 0.65, 0.85, 0.95):
                    prm = row_params(V, 1.0, k, p)
                    a = sample_row(x, prm, 0.5, want_alternatives=False)
                    b = sample_row(x, prm, 0.5, order="p_then_k", want_alternatives=False)
                    assert a.kept <= b.kept
                    assert set(np.flatnonzero(a.r > 0)) == set(pi[:a.kept].tolist())
                    w = np.exp(x - x.max())[pi][:k]
                    w = w / w.sum()
                    assert w[:a.kept - 1].sum() < p
                    assert a.kept == k or w[:a.kept].sum() >= p
                    differ += a.kept != b.kept
    assert differ > 0


# ------------------------------------------------------------- the draw --

def test_draw_matches_searchsorted():
    rng = np.random.default_rng(6)
    for _ in range(200):
        V = int(rng.integers(1, 300))
        x = rng.normal(0, 2, V)
        prm = row_params(V, float(rng.uniform(0.3, 2)), int(rng.integers(-1, V + 2)),
                         float(rng.uniform(0.05, 1.2)))
        u = float(rng.integers(0, 1 << 24)) * 2 ** -24
        res = sample_row(x, prm, u)
        c = np.cumsum(res.r)
        if c[-1] > u:
            assert res.token == int(np.searchsorted(c, u, side="right"))
        assert res.r[res.token] > 0


def test_draw_measure_brute_force():
    """Sweeping u over a 2^-16 grid, token i is drawn for a measure r_i."""
    x = np.array([1.0, -0.5, 2.0, 0.25, 2.0])
    prm = row_params(5, 0.8, 4, 0.97)
    base = sample_row(x, prm, 0.0)
    counts = np.zeros(5)
    n = 1 << 16
    for j in range(n):
        counts[inverse_cdf(base.r, j / n)] += 1
    np.testing.assert_allclose(counts / n, base.r, atol=1.0 / n)
    # dyadic masses put every CDF boundary on the grid: token i owns exactly the
    # half-open interval [C_{i-1}, C_i), i.e. r_i * n grid points
    r = np.array([0.5, 0.0, 0.25, 0.125, 0.125])
    counts = np.zeros(5)
    for j in range(n):
        counts[inverse_cdf(r, j / n)] += 1
    assert np.array_equal(counts, r * n)
    assert inverse_cdf(r, 0.5) == 2 and inverse_cdf(r, 0.0) == 0


def test_batch_permutation_and_resume():
    """Tokens follow (seed, uid, step), not the row position."""
    rng = np.random.default_rng(7)
    B, V = 12, 256
    X = rng.normal(0, 2, (B, V)).astype(np.float32)
    T = rng.uniform(0.3, 1.5, B).astype(np.float32)
    k = rng.choice([-1, 5, 50], B).astype(np.int32)
    p = rng.choice([1.0, 0.9], B).astype(np.float32)
    uid = rng.integers(0, 10 ** 9, B)
    a = [r.token for r in sample_batch(X, "f32", T, k, p, uid, 17, 42)]
    perm = rng.permutation(B)
    b = [r.token for r in sample_batch(X[perm], "f32", T[perm], k[perm], p[perm], uid[perm], 17, 42)]
    assert [a[i] for i in perm] == b
    c = [r.token for r in sample_batch(X, "f32", T, k, p, uid, 17, 42)]
    assert a == c


# ----------------------------------------------------------- prepare ----

def test_prepare_clamps():
    V = 100
    assert row_params(V, 0.0, 5, 0.5).greedy
    assert row_params(V, float(np.float32(1e-6)), 5, 0.5).greedy
    assert not row_params(V, 1.1e-6, 5, 0.5).greedy
    assert row_params(V, 0.7, 0, 1.0).k == V
    assert row_params(V, 0.7, -1, 1.0).k == V
    assert row_params(V, 0.7, V, 1.0).k == V
    assert row_params(V, 0.7, V + 3, 1.0).k == V
    assert row_params(V, 0.7, V - 1, 1.0).k == V - 1
    assert row_params(V, 0.7, 5, 0.0).p == float(np.float32(1e-6))
    assert row_params(V, 0.7, 5, 2.0).p == 1.0
    assert row_params(V, 0.7, 5, float("nan")).p == float(np.float32(1e-6))
    assert row_params(V, float("nan"), 5, 0.5).greedy


# ------------------------------------------------------- write-back -----

def test_write_tokens_matches_fancy_index():
    rng = np.random.default_rng(8)
    R, C, B = 16, 40, 10
    pool = rng.integers(0, 1000, (R, C)).astype(np.int32)
    rows = rng.permutation(R)[:B].astype(np.int64)
    cols = rng.integers(-1, C, B).astype(np.int64)
    cols[:2] = -1                      # "do not write": lands in the last column
    toks = rng.integers(0, 1 << 20, B).astype(np.int32)
    new, host, bad = write_tokens(pool, rows, cols, toks)
    want = pool.copy()
    want[rows, cols % C] = toks
    assert np.array_equal(new, want) and np.array_equal(host, toks) and not bad
    _, _, bad = write_tokens(pool, np.array([0, R]), np.array([0, 0]), np.array([1, 2]))
    assert bad
    _, _, bad = write_tokens(pool, np.array([0]), np.array([-2]), np.array([1]))
    assert bad


# ------------------------------------------------------- input gather ---

def test_gather_tokens_matches_fancy_index():
    rng = np.random.default_rng(9)
    R, C, n = 12, 50, 300
    pool = rng.integers(-5, 1 << 20, (R, C)).astype(np.int32)
    rows = rng.integers(0, R, n).astype(np.int64)      # repeats allowed (prefill spans)
    pos = rng.integers(0, C, n).astype(np.int64)
    ids, bad = gather_tokens(pool, rows, pos)
    assert ids.dtype == np.int32 and np.array_equal(ids, pool[rows, pos]) and not bad
    ids, bad = gather_tokens(pool, np.zeros(0, np.int64), np.zeros(0, np.int64))
    assert ids.shape == (0,) and not bad


def test_gather_tokens_out_of_range_is_reported_not_wrapped():
    pool = np.arange(12, dtype=np.int32).reshape(3, 4)
    for r, c in ((3, 0), (0, 4), (-1, 0), (0, -1), (1 << 40, 0)):
        ids, bad = gather_tokens(pool, np.array([1, r]), np.array([2, c]))
        assert bad and ids[0] == 6 and ids[1] == -1, (r, c)


def test_write_then_gather_round_trip():
    """The next step's input at (row, device_len) is the token just written
    there; a column of -1 was written to the last column."""
    rng = np.random.default_rng(10)
    R, C, B = 32, 64, 20
    pool = rng.integers(0, 1000, (R, C)).astype(np.int32)
    rows = rng.permutation(R)[:B].astype(np.int64)
    cols = rng.integers(0, C, B).astype(np.int64)
    cols[::5] = -1
    toks = rng.integers(1000, 2000, B).astype(np.int32)
    new, _, _ = write_tokens(pool, rows, cols, toks)
    ids, bad = gather_tokens(new, rows, np.where(cols == -1, C - 1, cols))
    assert np.array_equal(ids, toks) and not bad


def test_input_tuple_hand_worked_batch():
    """A prefill of 4 tokens, a decode at position 7 and a one-token chunk at
    position 2, packed request after request."""
    rows, pos = input_tuple([3, 0, 5], [0, 7, 2], [4, 8, 3])
    assert rows.tolist() == [3, 3, 3, 3, 0, 5] and pos.tolist() == [0, 1, 2, 3, 7, 2]
    rows, pos = input_tuple([1], [5], [5])                 # nothing to run
    assert rows.shape == (0,) and pos.shape == (0,)


def test_gather_equals_concatenated_request_slices():
    """Driving the engine by hand ("The engine and the sampler"), the batch's
    input is the concatenation of every request's ids[cached_len:device_len];
    with each request's ids stored in its pool row, gathering the input tuple
    gives the same array."""
    rng = np.random.default_rng(11)
    R, C = 8, 96
    pool = np.full((R, C), -9, dtype=np.int32)
    table_idx = rng.permutation(R)[:5]
    reqs = []
    for t in table_idx:
        L = int(rng.integers(1, C))
        ids = rng.integers(0, 50000, L).astype(np.int32)
        pool[t, :L] = ids
        lo = int(rng.integers(0, L))
        reqs.append((t, lo, L, ids))
    rows, pos = input_tuple([r[0] for r in reqs], [r[1] for r in reqs], [r[2] for r in reqs])
    got, bad = gather_tokens(pool, rows, pos)
    want = np.concatenate([ids[lo:hi] for _, lo, hi, ids in reqs])
    assert np.array_equal(got, want) and not bad


# ------------------------------------------------------------ prepare ---

def test_prepare_hand_worked_batch():
    """Greedy requests get the tiny temperature, top-k below 1 becomes V,
    top-p is clamped into [1e-6, 1] ("The engine and the sampler", section
    "The sampler")."""
    V = 100
    T = np.array([0.0, 0.7, -1.0, 1.3, 2e-7], dtype=np.float32)
    k = np.array([-1, 50, 0, 1, 103], dtype=np.int32)
    p = np.array([0.9, 1.0, 1.5, 1e-9, 0.25], dtype=np.float32)
    ts, ks, ps = prepare(V, T, k, p)
    assert ts.dtype == np.float32 and ks.dtype == np.int32 and ps.dtype == np.float32
    assert ts.tolist() == [np.float32(1e-6), np.float32(0.7), np.float32(1e-6), np.float32(1.3),
                           np.float32(1e-6)]
    assert ks.tolist() == [100, 50, 100, 1, 103]
    assert ps.tolist() == [np.float32(0.9), 1.0, 1.0, np.float32(1e-6), 0.25]


def test_prepare_none_rules():
    V = 64
    # every request greedy: no tensors at all (the plain argmax path)
    assert prepare(V, np.array([0.0, -2.0], np.float32), np.array([5, 7], np.int32),
                   np.array([0.5, 0.5], np.float32)) == (None, None, None)
    assert prepare(V, None, np.array([5], np.int32), None) == (None, None, None)
    T = np.array([0.0, 0.8], np.float32)
    # top-k set by nobody (every entry ends up V), top-p never below 1
    ts, ks, ps = prepare(V, T, np.array([-1, V], np.int32), np.array([1.0, 3.0], np.float32))
    assert ts is not None and ks is None and ps is None
    ts, ks, ps = prepare(V, T, None, None)
    assert ks is None and ps is None
    # one request is enough to build each tensor
    _, ks, ps = prepare(V, T, np.array([-1, V + 1], np.int32), np.array([1.0, 0.99999], np.float32))
    assert ks.tolist() == [V, V + 1] and ps is not None and ps[1] < 1.0


def test_prepare_keeps_every_rows_routing():
    """sample_batch clamps the prepared tensors again; for every request the
    effective (greedy, T, k, p) equals that of its raw parameters."""
    rng = np.random.default_rng(12)
    V, B = 500, 400
    T = rng.choice(np.array([0.0, -1.0, 1e-9, 5e-7, 1e-6, 2e-6, 0.3, 0.7, 1.5], np.float32), B)
    k = rng.choice(np.array([-7, -1, 0, 1, 2, 50, V - 1, V, V + 9], np.int32), B)
    p = rng.choice(np.array([1e-12, 1e-6, 0.2, 0.9, 1.0, 1.7], np.float32), B)
    ts, ks, ps = prepare(V, T, k, p)
    for b in range(B):
        raw = row_params(V, float(max(T[b], 0.0)), int(k[b]), float(p[b]))
        prep = row_params(V, float(ts[b]), None if ks is None else int(ks[b]),
                          None if ps is None else float(ps[b]))
        assert raw == prep, (b, T[b], k[b], p[b])


# -------------------------------------------------------------- min_p ---

def test_min_p_on_the_pages_logits():
    """The pages' worked logits [5, 4, 3, 0, 0, 0] at T = 1: probabilities
    relative to the maximum are 1, 1/e, 1/e^2, 1/e^5 ... min_p 0.2 keeps
    {0, 1} (as top-k 2: token 0 with probability e/(1+e)), min_p 0.1 keeps
    {0, 1, 2}, min_p 1 keeps the maximum only."""
    x = np.array([5.0, 4.0, 3.0, 0.0, 0.0, 0.0])
    e = np.e
    for mp, kept, r0 in ((0.2, 2, e / (1 + e)), (0.1, 3, e * e / (e * e + e + 1)), (1.0, 1, 1.0),
                         (np.exp(-5) * 0.999, 6, None)):
        prm = row_params(6, 1.0, -1, 1.0, mp)
        res = sample_row(x, prm, 0.5)
        assert res.kept == kept, mp
        if r0 is not None:
            assert abs(res.r[0] - r0) < 1e-15
    # min_p 1 with a tie at the maximum keeps both maxima
    res = sample_row(np.array([2.0, 7.0, 7.0, 1.0]), row_params(4, 0.5, -1, 1.0, 1.0), 0.7)
    assert res.kept == 2 and set(np.flatnonzero(res.r)) == {1, 2}


def test_min_p_is_the_intersection_of_masks():
    """By brute force: the kept set equals (top-k then top-p mask) AND
    (p_i >= p_max * min_p), computed on token indices."""
    rng = np.random.default_rng(14)
    for _ in range(300):
        V = int(rng.integers(2, 9))
        x = np.round(rng.standard_normal(V) * 2, 1)
        T = float(rng.choice([0.5, 1.0, 1.7]))
        k = int(rng.integers(1, V + 1))
        p = float(rng.choice([0.3, 0.6, 0.9, 1.0]))
        mp = float(rng.choice([0.05, 0.2, 0.5, 0.9]))
        res = sample_row(x, row_params(V, T, k, p, mp), 0.3)
        if res.cutoff_ambiguous:
            continue
        prob = np.exp((x - x.max()) / T)
        prob /= prob.sum()
        order = np.argsort(-x, kind="stable")
        n_kp = sample_row(x, row_params(V, T, k, p), 0.3).kept
        mask_kp = np.zeros(V, bool)
        mask_kp[order[:n_kp]] = True
        mask_min = prob >= prob.max() * mp
        assert set(np.flatnonzero(res.r > 0)) == set(np.flatnonzero(mask_kp & mask_min))


def test_min_p_logit_threshold_and_zero():
    """p_i >= p_max * min_p  <=>  x_i >= m + T ln(min_p); min_p 0 changes
    nothing."""
    rng = np.random.default_rng(15)
    for _ in range(50):
        V = 3000
        x = rng.standard_normal(V) * 3
        T = float(rng.uniform(0.3, 2.0))
        mp = float(rng.uniform(0.001, 0.9))
        prob = np.exp((x - x.max()) / T)
        q_sorted = np.sort(prob)[::-1] / prob.sum()
        assert min_p_count(q_sorted, mp) == int(np.count_nonzero(x >= x.max() + T * np.log(mp)))
        a = sample_row(x, row_params(V, T, 40, 0.9), 0.42)
        b = sample_row(x, row_params(V, T, 40, 0.9, 0.0), 0.42)
        assert a.kept == b.kept and a.token == b.token and np.array_equal(a.r, b.r)
    assert row_params(10, 1.0, -1, 1.0, -0.5).min_p == 0.0
    assert row_params(10, 1.0, -1, 1.0, float("nan")).min_p == 0.0
    assert row_params(10, 1.0, -1, 1.0, 3.0).min_p == 1.0


# --------------------------------------------------------- page table ---

def test_page_aligned_allocation_pages_test():
    """The pages' test of page-aligned allocation ("CacheManager: allocation,
    release and admission control", section "Tests"): 8 pages of 4 tokens; a
    6-token prompt in table row 2 takes 2 pages (row [0..7], 6 pages free);
    device_len 7 needs none; device_len 9 takes a third page whose location
    is a multiple of 4 (5 free)."""
    pool = PagePool(num_pages=8, page_size=4)
    table = np.full((4, 32), -1, dtype=np.int32)
    table, _ = pool.allocate_paged(table, [2], [0], [6])
    assert table[2, :8].tolist() == [0, 1, 2, 3, 4, 5, 6, 7] and len(pool.free_slots) == 6
    table, _ = pool.allocate_paged(table, [2], [6], [7])
    assert len(pool.free_slots) == 6
    table, _ = pool.allocate_paged(table, [2], [8], [9])
    assert len(pool.free_slots) == 5 and table[2, 8] % 4 == 0
    assert table[2, 8:12].tolist() == [8, 9, 10, 11]


def test_paged_info_worked_count():
    """Page size 4, cached_len 6, device_len 9: pages 0-1 exist, 3 are needed,
    one is allocated (same page, section "Allocating pages for this step's
    tokens")."""
    info, needed = paged_info([5], [6], [9], 4)
    assert needed == 1 and info == [(5, 2, 3)]
    info, needed = paged_info([0, 1, 2], [0, 3, 7], [1, 4, 7], 1)
    assert needed == 2 and info == [(0, 0, 1), (1, 3, 4)]


def test_page_table_brute_force():
    """Every written position holds its own page's first location plus its
    offset, no location is written twice, and nothing else changes."""
    rng = np.random.default_rng(13)
    for ps in (1, 2, 4, 16):
        R, C = 24, 256
        table0 = rng.integers(-50, -1, (R, C)).astype(np.int32)
        n = 12
        tidx = rng.permutation(R)[:n]
        dev = rng.integers(0, C + 1, n)
        cached = np.minimum(dev, rng.integers(0, C + 1, n))
        info, needed = paged_info(tidx, cached, dev, ps)
        starts = rng.permutation(4 * needed + 8)[:needed] * ps
        table, bad = write_page_table(table0, page_to_token(starts, ps), info, ps)
        assert not bad
        seen = set()
        k = 0
        touched = np.zeros_like(table0, dtype=bool)
        for t, first, last in info:
            for page in range(first, last):
                for o in range(ps):
                    v = int(table[t, page * ps + o])
                    assert v == starts[k] + o and v not in seen
                    seen.add(v)
                    touched[t, page * ps + o] = True
                k += 1
        assert k == needed and np.array_equal(table[~touched], table0[~touched])


def test_draw_band_accepts_exactly_the_near_tokens():
    """The draw's tolerance: with dyadic masses the CDF boundaries are exact
    (0.25, 0.5, 1), so which tokens a u near a boundary may give is known by
    hand: both neighbours within 1e-5 of the boundary, only the owner beyond,
    never a token of zero mass ("The engine and the sampler", section "The
    sampler": one categorical draw from the kept distribution)."""
    r = np.array([0.25, 0.0, 0.25, 0.5])
    cases = [
        (0.5 - 0.5e-5, True, [2, 3]),
        (0.5 - 2e-5, False, [2]),
        (0.5 + 0.5e-5, True, [2, 3]),
        (0.5 + 2e-5, False, [3]),
        (0.25 + 0.5e-5, True, [0, 2]),
        (0.25 - 2e-5, False, [0]),
        (0.75, False, [3]),
    ]
    for u, near, toks in cases:
        got_near, got = sr._acceptable(r, u)
        assert got_near == near and got == toks, (u, got_near, got)
        assert sr.inverse_cdf(r, u) in got


def test_cutoff_band_hand_worked():
    """Which kept lengths rounding of the top-p prefixes may give.  With
    masses (1/2, 1/4, 1/8, 1/8) the exclusive prefixes 0, 0.5, 0.75, 0.875
    are exact, so a p within 1e-6 of 0.75 may keep 2 or 3 and a p 5e-6 away
    keeps exactly one of them.  The first prefix is exactly 0: at the
    clamped top_p = float32(1e-6) only the first token is kept, with no
    alternative ("The engine and the sampler", section "The sampler": the
    top rank, with nothing before it, survives every cut)."""
    q = np.array([0.5, 0.25, 0.125, 0.125])
    assert sr.cutoff_alternatives(q, 4, 0.75 - 5e-7) == {2, 3}
    assert sr.cutoff_alternatives(q, 4, 0.75 + 5e-7) == {2, 3}
    assert sr.cutoff_alternatives(q, 4, 0.75 - 5e-6) == {2}
    assert sr.cutoff_alternatives(q, 4, 0.75 + 5e-6) == {3}
    assert sr.cutoff_alternatives(q, 4, float(np.float32(1e-6))) == {1}
    assert sr.cutoff_alternatives(q, 4, 1.0) == {4}
    # top-k 2 renormalises first: (2/3, 1/3), prefixes 0, 2/3
    assert sr.cutoff_alternatives(q, 2, 2.0 / 3.0 + 5e-7) == {1, 2}
    assert sr.cutoff_alternatives(q, 2, 0.7) == {2}
    res = sr.sample_row(np.array([3.0, 1.0, 0.5, 0.2, 0.1, 0.0]), sr.row_params(6, 1.0, -1, 1e-9), 0.3)
    assert res.kept == 1 and not res.cutoff_ambiguous and res.token == 0


def test_min_p_band_hand_worked():
    """The min_p threshold's tolerance: a token 1e-10 from the threshold in
    log-probability may go either way, one 1e-8 away may not ("The engine and
    the sampler", section "Exercises", exercise 2: p_i >= min_p * p_max)."""
    prm = sr.row_params(5, 1.0, -1, 1.0, min_p=0.5)
    thr = float(np.log(prm.min_p))
    for off, want in [(1e-10, {1, 2}), (-1e-10, {1, 2}), (1e-8, {2}), (-1e-8, {1})]:
        x = np.array([0.0, thr + off, -5.0, -6.0, -7.0])
        assert sr.min_p_alternatives(x, prm.T, prm.min_p) == want, off
        res = sr.sample_row(x, prm, 0.3)
        assert res.kept == (2 if off > 0 else 1)
        assert res.cutoff_ambiguous == (abs(off) < 1e-9)
    assert sr.min_p_alternatives(np.array([0.0, -1.0]), 1.0, 0.0) == set()


def test_module_header_marks_test_infrastructure():
    assert "TEST INFRASTRUCTURE" in oracle.__doc__
