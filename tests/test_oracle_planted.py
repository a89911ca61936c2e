"""Plant plausible mistakes in the oracle (CPU only) and check that a pin
catches each one.  This guards the pins themselves: a pin that passes on a
broken oracle would prove nothing."""
import numpy as np
import pytest

import oracle.philox as ph
import oracle.sampler_ref as sr
from tests import test_oracle_pins as pins


def _inclusive_prefix(q_sorted, k, p, order="k_then_p"):
    k = min(k, len(q_sorted))
    if p >= 1.0:
        return k
    q = q_sorted[:k] / q_sorted[:k].sum()
    return int(np.count_nonzero(np.cumsum(q) < p))


def _non_strict(q_sorted, k, p, order="k_then_p"):
    k = min(k, len(q_sorted))
    if p >= 1.0:
        return k
    q = q_sorted[:k] / q_sorted[:k].sum()
    before = np.concatenate(([0.0], np.cumsum(q)[:-1]))
    return int(np.count_nonzero(before <= p))


def _no_renormalise(q_sorted, k, p, order="k_then_p"):
    k = min(k, len(q_sorted))
    if p >= 1.0:
        return k
    q = q_sorted[:k]
    before = np.concatenate(([0.0], np.cumsum(q)[:-1]))
    return int(np.count_nonzero(before < p))


_real_filter = sr.filter_sorted


def _p_then_k(q_sorted, k, p, order="k_then_p"):
    return _real_filter(q_sorted, k, p, "p_then_k")


def _distribution_times_T(x, T, pi, n):
    return _real_distribution(x, 1.0 / T, pi, n)


_real_distribution = sr._distribution
_real_order = sr.descending_order


def _last_index_ties(x):
    # descending by value but ties by descending index
    return np.lexsort((-np.arange(len(x)), -x))


def _draw_ge(r, u):
    c = np.cumsum(r)
    hit = np.flatnonzero(c >= u)
    return int(hit[0]) if hit.size else int(np.flatnonzero(r > 0)[-1])


def _philox_no_key_bump(counter, key, rounds=10):
    x0, x1, x2, x3 = (int(c) & ph.M64 for c in counter)
    k0, k1 = (int(k) & ph.M64 for k in key)
    for _ in range(rounds):
        p0, p1 = ph.PHILOX_M0 * x0, ph.PHILOX_M1 * x2
        x0, x1, x2, x3 = ((p1 >> 64) ^ x1 ^ k0, p1 & ph.M64, (p0 >> 64) ^ x3 ^ k1, p0 & ph.M64)
    return (x0, x1, x2, x3)


def _write_minus_one_to_first(pool, rows, cols, tokens):
    return _real_write(pool, rows, np.where(np.asarray(cols) == -1, 0, cols), tokens)


_real_write = sr.write_tokens
_real_gather = sr.gather_tokens
_real_input_tuple = sr.input_tuple


def _gather_transposed(pool, rows, positions):
    # operands swapped: reads pool[position, row] (square pools hide it)
    R, C = pool.shape
    ids = np.full(len(rows), -1, dtype=np.int32)
    bad = False
    for i in range(len(rows)):
        r, c = int(positions[i]), int(rows[i])
        if 0 <= r < R and 0 <= c < C:
            ids[i] = pool[r, c]
        else:
            bad = True
    return ids, bad


def _gather_wraps_negative(pool, rows, positions):
    # NumPy-style wrap of negative indices instead of a reported miss
    R, C = pool.shape
    r = np.asarray(rows, dtype=np.int64)
    c = np.asarray(positions, dtype=np.int64)
    ok = (r >= -R) & (r < R) & (c >= -C) & (c < C)
    ids = np.full(len(r), -1, dtype=np.int32)
    ids[ok] = pool[r[ok], c[ok]]
    return ids, bool((~ok).any())


_real_prepare = sr.prepare


def _prepare_k_strict(V, temperature, top_k, top_p):
    # "k > 1" for "k >= 1": a top-k of 1 would be dropped
    k2 = None if top_k is None else np.where(np.asarray(top_k) == 1, -1, top_k).astype(np.int32)
    return _real_prepare(V, temperature, k2, top_p)


def _prepare_p_tensor_always(V, temperature, top_k, top_p):
    ts, ks, ps = _real_prepare(V, temperature, top_k, top_p)
    if ts is not None and ps is None:
        ps = np.ones(len(ts), dtype=np.float32)
    return ts, ks, ps


_real_paged_info = sr.paged_info
_real_page_to_token = sr.page_to_token


def _paged_info_floor(table_idx, cached_len, device_len, page_size):
    # floor instead of ceil for the first page: a partly filled page again
    info, needed = [], 0
    for t, c, d in zip(table_idx, cached_len, device_len):
        first, last = int(c) // page_size, -(-int(d) // page_size)
        if last > first:
            needed += last - first
            info.append((int(t), first, last))
    return info, needed


def _page_to_token_scaled(page_starts, page_size):
    # treats the free slots as page numbers
    return _real_page_to_token(np.asarray(page_starts) * page_size, page_size)


def _min_p_strict(q_sorted, min_p):
    # ">" for ">=": a token exactly at the threshold (or the maximum itself
    # at min_p 1) is dropped
    if min_p <= 0.0:
        return len(q_sorted)
    return int(np.count_nonzero(q_sorted > q_sorted[0] * min_p))


def _min_p_absolute(q_sorted, min_p):
    # threshold on the probability itself, not relative to the maximum
    if min_p <= 0.0:
        return len(q_sorted)
    return max(1, int(np.count_nonzero(q_sorted >= min_p)))


def _input_tuple_inclusive(table_idx, cached_len, device_len):
    # off by one: runs [cached_len, device_len]
    return _real_input_tuple(table_idx, cached_len, [int(d) + 1 for d in device_len])


def _acceptable_wide(r, u):
    # the draw band ten times too wide
    c = np.cumsum(r)
    prev = np.concatenate(([0.0], c[:-1]))
    kept = r > 0
    band = 1e-4
    ok = np.flatnonzero(kept & (prev - band <= u) & (u < c + band))
    near = np.abs(np.concatenate((prev[kept], c[kept])) - u).min() < band
    return bool(near), [int(i) for i in ok]


def _acceptable_zero_mass(r, u):
    # tokens of zero mass accepted next to a boundary
    c = np.cumsum(r)
    prev = np.concatenate(([0.0], c[:-1]))
    band = sr.DRAW_BAND
    ok = np.flatnonzero((prev - band <= u) & (u < c + band))
    near = np.abs(np.concatenate((prev, c)) - u).min() < band
    return bool(near), [int(i) for i in ok]


def _cutoff_band_includes_first(q_sorted, k, p):
    # the exact S_0 = 0 treated as if rounding could move it
    k = min(k, len(q_sorted))
    if p >= 1.0:
        return {k}
    q = q_sorted[:k] / q_sorted[:k].sum()
    before = np.concatenate(([0.0], np.cumsum(q)[:-1]))
    n = int(np.count_nonzero(before < p))
    out = {n}
    if np.any(np.abs(before - p) < sr.CUT_BAND):
        out |= {a for a in (n - 1, n + 1) if 1 <= a <= k}
    return out


_real_cutoff_alternatives = sr.cutoff_alternatives


def _cutoff_band_wide(q_sorted, k, p):
    old = sr.CUT_BAND
    sr.CUT_BAND = 1e-5
    try:
        return _real_cutoff_alternatives(q_sorted, k, p)
    finally:
        sr.CUT_BAND = old


_real_min_p_alternatives = sr.min_p_alternatives


def _min_p_band_wide(x_sorted, T, min_p):
    old = sr.MIN_P_BAND
    sr.MIN_P_BAND = 1e-7
    try:
        return _real_min_p_alternatives(x_sorted, T, min_p)
    finally:
        sr.MIN_P_BAND = old


def _run_pins(names):
    for name in names:
        fn = getattr(pins, name)
        if name == "test_top_p_cutoffs_exact":
            for args in [((0.5, 0.25, 0.125, 0.125), 4, 0.75, 2),
                         ((0.5, 0.25, 0.125, 0.125), 2, 0.6, 1),
                         ((0.4, 0.3, 0.2, 0.1), 3, 0.42, 1)]:
                fn(*args)
        elif name == "test_philox_matches_numpy":
            fn((7, 1999, 0, 0), (42, 0))
        else:
            fn()


PLANTS = [
    ("filter_sorted", _inclusive_prefix, ["test_pages_example_supports_and_closed_form"]),
    ("filter_sorted", _non_strict, ["test_top_p_cutoffs_exact"]),
    ("filter_sorted", _no_renormalise, ["test_top_p_cutoffs_exact"]),
    ("filter_sorted", _p_then_k, ["test_filter_order_brute_force"]),
    ("_distribution", _distribution_times_T, ["test_two_token_closed_form"]),
    ("descending_order", _last_index_ties, ["test_topk_set_matches_heapq_with_index_ties"]),
    ("inverse_cdf", _draw_ge, ["test_draw_measure_brute_force"]),
    ("write_tokens", _write_minus_one_to_first, ["test_write_tokens_matches_fancy_index"]),
    ("gather_tokens", _gather_transposed, ["test_gather_tokens_matches_fancy_index"]),
    ("gather_tokens", _gather_wraps_negative,
     ["test_gather_tokens_out_of_range_is_reported_not_wrapped"]),
    ("input_tuple", _input_tuple_inclusive, ["test_input_tuple_hand_worked_batch"]),
    ("prepare", _prepare_k_strict, ["test_prepare_hand_worked_batch"]),
    ("prepare", _prepare_p_tensor_always, ["test_prepare_none_rules"]),
    ("paged_info", _paged_info_floor, ["test_paged_info_worked_count"]),
    ("min_p_count", _min_p_strict, ["test_min_p_on_the_pages_logits"]),
    ("min_p_count", _min_p_absolute, ["test_min_p_on_the_pages_logits"]),
    ("page_to_token", _page_to_token_scaled, ["test_page_aligned_allocation_pages_test"]),
    ("_acceptable", _acceptable_wide, ["test_draw_band_accepts_exactly_the_near_tokens"]),
    ("_acceptable", _acceptable_zero_mass, ["test_draw_band_accepts_exactly_the_near_tokens"]),
    ("cutoff_alternatives", _cutoff_band_includes_first, ["test_cutoff_band_hand_worked"]),
    ("cutoff_alternatives", _cutoff_band_wide, ["test_cutoff_band_hand_worked"]),
    ("min_p_alternatives", _min_p_band_wide, ["test_min_p_band_hand_worked"]),
]


@pytest.mark.parametrize("attr,bad,pin_names", PLANTS, ids=[p[1].__name__ for p in PLANTS])
def test_planted_sampler_mistake_is_caught(monkeypatch, attr, bad, pin_names):
    monkeypatch.setattr(sr, attr, bad)
    for mod_name in ("filter_sorted", "inverse_cdf", "write_tokens", "gather_tokens",
                     "input_tuple", "prepare", "paged_info", "page_to_token", "min_p_count"):
        if attr == mod_name:
            monkeypatch.setattr(pins, mod_name, bad)
    with pytest.raises(Exception):    # a failed assertion, or the oracle breaking outright
        _run_pins(pin_names)


def test_planted_philox_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(pins, "philox4x64", _philox_no_key_bump)
    with pytest.raises(AssertionError):
        _run_pins(["test_philox_matches_numpy"])
