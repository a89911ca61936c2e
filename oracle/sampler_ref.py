"""fp64 CPU oracle of the per-step batched sampler and the token write-back.

TEST INFRASTRUCTURE.  This is the plain, slow, obviously-correct statement of
what the sampler computes; it is never on the product path.  Only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import it.
It shares no code with the HIP library and imports nothing from it.

It follows the mini-sglang pages step by step, in float64:

* "The engine and the sampler", section "The sampler" -- ``Sampler.prepare``
  (clamps ``MIN_T = MIN_P = 1e-6``, ``top_k < 1`` means the whole vocabulary,
  ``top_p`` clamped to [1e-6, 1], an all-greedy batch carries no temperature
  array and is decided by argmax) and ``sample_torch`` (softmax of
  logits / T, sort descending, top-k mask by rank, renormalise, mask the
  ranks whose preceding mass is already >= top_p, scatter back to index
  order, one categorical draw).  The same section states the order: top-k
  first, then top-p; the top rank has an empty prefix, so it survives every cut.
* "The engine and the sampler", section "forward_batch": tokens are int32;
  one copy stays on the device, one goes to the host.
* "The scheduler skeleton and the offline interface", section "Preparing a
  batch" (``_make_write_tuple``) and ``_forward``: the token is written to
  ``token_pool[row, col]``; a column of -1 lands in the last column.

Readings taken where the pages leave a step open (each is listed in the
design notes):

* a row is greedy iff its temperature is not above float32(1e-6); greedy
  rows take the exact argmax (lowest index on ties), not a tiny-T softmax;
* NaN temperature -> greedy; NaN top_p -> 1e-6 (clamp order max then min);
* the descending order ranks by the logit value with ties by ascending index
  (softmax is strictly monotone for T > 0), and -0.0 equals +0.0;
* ``top_k >= V`` is the same as disabled; ``top_p >= 1`` disables top-p;
* the top-p test is strict: keep rank j iff the exclusive prefix of the
  renormalised post-top-k masses is < top_p;
* the categorical draw is an inverse CDF in ascending token index with a
  strict ``>``: token = min{i : C_i > u}, ``u`` from the keyed Philox stream;
* the final distribution is the kept masses divided by their sum.

Ambiguity flags (decisions that rounding order may legitimately flip):
``draw_ambiguous`` when ``u`` lies within 1e-5 of a CDF boundary, and
``cutoff_ambiguous`` when a comparison that sets the kept length could be
flipped by rounding: an exclusive prefix after the first rank within 1e-6 of
top_p (the first rank's prefix is exactly 0 and is always kept), or a token
within 1e-9 of the min_p threshold in log-probability.  The alternative kept
lengths are exactly the ones those flips can give (``cutoff_alternatives``,
``min_p_alternatives``).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

from .philox import request_uniform, request_word

MIN_T = float(np.float32(1e-6))
MIN_P = float(np.float32(1e-6))
DRAW_BAND = 1e-5
CUT_BAND = 1e-6
MIN_P_BAND = 1e-9      # min_p: |log(p_i / p_max) - log(min_p)| below this is ambiguous


def widen_logits(logits: np.ndarray, dtype: str) -> np.ndarray:
    """Logits as float64: bf16 bit patterns shifted into the top half of a
    float32, or float32 values, both widened exactly."""
    if dtype == "bf16":
        f32 = (np.asarray(logits).astype(np.uint32) << np.uint32(16)).view(np.float32)
        return f32.astype(np.float64)
    return np.asarray(logits, dtype=np.float32).astype(np.float64)


@dataclass
class RowParams:
    greedy: bool
    T: float          # effective temperature (float32 value, widened)
    k: int            # effective top-k (V when disabled)
    p: float          # effective top-p (1.0 when disabled)
    min_p: float = 0.0  # effective min_p (0.0 when disabled)


def row_params(V: int, T: Optional[float], k: Optional[int], p: Optional[float],
               min_p: Optional[float] = None) -> RowParams:
    """``Sampler.prepare``'s clamps for one request, evaluated in float32.
    min_p (the pages' exercise, "The engine and the sampler", section
    "Exercises"): a value not above 0 (or NaN) disables it, values above 1
    act as 1."""
    if T is None:
        return RowParams(True, MIN_T, 1, 1.0)
    t32 = np.float32(T)
    greedy = not (t32 > np.float32(MIN_T))
    T_eff = float(t32) if not greedy else MIN_T
    k_eff = V if (k is None or int(k) < 1 or int(k) >= V) else int(k)
    if p is None:
        p_eff = 1.0
    else:
        p32 = np.float32(p)
        p_eff = float(p32) if p32 > np.float32(MIN_P) else MIN_P
        p_eff = min(p_eff, 1.0)
    mp_eff = 0.0
    if min_p is not None:
        m32 = np.float32(min_p)
        mp_eff = min(float(m32), 1.0) if m32 > 0 else 0.0
    return RowParams(greedy, T_eff, k_eff, p_eff, mp_eff)


def descending_order(x: np.ndarray) -> np.ndarray:
    """Ranks by value descending, ties by ascending index (stable sort of -x)."""
    return np.argsort(-x, kind="stable")


def filter_sorted(q_sorted: np.ndarray, k: int, p: float, order: str = "k_then_p") -> int:
    """Length n of the kept prefix of descending-sorted probabilities.

    ``k_then_p`` (the pages' order): zero the ranks >= k, renormalise, keep a
    rank while the mass strictly before it is < p.  ``p_then_k`` applies the
    same two masks in the opposite order (used only to show that the order
    matters).
    """
    V = len(q_sorted)
    k = min(k, V)
    if order == "k_then_p":
        if p >= 1.0:
            return k
        q = q_sorted[:k] / q_sorted[:k].sum()
        before = np.concatenate(([0.0], np.cumsum(q)[:-1]))
        return int(np.count_nonzero(before < p))
    if order == "p_then_k":
        n = V
        if p < 1.0:
            q = q_sorted / q_sorted.sum()
            before = np.concatenate(([0.0], np.cumsum(q)[:-1]))
            n = int(np.count_nonzero(before < p))
        return min(n, k)
    raise ValueError(order)


def min_p_count(q_sorted: np.ndarray, min_p: float) -> int:
    """Length of the prefix kept by min_p: the tokens whose probability is at
    least the maximum probability times min_p ("The engine and the sampler",
    section "Exercises", exercise 2 and its answer: the mask is taken on the
    full temperature-scaled distribution and intersected with the top-k /
    top-p mask; both masks are prefixes of the descending order, so the
    intersection is the shorter prefix)."""
    if min_p <= 0.0:
        return len(q_sorted)
    return int(np.count_nonzero(q_sorted >= q_sorted[0] * min_p))


def inverse_cdf(r: np.ndarray, u: float) -> int:
    """min{i : sum_{j<=i} r_j > u} in ascending token index; if rounding
    leaves the last partial sum <= u, the largest index with r_i > 0."""
    c = np.cumsum(r)
    hit = np.flatnonzero(c > u)
    if hit.size:
        return int(hit[0])
    return int(np.flatnonzero(r > 0)[-1])


@dataclass
class RowResult:
    token: int
    greedy: bool
    r: np.ndarray                 # final distribution over V (float64)
    kept: int                     # length of the kept prefix of the descending order
    order_prefix: np.ndarray      # descending-order indices of the first min(k_eff, 64) ranks
    u: float
    word0: int
    params: RowParams
    draw_ambiguous: bool = False
    acceptable: List[int] = field(default_factory=list)
    cutoff_ambiguous: bool = False
    alt_r: Dict[int, np.ndarray] = field(default_factory=dict)   # kept count -> r
    alt_acceptable: Dict[int, List[int]] = field(default_factory=dict)


def _distribution(x: np.ndarray, T: float, pi: np.ndarray, n: int) -> np.ndarray:
    m = x.max()
    w = np.exp((x - m) / T)
    prob = w / w.sum()
    r = np.zeros_like(prob)
    keep = pi[:n]
    r[keep] = prob[keep]
    return r / r.sum()


def _acceptable(r: np.ndarray, u: float):
    """(near, tokens): whether ``u`` lies within DRAW_BAND of a CDF boundary
    of a kept token, and the kept tokens whose interval [C_{i-1}, C_i),
    widened by DRAW_BAND on both sides, contains ``u``."""
    c = np.cumsum(r)
    prev = np.concatenate(([0.0], c[:-1]))
    kept = r > 0
    ok = np.flatnonzero(kept & (prev - DRAW_BAND <= u) & (u < c + DRAW_BAND))
    near = np.abs(np.concatenate((prev[kept], c[kept])) - u).min() < DRAW_BAND
    return bool(near), [int(i) for i in ok]


def cutoff_alternatives(q_sorted: np.ndarray, k: int, p: float) -> set:
    """Kept lengths of the top-k-then-top-p filter that rounding of the
    exclusive prefixes may also give.  Rank j is kept iff S_j < p; S_0 = 0 is
    exact (the first rank is always kept), and every later S_j is a sum that
    rounding may move by up to CUT_BAND.  Since S_j never decreases along the
    order, the reachable lengths are every count between the one at
    p - CUT_BAND and the one at p + CUT_BAND ("The engine and the sampler",
    section "The sampler": the top-p test on the renormalised top-k masses).
    Returns the set of lengths (the exact one included)."""
    k = min(k, len(q_sorted))
    if p >= 1.0:
        return {k}
    q = q_sorted[:k] / q_sorted[:k].sum()
    before = np.cumsum(q)[:-1]          # S_1 .. S_{k-1}
    n_lo = 1 + int(np.count_nonzero(before < p - CUT_BAND))
    n_hi = 1 + int(np.count_nonzero(before < p + CUT_BAND))
    return set(range(n_lo, n_hi + 1))


def min_p_alternatives(x_sorted: np.ndarray, T: float, min_p: float) -> set:
    """Kept lengths of the min_p filter that rounding may also give: rank j
    is kept iff d_j = (x_j - x_0)/T - ln(min_p) >= 0 (the probability at least
    min_p times the largest); a d_j within MIN_P_BAND of 0 may go either way.
    d never increases along the order, so the reachable lengths run from
    #{d >= MIN_P_BAND} to #{d > -MIN_P_BAND}.  Returns the set of lengths
    (the exact one included); empty when min_p is off."""
    if min_p <= 0.0:
        return set()
    d = (x_sorted - x_sorted[0]) / T - np.log(min_p)
    lo = int(np.count_nonzero(d >= MIN_P_BAND))
    hi = int(np.count_nonzero(d > -MIN_P_BAND))
    return set(range(lo, hi + 1))


def sample_row(x: np.ndarray, params: RowParams, u: float, word0: int = 0,
               order: str = "k_then_p", want_alternatives: bool = True) -> RowResult:
    """One request: greedy argmax, or softmax -> top-k -> top-p -> draw."""
    V = len(x)
    if params.greedy:
        tok = int(np.argmax(x))
        r = np.zeros(V)
        r[tok] = 1.0
        return RowResult(tok, True, r, 1, np.array([tok]), u, word0, params)

    pi = descending_order(x)
    m = x.max()
    w = np.exp((x - m) / params.T)          # softmax(logits / T), max subtracted
    prob = w / w.sum()
    q_sorted = prob[pi]
    n_kp = filter_sorted(q_sorted, params.k, params.p, order)
    n_min = min_p_count(q_sorted, params.min_p)
    n = min(n_kp, n_min)
    r = _distribution(x, params.T, pi, n)
    tok = inverse_cdf(r, u)
    res = RowResult(tok, False, r, n, pi[:min(params.k, 64)].copy(), u, word0, params)
    res.draw_ambiguous, res.acceptable = _acceptable(r, u)

    if not want_alternatives:
        return res
    # kept lengths that rounding at a cut-off may also give
    kp_alts = cutoff_alternatives(q_sorted, params.k, params.p) if order == "k_then_p" else {n_kp}
    min_alts = min_p_alternatives(x[pi], params.T, params.min_p) or {n_min}
    alts = {min(a, b) for a in kp_alts for b in min_alts} - {n}
    alts = {a for a in alts if a >= 1}
    if alts:
        res.cutoff_ambiguous = True
        for n_alt in sorted(alts):
            r_alt = _distribution(x, params.T, pi, n_alt)
            res.alt_r[n_alt] = r_alt
            res.alt_acceptable[n_alt] = _acceptable(r_alt, u)[1] + [inverse_cdf(r_alt, u)]
    return res


def _opt(a: Optional[np.ndarray], b: int):
    return None if a is None else a[b]


def sample_batch(logits: np.ndarray, dtype: str, temperature: Optional[np.ndarray],
                 top_k: Optional[np.ndarray], top_p: Optional[np.ndarray],
                 uid: np.ndarray, step: int, seed: int, rows=None,
                 order: str = "k_then_p", min_p: Optional[np.ndarray] = None) -> List[RowResult]:
    """Every request of one decode step (or the subset ``rows``)."""
    X = widen_logits(logits, dtype)
    B, V = X.shape
    out = []
    for b in (range(B) if rows is None else rows):
        prm = row_params(V, _opt(temperature, b), _opt(top_k, b), _opt(top_p, b),
                         _opt(min_p, b))
        if temperature is None:
            u, w0 = 0.0, 0
        else:
            w0 = request_word(seed, int(uid[b]), step)
            u = request_uniform(seed, int(uid[b]), step)
        out.append(sample_row(X[b], prm, u, w0, order))
    return out


def write_tokens(pool: np.ndarray, rows: np.ndarray, cols: np.ndarray, tokens: np.ndarray):
    """``token_pool[rows, cols] = tokens`` with column -1 meaning the last
    column; an out-of-range (row, col) is skipped and reported.

    Returns (new pool, host copy of the tokens, out_of_range flag)."""
    out = pool.copy()
    R, C = out.shape
    bad = False
    for b in range(len(tokens)):
        r, c = int(rows[b]), int(cols[b])
        if c == -1:
            c = C - 1
        if 0 <= r < R and 0 <= c < C:
            out[r, c] = np.int32(tokens[b])
        else:
            bad = True
    return out, np.asarray(tokens, dtype=np.int32).copy(), bad


def gather_tokens(pool: np.ndarray, rows: np.ndarray, positions: np.ndarray):
    """``token_pool[rows, positions]``: the step's input ids ("The scheduler
    skeleton and the offline interface", sections "Preparing a batch" and
    "_forward").  Indices are used as given; an entry outside the pool gives
    -1 and is reported.

    Returns (ids int32 [n], out_of_range flag)."""
    R, C = pool.shape
    ids = np.full(len(rows), -1, dtype=np.int32)
    bad = False
    for i in range(len(rows)):
        r, c = int(rows[i]), int(positions[i])
        if 0 <= r < R and 0 <= c < C:
            ids[i] = pool[r, c]
        else:
            bad = True
    return ids, bad


def input_tuple(table_idx, cached_len, device_len):
    """(rows, positions) of one batch: every request contributes its positions
    [cached_len, device_len) in order, request after request (same page,
    section "Preparing a batch")."""
    rows, pos = [], []
    for r, lo, hi in zip(table_idx, cached_len, device_len):
        for c in range(int(lo), int(hi)):
            rows.append(int(r))
            pos.append(c)
    return np.asarray(rows, dtype=np.int64), np.asarray(pos, dtype=np.int64)


def prepare(V: int, temperature, top_k, top_p, min_p=None):
    """``Sampler.prepare`` for a batch ("The engine and the sampler", section
    "The sampler"), from request-level parameters (each array may be None:
    not set by any request).  A request is greedy iff its temperature is
    <= 0.  The values are computed on Python floats as the pages do, then
    stored as float32 / int32.

    min_p (the pages' exercise) follows the same rule: a tensor only when
    some request sets a value above 0; the value is passed as given and
    clamped where it is used.

    Returns (temperature, top_k, top_p), or (temperature, top_k, top_p,
    min_p) when ``min_p`` is given: float32 / int32 / float32 (/ float32)
    arrays, or None where the pages pass None."""
    B = 0
    for a in (temperature, top_k, top_p, min_p):
        if a is not None:
            B = len(a)
    T = [0.0] * B if temperature is None else [float(np.float32(t)) for t in temperature]
    greedy = [not (t > 0.0) if t == t else False for t in T]       # NaN is not greedy
    if all(greedy):
        return (None, None, None) if min_p is None else (None, None, None, None)
    min_t = min_p_clamp = 1e-6
    ts = [max(0.0 if g else t, min_t) for g, t in zip(greedy, T)]
    ks_in = [-1] * B if top_k is None else [int(k) for k in top_k]
    ks = [k if k >= 1 else V for k in ks_in]
    ps_in = [1.0] * B if top_p is None else [float(np.float32(p)) for p in top_p]
    ps = [min(max(p, min_p_clamp), 1.0) for p in ps_in]
    out_k = np.array(ks, dtype=np.int32) if any(k != V for k in ks) else None
    out_p = np.array(ps, dtype=np.float32) if any(p < 1.0 for p in ps) else None
    if min_p is None:
        return np.array(ts, dtype=np.float32), out_k, out_p
    mps = [float(np.float32(v)) for v in min_p]
    out_m = np.array(mps, dtype=np.float32) if any(v > 0.0 for v in mps) else None
    return np.array(ts, dtype=np.float32), out_k, out_p, out_m


def _div_ceil(a: int, b: int) -> int:
    return -(-int(a) // int(b))


def page_to_token(page_starts, page_size: int) -> np.ndarray:
    """Token locations of allocated pages: each page's first location plus
    every offset inside the page ("CacheManager: allocation, release and
    admission control", section "The free-page list": free slots hold the
    first token location of each page).  The pages do not print
    ``_page_to_token``; this is the plainest reading of that section."""
    starts = np.asarray(page_starts, dtype=np.int64)
    return (starts[:, None] + np.arange(page_size, dtype=np.int64)[None, :]).reshape(-1)


def write_page_table(page_table: np.ndarray, allocated: np.ndarray, info, page_size: int):
    """``_write_page_table`` (same page, section "Allocating pages for this
    step's tokens"): (row, column) pairs built on the host request by request
    over [first_page * page_size, last_page * page_size), then one indexed
    assignment of the allocated token locations.  An out-of-range
    pair is skipped and reported.

    Returns (new page table, out_of_range flag)."""
    rows, cols = [], []
    for table_idx, first_page, last_page in info:
        lo, hi = first_page * page_size, last_page * page_size
        rows.extend([int(table_idx)] * (hi - lo))
        cols.extend(range(lo, hi))
    assert len(rows) == len(allocated), "allocated locations must match the positions"
    out = page_table.copy()
    R, C = out.shape
    bad = False
    for r, c, v in zip(rows, cols, allocated):
        if 0 <= r < R and 0 <= c < C:
            out[r, c] = np.int32(v)
        else:
            bad = True
    return out, bad


def paged_info(table_idx, cached_len, device_len, page_size: int):
    """``allocate_paged``'s per-request page ranges (same page and section):
    pages [ceil(cached_len /
    page_size), ceil(device_len / page_size)) are new; requests without a new
    page are left out.  Returns (info list, number of new pages)."""
    info, needed = [], 0
    for t, c, d in zip(table_idx, cached_len, device_len):
        first, last = _div_ceil(c, page_size), _div_ceil(d, page_size)
        if last > first:
            needed += last - first
            info.append((int(t), first, last))
    return info, needed


class PagePool:
    """The free-page list of the cache manager with the naive cache (no
    eviction; same page, sections "The free-page list" and "_allocate"): free
    slots start as every page's first token location, and allocation takes
    pages from the front."""

    def __init__(self, num_pages: int, page_size: int):
        self.page_size = page_size
        self.free_slots = np.arange(num_pages, dtype=np.int64) * page_size

    def allocate(self, needed_pages: int) -> np.ndarray:
        assert needed_pages <= len(self.free_slots), "not enough free pages"
        out = self.free_slots[:needed_pages].copy()
        self.free_slots = self.free_slots[needed_pages:]
        return out

    def allocate_paged(self, page_table: np.ndarray, table_idx, cached_len, device_len):
        """Allocate this step's pages and write them into the page table.
        Returns (new page table, page starts allocated)."""
        info, needed = paged_info(table_idx, cached_len, device_len, self.page_size)
        if needed == 0:
            return page_table.copy(), np.zeros(0, dtype=np.int64)
        starts = self.allocate(needed)
        out, bad = write_page_table(page_table, page_to_token(starts, self.page_size), info,
                                    self.page_size)
        assert not bad
        return out, starts
