"""Seeded synthetic inputs for the per-step batched sampler.

This module only *draws* inputs: logits, per-request sampling parameters,
request uids, token pools and write positions.  It holds none of the
sampler's arithmetic (no softmax, no filtering, no draw), so both the fp64
oracle under ``oracle/`` and the HIP path can be fed from it without sharing
any code with each other.

Workloads follow the decode-step sampler of the mini-sglang pages
("The engine and the sampler", section "The sampler"): a ``[B, V]`` logits
tensor, per-request ``temperature`` / ``top_k`` / ``top_p`` arrays (each may
be absent), and a token pool written at ``(row, col)`` per request ("The
scheduler skeleton and the offline interface", section "Preparing a batch").

Shapes and distributions (all seeded with ``numpy.random.default_rng``):

* ``c0`` -- B=4, V=1024, fp32 N(0, 2); rows 0-1 greedy, rows 2-3
  T=0.7, top_k=50, top_p=0.9; pool [4, 64].
* ``c1`` -- B=64, V=32000, fp32 N(0, 2) plus 8 spikes of +U[6, 10] per row;
  3 rows (5 %) get an exact copy of their maximum at another index; all
  greedy (no temperature array); pool [64, 128].
* ``c2`` -- B=256, V=128256, bf16 N(0, 3); even uids greedy, odd uids
  T=0.7, top_p=0.9, no top_k array; pool [256, 4096].
* ``c3`` -- B=256, V=151936, fp32 2*Gumbel(0, 1) + 1.5*(A W^T)/2 with
  A[B,4], W[V,4] ~ N(0, 1) (a rank-4 term of entrywise std 1.5);
  T ~ U[0.3, 1.5], top_k from {1, 20, 50, -1}, top_p from {1, 0.95, 0.8};
  pool [256, 4096].
* ``c4`` -- decode loop, B=512, V=152064, bf16 N(0, 2.5) regenerated per
  step from ``default_rng([1004, step])``; parameters drawn once per request
  from c3's distributions (``c4b``: c2's half-greedy mix); pool [512, 4096]
  written at ``pos0 + step`` with ``pos0 ~ U[1, 2048]``.

bf16 logits are produced from float32 draws by round-to-nearest-even and
are carried as their raw ``uint16`` bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

SAMPLER_SEED = 42  # the engine seeds its generator with 42

F32 = "f32"
BF16 = "bf16"


@dataclass
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16"
    logits: np.ndarray              # [B, V] float32, or uint16 bf16 bit patterns
    temperature: Optional[np.ndarray]  # [B] float32 or None (whole batch greedy)
    top_k: Optional[np.ndarray]     # [B] int32 or None (disabled)
    top_p: Optional[np.ndarray]     # [B] float32 or None (disabled)
    uid: np.ndarray                 # [B] int64
    step: int
    pool: np.ndarray                # [R, C] int32, initial contents
    rows: np.ndarray                # [B] int64
    cols: np.ndarray                # [B] int64 (-1 => last column)
    seed: int = SAMPLER_SEED
    meta: dict = field(default_factory=dict)
    min_p: Optional[np.ndarray] = None  # [B] float32 or None (disabled)

    @property
    def B(self) -> int:
        return int(self.logits.shape[0])

    @property
    def V(self) -> int:
        return int(self.logits.shape[1])

    @property
    def bytes_per_logit(self) -> int:
        return 4 if self.dtype == F32 else 2

    def with_logits(self, logits: np.ndarray, step: Optional[int] = None) -> "Workload":
        return replace(self, logits=logits, step=self.step if step is None else step)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    chunk = 1 << 22
    flat_b = b.reshape(-1)
    flat_o = out.reshape(-1)
    for s in range(0, flat_b.size, chunk):
        v = flat_b[s:s + chunk]
        r = (v >> np.uint32(16)) & np.uint32(1)
        r += np.uint32(0x7FFF)
        r += v
        r >>= np.uint32(16)
        flat_o[s:s + chunk] = r.astype(np.uint16)
    return out


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for building inputs)."""
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _c3_params(rng: np.random.Generator, B: int):
    T = rng.uniform(0.3, 1.5, B).astype(np.float32)
    k = rng.choice(np.array([1, 20, 50, -1], dtype=np.int32), B)
    p = rng.choice(np.array([1.0, 0.95, 0.8], dtype=np.float32), B)
    return T, k.astype(np.int32), p.astype(np.float32)


def _c2_params(B: int):
    uid = np.arange(B)
    greedy = (uid % 2) == 0
    T = np.where(greedy, 0.0, 0.7).astype(np.float32)
    p = np.where(greedy, 1.0, 0.9).astype(np.float32)
    return T, None, p


def c0() -> Workload:
    rng = np.random.default_rng(1000)
    B, V = 4, 1024
    logits = rng.normal(0.0, 2.0, (B, V)).astype(np.float32)
    T = np.array([0.0, 0.0, 0.7, 0.7], dtype=np.float32)
    k = np.array([-1, -1, 50, 50], dtype=np.int32)
    p = np.array([1.0, 1.0, 0.9, 0.9], dtype=np.float32)
    pool = rng.integers(0, V, (4, 64)).astype(np.int32)
    rows = np.arange(4, dtype=np.int64)
    cols = rng.integers(1, 64, 4).astype(np.int64)
    return Workload("c0", F32, logits, T, k, p, np.arange(B, dtype=np.int64), 0,
                    pool, rows, cols)


def c0_permuted() -> Workload:
    """c0 with the greedy rows moved to positions 1 and 3."""
    w = c0()
    perm = np.array([2, 0, 3, 1])
    return replace(w, name="c0_permuted", logits=w.logits[perm].copy(),
                   temperature=w.temperature[perm].copy(), top_k=w.top_k[perm].copy(),
                   top_p=w.top_p[perm].copy(), uid=w.uid[perm].copy(),
                   rows=w.rows[perm].copy(), cols=w.cols[perm].copy())


def c1() -> Workload:
    rng = np.random.default_rng(1001)
    B, V = 64, 32000
    logits = rng.normal(0.0, 2.0, (B, V)).astype(np.float32)
    for b in range(B):
        idx = rng.choice(V, 8, replace=False)
        logits[b, idx] += rng.uniform(6.0, 10.0, 8).astype(np.float32)
    tie_rows = rng.choice(B, 3, replace=False)
    below = False
    ties = []
    for n, b in enumerate(tie_rows):
        i_star = int(np.argmax(logits[b]))
        if n == len(tie_rows) - 1 and not below and i_star > 0:
            j = int(rng.integers(0, i_star))
        else:
            j = int(rng.integers(0, V - 1))
            j = j + 1 if j >= i_star else j
        below |= j < i_star
        logits[b, j] = logits[b, i_star]
        ties.append((int(b), i_star, j))
    pool = rng.integers(0, V, (B, 128)).astype(np.int32)
    rows = rng.permutation(B).astype(np.int64)
    cols = rng.integers(1, 128, B).astype(np.int64)
    return Workload("c1", F32, logits, None, None, None, np.arange(B, dtype=np.int64), 0,
                    pool, rows, cols, meta={"tie_rows": [int(r) for r in tie_rows], "ties": ties})


def c2() -> Workload:
    rng = np.random.default_rng(1002)
    B, V = 256, 128256
    x = rng.standard_normal((B, V), dtype=np.float32)
    x *= np.float32(3.0)
    logits = to_bf16_bits(x)
    T, k, p = _c2_params(B)
    pool = rng.integers(0, V, (B, 4096)).astype(np.int32)
    rows = rng.permutation(B).astype(np.int64)
    cols = rng.integers(1, 2049, B).astype(np.int64)
    return Workload("c2", BF16, logits, T, k, p, np.arange(B, dtype=np.int64), 0,
                    pool, rows, cols)


def c3() -> Workload:
    rng = np.random.default_rng(1003)
    B, V = 256, 151936
    g = rng.gumbel(0.0, 1.0, (B, V))
    A = rng.standard_normal((B, 4))
    W = rng.standard_normal((V, 4))
    x = 2.0 * g
    x += 1.5 * (A @ W.T) / 2.0
    logits = x.astype(np.float32)
    del g, x
    T, k, p = _c3_params(rng, B)
    pool = rng.integers(0, V, (B, 4096)).astype(np.int32)
    rows = rng.permutation(B).astype(np.int64)
    cols = rng.integers(1, 2049, B).astype(np.int64)
    return Workload("c3", F32, logits, T, k, p, np.arange(B, dtype=np.int64), 0,
                    pool, rows, cols)


C4_B, C4_V, C4_STEPS = 512, 152064, 64


def c4_logits(step: int) -> np.ndarray:
    rng = np.random.default_rng([1004, step])
    x = rng.standard_normal((C4_B, C4_V), dtype=np.float32)
    x *= np.float32(2.5)
    return to_bf16_bits(x)


def c4(step: int = 0, half_greedy: bool = False) -> Workload:
    """One step of the decode loop (``half_greedy``: the c2-style parameter mix)."""
    rng = np.random.default_rng(2004)
    B, V = C4_B, C4_V
    if half_greedy:
        T, k, p = _c2_params(B)
    else:
        T, k, p = _c3_params(rng, B)
    prng = np.random.default_rng(3004)
    pool = prng.integers(0, V, (B, 4096)).astype(np.int32)
    pos0 = prng.integers(1, 2049, B).astype(np.int64)
    rows = np.arange(B, dtype=np.int64)
    return Workload("c4b" if half_greedy else "c4", BF16, c4_logits(step), T, k, p,
                    np.arange(B, dtype=np.int64), step, pool, rows, pos0 + step,
                    meta={"pos0": pos0})


CONFIGS = {"c0": c0, "c1": c1, "c2": c2, "c3": c3, "c4": c4}

LOOP_B, LOOP_V, LOOP_POOL = 64, 4096, (64, 256)


def loop_small_logits(step: int) -> np.ndarray:
    rng = np.random.default_rng([1104, step])
    x = rng.standard_normal((LOOP_B, LOOP_V), dtype=np.float32)
    x *= np.float32(2.5)
    return to_bf16_bits(x)


def loop_small(step: int = 0) -> Workload:
    """c4's decode loop at a size the oracle runs every row of: B=64, V=4096
    bf16 N(0, 2.5) per step, c3's parameter mix, pool [64, 256] written at
    ``pos0 + step`` with ``pos0 ~ U[1, 128]``."""
    rng = np.random.default_rng(2104)
    T, k, p = _c3_params(rng, LOOP_B)
    prng = np.random.default_rng(3104)
    pool = prng.integers(0, LOOP_V, LOOP_POOL).astype(np.int32)
    pos0 = prng.integers(1, 129, LOOP_B).astype(np.int64)
    rows = prng.permutation(LOOP_POOL[0])[:LOOP_B].astype(np.int64)
    return Workload("loop_small", BF16, loop_small_logits(step), T, k, p,
                    np.arange(100, 100 + LOOP_B, dtype=np.int64), step, pool, rows, pos0 + step,
                    meta={"pos0": pos0})


def mixed_input_batch(seed: int, n_req: int = 64, n_prefill: int = 8, pool_rows: int = 256,
                      pool_cols: int = 4096):
    """A step's requests as (table_idx, cached_len, device_len): ``n_prefill``
    prefill or chunked-prefill spans of 1..2048 tokens among single-token
    decode requests, in distinct pool rows; the pool holds random ids."""
    rng = np.random.default_rng(seed)
    pool = rng.integers(0, 152064, (pool_rows, pool_cols)).astype(np.int32)
    table_idx = rng.permutation(pool_rows)[:n_req].astype(np.int64)
    device_len = rng.integers(1, pool_cols + 1, n_req).astype(np.int64)
    cached_len = device_len - 1
    pre = rng.permutation(n_req)[:n_prefill]
    span = rng.integers(1, 2049, n_prefill)
    cached_len[pre] = np.maximum(device_len[pre] - span, 0)
    return pool, table_idx, cached_len, device_len


def tiny(rng: np.random.Generator, B: int, V: int, dtype: str = F32, scale: float = 2.0,
         greedy_frac: float = 0.25, pool_cols: int = 64) -> Workload:
    """A small random mixed batch with per-request parameters of every kind."""
    x = (rng.standard_normal((B, V)) * scale).astype(np.float32)
    logits = to_bf16_bits(x) if dtype == BF16 else x
    T = rng.uniform(0.2, 1.6, B).astype(np.float32)
    T[rng.random(B) < greedy_frac] = 0.0
    k = rng.choice(np.array([-1, 0, 1, 2, 5, 20, 64, 100, V - 1, V, V + 5], dtype=np.int64), B)
    p = rng.choice(np.array([1.0, 0.99, 0.9, 0.5, 0.1, 1e-9, 1.5], dtype=np.float64), B)
    pool = rng.integers(0, V, (B, pool_cols)).astype(np.int32)
    rows = rng.permutation(B).astype(np.int64)
    cols = rng.integers(0, pool_cols, B).astype(np.int64)
    cols[rng.random(B) < 0.1] = -1
    cols[0] = -1
    uid = rng.integers(-(1 << 40), 1 << 40, B).astype(np.int64)
    return Workload(f"tiny_{B}x{V}_{dtype}", dtype, logits, T, k.astype(np.int32),
                    p.astype(np.float32), uid, int(rng.integers(0, 1 << 20)), pool, rows, cols)


def paged_batch(seed: int, n_req: int = 300, table_rows: int = 512, table_cols: int = 4096,
                page_size: int = 1, prefill_frac: float = 0.25):
    """One step's requests for the page-table write: distinct table rows,
    prefill spans (cached_len 0 or a chunk boundary, device_len up to the
    table width) and decode requests (one new token); a free list of page
    starts (multiples of page_size, shuffled) large enough for the step."""
    rng = np.random.default_rng(seed)
    table_idx = rng.permutation(table_rows)[:n_req].astype(np.int64)
    device_len = rng.integers(1, table_cols + 1, n_req).astype(np.int64)
    cached_len = device_len - 1
    pre = rng.random(n_req) < prefill_frac
    cached_len[pre] = np.maximum(device_len[pre] - rng.integers(1, 2049, int(pre.sum())), 0)
    num_pages = (table_rows * table_cols) // page_size
    free_slots = rng.permutation(num_pages).astype(np.int64) * page_size
    return table_idx, cached_len, device_len, free_slots

def with_min_p(w: Workload, values, seed: int = 0) -> Workload:
    """The same batch with a per-request min_p drawn from ``values``."""
    rng = np.random.default_rng([5000, seed])
    mp = rng.choice(np.asarray(values, dtype=np.float32), w.B).astype(np.float32)
    return replace(w, name=f"{w.name}+min_p", min_p=mp)