"""Helpers that run a workload through the HIP library and compare it with the
oracle under the acceptance rules:

* greedy rows, argmax rows (top_k = 1) and top-k index lists: bit-exact;
* the Philox word of each row: bit-exact;
* token pool and host copy: bit-exact;
* kept-prefix length: equal, or (only when the oracle flags the top-p cut-off
  as within 1e-6 of p) one of the neighbouring lengths;
* sampled token: equal, unless u lies within 1e-5 of a CDF boundary, then one
  of the oracle's acceptable tokens for that kept length;
* final probabilities: max |diff| <= 1e-6 over the row.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import decode_step_token_amd as dst
import oracle
from workloads import Workload

PROB_TOL = 1e-6
M64 = (1 << 64) - 1


def log(msg: str) -> None:
    print(f"[parity {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def to_device_logits(w: Workload, pad: int = 0) -> torch.Tensor:
    a = w.logits.view(np.int16) if w.dtype == "bf16" else w.logits
    t = torch.from_numpy(np.ascontiguousarray(a))
    if pad:
        t = torch.nn.functional.pad(t, (0, pad))
    return t.cuda()


def opt(a, dtype):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dtype).cuda()


def run_gpu(w: Workload, sampler: dst.Sampler = None, debug: bool = True, pad: int = 0,
            host: bool = True, logits_dev: torch.Tensor = None, force_exact: bool = False,
            path: str = None):
    """Run sample_batch + write_tokens for one step; returns numpy results.
    ``path``: None (the library's choice), "exact", "stream" or "split"."""
    if force_exact:
        path = "exact"
    own = sampler is None
    if own:
        sampler = dst.Sampler(0, max(w.B, 1), w.V, w.dtype, w.seed)
    try:
        B, V = w.B, w.V
        logits = to_device_logits(w, pad) if logits_dev is None else logits_dev
        T = opt(w.temperature, torch.float32)
        k = opt(w.top_k, torch.int32)
        p = opt(w.top_p, torch.float32)
        uid = opt(w.uid, torch.int64)
        dbg = None
        if debug:
            dbg = {"probs_out": torch.full((B, V), -1.0, dtype=torch.float32, device="cuda"),
                   "kept_out": torch.full((B,), -7, dtype=torch.int32, device="cuda"),
                   "topk_idx_out": torch.full((B, 64), -7, dtype=torch.int32, device="cuda"),
                   "rand_out": torch.full((B,), -7, dtype=torch.int64, device="cuda")}
        if path is not None:
            assert path in ("exact", "stream", "split"), path
            dbg = dict(dbg or {}, **{f"force_{path}": True})
        toks = sampler.sample(logits, temperature=T, top_k=k, top_p=p, uid=uid, step=w.step,
                              debug=dbg, min_p=opt(w.min_p, torch.float32))
        pool = torch.from_numpy(w.pool.copy()).cuda()
        rows = opt(w.rows, torch.int64)
        cols = opt(w.cols, torch.int64)
        host_out = torch.full((B,), -7, dtype=torch.int32).pin_memory() if host else None
        ticket = sampler.write(pool, rows, cols, toks, host_out)
        sampler.wait(ticket)
        out = {"tokens": toks.cpu().numpy(), "pool": pool.cpu().numpy(),
               "host": None if host_out is None else host_out.numpy().copy()}
        if dbg:
            for name, t in dbg.items():
                if isinstance(t, torch.Tensor):
                    out[name] = t.cpu().numpy()
        return out
    finally:
        if own:
            sampler.close()


def run_oracle(w: Workload, rows=None):
    return oracle.sample_batch(w.logits, w.dtype, w.temperature, w.top_k, w.top_p, w.uid,
                               w.step, w.seed, rows=rows, min_p=w.min_p)


def compare(w: Workload, gpu: dict, ref, rows=None, check_probs_rows=None) -> dict:
    """Assert the acceptance rules; returns a small summary of ambiguous rows."""
    rows = list(range(w.B)) if rows is None else list(rows)
    stats = {"draw_ambiguous": 0, "cutoff_ambiguous": 0, "rows": len(rows)}
    for res, b in zip(ref, rows):
        tok = int(gpu["tokens"][b])
        where = f"{w.name} row {b}"
        if "rand_out" in gpu and w.temperature is not None:
            assert (int(gpu["rand_out"][b]) & M64) == res.word0, f"{where}: Philox word"
        if res.greedy or res.params.k == 1:
            assert tok == res.token, f"{where}: argmax {tok} != {res.token}"
            if "kept_out" in gpu:
                assert gpu["kept_out"][b] == 1, where
            if "topk_idx_out" in gpu:
                assert gpu["topk_idx_out"][b][0] == res.token and np.all(gpu["topk_idx_out"][b][1:] == -1)
        else:
            if "topk_idx_out" in gpu:
                want = np.full(64, -1)
                want[:len(res.order_prefix)] = res.order_prefix
                assert np.array_equal(gpu["topk_idx_out"][b], want), f"{where}: top-k index list"
            kept = int(gpu["kept_out"][b]) if "kept_out" in gpu else res.kept
            if kept == res.kept:
                r, acceptable = res.r, res.acceptable
                exact = not res.draw_ambiguous
                want_tok = res.token
            else:
                assert res.cutoff_ambiguous and kept in res.alt_r, \
                    f"{where}: kept {kept} != {res.kept} (cut-off ambiguous: {res.cutoff_ambiguous})"
                r, acceptable, exact, want_tok = res.alt_r[kept], res.alt_acceptable[kept], False, None
            stats["cutoff_ambiguous"] += res.cutoff_ambiguous
            stats["draw_ambiguous"] += res.draw_ambiguous
            if exact:
                assert tok == want_tok, f"{where}: token {tok} != {want_tok} (u={res.u})"
            else:
                assert tok in acceptable, f"{where}: token {tok} not in {acceptable[:10]}"
            assert r[tok] > 0, f"{where}: token outside the kept set"
        if "probs_out" in gpu and (check_probs_rows is None or b in check_probs_rows):
            kept = int(gpu["kept_out"][b]) if "kept_out" in gpu else res.kept
            r = res.r if (kept == res.kept or res.greedy) else res.alt_r[kept]
            err = np.abs(gpu["probs_out"][b].astype(np.float64) - r).max()
            assert err <= PROB_TOL, f"{where}: probs max err {err}"
    # the write-back is compared bit-exactly with the oracle's scatter of the
    # same tokens (callers that check the pool themselves pass none)
    if "pool" in gpu:
        want_pool, want_host, bad = oracle.write_tokens(w.pool, w.rows, w.cols, gpu["tokens"])
        assert np.array_equal(gpu["pool"], want_pool), f"{w.name}: token pool"
    if gpu.get("host") is not None:
        assert np.array_equal(gpu["host"], gpu["tokens"]), f"{w.name}: host copy"
    return stats
