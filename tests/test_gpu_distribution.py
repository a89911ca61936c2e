"""The draw's distribution ("The engine and the sampler", section "Tests": the
sampled frequencies follow the filtered distribution): more than 10^5 draws
per case, from rows that repeat one logits vector under distinct request ids
and advancing step counters, so every draw has its own Philox uniform.  The
counts are compared with the oracle's final distribution r by a chi-square
test (categories with fewer than 5 expected draws pooled).

Cases: a V = 1024 row with top-k 50 and top-p 0.9 (the listed route), a
V = 1024 row with top-p 0.99 alone (a nucleus of hundreds of tokens, drawn
from per-tile kept weights), and a flat top-p row at V = 151936, T = 1.5,
N(0, 2.5) logits, whose nucleus holds tens of thousands of tokens; there the tokens are pooled
into 200 runs of consecutive ids of about equal expected mass, since the
draw walks the kept mass in id order.  Each case runs on both row kernels."""
import numpy as np
import pytest
import scipy.stats
import torch

import decode_step_token_amd as dst
import oracle
from tests.parity import log

pytestmark = pytest.mark.gpu

P_MIN = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    dst.load()
    yield
    torch.cuda.synchronize()


def _draw_counts(x, T, k, p, B, steps, path):
    """Token counts of B * steps draws from one row x (float32 [V])."""
    V = x.shape[0]
    dev = torch.device("cuda:0")
    logits = torch.from_numpy(np.ascontiguousarray(np.tile(x, (B, 1)))).to(dev)
    temp = torch.full((B,), T, dtype=torch.float32, device=dev)
    topk = None if k is None else torch.full((B,), k, dtype=torch.int32, device=dev)
    topp = torch.full((B,), p, dtype=torch.float32, device=dev)
    uid = torch.arange(B, dtype=torch.int64, device=dev) * 7919 + 11
    s = dst.Sampler(0, B, V, "f32", 4242)
    toks = torch.empty((steps, B), dtype=torch.int32, device=dev)
    try:
        for st in range(steps):
            s.sample(logits, temperature=temp, top_k=topk, top_p=topp, uid=uid, step=1000 + st,
                     tokens_out=toks[st], debug={f"force_{path}": True})
        torch.cuda.synchronize()
        s.check()
    finally:
        s.close()
    return np.bincount(toks.cpu().numpy().ravel(), minlength=V)


def _oracle_r(x, T, k, p):
    V = x.shape[0]
    prm = oracle.row_params(V, T, -1 if k is None else k, p)
    return oracle.sample_row(x.astype(np.float64), prm, 0.5, want_alternatives=False).r


def _chi2(counts, expected_prob, groups=None):
    n = counts.sum()
    if groups is not None:
        counts = np.add.reduceat(counts, groups)
        expected_prob = np.add.reduceat(expected_prob, groups)
    exp = expected_prob * n
    big = exp >= 5
    obs = np.append(counts[big], counts[~big].sum())
    e = np.append(exp[big], exp[~big].sum())
    keep = e > 0
    stat, pval = scipy.stats.chisquare(obs[keep], e[keep] * obs[keep].sum() / e[keep].sum())
    return stat, pval, int(keep.sum())


@pytest.mark.parametrize("path", ["stream", "split"])
@pytest.mark.parametrize("k,p", [(50, 0.9), (None, 0.99)])
def test_small_row(path, k, p):
    x = np.random.default_rng(15).normal(0, 2, 1024).astype(np.float32)
    log(f"case chi-square V=1024 k={k} p={p} path={path}")
    counts = _draw_counts(x, 1.0, k, p, 4096, 25, path)
    r = _oracle_r(x, 1.0, k, p)
    assert counts[r == 0].sum() == 0, "a token outside the kept set was drawn"
    stat, pval, cats = _chi2(counts, r)
    log(f"  {counts.sum()} draws, support {int((r > 0).sum())}, chi2={stat:.1f} over {cats} categories, p={pval:.3g}")
    assert pval > P_MIN


@pytest.mark.parametrize("path", ["stream", "split"])
def test_flat_row(path):
    x = (np.random.default_rng(16).standard_normal(151936) * 2.5).astype(np.float32)
    log(f"case chi-square flat V=151936 T=1.5 p=0.95 path={path}")
    counts = _draw_counts(x, 1.5, None, 0.95, 256, 400, path)
    r = _oracle_r(x, 1.5, None, 0.95)
    assert counts[r == 0].sum() == 0, "a token outside the kept set was drawn"
    # runs of consecutive ids of about equal expected mass
    cum = np.cumsum(r)
    groups = np.unique(np.searchsorted(cum, np.linspace(0.0, cum[-1], 201)[:-1], side="right"))
    stat, pval, cats = _chi2(counts, r, groups)
    log(f"  {counts.sum()} draws, support {int((r > 0).sum())}, chi2={stat:.1f} over {cats} runs, p={pval:.3g}")
    assert pval > P_MIN
