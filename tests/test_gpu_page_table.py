"""write_page_table (the cache manager's paged allocation write), through the
C ABI: the page table equals the oracle's ``_write_page_table`` bit for bit,
on the pages' own allocation test and on random prefill/decode batches."""
import ctypes

import numpy as np
import pytest
import torch

import decode_step_token_amd as dst
import oracle
import workloads as wl
from tests.parity import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    dst.load()
    yield
    torch.cuda.synchronize()


def _step(s, pool, table_np, table_dev, tidx, cached, dev_len):
    """One allocate_paged: pages from the oracle's free list, written by the
    library on the device and by the oracle on the host."""
    want, starts = pool.allocate_paged(table_np, tidx, cached, dev_len)
    ps_dev = torch.from_numpy(starts.astype(np.int32)).cuda() if len(starts) else None
    s.write_page_table(table_dev, np.asarray(tidx, np.int64), np.asarray(cached, np.int64),
                       np.asarray(dev_len, np.int64), ps_dev, pool.page_size)
    return want


def test_pages_allocation_test():
    log("case page table: the pages' allocation test")
    pool = oracle.PagePool(num_pages=8, page_size=4)
    table = np.full((4, 32), -1, dtype=np.int32)
    with dst.Sampler(0, 4, 8) as s:
        dev = torch.from_numpy(table.copy()).cuda()
        table = _step(s, pool, table, dev, [2], [0], [6])
        got = dev.cpu().numpy()
        assert got[2, :8].tolist() == [0, 1, 2, 3, 4, 5, 6, 7] and len(pool.free_slots) == 6
        table = _step(s, pool, table, dev, [2], [6], [7])
        assert len(pool.free_slots) == 6
        table = _step(s, pool, table, dev, [2], [8], [9])
        got = dev.cpu().numpy()
        s.check()
        assert len(pool.free_slots) == 5 and got[2, 8] % 4 == 0
        assert np.array_equal(got, table)


@pytest.mark.parametrize("ps", [1, 4, 16])
def test_random_prefill_and_decode_batches(ps):
    tidx, cached, dev_len, free = wl.paged_batch(40 + ps, page_size=ps)
    log(f"case page table random batch ps={ps} requests={len(tidx)}")
    table0 = np.random.default_rng(ps).integers(-100, -1, (512, 4096)).astype(np.int32)
    info, needed = oracle.paged_info(tidx, cached, dev_len, ps)
    starts = free[:needed]
    want, bad = oracle.write_page_table(table0, oracle.page_to_token(starts, ps), info, ps)
    assert not bad
    with dst.Sampler(0, len(tidx), 8) as s:
        dev = torch.from_numpy(table0.copy()).cuda()
        s.write_page_table(dev, tidx, cached, dev_len,
                           torch.from_numpy(starts.astype(np.int32)).cuda(), ps)
        s.check()
        assert np.array_equal(dev.cpu().numpy(), want)


@pytest.mark.parametrize("ps", [1, 16])
def test_decode_steps(ps):
    """64 decode steps of 512 requests: a new page for a request every
    page_size steps, written while the rows fill up."""
    B, steps = 512, 64
    rng = np.random.default_rng(7)
    tidx = rng.permutation(B).astype(np.int64)
    dlen = rng.integers(1, 2049, B).astype(np.int64)
    pool = oracle.PagePool(num_pages=(B * 4096) // ps, page_size=ps)
    table = np.full((B, 4096), -1, dtype=np.int32)
    log(f"case page table decode steps ps={ps}")
    with dst.Sampler(0, B, 8) as s:
        dev = torch.from_numpy(table.copy()).cuda()
        table = _step(s, pool, table, dev, tidx, np.zeros(B, np.int64), dlen)   # prefill
        for _ in range(steps):
            table = _step(s, pool, table, dev, tidx, dlen, dlen + 1)
            dlen = dlen + 1
        s.check()
        assert np.array_equal(dev.cpu().numpy(), table)


def test_errors_and_empty():
    log("case page table errors")
    with dst.Sampler(0, 4, 8) as s:
        dev = torch.full((4, 32), -1, dtype=torch.int32, device="cuda")
        starts = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
        one = lambda *v: np.array(v, dtype=np.int64)
        for args in [
            (one(1), one(0), one(12), starts, 4),        # needs 3 pages, 2 given
            (one(4), one(0), one(8), starts, 4),         # row outside the table
            (one(1), one(24), one(36), starts, 4),       # pages past the last column
            (one(1), one(-4), one(8), starts, 4),        # negative length
            (one(1), one(0), one(8), starts, 0),         # page size 0
        ]:
            with pytest.raises(dst.SamplerError) as e:
                s.write_page_table(dev, *args)
            assert e.value.code == -1
        with pytest.raises(dst.SamplerError):                      # n_req > max_batch
            s.write_page_table(dev, one(0, 1, 2, 3, 0), one(0, 0, 0, 0, 0), one(1, 1, 1, 1, 1),
                               torch.zeros(5, dtype=torch.int32, device="cuda"), 1)
        # no new page: nothing enqueued, table unchanged
        s.write_page_table(dev, one(1, 2), one(5, 7), one(5, 8), None, 4)
        s.check()
        assert torch.all(dev == -1)


def test_staging_rotation_under_load():
    n = 3 * dst._binding.PREP_SLOTS
    log(f"case page table staging rotation, {n} calls")
    ps = 4
    pool = oracle.PagePool(num_pages=4096, page_size=ps)
    table = np.full((64, 256), -1, dtype=np.int32)
    rng = np.random.default_rng(3)
    calls = []
    for i in range(n):
        tidx = rng.permutation(64)[:16].astype(np.int64)
        d = rng.integers(1, 257, 16).astype(np.int64)
        c = np.maximum(d - rng.integers(1, 40, 16), 0)
        table, starts = pool.allocate_paged(table, tidx, c, d)
        calls.append((tidx, c, d, starts))
    with dst.Sampler(0, 16, 8) as s:
        dev = torch.full((64, 256), -1, dtype=torch.int32, device="cuda")
        starts_dev = [torch.from_numpy(st.astype(np.int32)).cuda() for *_, st in calls]
        torch.cuda._sleep(int(2e6))            # keep the stream busy while calls pile up
        for (tidx, c, d, _), sd in zip(calls, starts_dev):
            s.write_page_table(dev, tidx, c, d, sd if sd.numel() else None, ps)
        torch.cuda.synchronize()
        s.check()
        assert np.array_equal(dev.cpu().numpy(), table)
