"""The whole configured decode loop at full size: 64 overlapped steps of c4
(B = 512, V = 152064 bf16; "The scheduler skeleton and the offline
interface", section "_forward" and its overlap loop), every row of every
step compared with the fp64 oracle -- token, kept length and Philox word.

The host work runs in a pool of spawned worker processes (they never touch
the GPU), as the bench's CPU baseline does: they generate each step's logits
(handed to the GPU process through shared memory, then freed) and afterwards
run the oracle on each step and compare it with the loop's outputs."""
import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor
from multiprocessing import shared_memory

import numpy as np
import pytest
import torch

import decode_step_token_amd as dst
import workloads as wl
from tests.parity import log

pytestmark = pytest.mark.gpu

STEPS = 64


def _make_logits(step):
    """Worker: the step's bf16 logits into a new shared-memory block."""
    x = wl.c4_logits(step)
    shm = shared_memory.SharedMemory(create=True, size=x.nbytes)
    np.ndarray(x.shape, dtype=x.dtype, buffer=shm.buf)[...] = x
    name = shm.name
    shm.close()
    return name, x.shape, x.dtype.str


def _check_step(task):
    """Worker: the oracle on every row of one step, compared with the loop's
    tokens / kept lengths / Philox words; returns (step, ambiguity counts)."""
    from tests.parity import compare, run_oracle
    step, tokens, kept, rand = task
    w = wl.c4(step)
    stats = compare(w, {"tokens": tokens, "kept_out": kept, "rand_out": rand}, run_oracle(w))
    return step, stats["draw_ambiguous"], stats["cutoff_ambiguous"]


@pytest.mark.timeout(900)
def test_c4_loop_all_steps_every_row():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    dst.load()
    w0 = wl.c4(0)
    B, V = w0.B, w0.V
    workers = max(1, min(len(os.sched_getaffinity(0)), 16))
    log(f"case c4 loop: {STEPS} steps, B={B} V={V}, {workers} host workers")
    ctx = multiprocessing.get_context("spawn")
    with ProcessPoolExecutor(workers, mp_context=ctx) as ex:
        futs = [ex.submit(_make_logits, st) for st in range(STEPS)]
        logits = []
        for st, f in enumerate(futs):
            name, shape, dt = f.result()
            shm = shared_memory.SharedMemory(name=name)
            try:
                host = np.ndarray(shape, dtype=np.dtype(dt), buffer=shm.buf)
                logits.append(torch.from_numpy(host.view(np.int16)).cuda().view(torch.bfloat16))
                torch.cuda.synchronize()
            finally:
                shm.close()
                shm.unlink()
            if st % 16 == 15:
                log(f"  logits of steps 0..{st} resident")

        dev = torch.device("cuda:0")
        pool = torch.from_numpy(w0.pool.copy()).to(dev)
        rows = torch.from_numpy(w0.rows).to(dev)
        pos0 = w0.meta["pos0"]
        out_pos = [torch.from_numpy(pos0 + st).to(dev) for st in range(STEPS)]
        blocks = [torch.empty(dst._binding.PREP_BYTES_PER_REQUEST * B, dtype=torch.uint8, device=dev)
                  for _ in range(2)]
        ring = [torch.full((B,), -7, dtype=torch.int32).pin_memory() for _ in range(2)]
        toks = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(STEPS)]
        kept = [torch.full((B,), -7, dtype=torch.int32, device=dev) for _ in range(STEPS)]
        rand = [torch.full((B,), -7, dtype=torch.int64, device=dev) for _ in range(STEPS)]
        host = []
        with dst.Sampler(0, B, V, "bf16", w0.seed) as s:
            prev = None
            for st in range(STEPS):
                args = s.prepare(B, w0.temperature, w0.top_k, w0.top_p, w0.uid, dev_block=blocks[st % 2])
                s.sample(logits[st], step=st, tokens_out=toks[st],
                         debug={"kept_out": kept[st], "rand_out": rand[st]}, **args)
                t = s.write(pool, rows, out_pos[st], toks[st], ring[st % 2])
                if prev is not None:
                    s.wait(prev)
                    host.append(ring[(st - 1) % 2].numpy().copy())
                prev = t
            s.wait(prev)
            host.append(ring[(STEPS - 1) % 2].numpy().copy())
            s.check()
        del logits
        tk = [x.cpu().numpy() for x in toks]
        kp = [x.cpu().numpy() for x in kept]
        rd = [x.cpu().numpy() for x in rand]
        for st in range(STEPS):
            assert np.array_equal(host[st], tk[st]), f"step {st}: host copy"
        log(f"  loop done; oracle on {STEPS} x {B} rows")
        amb_d = amb_c = 0
        for st, d, c in ex.map(_check_step, [(st, tk[st], kp[st], rd[st]) for st in range(STEPS)]):
            amb_d += d
            amb_c += c
            if st % 16 == 15:
                log(f"  steps 0..{st} match the oracle")
    log(f"  ok: {STEPS * B} rows, draw-ambiguous {amb_d}, cut-off-ambiguous {amb_c}")
