"""Two host threads drive the whole pass at once, each on its own stream with
its own buffers (the calls are reentrant: no state beyond a lock-guarded
per-kernel LDS limit and the device's CU count): every result equals the
single-threaded one -- counts and top-P exactly, Y within the bf16 parity
bar (the value sums are float atomics, added in any order)."""
import threading

import numpy as np
import pytest

import oracle
from adaptive_vector_quantized_amd import gen
from parity_util import say, to_device

pytestmark = pytest.mark.gpu


def _inputs(seed):
    import torch
    cfg = gen.CONFIGS["grid64"].replace(H=4, N=2048 + 64 + 5, grid=None, M0=100)
    data = gen.make(cfg, seed=seed, checker=oracle.MarginChecker())
    cb = torch.from_numpy(data["codebook"]).to(torch.bfloat16).contiguous().cuda()
    return cfg, {k: to_device(data[k], cfg.dtype, cfg.B, cfg.H) for k in ("Q", "K", "V")}, cb


def _pass(cfg, t, cb, stream, reps):
    import torch
    from adaptive_vector_quantized_amd import _lib
    with torch.cuda.stream(stream):
        for _ in range(reps):
            vsum, counts, _ = _lib.assign_aggregate(t["K"], t["V"], cb, cfg.C)
            Y, topp, _ = _lib.attention_fwd(t["Q"], cb, vsum, counts, cfg.C, cfg.P, cfg.block_q, cfg.scale,
                                           want_topp=True)
        stream.synchronize()
    return counts.cpu().numpy(), topp.cpu().numpy(), Y.cpu().numpy()


def test_two_threads_two_streams():
    import torch
    say("[threads] two host threads, two streams")
    jobs = [_inputs(seed) for seed in (71, 72)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    alone = [_pass(cfg, t, cb, streams[i], 1) for i, (cfg, t, cb) in enumerate(jobs)]
    out = [None, None]
    errs = []

    def run(i):
        try:
            cfg, t, cb = jobs[i]
            out[i] = _pass(cfg, t, cb, streams[i], 20)
        except Exception as e:  # surfaced below
            errs.append(e)
    th = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for x in th:
        x.start()
    for x in th:
        x.join()
    torch.cuda.synchronize()
    assert not errs, errs
    for i in range(2):
        c0, p0, y0 = alone[i]
        c1, p1, y1 = out[i]
        assert np.array_equal(c0, c1) and np.array_equal(p0, p1)
        err = np.abs(y1.astype(np.float64) - y0).max() / np.abs(y0).max()
        say(f"  job {i}: max|dY|/max|Y| between runs = {err:.2e}")
        # the value sums are float atomics in any order, and their fp16 operand
        # rounding can turn a last-bit difference into more: the bf16 parity bar
        assert err <= 2e-3
