"""Calls on separate streams at once give the results of one stream.

The library keeps no state between calls, so calls on different streams
whose outputs and workspaces are disjoint may overlap on the device. Two
rounds of different workloads (a uniform and a ragged batch, each with its
own bounds, outputs and workspaces) run concurrently:
- on two streams from one host thread;
- from two host threads, each with its own stream. The binding's ctypes calls
  release the GIL, so both threads are inside the library at once.
Every output equals the same round run alone, bit for bit.
"""
import threading

import pytest
import torch

from tests.test_gpu_graph_replay import Round, _same, _workload

pytestmark = pytest.mark.gpu


def _rounds():
    rounds = [Round(_workload(False)), Round(_workload(True))]
    refs = []
    for r in rounds:
        r.per_step()
        torch.cuda.synchronize()
        refs.append([t.clone() for t in r.outputs()])
    return rounds, refs


def _scramble(r):
    for t in r.outputs()[:-1]:  # outputs (not the bounds) start from garbage
        t.fill_(-3 if t.dtype == torch.int32 else 7.0)


def _check(rounds, refs, tag):
    for j, (r, ref) in enumerate(zip(rounds, refs)):
        for i, (a, b) in enumerate(zip(r.outputs(), ref)):
            assert _same(a, b), (tag, j, i)


def test_two_streams_one_thread():
    print("two rounds on two streams, one thread", flush=True)
    rounds, refs = _rounds()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for r in rounds:
            _scramble(r)
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        # interleave the two rounds' launches so that their kernels overlap
        for j in range(rounds[0].g):
            for r, s in zip(rounds, streams):
                with torch.cuda.stream(s):
                    r.step(j)
        for r, s in zip(rounds, streams):
            with torch.cuda.stream(s):
                r.verify_and_sample()
        torch.cuda.synchronize()
        _check(rounds, refs, rep)


def test_two_threads_two_streams():
    print("two rounds from two host threads, a stream each", flush=True)
    rounds, refs = _rounds()
    errors = []
    start = threading.Barrier(2)

    def worker(r, dev):
        try:
            torch.cuda.set_device(dev)
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                for _ in range(3):
                    r.per_step()
            s.synchronize()
        except BaseException as e:  # reported by the main thread
            errors.append(e)

    for r in rounds:
        _scramble(r)
    torch.cuda.synchronize()
    dev = torch.cuda.current_device()
    threads = [threading.Thread(target=worker, args=(r, dev)) for r in rounds]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    _check(rounds, refs, "threads")


def test_explicit_stream_argument_keeps_internal_buffers():
    """Calls given stream=<a side stream>, with no workspace or outputs passed
    in, allocate them on the current stream. The binding records them on the
    side stream too, so memory the current stream allocates and fills while
    the side stream's kernels still run never lands in them."""
    import numpy as np

    import oracle
    import self_sparse_speculative_paged_amd as s3r
    from tests.parity import check_tokens

    print("stream= side stream with internal workspaces", flush=True)
    g = torch.Generator().manual_seed(17)
    B, gamma, V = 32, 6, 151936
    d = torch.randn((B, gamma, V), generator=g) * 2.0
    t = torch.cat([d + torch.randn((B, gamma, V), generator=g) * 0.5,
                   torch.randn((B, 1, V), generator=g) * 2.0], dim=1)
    x = torch.from_numpy(oracle.draw_draft_tokens(d.double().numpy(), 1.0, seed=1, offset=0))
    dd, td, xd = d.cuda(), t.cuda(), x.cuda().int()
    ref_out, ref_n = s3r.spec_sample(dd, td, xd, 1.0, 0, 3)
    ref_draw = s3r.draft_sample(dd, 1.0, 5, 0)
    ref_alpha = s3r.acceptance_rate(dd, td, 1.0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    big = torch.randn((4096, 4096), device="cuda")
    with torch.cuda.stream(side):
        for _ in range(30):  # keep the side stream busy so the calls below queue behind it
            big = big @ big * 1e-3
    out, n = s3r.spec_sample(dd, td, xd, 1.0, 0, 3, stream=side)
    draw = s3r.draft_sample(dd, 1.0, 5, 0, stream=side)
    alpha = s3r.acceptance_rate(dd, td, 1.0, stream=side)
    junk = [torch.full((1 << 18,), 7, dtype=torch.float32, device="cuda") for _ in range(64)]
    junk += [torch.full((1 << 16,), -1, dtype=torch.int32, device="cuda") for _ in range(64)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out, ref_out) and torch.equal(n, ref_n)
    assert torch.equal(draw, ref_draw) and torch.equal(alpha, ref_alpha)
    ro, rn, dec = oracle.spec_sample(d.double().numpy(), t.double().numpy(), x.numpy(), 1.0, 0, 3)
    assert check_tokens(out.cpu().numpy(), n.cpu().numpy(), ro, rn, dec) >= B // 2
    assert np.max(np.abs(alpha.cpu().numpy() - oracle.acceptance_rate(d.double().numpy(), t.double().numpy(),
                                                                       1.0))) <= 5e-6
