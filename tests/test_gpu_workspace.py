"""The library's stream-ordered workspace on the GPU: each stream keeps a
cached buffer that later calls on it reuse without allocating or freeing,
so a call returns without waiting for the GPU; calls on different streams
(more of them than the cache holds) get results identical to one stream's."""
import time

import numpy as np
import pytest
import torch

import sliding_tile_attention_amd as sta
from tests.gpu_util import say
from tests.inputs import tensors

pytestmark = pytest.mark.gpu


def _inputs(grid, tile, H, D, seed):
    B, N = 1, int(np.prod(grid))
    q, k, v, do = (torch.from_numpy(x).to("cuda").to(torch.bfloat16)
                   for x in tensors(B, H, N, D, "bf16", seed, with_dout=True))
    return q, k, v, do


def _layer(q, k, v, do, geom, idx, stream):
    with torch.cuda.stream(stream):
        o, lse = sta.forward(q, k, v, geom, idx, stream=stream)
        dq, dk, dv = sta.backward(q, k, v, o, lse, do, geom, idx, stream=stream)
    return o, lse, dq, dk, dv


def test_streams_get_identical_results_growing_and_evicted():
    """Forward + backward of several inputs on one stream, then the same on
    4 concurrent streams (first a small and then a larger geometry, so each
    stream's buffer grows), then on 18 streams one after another (more than
    the 16 cached per device, so slots are evicted): every output identical."""
    cases = [((4, 16, 24), (2, 8, 8), [(3, 3, 3), (1, 3, 3)]), ((8, 16, 24), (2, 8, 8), [(3, 3, 5), (3, 3, 3)])]
    main = torch.cuda.current_stream()
    for grid, tile, windows in cases:
        geom = sta.Geometry(grid, tile)
        idx = sta.StaIndex(geom, windows)
        ins = [_inputs(grid, tile, 2, 64, 300 + i) for i in range(4)]
        ref = [_layer(*x, geom, idx, main) for x in ins]
        torch.cuda.synchronize()
        say("workspace: %s on 4 concurrent streams" % (grid,))
        streams = [torch.cuda.Stream() for _ in ins]
        for s in streams:
            s.wait_stream(main)
        got = [_layer(*x, geom, idx, s) for x, s in zip(ins, streams)]
        torch.cuda.synchronize()
        for r, g in zip(ref, got):
            for a, b in zip(r, g):
                assert torch.equal(a, b)
    say("workspace: 18 streams in turn")
    grid, tile, windows = cases[0]
    geom = sta.Geometry(grid, tile)
    idx = sta.StaIndex(geom, windows)
    x = _inputs(grid, tile, 2, 64, 310)
    ref = _layer(*x, geom, idx, main)
    torch.cuda.synchronize()
    for _ in range(18):
        s = torch.cuda.Stream()
        s.wait_stream(main)
        got = _layer(*x, geom, idx, s)
        main.wait_stream(s)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)
    torch.cuda.synchronize()


def test_calls_return_before_the_gpu_finishes():
    """Four forwards of the 720p grid with 4 heads (a few ms of GPU work
    each) are enqueued in a small fraction of the time the GPU takes for
    them: no call waits for an earlier one (a free per call would)."""
    grid, tile = (30, 48, 80), (6, 8, 8)
    geom = sta.Geometry(grid, tile)
    idx = sta.StaIndex(geom, [(3, 3, 5)] * 4)
    q, k, v, _ = _inputs(grid, tile, 4, 128, 320)
    for _ in range(2):
        sta.forward(q, k, v, geom, idx)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(4):
        sta.forward(q, k, v, geom, idx)
    t1 = time.perf_counter()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    say("workspace: enqueue %.2f ms, GPU done after %.2f ms" % ((t1 - t0) * 1e3, (t2 - t0) * 1e3))
    assert t1 - t0 < 0.3 * (t2 - t0)


def test_threads_on_streams_and_one_shared_stream():
    """Four host threads, each calling forward + backward ten times on a
    stream of its own, then on one shared stream (a buffer in use by one
    thread's call sends the other to pool memory): every result identical to
    the single-thread reference."""
    import threading
    grid, tile, windows = (4, 16, 24), (2, 8, 8), [(3, 3, 3), (1, 3, 3)]
    geom = sta.Geometry(grid, tile)
    idx = sta.StaIndex(geom, windows)
    main = torch.cuda.current_stream()
    ins = [_inputs(grid, tile, 2, 64, 330 + i) for i in range(4)]
    ref = [_layer(*x, geom, idx, main) for x in ins]
    torch.cuda.synchronize()
    shared = torch.cuda.Stream()
    for label, streams in (("own streams", [torch.cuda.Stream() for _ in ins]), ("one stream", [shared] * 4)):
        say("workspace: 4 threads, %s" % label)
        for s in set(streams):
            s.wait_stream(main)
        errors = []

        def work(t):
            try:
                torch.cuda.set_device(0)
                for _ in range(10):
                    got = _layer(*ins[t], geom, idx, streams[t])
                    streams[t].synchronize()
                    if not all(torch.equal(a, b) for a, b in zip(got, ref[t])):
                        errors.append("thread %d differs" % t)
                        return
            except Exception as e:                      # reported below
                errors.append("thread %d: %r" % (t, e))

        threads = [threading.Thread(target=work, args=(t,)) for t in range(4)]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        torch.cuda.synchronize()
        assert not errors, errors
