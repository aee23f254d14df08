"""The boundary's promises on the GPU: no call allocates device memory, the
first call of a process can be captured into a HIP graph, and calls that
overlap in time are independent when each has its own workspace."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import gemm_q4_amd as q4
import oracle
import synth
from gpu_util import DEV, TOL_GEMM, TOL_SMALL_N, packed_from_blocks, to_dev

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def test_first_call_of_a_process_captures_into_a_graph():
    """In a fresh process, the first library calls (repacks, decode with the
    activation pre-pass, decode with a split K range, prefill, the head's
    greedy pick) are made inside a graph capture; every replay equals the
    eager calls made afterwards, bit for bit."""
    print("cold capture in a child process", flush=True)
    r = subprocess.run([sys.executable, os.path.join(HERE, "cold_capture.py")],
                       capture_output=True, text=True, timeout=300)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0
    res = json.loads(r.stdout.strip().splitlines()[-1])
    assert res and all(res.values()), res


def test_calls_allocate_no_device_memory():
    """Free device memory is the same before and after a run of calls of
    every compute entry point with caller-owned buffers (after one warm-up
    round that loads the kernels' code)."""
    shapes = [(8, 9728, 2560, np.float32), (1, 9728, 2560, np.float32),
              (4, 2560, 9728, np.float32), (512, 2560, 9728, np.float16)]
    calls = []
    for i, (n, out, in_, dt) in enumerate(shapes):
        blk = synth.make_blocks(out, in_, seed=i)
        p = packed_from_blocks(blk, out, in_)
        x = to_dev(synth.make_x(n, in_, seed=i, dtype=dt))
        y = torch.empty((n, out), device=DEV)
        need = q4.q4_0_matmul_workspace_size(n, out, in_, q4.dtype_code(x))
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
        calls.append(lambda p=p, x=x, y=y, n=n, out=out, in_=in_, ws=ws, need=need:
                     q4.q4_0_matmul(p, x, q4.dtype_code(x), y, n, out, in_, ws, need))
    # grouped, greedy pick, routed, W4A8
    hp = packed_from_blocks(synth.make_blocks(4096, 2560, seed=9), 4096, 2560)
    kp = packed_from_blocks(synth.make_blocks(1024, 2560, seed=10), 1024, 2560)
    x8 = to_dev(synth.make_x(8, 2560, seed=11))
    yq, yk = torch.empty((8, 4096), device=DEV), torch.empty((8, 1024), device=DEV)
    lins = [(hp, x8, yq, 4096, 2560), (kp, x8, yk, 1024, 2560)]
    gneed = q4.q4_0_grouped_workspace_size(lins, q4.F32, 8)
    gws = torch.empty(max(gneed, 256), dtype=torch.uint8, device=DEV)
    calls.append(lambda: q4.q4_0_matmul_grouped(lins, q4.F32, 8, gws, gneed))
    mv, mi = torch.empty(8, device=DEV), torch.empty(8, dtype=torch.int32, device=DEV)
    aneed = q4.q4_0_argmax_workspace_size(8, 4096, 2560)
    aws = torch.empty(aneed, dtype=torch.uint8, device=DEV)
    calls.append(lambda: q4.q4_0_matmul_argmax(hp, x8, q4.F32, None, 8, 4096, 2560, mv, mi,
                                               aws, aneed))
    n_exp, out, in_ = 4, 300, 2560
    stack = torch.cat([packed_from_blocks(synth.make_blocks(out, in_, seed=20 + e), out, in_)
                       for e in range(n_exp)])
    route = to_dev(np.array([[0, 3], [2, 1], [1, 1]], dtype=np.int32))
    x3 = to_dev(synth.make_x(3, in_, seed=21))
    yr = torch.empty((6, out), device=DEV)
    for rk in (q4.ROUTE_BY_COLUMN, q4.ROUTE_BY_EXPERT):
        rneed = q4.q4_0_routed_workspace_size(3, 2, n_exp, out, in_, rk)
        rws = torch.empty(max(rneed, 256), dtype=torch.uint8, device=DEV)
        calls.append(lambda rk=rk, rws=rws, rneed=rneed: q4.q4_0_matmul_routed_ex(
            stack, n_exp, x3, q4.F32, route, 2, yr, 3, out, in_, rk, rws, rneed))
    q8, d8 = q4.quantize_x8(x8)
    wneed = q4.q4_0_w4a8_workspace_size(8, 4096, 2560)
    wws = torch.empty(max(wneed, 256), dtype=torch.uint8, device=DEV)
    calls.append(lambda: q4.q4_0_matmul_w4a8(hp, q8, d8, yq, 8, 4096, 2560, wws, wneed))
    for c in calls:                                  # warm-up: code objects load
        c()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(5):
        for c in calls:
            c()
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    assert free1 == free0, (free0, free1)


def test_graphs_captured_on_one_stream_replay_concurrently():
    """Two graphs captured one after the other on the same stream, each call
    with its own workspace, replayed at the same time on two streams (with
    the split-K decode and the activation pre-pass, which use the
    workspace): each replay gives its own eager result."""
    cases = []
    for i, (n, out, in_) in enumerate([(4, 2560, 9728), (20, 9728, 2560)]):
        blk = synth.make_blocks(out, in_, seed=60 + i)
        p = packed_from_blocks(blk, out, in_)
        x = to_dev(synth.make_x(n, in_, seed=61 + i))
        ref = q4.matmul(p, x, out)
        y = torch.empty((n, out), device=DEV)
        need = q4.q4_0_matmul_workspace_size(n, out, in_)
        assert need > 0
        ws = torch.empty(need, dtype=torch.uint8, device=DEV)
        cases.append((p, x, y, n, out, in_, ws, need, ref))
    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    graphs = []
    for p, x, y, n, out, in_, ws, need, _ in cases:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            for _ in range(4):
                q4.q4_0_matmul(p, x, q4.F32, y, n, out, in_, ws, need, cs)
        graphs.append(g)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(5):
        for c in cases:
            c[2].fill_(float("nan"))
        torch.cuda.synchronize()
        sa.wait_stream(torch.cuda.current_stream())
        sb.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(sa):
            graphs[0].replay()
        with torch.cuda.stream(sb):
            graphs[1].replay()
        torch.cuda.synchronize()
        for i, c in enumerate(cases):
            assert torch.equal(c[2], c[8]), (rep, i)


def test_workspace_contents_on_entry_do_not_matter():
    """A workspace full of NaN bits, or left over from another call, gives
    the same result as a fresh one (nothing is read before it is written)."""
    out, in_, n = 2560, 9728, 6
    blk = synth.make_blocks(out, in_, seed=70)
    p = packed_from_blocks(blk, out, in_)
    x = to_dev(synth.make_x(n, in_, seed=71))
    need = q4.q4_0_matmul_workspace_size(n, out, in_)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y0 = torch.empty((n, out), device=DEV)
    ws.fill_(0xFF)
    q4.q4_0_matmul(p, x, q4.F32, y0, n, out, in_, ws, need)
    y1 = torch.empty((n, out), device=DEV)
    q4.q4_0_matmul(p, x, q4.F32, y1, n, out, in_, ws, need)     # leftover contents
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    y_ref, den = oracle.matmul(blk, x.cpu().numpy(), out, in_)
    assert oracle.max_ratio(y0.cpu().numpy(), y_ref, den) <= TOL_SMALL_N


def test_stream_read_aid_reads_every_byte():
    """The streaming-read measurement aid: the XOR of every workgroup's
    checksum equals the XOR of the buffer's 32-bit words (each word read
    once), and an empty launch writes zeros."""
    nbytes = 16 * 1000 * 37
    rng = np.random.default_rng(3)
    words = rng.integers(0, 2 ** 23, size=nbytes // 4, dtype=np.uint32)
    src = to_dev(words.view(np.uint8))
    for wgs in (1, 7, 256, 1024):
        sink = torch.full((wgs,), float("nan"), device=DEV)
        q4.q4_0_stream_read(src, nbytes, sink, wgs)
        torch.cuda.synchronize()
        got = 0
        for v in sink.cpu().numpy().astype(np.uint32).tolist():
            got ^= v
        want = int(np.bitwise_xor.reduce(words)) & 0x7FFFFF
        assert got == want, wgs
    sink = torch.full((64,), float("nan"), device=DEV)
    q4.q4_0_stream_read(None, 0, sink, 64)
    torch.cuda.synchronize()
    assert torch.equal(sink, torch.zeros_like(sink))


@pytest.mark.parametrize("n,out,in_,dt", [(8, 1024, 2560, np.float32),
                                           (512, 2560, 9728, np.float16)])
def test_workspace_of_the_maximum_size_serves_any_call(n, out, in_, dt):
    """One Q4_0_WORKSPACE_MAX buffer passed with its full size serves calls
    that need less."""
    blk = synth.make_blocks(out, in_, seed=80)
    p = packed_from_blocks(blk, out, in_)
    x = synth.make_x(n, in_, seed=81, dtype=dt)
    ws = torch.empty(q4.WORKSPACE_MAX, dtype=torch.uint8, device=DEV)
    y = torch.empty((n, out), device=DEV)
    q4.q4_0_matmul(p, to_dev(x), q4.dtype_code(to_dev(x)), y, n, out, in_, ws)
    torch.cuda.synchronize()
    y_ref, den = oracle.matmul(blk, x, out, in_)
    tol = TOL_GEMM if n > 8 else TOL_SMALL_N
    assert oracle.max_ratio(y.cpu().numpy(), y_ref, den) <= tol
