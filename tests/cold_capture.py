"""Run by tests/test_gpu_boundary.py in a fresh process: the first library
calls of the process are made inside a HIP graph capture (no call before it,
on any stream), then the graph is replayed and compared with eager calls
made afterwards.  Prints one JSON line with the outcome of each case."""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import gemm_q4_amd as q4  # noqa: E402
import synth  # noqa: E402


def main():
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cases = [  # (name, n, out, in, x dtype): pre-pass, split K + reduction, prefill
        ("decode_n20_prepass", 20, 9728, 2560, np.float32),
        ("decode_n4_ksplit", 4, 2560, 9728, np.float32),
        ("prefill_512", 512, 2560, 9728, np.float16),
    ]
    bufs = []
    for i, (name, n, out, in_, dt) in enumerate(cases):
        blk = torch.from_numpy(synth.make_blocks(out, in_, seed=20 + i).reshape(-1)).to(dev)
        packed = torch.empty(q4.q4_0_packed_bytes(out, in_), dtype=torch.uint8, device=dev)
        x = torch.from_numpy(synth.make_x(n, in_, seed=30 + i, dtype=dt)).to(dev)
        y = torch.full((n, out), float("nan"), device=dev)
        need = q4.q4_0_matmul_workspace_size(n, out, in_, q4.dtype_code(x))
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
        bufs.append((name, n, out, in_, blk, packed, x, y, ws, need))
    # the head's greedy pick (workspace always needed)
    hb = torch.from_numpy(synth.make_blocks(151936, 2560, seed=40).reshape(-1)).to(dev)
    hp = torch.empty(q4.q4_0_packed_bytes(151936, 2560), dtype=torch.uint8, device=dev)
    hx = torch.from_numpy(synth.make_x(1, 2560, seed=41)).to(dev)
    hneed = q4.q4_0_argmax_workspace_size(1, 151936, 2560)
    hws = torch.empty(hneed, dtype=torch.uint8, device=dev)
    mv = torch.empty(1, device=dev)
    mi = torch.empty(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        # the repacks and the products: the process's first library calls
        for name, n, out, in_, blk, packed, x, y, ws, need in bufs:
            q4.q4_0_repack(blk, packed, out, in_, cs)
            q4.q4_0_matmul(packed, x, q4.dtype_code(x), y, n, out, in_, ws, need, cs)
        q4.q4_0_repack(hb, hp, 151936, 2560, cs)
        q4.q4_0_matmul_argmax(hp, hx, q4.F32, None, 1, 151936, 2560, mv, mi, hws, hneed, cs)
    print("captured", flush=True)
    res = {}
    for rep in range(3):
        for b in bufs:
            b[7].fill_(float("nan"))
        mv.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, n, out, in_, blk, packed, x, y, ws, need in bufs:
            ref = q4.matmul(packed, x, out)
            torch.cuda.synchronize()
            ok = bool(torch.equal(y, ref))
            res[name] = res.get(name, True) and ok
        rv, ri = q4.matmul_argmax(hp, hx, 151936)
        torch.cuda.synchronize()
        res["argmax_head"] = res.get("argmax_head", True) and bool(
            torch.equal(rv, mv) and torch.equal(ri, mi))
        print(f"replay {rep}: {res}", flush=True)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
