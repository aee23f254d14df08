"""Benchmark of the Q4_0 matmul library on one MI355X.

One step = one pass of the hot path over one batch of synthetic input: for the
headline workload (FFN-up decode GEMV, W 9728 x 2560 in Q4_0, x float32
1 x 2560) that is one q4_0_matmul call.  Inputs are resident in HBM before
the timed region.  Successive steps rotate through copies of the repacked
weights totalling at least 1 GiB, so that the 256 MB Infinity Cache cannot
serve them and the figure is HBM bandwidth.

Timing: the steps' launches are recorded in HIP graphs and replayed between
two HIP events on the launch stream, exactly --steps steps; an untimed replay
is enqueued just before the first event, so the device is busy while the
timed replays are submitted and no host latency enters the timed region.

Prints ONE JSON line (rank 0, N = 1): effective weight GB/s (Q4_0 bytes, 18
per 32 weights, over the per-step time), the roofline object for the kernel
that runs (algorithmic bytes per launch over the events' per-launch time,
against 8 TB/s and against the measured single-launch read of the same
bytes), the oracle's CPU baseline on all host cores and on one, and under
"extra" the other workloads (small GEMV, batched decode of a 4B-class block,
logit head, mid-n band, W4A8, routed mixture of experts, prefill GEMMs) each
with its own roofline fractions, plus the calibration: the cost of an empty
launch and the plain streaming read rate at each workload's size.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Q4_0 matmul effective weight GB/s (n≤8) and TFLOP/s (n=512), % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFS = 2500.0     # MI355X dense fp16 MFMA
ROTATE_BYTES = 1 << 30
PROFILES = os.path.join(ROOT, "profiles")
GRAPH_MAX_STEPS = 1000         # steps recorded in one graph at most
# Fewest steps timed by graph replay.  Each graph launch costs about 12 us of
# device time at its head on this part (measured: FFN-up n = 1 reads 6.43 us
# per step over 20-step replays, 5.83 us over 1000-step replays), which one
# step of a real decode loop would share among all the kernels of a model;
# so the timed region holds at least this many steps, and the line reports
# both the steps requested and the steps timed.
MIN_TIMED_STEPS = 1000


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000,
                    help="steps to time; graph timing takes at least MIN_TIMED_STEPS "
                         "(the line reports both)")
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="ffn_up_decode",
                    choices=["gemv_1024", "ffn_up_decode", "block_decode",
                             "logit_head", "prefill", "moe_routed", "launch_floor",
                             "stream_read"])
    ap.add_argument("--n", type=int, default=None, help="rows of x (decode workloads)")
    ap.add_argument("--kernel", default="auto",
                    choices=["auto", "gemv_dpp", "gemv_mfma", "gemm"])
    ap.add_argument("--grouped", action="store_true",
                    help="block_decode: run the projections as grouped launches "
                         "(Q,K,V | O | gate,up | down)")
    ap.add_argument("--one-group", action="store_true",
                    help="block_decode: all seven projections, each with its own x, in one "
                         "grouped call")
    ap.add_argument("--w4a8", action="store_true",
                    help="decode workloads: int8 activations (q4_0_quantize_x8 + "
                         "q4_0_matmul_w4a8 per linear)")
    ap.add_argument("--argmax", action="store_true",
                    help="decode workloads: q4_0_matmul_argmax with no y stored")
    ap.add_argument("--bytes", type=int, default=14008320,
                    help="stream_read workload: bytes per launch")
    ap.add_argument("--quick", action="store_true",
                    help="headline workload only (no extra workloads, no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the empty-launch and streaming-read legs (counter runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--isolated", action="store_true",
                    help="profiling aid: only --steps launches of one linear (or of the "
                         "empty launch), each followed by a synchronisation, so a kernel "
                         "trace sees each dispatch alone")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


def kernel_code(q4, name):
    return {"auto": q4.KERNEL_AUTO, "gemv_dpp": q4.KERNEL_GEMV_DPP,
            "gemv_mfma": q4.KERNEL_GEMV_MFMA, "gemm": q4.KERNEL_GEMM}[name]


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_q4_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def ws_tensor(torch, nbytes):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")


class Case:
    """One linear: repacked copies of W, copies of x (the same values: step i
    reads x copy i % copies, so x comes from memory, as an activation just
    written by the previous kernel would, not from a cache warmed by the
    step before; warm_x keeps one copy), a y and a workspace on the device."""

    def __init__(self, torch, q4, synth, out, in_, n, x_dtype, seed, copies, kernel=0,
                 warm_x=False):
        self.out, self.in_, self.n = out, in_, n
        blk = synth.make_blocks(out, in_, seed=seed)
        b = torch.from_numpy(blk.reshape(-1)).cuda()
        base = q4.repacked(b, out, in_)
        del b
        self.packed = [base] + [base.clone() for _ in range(copies - 1)]
        npdt = np.float16 if x_dtype == "f16" else np.float32
        x0 = torch.from_numpy(synth.make_x(n, in_, seed=seed + 1000, dtype=npdt)).cuda()
        self.xs = [x0] + [x0.clone() for _ in range(0 if warm_x else copies - 1)]
        self.x = x0
        self.xcode = q4.F16 if x_dtype == "f16" else q4.F32
        self.y = torch.empty((n, out), dtype=torch.float32, device="cuda")
        self.wbytes = q4.q4_0_blocks_bytes(out, in_)
        self.xbytes = n * in_ * (2 if x_dtype == "f16" else 4)
        self.ybytes = n * out * 4
        self.flops = 2.0 * n * out * in_
        self.kernel = kernel
        self.ws_need = q4.q4_0_matmul_workspace_size(n, out, in_, self.xcode, kernel)
        self.ws = ws_tensor(torch, self.ws_need)


# The block's projections grouped as one decoder block runs them: Q, K and V
# read the same input, so do gate and up; O and down each wait for the
# previous step of the block.
BLOCK_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


def timed_steps(steps, graph=True):
    """Steps actually timed for a request of `steps`."""
    return max(steps, MIN_TIMED_STEPS) if graph else steps


def time_steps(torch, step, steps, warmup, graph=True):
    """Time timed_steps(steps) calls step(i, stream) (step i uses weight copy
    i % copies); return ms per step.

    graph=True: the steps are recorded in HIP graphs of at most
    GRAPH_MAX_STEPS steps (plus one graph for the remainder) and replayed;
    the device runs the same kernels on the same buffers without the Python
    and driver launch cost between them, as a decode loop would run them.
    One untimed replay is enqueued right before the first event, so the
    device is busy while the timed replays are submitted."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i, stream.cuda_stream)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if not graph:
        step(0, stream.cuda_stream)
        e0.record(stream)
        for i in range(steps):
            step(i, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps
    steps = timed_steps(steps)
    gsteps = min(steps, GRAPH_MAX_STEPS)
    reps, rem = divmod(steps, gsteps)
    cs = torch.cuda.Stream()
    cs.wait_stream(stream)

    def capture(count, first):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            for i in range(first, first + count):
                step(i, cs.cuda_stream)
        return g

    g = capture(gsteps, 0)
    gr = capture(rem, gsteps * reps) if rem else None
    g.replay()                      # untimed: the first replay uploads the graph
    if gr is not None:
        gr.replay()
    torch.cuda.synchronize()
    g.replay()                      # untimed, not awaited: keeps the device busy
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    if gr is not None:
        gr.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def timed(torch, q4, cases, steps, warmup, graph=True, groups=None, argmax=False, w4a8=False):
    """Time `steps` steps (each step = every case once, on its next weight
    copy); return ms per step.

    With `groups` (lists of case indices) each group runs as one
    q4_0_matmul_grouped call (its linears keep their own x).  With `argmax`
    each case runs as q4_0_matmul_argmax with no y stored (the greedy pick of
    a logit head).  With `w4a8` each case quantizes its x to int8
    (q4_0_quantize_x8) and runs q4_0_matmul_w4a8 on the codes."""
    ncopy = len(cases[0].packed)
    if argmax:
        for c in cases:
            c.mv = torch.empty(c.n, dtype=torch.float32, device="cuda")
            c.mi = torch.empty(c.n, dtype=torch.int32, device="cuda")
            c.aneed = q4.q4_0_argmax_workspace_size(c.n, c.out, c.in_, c.xcode)
            c.aws = ws_tensor(torch, c.aneed)
    if w4a8:
        for c in cases:
            c.q8 = torch.empty((c.n, c.in_), dtype=torch.int8, device="cuda")
            c.d8 = torch.empty((c.n, c.in_ // 32), dtype=torch.float32, device="cuda")
            c.wneed = q4.q4_0_w4a8_workspace_size(c.n, c.out, c.in_)
            c.wws = ws_tensor(torch, c.wneed)
    gws = []
    for grp in groups or ():
        lin = [(cases[k].packed[0], cases[k].x, cases[k].y, cases[k].out, cases[k].in_)
               for k in grp]
        need = q4.q4_0_grouped_workspace_size(lin, cases[grp[0]].xcode, cases[grp[0]].n)
        gws.append((ws_tensor(torch, need), need))

    def step(i, sh):
        if w4a8:
            for c in cases:
                q4.q4_0_quantize_x8(c.xs[i % len(c.xs)], c.xcode, c.q8, c.d8, c.n, c.in_, sh)
                q4.q4_0_matmul_w4a8(c.packed[i % ncopy], c.q8, c.d8, c.y, c.n, c.out, c.in_,
                                    c.wws, c.wneed, sh)
            return
        if argmax:
            for c in cases:
                q4.q4_0_matmul_argmax(c.packed[i % ncopy], c.xs[i % len(c.xs)], c.xcode, None,
                                      c.n, c.out, c.in_, c.mv, c.mi, c.aws, c.aneed, sh)
            return
        if groups is None:
            for c in cases:
                q4.q4_0_matmul_ex(c.packed[i % ncopy], c.xs[i % len(c.xs)], c.xcode, c.y, c.n,
                                  c.out, c.in_, c.kernel, c.ws, c.ws_need, sh)
            return
        for grp, (ws, need) in zip(groups, gws):
            q4.q4_0_matmul_grouped(
                [(cases[k].packed[i % ncopy], cases[k].xs[i % len(cases[k].xs)], cases[k].y,
                  cases[k].out, cases[k].in_) for k in grp], cases[grp[0]].xcode,
                cases[grp[0]].n, ws, need,
                sh)

    return time_steps(torch, step, steps, warmup, graph)


def copies_for(total_bytes):
    return max(2, -(-ROTATE_BYTES // max(1, total_bytes)))


class Calibration:
    """Attainable rates on this part, measured in this run with the library's
    measurement aids (q4_0_stream_read): the cost of one empty launch, and
    for a given byte count the best rate of a plain streaming read of that
    many bytes in one launch (over rotating buffers of at least 1 GiB, graph
    replay, the best of several grid sizes)."""

    GRIDS = (256, 512, 1024, 2048, 4096)
    FLOOR_GRID = 250      # the empty launch's grid: told apart from the reads in a trace

    def __init__(self, torch, q4):
        self.torch, self.q4 = torch, q4
        self.sink = torch.empty(65536, dtype=torch.float32, device="cuda")
        self.reads = {}
        self.floor = None
        self.floor_isolated = None

    def isolated_us(self, step, reps=200):
        """Median time of one launch run alone: event, the launch, event,
        then a synchronisation before the next (what a profiler's per-dispatch
        duration measures, launch ramp included), in us."""
        torch = self.torch
        stream = torch.cuda.current_stream()
        times = []
        for i in range(reps + 10):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(i, stream.cuda_stream)
            e1.record(stream)
            e1.synchronize()
            if i >= 10:
                times.append(e0.elapsed_time(e1) * 1e3)
        return round(float(np.median(times)), 3)

    def launch_floor_us(self, steps=500):
        if self.floor is None:
            q4, sink = self.q4, self.sink
            g = self.FLOOR_GRID
            ms = time_steps(self.torch, lambda i, sh: q4.q4_0_stream_read(None, 0, sink, g, sh),
                            steps, 20)
            self.floor = round(ms * 1e3, 3)
            self.floor_isolated = self.isolated_us(
                lambda i, sh: q4.q4_0_stream_read(None, 0, sink, g, sh))
        return self.floor

    def read(self, nbytes, steps=200):
        nbytes = -(-nbytes // 16) * 16
        if nbytes in self.reads:
            return self.reads[nbytes]
        torch, q4, sink = self.torch, self.q4, self.sink
        slot = -(-nbytes // 4096) * 4096
        copies = copies_for(slot)
        buf = torch.empty(slot * copies, dtype=torch.uint8, device="cuda")
        buf.fill_(1)
        best = None
        for wgs in self.GRIDS:
            def step(i, sh, wgs=wgs):
                off = (i % copies) * slot
                q4.q4_0_stream_read(buf[off:off + nbytes], nbytes, sink, wgs, sh)
            ms = time_steps(torch, step, steps, 10)
            if best is None or ms < best[0]:
                best = (ms, wgs)
        del buf
        torch.cuda.empty_cache()
        res = {"bytes": nbytes, "us": round(best[0] * 1e3, 3),
               "GB/s": round(nbytes / (best[0] * 1e-3) / 1e9, 1), "workgroups": best[1]}
        self.reads[nbytes] = res
        return res

    def summary(self):
        return {"launch_floor_us": self.floor, "launch_floor_isolated_us": self.floor_isolated,
                "stream_read": sorted(self.reads.values(), key=lambda r: r["bytes"]),
                "note": "empty launch and plain 16-byte non-temporal streaming read "
                        "(q4_0_stream_read), graph replay, weights rotated over >= 1 GiB"}


def parity_check(q4, oracle, synth, case, seed, rows=64):
    """Oracle check of the benched configuration on sampled rows."""
    blk = synth.make_blocks(case.out, case.in_, seed=seed)
    x = case.x.cpu().numpy()
    rng = np.random.default_rng(seed)
    r = np.unique(rng.integers(0, case.out, size=rows))
    y_ref, den = oracle.matmul(blk, x, case.out, case.in_, rows=r)
    y = case.y.cpu().numpy()[:, r]
    return oracle.max_ratio(y, y_ref, den)


def traffic_for(workload):
    """Counter-measured HBM bytes per launch, if taken on the current sources."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    ent = data.get(workload)
    if not ent or ent.get("src_sha") != source_hash():
        return None
    return ent.get("bytes_per_launch")


def decode_line(torch, q4, synth, cal, name, linears, n, kernel, steps, warmup, groups=None,
                argmax=False, w4a8=False, launches=None, names=None):
    """One decode configuration: ms per step, effective weight GB/s, and the
    fraction of 8 TB/s and of the measured single-launch read of the step's
    weight bytes.  With `names` (one call per linear), each linear is also
    timed alone on the same buffers: `per_linear` gives its us per call."""
    total_w = sum(q4.q4_0_blocks_bytes(o, i) for o, i in linears)
    copies = copies_for(total_w)
    cases = [Case(torch, q4, synth, o, i, n, "f32", seed=k, copies=copies, kernel=kernel)
             for k, (o, i) in enumerate(linears)]
    ms = timed(torch, q4, cases, steps, warmup, groups=groups, argmax=argmax, w4a8=w4a8)
    ms_eager = timed(torch, q4, cases, min(steps, 200), 5, graph=False, groups=groups,
                     argmax=argmax, w4a8=w4a8)
    gbs = total_w / (ms * 1e-3) / 1e9
    alg = sum(c.wbytes + c.xbytes + c.ybytes for c in cases)
    kern = ["w4a8"] if w4a8 else sorted(
        {q4.KERNEL_NAMES[q4.q4_0_select_kernel(n, o, i) if kernel == 0 else kernel]
         for o, i in linears})
    att = cal.read(total_w)
    res = {"workload": name, "n": n, "ms_per_step": round(ms, 5),
           "steps": timed_steps(steps),
           "ms_per_step_eager": round(ms_eager, 5),
           "weight_bytes": total_w, "algorithmic_bytes": alg, "GB/s": round(gbs, 1),
           "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
           "attainable_GB/s": att["GB/s"], "frac_attainable": round(gbs / att["GB/s"], 4),
           "kernels": kern,
           "calls_per_step": launches or (len(linears) if groups is None else len(groups)),
           "grouped": groups is not None, "argmax": argmax, "w4a8": w4a8,
           "rotation_copies": copies}
    del cases
    torch.cuda.empty_cache()
    if names is not None and groups is None and not argmax and not w4a8:
        # each linear alone, its own copies rotated over at least 1 GiB
        per = {}
        for k, (nm, (o, i)) in enumerate(zip(names, linears)):
            c = Case(torch, q4, synth, o, i, n, "f32", seed=k,
                     copies=copies_for(q4.q4_0_blocks_bytes(o, i)), kernel=kernel)
            per[f"{nm} {o}x{i}"] = round(timed(torch, q4, [c], steps, warmup) * 1e3, 3)
            del c
            torch.cuda.empty_cache()
        res["per_linear_us"] = per
        res["per_linear_sum_us"] = round(sum(per.values()), 3)
    return res


def routed_line(torch, q4, synth, cal, n, steps, warmup, n_exp=128, k=8, out=768, in_=2048,
                hot=0, auto_only=False):
    """Routed (mixture-of-experts) decode, synthetic: n rows of x, each through
    k distinct experts drawn from n_exp experts of out x in (an expert FFN
    projection of a mid-size mixture model; the experts' shape is chosen, not
    taken from a page), or with hot > 0 from the same first `hot` experts
    (concentrated routing).  One q4_0_matmul_routed call per step, timed by
    column, by expert and as AUTO picks, and for n <= 4 against the same pairs
    as n*k single-row q4_0_matmul calls (auto_only: the form AUTO picks alone,
    for counter runs).  GB/s counts the distinct experts' Q4_0 bytes of a
    step."""
    eb = q4.q4_0_blocks_bytes(out, in_)
    pb = q4.q4_0_packed_bytes(out, in_)
    copies = copies_for(n_exp * eb)
    parts = []
    for e in range(n_exp):
        b = torch.from_numpy(synth.make_blocks(out, in_, seed=500 + e).reshape(-1)).cuda()
        parts.append(q4.repacked(b, out, in_))
    base = torch.cat(parts)
    del parts
    stacks = [base] + [base.clone() for _ in range(copies - 1)]
    x = torch.from_numpy(synth.make_x(n, in_, seed=501)).cuda()
    rng = np.random.default_rng(502)
    pool = hot if hot else n_exp
    route_np = np.stack([rng.permutation(pool)[:k] for _ in range(n)]).astype(np.int32)
    route = torch.from_numpy(route_np).cuda()
    y = torch.empty((n * k, out), dtype=torch.float32, device="cuda")
    uniq = len(np.unique(route_np))

    def routed(rk):
        need = q4.q4_0_routed_workspace_size(n, k, n_exp, out, in_, rk)
        ws = ws_tensor(torch, need)

        def step(i, sh):
            q4.q4_0_matmul_routed_ex(stacks[i % copies], n_exp, x, q4.F32, route, k, y, n, out,
                                     in_, rk, ws, need, sh)
        return step

    sneed = q4.q4_0_matmul_workspace_size(1, out, in_, q4.F32, q4.KERNEL_GEMV_MFMA)
    sws = ws_tensor(torch, sneed)

    def singles(i, sh):
        st = stacks[i % copies]
        for t in range(n):
            for j in range(k):
                e, p = int(route_np[t, j]), t * k + j
                q4.q4_0_matmul_ex(st[e * pb:(e + 1) * pb], x[t:t + 1], q4.F32, y[p:p + 1], 1,
                                  out, in_, q4.KERNEL_GEMV_MFMA, sws, sneed, sh)

    auto = q4.q4_0_select_route(n, k, n_exp, out, in_)
    ms = {}
    for name, rk in (("by_column", q4.ROUTE_BY_COLUMN), ("by_expert", q4.ROUTE_BY_EXPERT)):
        if auto_only and rk != auto:
            ms[name] = None
            continue
        try:
            ms[name] = time_steps(torch, routed(rk), steps, warmup)
        except q4.Q4Error:
            ms[name] = None
    best = ms["by_column" if auto == q4.ROUTE_BY_COLUMN else "by_expert"]
    gbs = uniq * eb / (best * 1e-3) / 1e9
    att = cal.read(uniq * eb)
    res = {"workload": "moe_routed_decode" + (f"_hot{hot}" if hot else ""), "n": n,
           "experts": n_exp, "k": k,
           "expert_shape": [out, in_], "distinct_experts": uniq,
           "auto": "by_column" if auto == q4.ROUTE_BY_COLUMN else "by_expert",
           "ms_per_step": round(best, 5), "steps": timed_steps(steps),
           "ms_by_column": ms["by_column"] and round(ms["by_column"], 5),
           "ms_by_expert": ms["by_expert"] and round(ms["by_expert"], 5),
           "weight_bytes": uniq * eb, "GB/s": round(gbs, 1),
           "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
           "attainable_GB/s": att["GB/s"], "frac_attainable": round(gbs / att["GB/s"], 4),
           "rotation_copies": copies}
    if n <= 4 and not auto_only:
        res["ms_single_calls"] = round(time_steps(torch, singles, steps, warmup), 5)
    del stacks, base
    torch.cuda.empty_cache()
    return res


def mfma_loop_peak(torch, q4, reps=3):
    """Sustained rate of back-to-back v_mfma_f32_32x32x16_f16 on every SIMD
    (the library's measurement aid), best of `reps` launches, in TFLOP/s."""
    wgs, iters = 256, 4000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    best = 0.0
    for _ in range(reps + 1):                 # the first launch warms the clock up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        flops = q4.q4_0_mfma_loop(sink, wgs, iters, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        best = max(best, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return round(best, 1)


def dense_f16_library_ms(torch, o, i, n, steps, warmup, copies=4):
    """Context for the prefill lines: the platform's dense binary16 GEMM
    (torch.matmul, which calls the vendor BLAS library) on the same shape with
    binary16 weights (four times the bytes, no decode), timed the same way."""
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn(n, i, device="cuda", dtype=torch.float16, generator=g)
    ws = [torch.randn(o, i, device="cuda", dtype=torch.float16, generator=g)
          for _ in range(copies)]
    ys = [torch.empty(n, o, device="cuda", dtype=torch.float16) for _ in range(copies)]
    ms = time_steps(torch, lambda k, s: torch.matmul(x, ws[k % copies].t(), out=ys[k % copies]),
                    steps, warmup)
    del x, ws, ys
    torch.cuda.empty_cache()
    return ms


def prefill_line(torch, q4, synth, kernel, steps, warmup):
    loop_peak = mfma_loop_peak(torch, q4)
    res = []
    for li, (o, i) in enumerate([(9728, 2560), (2560, 9728)]):
        c = Case(torch, q4, synth, o, i, 512, "f16", seed=li, copies=4, kernel=kernel)
        ms = timed(torch, q4, [c], steps, warmup)
        tfs = c.flops / (ms * 1e-3) / 1e12
        flops = c.flops
        del c
        torch.cuda.empty_cache()
        lib = dense_f16_library_ms(torch, o, i, 512, steps, warmup)
        res.append({"linear": f"{o}x{i}", "n": 512, "ms_per_step": round(ms, 5),
                    "TFLOP/s": round(tfs, 2), "frac_mfma_f16": round(tfs / F16_MFMA_PEAK_TFS, 4),
                    "mfma_loop_TFLOP/s": loop_peak, "frac_mfma_loop": round(tfs / loop_peak, 4),
                    "kernel": q4.KERNEL_NAMES[q4.q4_0_select_kernel(512, o, i, q4.F16)
                                              if kernel == 0 else kernel],
                    "dense_f16_library_ms": round(lib, 5),
                    "dense_f16_library_TFLOP/s": round(flops / (lib * 1e-3) / 1e12, 2)})
    return res


def cpu_baseline(oracle, synth, out, in_, n, seconds):
    """The oracle as it stands, on all host cores and on one, over repeated
    full passes of the workload."""
    blk = synth.make_blocks(out, in_, seed=0)
    x = synth.make_x(n, in_, seed=1000)
    wbytes = out * (in_ // 32) * 18

    def run(nthreads, budget):
        times, threads = [], 0
        t_end = time.perf_counter() + budget
        while True:
            t0 = time.perf_counter()
            _, _, threads = oracle.matmul(blk, x, out, in_, nthreads=nthreads,
                                          return_threads=True)
            times.append(time.perf_counter() - t0)
            if time.perf_counter() > t_end and len(times) >= 3:
                break
        return float(np.median(times)), int(threads), times

    t, threads, times = run(0, seconds)
    t1, _, times1 = run(1, seconds / 2)
    return {"value": round(wbytes / t / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(times)} full oracle passes of the {out}x{in_} n={n} workload "
                      f"(median {t * 1e3:.2f} ms each, ~{sum(times):.0f} s total)",
            "single_thread": {"value": round(wbytes / t1 / 1e9, 4), "unit": "GB/s",
                              "cores": 1,
                              "sample": f"{len(times1)} passes, median {t1 * 1e3:.1f} ms"}}


def calibration_main(torch, q4, cal, args):
    """--workload launch_floor / stream_read: the measurement aids alone (for
    profiling them under the same trace as the products)."""
    if args.workload == "launch_floor":
        us = cal.launch_floor_us(args.steps)
        return {"workload": "launch_floor", "us_per_launch": us}
    r = cal.read(args.bytes, args.steps)
    return {"workload": "stream_read", **r}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only (--gpus must be 1); sharding is described, not run",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    import torch
    import gemm_q4_amd as q4
    import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    cal = Calibration(torch, q4)
    if args.workload == "launch_floor" and args.isolated:
        g = Calibration.FLOOR_GRID
        us = cal.isolated_us(lambda i, sh: q4.q4_0_stream_read(None, 0, cal.sink, g, sh),
                             reps=args.steps)
        print(json.dumps({"workload": "launch_floor", "isolated": True,
                          "us_per_launch_isolated": us}), flush=True)
        return
    if args.workload in ("launch_floor", "stream_read"):
        print(json.dumps(calibration_main(torch, q4, cal, args)), flush=True)
        return
    if args.workload == "moe_routed":
        # the routed decode alone: the form AUTO picks, n rows (default 4)
        n = args.n if args.n is not None else 4
        line = routed_line(torch, q4, synth, cal, n, args.steps, args.warmup, auto_only=True)
        roof = {"bound": "hbm", "achieved": line["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": line["frac_hbm"], "traffic": traffic_for(f"moe_routed_n{n}"),
                "attainable_GB/s": line["attainable_GB/s"],
                "frac_attainable": line["frac_attainable"]}
        rec = {"metric": METRIC, "value": line["GB/s"], "unit": "GB/s", "n_gpus": 1,
               "steps": timed_steps(args.steps), "steps_requested": args.steps,
               "warmup": args.warmup, "ms_per_step": line["ms_per_step"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
               "dtype": "f16", "data": "synthetic",
               "config": {"workload": "moe_routed_decode", "n": n, "experts": line["experts"],
                          "k": line["k"], "expert_shape": line["expert_shape"],
                          "route": line["auto"]},
               "roofline": roof, "extra": {"routed": [line], "calibration": cal.summary()},
               "source_sha": source_hash()}
        print(json.dumps(rec), flush=True)
        return
    kernel = kernel_code(q4, args.kernel)
    wl = synth.WORKLOADS[args.workload]
    n = args.n if args.n is not None else wl.ns[0]

    if args.workload == "prefill":
        lines = prefill_line(torch, q4, synth, kernel, args.steps, args.warmup)
        head = lines[0]
        value, unit, ms = head["TFLOP/s"], "TFLOP/s", head["ms_per_step"]
        roof = {"bound": "mfma", "achieved": value, "peak": F16_MFMA_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(value / F16_MFMA_PEAK_TFS, 4),
                "traffic": traffic_for("prefill")}
        cfg = {"workload": "prefill", "linears": [l["linear"] for l in lines], "n": 512,
               "x_dtype": "f16", "kernel": head["kernel"]}
        dtype = "f16"
        extra = {"prefill": lines}
        parity = None
    else:
        linears = [(l.out, l.in_) for l in wl.linears]
        total_w = sum(q4.q4_0_blocks_bytes(o, i) for o, i in linears)
        copies = copies_for(total_w)
        cases = [Case(torch, q4, synth, o, i, n, "f32", seed=k, copies=copies, kernel=kernel)
                 for k, (o, i) in enumerate(linears)]
        if args.isolated:
            c = cases[0]
            ncp = len(c.packed)
            us = cal.isolated_us(lambda i, sh: q4.q4_0_matmul_ex(
                c.packed[i % ncp], c.xs[i % len(c.xs)], c.xcode, c.y, c.n, c.out, c.in_,
                c.kernel, c.ws, c.ws_need, sh), reps=args.steps)
            print(json.dumps({"workload": args.workload, "n": n, "isolated": True,
                              "linear": f"{c.out}x{c.in_}", "us_per_launch_isolated": us,
                              "source_sha": source_hash()}), flush=True)
            return
        groups = None
        names = [l.name for l in wl.linears]
        if args.workload == "block_decode" and args.grouped:
            groups = [[names.index(nm) for nm in grp] for grp in BLOCK_GROUPS]
        elif args.workload == "block_decode" and args.one_group:
            groups = [list(range(len(names)))]
        ms = timed(torch, q4, cases, args.steps, args.warmup, groups=groups,
                   argmax=args.argmax, w4a8=args.w4a8)
        ms_eager = timed(torch, q4, cases, min(args.steps, 500), 5, graph=False,
                         groups=groups, argmax=args.argmax, w4a8=args.w4a8)
        iso = None
        if groups is None and not args.argmax and not args.w4a8 and len(cases) == 1:
            c = cases[0]
            ncp = len(c.packed)
            iso = cal.isolated_us(lambda i, sh: q4.q4_0_matmul_ex(
                c.packed[i % ncp], c.xs[i % len(c.xs)], c.xcode, c.y, c.n, c.out, c.in_,
                c.kernel, c.ws, c.ws_need, sh))
        # the same steps with one x for every step (x warm in the caches)
        xs_saved = [c.xs for c in cases]
        for c in cases:
            c.xs = c.xs[:1]
        ms_warm_x = timed(torch, q4, cases, args.steps, args.warmup, groups=groups,
                          argmax=args.argmax, w4a8=args.w4a8)
        for c, xs in zip(cases, xs_saved):
            c.xs = xs
        parity = None if (args.argmax or args.w4a8) else max(
            parity_check(q4, __import__("oracle"), synth, c, seed=k) for k, c in enumerate(cases))
        value = total_w / (ms * 1e-3) / 1e9
        unit = "GB/s"
        kname = q4.KERNEL_NAMES[q4.q4_0_select_kernel(n, *linears[0]) if kernel == 0 else kernel]
        calls = len(linears) if groups is None else len(groups)
        alg = sum(c.wbytes + c.xbytes + c.ybytes for c in cases)
        # algorithmic bytes per call over the events' per-call time (one
        # launch per call for the headline: the kernel's launch duration)
        achieved = (alg / calls) / (ms / calls * 1e-3) / 1e9
        att = ({"GB/s": None, "us": None} if args.no_calibration else cal.read(total_w))
        floor = None if args.no_calibration else cal.launch_floor_us()
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_for(args.workload + ("_one_group" if args.one_group else "")
                                       + ("_grouped" if args.grouped else "")
                                       + ("_argmax" if args.argmax else "")
                                       + ("_w4a8" if args.w4a8 else "")
                                       + (f"_n{n}" if n != 1 else "")),
                "algorithmic_bytes_per_launch": alg // calls,
                "us_per_launch": round(ms / calls * 1e3, 4),
                "us_per_launch_isolated": iso,
                "attainable_GB/s": att["GB/s"], "attainable_us": att["us"],
                "frac_attainable": att["GB/s"] and round(achieved / att["GB/s"], 4),
                "launch_floor_us": floor}
        cfg = {"workload": args.workload, "linears": [f"{o}x{i}" for o, i in linears],
               "n": n, "x_dtype": "f32", "kernel": kname, "rotation_copies": copies,
               "weight_bytes_per_step": total_w,
               "timing": "HIP graph replay of the step's launches, events on the launch stream",
               "grouped": groups is not None, "argmax": args.argmax, "w4a8": args.w4a8,
               "ms_per_step_eager": round(ms_eager, 6),
               "ms_per_step_warm_x": round(ms_warm_x, 6),
               "x_copies": len(cases[0].xs),
               # the products: binary16 operands (x as high and low parts up to
               # 8 rows), float32 accumulation; W4A8: int8 operands, int32 sums
               "accumulate": "i32 then f32" if args.w4a8 else "f32"}
        dtype = "i8" if args.w4a8 else "f16"
        del cases
        torch.cuda.empty_cache()
        extra = {}
        if not args.quick:
            extra["decode"] = []
            extra["decode"].append(decode_line(torch, q4, synth, cal, "gemv_1024",
                                               [(1024, 1024)], 1, kernel, 2000, 100))
            blk = [(l.out, l.in_) for l in synth.WORKLOADS["block_decode"].linears]
            bnames = [l.name for l in synth.WORKLOADS["block_decode"].linears]
            bgroups = [[bnames.index(nm) for nm in grp] for grp in BLOCK_GROUPS]
            one = [list(range(len(blk)))]
            for nn in (1, 2, 4, 8):
                extra["decode"].append(decode_line(torch, q4, synth, cal, "block_decode", blk,
                                                   nn, kernel, 300, 30, names=bnames))
                if kernel == q4.KERNEL_AUTO:
                    extra["decode"].append(decode_line(torch, q4, synth, cal, "block_decode",
                                                       blk, nn, kernel, 300, 30,
                                                       groups=bgroups))
                    extra["decode"].append(decode_line(torch, q4, synth, cal,
                                                       "block_decode_one_group", blk, nn,
                                                       kernel, 300, 30, groups=one))
            for nn in (1, 4):
                extra["decode"].append(decode_line(torch, q4, synth, cal, "logit_head",
                                                   [(151936, 2560)], nn, kernel, 200, 20))
                if kernel == q4.KERNEL_AUTO:
                    extra["decode"].append(decode_line(torch, q4, synth, cal, "logit_head",
                                                       [(151936, 2560)], nn, kernel, 200, 20,
                                                       argmax=True))
            # the band between decode and prefill: the small-n kernel against
            # the tiled prefill product on the same shapes
            extra["mid_n"] = []
            up = [(9728, 2560)]
            for nn in (16, 32, 64):
                for kk in (q4.KERNEL_AUTO, q4.KERNEL_GEMM):
                    extra["mid_n"].append(decode_line(torch, q4, synth, cal, "ffn_up_decode", up,
                                                      nn, kk, 300, 20))
                extra["mid_n"].append(decode_line(torch, q4, synth, cal, "block_decode", blk, nn,
                                                  q4.KERNEL_AUTO, 200, 20, groups=bgroups))
            # W4A8: activations quantized to int8 per 32-value block, then the
            # integer product (both launches timed)
            extra["w4a8"] = [
                decode_line(torch, q4, synth, cal, "ffn_up_decode", up, 1, 0, 1000, 50,
                            w4a8=True),
                decode_line(torch, q4, synth, cal, "block_decode", blk, 4, 0, 200, 20,
                            w4a8=True),
                decode_line(torch, q4, synth, cal, "logit_head", [(151936, 2560)], 1, 0, 200,
                            20, w4a8=True)]
            extra["routed"] = [routed_line(torch, q4, synth, cal, nn, 300, 20)
                               for nn in (1, 4, 16, 32, 64)]
            extra["routed"] += [routed_line(torch, q4, synth, cal, nn, 300, 20, hot=16)
                                for nn in (16, 64)]
            extra["prefill"] = prefill_line(torch, q4, synth, 0, 200, 20)
        extra["calibration"] = cal.summary()

    if args.calib_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()

    rec = {"metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1,
           "steps": timed_steps(args.steps), "steps_requested": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": dtype, "data": "synthetic", "config": cfg, "roofline": roof}
    if parity is not None:
        rec["parity_max_ratio"] = parity
    if not args.quick and not args.no_cpu_baseline:
        import oracle
        o, i = wl.linears[0].out, wl.linears[0].in_
        rec["cpu_baseline"] = cpu_baseline(oracle, synth, o, i, n, args.cpu_seconds)
    if extra:
        rec["extra"] = extra
    rec["source_sha"] = source_hash()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
