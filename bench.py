"""Benchmark of the quantized-matmul hot path on one MI355X.

Prints ONE JSON line.  The headline value is the decode step on 8B-class
layer shapes (CQ W4A8, group 128, batch 1): for each of the four matrices
4096x4096, 1024x4096, 14336x4096, 4096x14336 one launch of cq_gemv_f32, which
quantizes the fp32 activations (A8) inside the GEMV launch.  ``value`` =
packed weight bytes (indices + fp16 norms) of the step / step time, in GB/s.  Weights are resident in HBM: the step cycles over
a pool of >= 1 GiB of distinct weight copies, so the 256 MB Infinity Cache
cannot hold them between uses.  After W warm-up steps, the K timed steps run
consecutively in one HIP graph (as a decode graph holds every layer's
launches), each on the next weight copy; the step time is their mean.

The same line carries: ``roofline`` for the dominant kernel (the fused CQ GEMV
on the 4096x14336 down-projection shape: mean launch duration over a HIP graph
of back-to-back HBM-cold launches, timed with HIP events on the launch stream), the prefill GEMM (512 tokens, TFLOP/s), the Minueza-shaped
Q4_0 decode pass and the same pass as a 512-token prefill (q4_0_gemm), the
bit-width sweep, the same decode layer shapes at 4, 16
and 32 tokens per call (``batched_decode_cb4``), and ``cpu_baseline``: the CPU
oracle timed on a bounded sample of the same workload.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
       python bench.py --only dominant|decode|prefill|q4_0|q4_0_prefill|q4_0_a8|sweep|batched|kmcu|floor|copy|c1
       (profiling runs)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0    # MI355X dense fp16/bf16 matrix, published
POOL_BYTES = 1 << 30             # >= 1 GiB of distinct weight copies per measurement
METRIC = "decode GEMV effective weight GB/s (% of HBM peak); prefill GEMM TFLOP/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "cq_gemv_4096x14336_traffic.json")
GEMV_SOURCES = [os.path.join(ROOT, "bit_quantized_matmul_amd", "csrc", f)
                for f in ("cq_gemv_impl.h", "cq_gemv_i4f.hip")]


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["dominant", "decode", "prefill", "q4_0", "q4_0_prefill", "sweep",
                                       "batched", "kmcu", "floor", "copy", "c1", "q4_0_a8"])
    ap.add_argument("--no-graph", action="store_true",
                    help="launch kernel-mean sequences eagerly (for counter collection)")
    return ap.parse_args()


EAGER = False


class Timer:
    """HIP events on the current (launch) stream."""

    def __init__(self):
        import torch
        self.torch = torch
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.s.record()

    def stop_ms(self) -> float:
        self.e.record()
        self.e.synchronize()
        return self.s.elapsed_time(self.e)


def graph_mean_ms(torch, launches, reps: int = 3) -> float:
    """Mean duration per launch of `launches` captured once in a HIP graph and
    replayed `reps` times between one HIP event pair on the launch stream (no
    host launch overhead between the kernels).  With --no-graph the sequence is
    launched eagerly instead (host-bound for short kernels)."""
    if EAGER:
        for fn in launches:
            fn()
        torch.cuda.synchronize()
        t = Timer()
        t.start()
        for _ in range(reps):
            for fn in launches:
                fn()
        return t.stop_ms() / (reps * len(launches))
    for fn in launches[:2]:
        fn()                                     # warm caches of device properties
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in launches:
            fn()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        g.replay()
    e.record()
    e.synchronize()
    ms = s.elapsed_time(e) / (reps * len(launches))
    del g
    return ms


def graph_repeats_ms(torch, launches, repeats: int = 5) -> list:
    """Per-launch mean of `launches` captured once in a HIP graph, for each of
    `repeats` separate replays (each replay timed alone between a HIP event
    pair on the launch stream)."""
    for fn in launches[:2]:
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for fn in launches:
            fn()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(repeats):
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        e.synchronize()
        out.append(s.elapsed_time(e) / len(launches))
    del g
    return out


def spread(values_ms, scale=1e3) -> dict:
    """min / median / max of repeated timings (ms -> us by default)."""
    v = sorted(x * scale for x in values_ms)
    return dict(min=v[0], median=v[len(v) // 2], max=v[-1], n=len(v))


def pool_copies(nbytes: int, minimum: int = 2) -> int:
    return max(minimum, math.ceil(POOL_BYTES / max(1, nbytes)))


def cold_pool(blob, existing=None):
    """>= 1 GiB of copies of `blob` (starting from `existing` ones), so that a
    sequence of launches cycling over them always reads from HBM."""
    pool = list(existing) if existing else [blob]
    while len(pool) < pool_copies(blob.numel()):
        pool.append(blob.clone())
    return pool


def payload_bytes(lay) -> int:
    """Algorithmic weight bytes: packed indices + fp16 norms."""
    return int(lay.idx_bytes + 2 * lay.norms_count)


# ----------------------------------------------------------------- workloads

def fit_codebooks(B, torch, dev):
    from bit_quantized_matmul_amd import inputs
    z = torch.from_numpy(inputs.gaussian_samples()).to(dev)
    out = {}
    for bits, levels in ((2, 4), (3, 8), (4, 16)):
        table, _ = B.cq_codebook_fit(z, levels, 200)
        out[bits] = table.cpu().numpy()
    return out


def codebook_for(code, cbs):
    return None if code in (1, 5, 6) else cbs[code]


def decode_setup(B, torch, dev, cbs):
    from bit_quantized_matmul_amd import inputs
    wl = inputs.cq_decode_8b()
    mats = []
    for (label, w), x in zip(wl.weights, wl.acts):
        rows, cols = w.shape
        lay = B.cq_pack_info(rows, cols, 128, 4)
        blob = B.cq_pack(torch.from_numpy(w).to(dev), lay, cbs[4])
        mats.append(dict(label=label, rows=rows, cols=cols, lay=lay, blob=blob,
                         x=torch.from_numpy(x).to(dev),
                         q=torch.empty((1, cols), dtype=torch.int8, device=dev),
                         s=torch.empty((1,), dtype=torch.float32, device=dev),
                         y=torch.empty((1, rows), dtype=torch.float32, device=dev)))
    step_bytes = sum(payload_bytes(m["lay"]) for m in mats)
    ncopies = pool_copies(step_bytes)
    pool = [[m["blob"]] + [m["blob"].clone() for _ in range(ncopies - 1)] for m in mats]
    torch.cuda.synchronize()
    return mats, pool, step_bytes, ncopies, wl


def run_step(B, mats, pool, slot, cb4):
    """One decode step: per matrix one launch (A8 fused into the GEMV)."""
    for i, m in enumerate(mats):
        B.cq_gemv_f32(pool[i][slot], m["lay"], cb4, m["x"], y=m["y"])


def run_step_two_launch(B, mats, pool, slot, cb4):
    """The same step as separate A8 and GEMV launches (reference figure)."""
    for i, m in enumerate(mats):
        B.act_fwht_quant_a8(m["x"], q=m["q"], scale=m["s"])
        B.cq_gemv(pool[i][slot], m["lay"], cb4, m["q"], m["s"], y=m["y"])


def bench_decode(B, torch, dev, cbs, steps, warmup):
    mats, pool, step_bytes, ncopies, _ = decode_setup(B, torch, dev, cbs)
    cb4 = cbs[4]
    run_step(B, mats, pool, 0, cb4)             # caches device properties before capture
    torch.cuda.synchronize()

    def graph_of(step_fn, slots):
        """One HIP graph of consecutive steps (as a model's decode graph holds
        every layer's launches), so a step pays no graph launch of its own."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for slot in slots:
                step_fn(B, mats, pool, slot, cb4)
        return g

    def per_step_ms(step_fn, slots_of, repeats=1):
        """W untimed warm-up steps, then exactly K timed steps, each run as one
        graph replay; slots_of(i) is step i's weight copy.  With repeats > 1
        the same K steps are timed again (each replay alone): the list of
        per-step times is returned, the first being the contract's run."""
        if warmup:
            gw = graph_of(step_fn, [slots_of(i) for i in range(warmup)])
            gw.replay()
            torch.cuda.synchronize()
            del gw
        g = graph_of(step_fn, [slots_of(warmup + i) for i in range(steps)])
        torch.cuda.synchronize()
        times = []
        for _ in range(repeats):
            t = Timer()
            t.start()
            g.replay()
            times.append(t.stop_ms() / steps)
        del g
        return times if repeats > 1 else times[0]

    # HBM-cold: the weight copies cycled in order, one per step; the first
    # timed run is the headline, four more give the spread
    reps = per_step_ms(run_step, lambda i: i % ncopies, repeats=5)
    ms = reps[0]
    # warm: the same copy every step (its weights stay in the Infinity Cache)
    ms_warm = per_step_ms(run_step, lambda i: 0)
    # the two-launch variant of the step (A8 and GEMV as separate kernels)
    ms_two = per_step_ms(run_step_two_launch, lambda i: i % ncopies)
    torch.cuda.synchronize()
    res = dict(ms_per_step=ms, step_us_repeats=spread(reps), step_bytes=step_bytes, pool_copies=ncopies,
               gbps=step_bytes / ms / 1e6, ms_two_launch=ms_two,
               gbps_two_launch=step_bytes / ms_two / 1e6, ms_warm=ms_warm,
               gbps_warm_infinity_cache=step_bytes / ms_warm / 1e6)
    # per-matrix fused GEMV launches, HBM-cold (each over its own >= 1 GiB pool),
    # averaged over graph replays
    per = {}
    for i, m in enumerate(mats):
        cp = cold_pool(pool[i][0], pool[i])
        d = graph_mean_ms(torch, [
            (lambda k=k: B.cq_gemv_f32(cp[k], m["lay"], cb4, m["x"], y=m["y"]))
            for k in range(len(cp))])
        b = payload_bytes(m["lay"])
        per[m["label"]] = dict(us=d * 1e3, gbps=b / d / 1e6, frac=b / d / 1e6 / HBM_PEAK_GBPS,
                               launches=len(cp))
        del cp
    res["gemv_per_matrix"] = per
    return res, mats, pool


def bench_dominant(B, torch, dev, cbs, steps, mats=None, pool=None):
    """Dominant kernel: fused CQ GEMV on 4096x14336; mean duration of HBM-cold
    launches (cycling >= 1 GiB of weight copies) replayed from a HIP graph."""
    if mats is None:
        mats, pool, _, _, _ = decode_setup(B, torch, dev, cbs)
    i = [m["label"] for m in mats].index("4096x14336")
    m = mats[i]
    cp = cold_pool(pool[i][0], pool[i])
    n = max(2 * len(cp), steps)
    times = graph_repeats_ms(torch, [
        (lambda k=k: B.cq_gemv_f32(cp[k % len(cp)], m["lay"], cbs[4], m["x"], y=m["y"]))
        for k in range(n)], repeats=5)
    d_ms = sorted(times)[len(times) // 2]                               # the median replay
    lay = m["lay"]
    algo = payload_bytes(lay) + lay.cols * 4 + lay.rows * 4           # weights + fp32 x + fp32 y
    return dict(kernel="cq_gemv_kernel, fused A8 (cq_gemv_f32: CQ 4-bit GEMV, 4096x14336, batch 1)",
                avg_us=d_ms * 1e3, us_repeats=spread(times), launches=n * len(times), algo_bytes=algo,
                achieved_gbps=algo / d_ms / 1e6)


def bench_c1(B, torch, dev, cbs):
    """The single CQ-W4A8 GEMV: 512x512 cb4, batch 1 (one cq_gemv_f32 launch,
    135 KB of weights: launch-bound).  Graph-timed warm (one copy) and
    HBM-cold (cycling >= 1 GiB of copies); y is returned for the parity check
    in the cpu_baseline leg."""
    from bit_quantized_matmul_amd import inputs
    wl = inputs.cq_single()
    w, xh = wl.weights[0][1], wl.acts[0]
    lay = B.cq_pack_info(512, 512, 128, 4)
    blob = B.cq_pack(torch.from_numpy(w).to(dev), lay, cbs[4])
    x = torch.from_numpy(xh).to(dev)
    y = torch.empty((1, 512), dtype=torch.float32, device=dev)
    warm = graph_repeats_ms(torch, [(lambda: B.cq_gemv_f32(blob, lay, cbs[4], x, y=y)) for _ in range(100)])
    pool = cold_pool(blob)
    cold = graph_repeats_ms(torch, [(lambda k=k: B.cq_gemv_f32(pool[k], lay, cbs[4], x, y=y))
                                    for k in range(len(pool))], repeats=3)
    B.cq_gemv_f32(blob, lay, cbs[4], x, y=y)
    torch.cuda.synchronize()
    nb = payload_bytes(lay)
    d = sorted(cold)[1]
    res = dict(workload="cq_single_512x512_b1 (cb4, group 128, fp32 x -> A8 fused)", bytes=nb,
               us_warm=spread(warm), us_hbm_cold=spread(cold), gbps_hbm_cold=nb / d / 1e6,
               pool_copies=len(pool))
    del pool
    return res, dict(w=w, x=xh, y=y.cpu().numpy(), blob=blob.cpu().numpy())


def bench_read_floor(torch, dev, rows: int = 4096, cols: int = 1852):
    """Vendor kernels reading about the dominant kernel's bytes (4096 x 1852
    fp32 = 30.3 MB, against the 4096x14336 GEMV's 30.35 MB), HBM-cold (cycling
    >= 1 GiB of buffers), timed like the GEMV: torch's row sums (the fastest
    plain streaming read found among torch's reductions) and torch's fp32
    GEMV; and a trivial kernel, the launch floor of any one launch."""
    nbytes = rows * cols * 4
    n = pool_copies(nbytes)
    pool = [torch.zeros((rows, cols), dtype=torch.float32, device=dev) for _ in range(n)]
    v = torch.zeros(cols, dtype=torch.float32, device=dev)
    d_sum = graph_mean_ms(torch, [(lambda k=k: pool[k].sum(dim=1)) for k in range(n)])
    d_mv = graph_mean_ms(torch, [(lambda k=k: torch.mv(pool[k], v)) for k in range(n)])
    tiny = torch.zeros(1, dtype=torch.float32, device=dev)
    e = graph_mean_ms(torch, [tiny.zero_ for _ in range(64)])
    del pool
    torch.cuda.empty_cache()
    rate = lambda d: dict(us=d * 1e3, gbps=nbytes / d / 1e6, frac=nbytes / d / 1e6 / HBM_PEAK_GBPS)
    return dict(bytes=nbytes, row_sums=rate(d_sum), fp32_gemv_torch_mv=rate(d_mv), empty_launch_us=e * 1e3)


def bench_prefill(B, torch, dev, cbs, steps, warmup):
    from bit_quantized_matmul_amd import inputs
    wl = inputs.cq_prefill()
    x = torch.from_numpy(wl.acts[0]).to(dev)
    q, s = B.act_fwht_quant_a8(x)
    out = {}
    t = Timer()
    for label, w in wl.weights:
        rows, cols = w.shape
        lay = B.cq_pack_info(rows, cols, 128, 4)
        blob = B.cq_pack(torch.from_numpy(w).to(dev), lay, cbs[4])
        y = torch.empty((q.shape[0], rows), dtype=torch.float32, device=dev)
        for _ in range(warmup):
            B.cq_gemm(blob, lay, cbs[4], q, s, y=y)
        times = graph_repeats_ms(torch, [(lambda: B.cq_gemm(blob, lay, cbs[4], q, s, y=y))
                                         for _ in range(max(steps, 10))], repeats=5)
        ms = sorted(times)[len(times) // 2]
        flops = 2.0 * q.shape[0] * rows * cols
        tf = flops / ms / 1e9
        out[label] = dict(m=int(q.shape[0]), us=ms * 1e3, us_repeats=spread(times), tflops=tf,
                          frac=tf / MFMA_F16_PEAK_TFLOPS)
        del blob, y
    # base-3 ternary at the wide shape: the base-3 GEMM (int8 MFMA, 8 k slots
    # a weight byte: 130 real of 224 slots a group; frac counts real MACs)
    label, w = wl.weights[0]
    rows, cols = w.shape
    lay = B.cq_pack_info(rows, cols, 128, 6)
    blob = B.cq_pack(torch.from_numpy(w).to(dev), lay, None)
    y = torch.empty((q.shape[0], rows), dtype=torch.float32, device=dev)
    B.cq_gemm(blob, lay, None, q, s, y=y)
    times = graph_repeats_ms(torch, [(lambda: B.cq_gemm(blob, lay, None, q, s, y=y))
                                     for _ in range(max(steps, 10))], repeats=5)
    ms = sorted(times)[len(times) // 2]
    tf = 2.0 * q.shape[0] * rows * cols / ms / 1e9
    out[f"ternary_base3_{label}"] = dict(m=int(q.shape[0]), us=ms * 1e3, us_repeats=spread(times), tops=tf,
                                         frac_int8_peak=tf / INT8_MFMA_PEAK_TOPS)
    del blob, y
    # context: the dense fp16 GEMM the format avoids (hipBLASLt via torch.mm,
    # contiguous [M, K] x [K, N] operands, fp16 weights of the same shape)
    m = q.shape[0]
    for label, w in wl.weights:
        rows, cols = w.shape
        a16 = x.to(torch.float16)
        wt16 = torch.from_numpy(w).to(dev).to(torch.float16).t().contiguous()
        d = graph_mean_ms(torch, [(lambda: torch.mm(a16, wt16)) for _ in range(20)])
        tf = 2.0 * m * rows * cols / d / 1e9
        out[f"dense_fp16_torch_mm_{label}"] = dict(m=int(m), us=d * 1e3, tflops=tf, frac=tf / MFMA_F16_PEAK_TFLOPS)
        del wt16
    # A8 on the 512 x 4096 prefill activations (graph-timed: eager launches
    # from Python are host-bound at this size)
    ms = graph_mean_ms(torch, [(lambda: B.act_fwht_quant_a8(x, q=q, scale=s)) for _ in range(max(steps, 20))])
    nb = x.numel() * 4 + q.numel() + s.numel() * 4
    out["act_fwht_quant_a8_512x4096"] = dict(us=ms * 1e3, gbps=nb / ms / 1e6)
    return out


def bench_q4_0(B, torch, dev, steps, warmup):
    from bit_quantized_matmul_amd import inputs
    wl = inputs.minueza_q4_0_pass()
    items = []
    total = 0
    for (label, w), x in zip(wl.weights, wl.acts):
        rows, cols = w.shape
        blocks = B.q4_0_pack(torch.from_numpy(w).to(dev))
        items.append((rows, cols, blocks, torch.from_numpy(x).to(dev),
                      torch.empty((1, rows), dtype=torch.float32, device=dev)))
        total += blocks.numel()

    def one_pass():
        for rows, cols, blocks, x, y in items:
            B.q4_0_gemv(blocks, rows, cols, x, y=y)

    one_pass()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_pass()
    for _ in range(warmup):
        g.replay()
    t = Timer()
    t.start()
    for _ in range(steps):
        g.replay()
    ms = t.stop_ms() / steps
    t.start()
    for _ in range(steps):
        one_pass()
    ms_eager = t.stop_ms() / steps
    # the tied head alone (the only matrix large enough to be bandwidth-bound),
    # graph-timed: eager launches from Python are host-bound at this size
    # each distinct matrix shape alone (the first layer's matrices), graph-timed, warm
    per_matrix = {}
    for (label, w), it in zip(wl.weights[:len(inputs.MINUEZA_LAYER_SHAPES)], items):
        r_, c_, b_, x_, y_ = it
        key = f"{r_}x{c_}"
        if key in per_matrix:
            continue
        ms_m = graph_mean_ms(torch, [(lambda: B.q4_0_gemv(b_, r_, c_, x_, y=y_)) for _ in range(max(steps, 20))])
        per_matrix[key] = dict(us=ms_m * 1e3, gbps=b_.numel() / ms_m / 1e6)
    rows, cols, blocks, x, y = items[-1]
    ms_head = graph_mean_ms(torch, [(lambda: B.q4_0_gemv(blocks, rows, cols, x, y=y)) for _ in range(max(steps, 20))])
    per_matrix[f"{rows}x{cols}"] = dict(us=ms_head * 1e3, gbps=blocks.numel() / ms_head / 1e6)
    # HBM-cold: >= 1 GiB of distinct copies of the whole pass, one graph of
    # consecutive passes each on the next copy (the 256 MB Infinity Cache
    # cannot hold them); the head alone likewise over its own pool
    ncop = pool_copies(total)
    copies = [[it[2]] + [it[2].clone() for _ in range(ncop - 1)] for it in items]
    torch.cuda.synchronize()

    def cold_pass(k):
        for i, (r_, c_, _, x_, y_) in enumerate(items):
            B.q4_0_gemv(copies[i][k], r_, c_, x_, y=y_)

    cold = graph_repeats_ms(torch, [(lambda k=k: cold_pass(k)) for k in range(ncop)], repeats=3)
    ms_cold = sorted(cold)[1]
    # stacked: each layer's q, k, v as one [520, 312] matrix and gate, up as
    # one [2184, 312] (the matrices that read the same activations, stacked
    # as inference engines do: row-major blocks concatenate): 41 launches of
    # the same kernels over the same bytes
    per = len(inputs.MINUEZA_LAYER_SHAPES)
    stacked = []
    for base in range(0, len(items) - 1, per):
        for grp in ((0, 1, 2), (3,), (4, 5), (6,)):
            its = [items[base + i] for i in grp]
            rows_s = sum(it[0] for it in its)
            stacked.append((rows_s, its[0][1], torch.cat([it[2] for it in its]), its[0][3],
                            torch.empty((1, rows_s), dtype=torch.float32, device=dev)))
    stacked.append(items[-1])
    st_copies = [[it[2]] + [it[2].clone() for _ in range(ncop - 1)] for it in stacked]
    torch.cuda.synchronize()

    def stacked_pass(k):
        for i, (r_, c_, _, x_, y_) in enumerate(stacked):
            B.q4_0_gemv(st_copies[i][k], r_, c_, x_, y=y_)

    ms_st = graph_mean_ms(torch, [(lambda: stacked_pass(0)) for _ in range(max(steps, 10))])
    st_cold = graph_repeats_ms(torch, [(lambda k=k: stacked_pass(k)) for k in range(ncop)], repeats=3)
    ms_st_cold = sorted(st_cold)[1]
    del st_copies
    head_pool = copies[-1] + [blocks.clone() for _ in range(max(0, pool_copies(blocks.numel()) - ncop))]
    hc = graph_repeats_ms(torch, [(lambda k=k: B.q4_0_gemv(head_pool[k], rows, cols, x, y=y))
                                  for k in range(len(head_pool))], repeats=3)
    ms_head_cold = sorted(hc)[1]
    del copies, head_pool
    torch.cuda.synchronize()
    return dict(launches=len(items), bytes=total, us_graph=ms * 1e3, gbps_graph=total / ms / 1e6,
                per_matrix_warm=per_matrix,
                us_eager=ms_eager * 1e3, head_us=ms_head * 1e3,
                head_gbps=blocks.numel() / ms_head / 1e6,
                note="us_graph / head_us: weights warm in the Infinity Cache (the 13 MB pass fits); "
                     "*_hbm_cold: cycling >= 1 GiB of copies",
                pass_us_hbm_cold=ms_cold * 1e3, pass_gbps_hbm_cold=total / ms_cold / 1e6,
                pass_copies=ncop, stacked_launches=len(stacked), stacked_us_graph=ms_st * 1e3,
                stacked_us_hbm_cold=ms_st_cold * 1e3, stacked_gbps_hbm_cold=total / ms_st_cold / 1e6,
                head_us_hbm_cold=ms_head_cold * 1e3,
                head_gbps_hbm_cold=blocks.numel() / ms_head_cold / 1e6,
                head_frac_hbm_cold=blocks.numel() / ms_head_cold / 1e6 / HBM_PEAK_GBPS)


FP32_MFMA_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix, published


def bench_q4_0_prefill(B, torch, dev, steps, warmup, m=512):
    """The Minueza Q4_0 pass as prefill: m prompt tokens through the same 71
    matrices, one q4_0_gemm launch each (fp32 activations, fp32 matrix cores)."""
    from bit_quantized_matmul_amd import inputs
    wl = inputs.minueza_q4_0_pass()
    rng = inputs.rng_for(12)
    items, flops = [], 0
    for (label, w) in wl.weights:
        rows, cols = w.shape
        blocks = B.q4_0_pack(torch.from_numpy(w).to(dev))
        x = torch.from_numpy(inputs.activations(rng, m, cols)).to(dev)
        items.append((label, rows, cols, blocks, x,
                      torch.empty((m, rows), dtype=torch.float32, device=dev)))
        flops += 2 * m * rows * cols

    def one_pass():
        for _, rows, cols, blocks, x, y in items:
            B.q4_0_gemm(blocks, rows, cols, x, y=y)

    one_pass()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        one_pass()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t = Timer()
    t.start()
    for _ in range(steps):
        g.replay()
    ms = t.stop_ms() / steps
    tf = flops / ms / 1e9
    # stacked: each layer's q, k, v as one [520, 312] matrix and gate, up as
    # one [2184, 312] (the matrices that read the same activations), 41 launches
    per = len(inputs.MINUEZA_LAYER_SHAPES)
    stacked = []
    for base in range(0, len(items) - 1, per):
        for grp in ((0, 1, 2), (3,), (4, 5), (6,)):
            its = [items[base + i] for i in grp]
            rows_s = sum(it[1] for it in its)
            stacked.append((rows_s, its[0][2], torch.cat([it[3] for it in its]), its[0][4],
                            torch.empty((m, rows_s), dtype=torch.float32, device=dev)))
    stacked.append(items[-1][1:])

    def stacked_pass():
        for rows, cols, blocks, x, y in stacked:
            B.q4_0_gemm(blocks, rows, cols, x, y=y)

    ms_st = graph_mean_ms(torch, [stacked_pass] * max(steps, 5))
    # the head alone (32002 x 312: the one launch large enough to fill the chip)
    _, rows, cols, blocks, x, y = items[-1]
    d = graph_mean_ms(torch, [(lambda: B.q4_0_gemm(blocks, rows, cols, x, y=y))] * 8)
    head_tf = 2 * m * rows * cols / d / 1e9
    return dict(tokens=m, launches=len(items), gflop=flops / 1e9, us_graph=ms * 1e3,
                tflops=tf, frac=tf / FP32_MFMA_PEAK_TFLOPS, stacked_launches=len(stacked),
                stacked_us_graph=ms_st * 1e3, stacked_tflops=flops / ms_st / 1e9,
                stacked_frac=flops / ms_st / 1e9 / FP32_MFMA_PEAK_TFLOPS, head_us=d * 1e3,
                head_tflops=head_tf, head_frac=head_tf / FP32_MFMA_PEAK_TFLOPS)


INT8_MFMA_PEAK_TOPS = 5000.0   # MI355X dense int8 matrix, published


def bench_q4_0_a8(B, torch, dev, steps, warmup, m=512):
    """The Minueza Q4_0 pass with int8 activations (A8, no rotation): decode
    (one token) and prefill (m tokens), graph-timed; each matrix's input is
    quantized with act_fwht_quant_a8 (group 1) then multiplied.  Times with
    the A8 launches and for the products alone are both given, and for decode
    the fused entry (one launch a matrix)."""
    from bit_quantized_matmul_amd import inputs
    wl = inputs.minueza_q4_0_pass()
    rng = inputs.rng_for(13)
    dec, pre, total, flops = [], [], 0, 0
    for (label, w), x in zip(wl.weights, wl.acts):
        rows, cols = w.shape
        blocks = B.q4_0_pack(torch.from_numpy(w).to(dev))
        total += blocks.numel()
        xd = torch.from_numpy(x).to(dev)
        q1, s1 = B.act_fwht_quant_a8(xd, group=1)
        dec.append((rows, cols, blocks, xd, q1, s1, torch.empty((1, rows), dtype=torch.float32, device=dev)))
        xp = torch.from_numpy(inputs.activations(rng, m, cols)).to(dev)
        qp, sp = B.act_fwht_quant_a8(xp, group=1)
        pre.append((rows, cols, blocks, xp, qp, sp, torch.empty((m, rows), dtype=torch.float32, device=dev)))
        flops += 2 * m * rows * cols
    torch.cuda.synchronize()

    def one(items, gemm, with_a8):
        def run():
            for rows, cols, blocks, x, q, s, y in items:
                if with_a8:
                    B.act_fwht_quant_a8(x, group=1, q=q, scale=s)
                (B.q4_0_gemm_a8 if gemm else B.q4_0_gemv_a8)(blocks, rows, cols, q, s, y=y)
        return run

    def t(fn):
        return sorted(graph_repeats_ms(torch, [fn] * max(steps, 5), repeats=5))[2]

    def fused():
        for rows, cols, blocks, x, q, s, y in dec:
            B.q4_0_gemv_a8_f32(blocks, rows, cols, x, y=y)

    d_a8, d_prod, d_fused = t(one(dec, False, True)), t(one(dec, False, False)), t(fused)
    # stacked as in the fp32 passes: q, k, v one matrix, gate, up one (41 launches a pass)
    per = len(inputs.MINUEZA_LAYER_SHAPES)

    def stack(items, nt):
        out = []
        for base in range(0, len(items) - 1, per):
            for grp in ((0, 1, 2), (3,), (4, 5), (6,)):
                its = [items[base + i] for i in grp]
                rows_s = sum(it[0] for it in its)
                out.append((rows_s, its[0][1], torch.cat([it[2] for it in its]), its[0][3], its[0][4], its[0][5],
                            torch.empty((nt, rows_s), dtype=torch.float32, device=dev)))
        out.append(items[-1])
        return out

    dec_st, pre_st = stack(dec, 1), stack(pre, m)

    def fused_st():
        for rows, cols, blocks, x, q, s, y in dec_st:
            B.q4_0_gemv_a8_f32(blocks, rows, cols, x, y=y)

    d_fused_st, p_prod_st = t(fused_st), t(one(pre_st, True, False))
    p_a8, p_prod = t(one(pre, True, True)), t(one(pre, True, False))
    rows, cols, blocks, x, q, s, y = pre[-1]
    head = sorted(graph_repeats_ms(torch, [lambda: B.q4_0_gemm_a8(blocks, rows, cols, q, s, y=y)] * 8))[2]
    head_tops = 2 * m * rows * cols / head / 1e9
    return dict(
        decode=dict(launches=2 * len(dec), bytes=total, us_with_a8=d_a8 * 1e3, us_products_only=d_prod * 1e3,
                    gbps_products_only=total / d_prod / 1e6, us_fused=d_fused * 1e3, fused_launches=len(dec),
                    us_fused_stacked=d_fused_st * 1e3, stacked_launches=len(dec_st),
                    note="weights warm in the Infinity Cache; us_fused: q4_0_gemv_a8_f32, the codes formed "
                         "in each product's launch"),
        prefill=dict(tokens=m, gop=flops / 1e9, us_with_a8=p_a8 * 1e3, us_products_only=p_prod * 1e3,
                     us_products_only_stacked=p_prod_st * 1e3,
                     tops_products_only=flops / p_prod / 1e9,
                     frac_int8_peak=flops / p_prod / 1e9 / INT8_MFMA_PEAK_TOPS,
                     head_us=head * 1e3, head_tops=head_tops, head_frac_int8_peak=head_tops / INT8_MFMA_PEAK_TOPS))


PCIE_PEAK_GBPS = 63.0   # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes x 128/130 / 8


def bench_kmcu_load(B, torch, dev, steps):
    """The tied Minueza image (92 tensors, 12.58 MiB: the file the KMCU page's
    section 1 prints) built from synthetic weights packed on the device, then
    parsed and moved into HBM with kmcu_upload_data.  The copy crosses the
    host link, so it is rated against PCIe, not HBM."""
    import time
    from bit_quantized_matmul_amd import inputs, kmcu
    wl = inputs.minueza_q4_0_pass(seed=3)
    packed = {lab: (w.shape, B.q4_0_pack(torch.from_numpy(w).to(dev)).cpu().numpy().tobytes())
              for lab, w in wl.weights}
    dim = inputs.MINUEZA_HEAD[2]
    ones = np.ones(dim, "<f4").tobytes()

    def q4(name, lab):
        (rows, cols), payload = packed[lab]
        return (name, kmcu.Q4, rows, cols, payload)

    tensors = [q4("tok_embed", "head")]
    for i in range(inputs.MINUEZA_LAYERS):
        tensors.append((f"L{i}.in_ln", kmcu.F32, 1, dim, ones))
        tensors += [q4(f"L{i}.{n}", f"L{i}.{n}") for n in ("q", "k", "v", "o")]
        tensors.append((f"L{i}.post_ln", kmcu.F32, 1, dim, ones))
        tensors += [q4(f"L{i}.{n}", f"L{i}.{n}") for n in ("gate", "up", "down")]
    tensors.append(("final_norm", kmcu.F32, 1, dim, ones))
    model = dict(n_layers=inputs.MINUEZA_LAYERS, dim=dim, n_heads=12, n_kv_heads=4, head_dim=26,
                 ffn_dim=1092, vocab_size=32002, max_seq=2048, bos_id=1, eos_id=32000, tied_embed=1,
                 rope_theta=10000.0, norm_eps=1e-6)
    file = bytes(kmcu.write(model, tensors))
    pinned = torch.empty((len(file),), dtype=torch.uint8, pin_memory=True)
    pinned.numpy()[:] = np.frombuffer(file, np.uint8)
    h = B.kmcu_header(file)
    data_bytes = len(file) - h.data_offset
    dst = torch.empty((data_bytes,), dtype=torch.uint8, device=dev)

    def rate(src):
        B.kmcu_upload_data(src, dst)                   # warm: page-in, staging buffers
        t0 = time.perf_counter()
        for _ in range(steps):
            B.kmcu_upload_data(src, dst)               # waits for its copy
        sec = (time.perf_counter() - t0) / steps
        return sec * 1e6, data_bytes / sec / 1e9

    pageable_us, pageable_gbps = rate(file)
    pinned_us, pinned_gbps = rate(pinned)
    t0 = time.perf_counter()
    _, loaded = B.kmcu_load(pinned)                    # parse + allocate + one copy
    load_us = (time.perf_counter() - t0) * 1e6
    ok = all(torch.equal(view.cpu(), pinned[t.offset:t.offset + t.nbytes]) for t, view in loaded.values())
    return dict(file_mib=len(file) / 2 ** 20, tensors=h.n_tensors, total_params=h.total_params,
                data_bytes=data_bytes, pageable_us=pageable_us, pageable_gbps=pageable_gbps,
                pinned_us=pinned_us, pinned_gbps=pinned_gbps, pinned_frac=pinned_gbps / PCIE_PEAK_GBPS,
                pcie_peak_gbps=PCIE_PEAK_GBPS, kmcu_load_us=load_us, bytes_match=bool(ok))


def bench_sweep(B, torch, dev, cbs, steps):
    from bit_quantized_matmul_amd import inputs
    wl = inputs.cq_bit_sweep()
    w = torch.from_numpy(wl.weights[0][1]).to(dev)
    rows, cols = w.shape
    acts = [torch.from_numpy(a).to(dev) for a in wl.acts]
    names = {1: "binary", 2: "cb2", 3: "cb3", 4: "cb4", 5: "ternary", 6: "ternary_base3"}
    out = {}
    for code in (1, 2, 3, 4, 5, 6):
        lay = B.cq_pack_info(rows, cols, 128, code)
        cb = codebook_for(code, cbs)
        blob = B.cq_pack(w, lay, cb)
        nb = payload_bytes(lay)
        n = pool_copies(nb)
        pool = [blob] + [blob.clone() for _ in range(n - 1)]
        for a in acts:
            batch = a.shape[0]
            q, s = B.act_fwht_quant_a8(a)
            y = torch.empty((batch, rows), dtype=torch.float32, device=dev)
            d = graph_mean_ms(torch, [
                (lambda k=k: B.cq_gemv(pool[k], lay, cb, q, s, y=y))
                for k in range(n)])
            out[f"{names[code]}_b{batch}"] = dict(us=d * 1e3, gbps=nb / d / 1e6,
                                                  frac=nb / d / 1e6 / HBM_PEAK_GBPS)
            if code in (1, 5):                   # the lookup-table kernel on the same weights
                d = graph_mean_ms(torch, [
                    (lambda k=k: B.cq_gemv_lut(pool[k], lay, q, s, y=y))
                    for k in range(n)])
                out[f"{names[code]}_lut_b{batch}"] = dict(us=d * 1e3, gbps=nb / d / 1e6,
                                                          frac=nb / d / 1e6 / HBM_PEAK_GBPS)
        del pool, blob
        torch.cuda.synchronize()
    return out


def bench_batched(B, torch, dev, cbs, steps, batches=(4, 16, 32)):
    """Several decode tokens at once on the 8B layer shapes (cb4): one cq_gemv per
    matrix, whose one pass over the weights on the matrix cores serves every token
    (32 tokens: two 16-token halves on the same weight fragments; their
    activations come from a stream of their own, so the 4- and 16-token inputs
    stay as they were)."""
    from bit_quantized_matmul_amd import inputs
    rng = inputs.rng_for(11)
    rng32 = inputs.rng_for(12)
    out = {}
    for (rows, cols) in inputs.DECODE_8B_SHAPES:
        w = torch.from_numpy(inputs.weight_matrix(rng, rows, cols, outliers=True)).to(dev)
        lay = B.cq_pack_info(rows, cols, 128, 4)
        blob = B.cq_pack(w, lay, cbs[4])
        del w
        nb = payload_bytes(lay)
        n = pool_copies(nb)
        pool = [blob] + [blob.clone() for _ in range(n - 1)]
        for batch in batches:
            x = torch.from_numpy(inputs.activations(rng if batch <= 16 else rng32, batch, cols)).to(dev)
            q, s = B.act_fwht_quant_a8(x)
            y = torch.empty((batch, rows), dtype=torch.float32, device=dev)
            d = graph_mean_ms(torch, [
                (lambda k=k: B.cq_gemv(pool[k], lay, cbs[4], q, s, y=y))
                for k in range(n)])
            out[f"{rows}x{cols}_b{batch}"] = dict(us=d * 1e3, gbps=nb / d / 1e6,
                                                  frac=nb / d / 1e6 / HBM_PEAK_GBPS)
        del pool, blob
        torch.cuda.synchronize()
    for batch in batches:
        us = sum(v["us"] for k, v in out.items() if k.endswith(f"_b{batch}"))
        out[f"step_b{batch}"] = dict(us=us, tokens_per_s=batch / us * 1e6)
    return out


def bench_copy(torch, dev, steps):
    """Plain 1 GiB device copy: the calibration kernel for FETCH_SIZE / WRITE_SIZE."""
    a = torch.empty(POOL_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    t = Timer()
    b.copy_(a)
    t.start()
    for _ in range(steps):
        b.copy_(a)
    ms = t.stop_ms() / steps
    return dict(bytes_read=POOL_BYTES, us=ms * 1e3, gbps=2 * POOL_BYTES / ms / 1e6)


# -------------------------------------------------------------- cpu baseline

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def c1_parity(c1, matmul, cq, a8, codebook):
    """The C1 GEMV's device result against the oracle, element by element:
    the oracle fits the codebook on the same samples and encodes W itself
    (its blob must equal the device's); the error is stated as
    max |y - ref| / magnitude and relative L2."""
    from bit_quantized_matmul_amd import inputs
    lv = codebook.shipped_table(codebook.lloyd_max_fit(inputs.gaussian_samples(), 16))
    idx, n16 = cq.encode(c1["w"], 128, 4, lv)
    blob_ok = bool(np.array_equal(cq.make_blob(idx, n16, 128, 4), c1["blob"]))
    q, s = a8.act_quant_a8(c1["x"], 128, "fp32")
    t0 = time.perf_counter()
    ref = matmul.cq_reference(idx, n16, 128, 4, lv, q, s)
    oracle_s = time.perf_counter() - t0
    mag = matmul.cq_magnitude(idx, n16, 128, 4, lv, q, s)
    err = np.abs(c1["y"].astype(np.float64) - ref)
    return dict(blob_bit_exact=blob_ok, max_err_over_magnitude=float(np.max(err / mag)),
                bound=1e-5, rel_l2=matmul.rel_l2(c1["y"], ref), max_abs_err=float(err.max()),
                oracle_product_ms=oracle_s * 1e3)


def cpu_baseline(reps: int = 60, rows_per_matrix: int = 512, c1=None):
    """The oracle (unchanged) on a bounded sample of the decode step: the
    plain definition (the reported value), the rotated-domain form, and the
    plain definition on one thread.  With `c1` (the 512x512 GEMV's device
    result) it also checks that result against the oracle."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from bit_quantized_matmul_amd import inputs
    from oracle import a8, codebook, cq, matmul
    wl = inputs.cq_decode_8b()
    lv = codebook.shipped_table(codebook.lloyd_max_quadrature(16))
    sample = []
    nbytes = 0
    for (label, w), x in zip(wl.weights, wl.acts):
        ws = w[:rows_per_matrix]
        idx, n16 = cq.encode(ws, 128, 4, lv)          # input preparation, not timed
        sample.append((idx, n16, x))
        nbytes += cq.pack_info(ws.shape[0], ws.shape[1], 128, 4)["idx_bytes"] + 2 * n16.size

    def timed(product, n):
        t0 = time.perf_counter()
        for _ in range(n):
            for idx, n16, x in sample:
                q, s = a8.act_quant_a8(x, 128, "fp32")
                product(idx, n16, 128, 4, lv, q, s)
        return time.perf_counter() - t0

    dt = timed(matmul.cq_reference, reps)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    rot_reps = max(1, reps // 3)
    dt_rot = timed(matmul.cq_rotated, rot_reps)
    one_reps = max(1, reps // 10)
    with threadpool_limits(limits=1):
        dt_one = timed(matmul.cq_reference, one_reps)
    c1_check = None if c1 is None else c1_parity(c1, matmul, cq, a8, codebook)
    return dict(value=reps * nbytes / dt / 1e9, unit="GB/s", cores=threads, kind="oracle",
                c1_parity=c1_check,
                seconds=dt,
                sample=f"first {rows_per_matrix} rows of each decode matrix (4096x4096, 1024x4096, "
                       f"14336x4096, 4096x14336), oracle A8 + plain-definition product "
                       f"(decode W_hat by FWHT, fp64 matmul), {reps} repetitions, "
                       f"{nbytes} packed bytes per repetition",
                rotated_domain=dict(value=rot_reps * nbytes / dt_rot / 1e9, seconds=dt_rot, reps=rot_reps,
                                    cores=threads),
                single_thread=dict(value=one_reps * nbytes / dt_one / 1e9, seconds=dt_one, reps=one_reps,
                                   cores=1),
                host=dict(cpu_count=os.cpu_count(), affinity=len(os.sched_getaffinity(0)),
                          blas_threads=threads, model=cpu_model()))


# ---------------------------------------------------------------------- main

def traffic_for_dominant():
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counters,
    only while the kernel source is the one that was profiled."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE))
        digest = hashlib.sha256(b"".join(open(f, "rb").read() for f in GEMV_SOURCES)).hexdigest()
        if rec.get("source_sha256") != digest:
            return None
        return float(rec["bytes_per_launch"])
    except Exception:
        return None


def main():
    global EAGER
    args = parse()
    EAGER = args.no_graph
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)
    import torch

    from bit_quantized_matmul_amd import binding as B
    B.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")

    if args.only == "copy":
        print(json.dumps(bench_copy(torch, dev, args.steps)))
        return
    if args.only == "kmcu":
        print(json.dumps(bench_kmcu_load(B, torch, dev, args.steps)))
        return
    if args.only == "floor":
        print(json.dumps(bench_read_floor(torch, dev)))
        return
    cbs = fit_codebooks(B, torch, dev)
    log("codebooks fitted on device")
    if args.only == "dominant":
        print(json.dumps(bench_dominant(B, torch, dev, cbs, args.steps)))
        return
    if args.only == "prefill":
        print(json.dumps(bench_prefill(B, torch, dev, cbs, args.steps, args.warmup)))
        return
    if args.only == "q4_0":
        print(json.dumps(bench_q4_0(B, torch, dev, args.steps, args.warmup)))
        return
    if args.only == "q4_0_prefill":
        print(json.dumps(bench_q4_0_prefill(B, torch, dev, args.steps, args.warmup)))
        return
    if args.only == "q4_0_a8":
        print(json.dumps(bench_q4_0_a8(B, torch, dev, args.steps, args.warmup)))
        return
    if args.only == "sweep":
        print(json.dumps(bench_sweep(B, torch, dev, cbs, args.steps)))
        return
    if args.only == "batched":
        print(json.dumps(bench_batched(B, torch, dev, cbs, args.steps)))
        return
    if args.only == "c1":
        print(json.dumps(bench_c1(B, torch, dev, cbs)[0]))
        return

    dec, mats, pool = bench_decode(B, torch, dev, cbs, args.steps, args.warmup)
    log(f"decode step {dec['ms_per_step'] * 1e3:.1f} us, {dec['gbps']:.0f} GB/s")
    dom = bench_dominant(B, torch, dev, cbs, args.steps, mats, pool)
    log(f"dominant {dom['avg_us']:.2f} us, {dom['achieved_gbps']:.0f} GB/s")
    del mats, pool
    torch.cuda.empty_cache()
    if args.only == "decode":
        print(json.dumps(dict(decode=dec, dominant=dom)))
        return
    pre = bench_prefill(B, torch, dev, cbs, args.steps, args.warmup)
    log(f"prefill {json.dumps({k: round(v.get('tflops', 0), 1) for k, v in pre.items()})}")
    q4 = bench_q4_0(B, torch, dev, args.steps, args.warmup)
    log(f"q4_0 pass {q4['us_graph']:.1f} us (graph)")
    q4p = bench_q4_0_prefill(B, torch, dev, args.steps, args.warmup)
    log(f"q4_0 prefill pass, {q4p['tokens']} tokens: {q4p['us_graph']:.1f} us, {q4p['tflops']:.1f} TFLOP/s")
    qa8 = bench_q4_0_a8(B, torch, dev, args.steps, args.warmup)
    log(f"q4_0 A8: decode pass {qa8['decode']['us_with_a8']:.1f} us with A8 ({qa8['decode']['us_products_only']:.1f} "
        f"products only); prefill {qa8['prefill']['us_with_a8']:.1f} us ({qa8['prefill']['tops_products_only']:.1f} TOP/s)")
    sweep = bench_sweep(B, torch, dev, cbs, args.steps)
    log("sweep done")
    bat = bench_batched(B, torch, dev, cbs, args.steps)
    log(f"batched decode step: 4 tokens {bat['step_b4']['us']:.1f} us, "
        f"16 tokens {bat['step_b16']['us']:.1f} us, 32 tokens {bat['step_b32']['us']:.1f} us")
    floor = bench_read_floor(torch, dev)
    log(f"30 MB vendor reads: row sums {floor['row_sums']['us']:.2f} us, fp32 mv {floor['fp32_gemv_torch_mv']['us']:.2f} us, "
        f"empty launch {floor['empty_launch_us']:.2f} us")
    km = bench_kmcu_load(B, torch, dev, args.steps)
    log(f"kmcu load: {km['file_mib']:.2f} MiB image, pinned {km['pinned_gbps']:.1f} GB/s, "
        f"pageable {km['pageable_gbps']:.1f} GB/s")
    c1, c1_data = bench_c1(B, torch, dev, cbs)
    log(f"C1 512x512: {c1['us_warm']['median']:.2f} us warm, {c1['us_hbm_cold']['median']:.2f} us HBM-cold")
    cpu = None if args.no_cpu_baseline else cpu_baseline(c1=c1_data)
    if cpu:
        log(f"cpu baseline {cpu['value']:.4f} GB/s in {cpu['seconds']:.1f} s")

    traffic = traffic_for_dominant()
    line = {
        "metric": METRIC,
        "value": round(dec["gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32 (4-bit codebook weights, int8 activations)",
        "data": "synthetic",
        "config": {
            "workload": "cq_w4a8_decode_8b_layers_b1: 4096x4096, 1024x4096, 14336x4096, 4096x14336 "
                        "[out,in], group 128, cb4, 1% outlier rows x8; per matrix one launch of "
                        "cq_gemv_f32 (A8 fused into the CQ GEMV); "
                        f"weights cycled over {dec['pool_copies']} HBM-resident copies "
                        f"({dec['pool_copies'] * dec['step_bytes'] / 2**30:.2f} GiB), one per step; "
                        f"the timed steps are consecutive in one HIP graph, as a decode graph "
                        f"holds every layer",
            "step_weight_bytes": dec["step_bytes"],
            "batch": 1,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom["kernel"],
            "achieved": round(dom["achieved_gbps"], 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dom["achieved_gbps"] / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algo_bytes_per_launch": dom["algo_bytes"],
            "avg_launch_us": round(dom["avg_us"], 3),
            "launch_us_repeats": {k: (round(v, 3) if isinstance(v, float) else v) for k, v in dom["us_repeats"].items()},
        },
        "cpu_baseline": (None if cpu is None else
                         {k: (round(v, 6) if isinstance(v, float) else v) for k, v in cpu.items()}),
        "decode": {k: v for k, v in dec.items() if k != "gemv_per_matrix"},
        "gemv_per_matrix": dec["gemv_per_matrix"],
        "prefill_gemm": pre,
        "q4_0_minueza_pass": q4,
        "q4_0_minueza_prefill_512": q4p,
        "q4_0_a8_minueza": qa8,
        "bit_sweep_14336x4096": sweep,
        "batched_decode_cb4": bat,
        "kmcu_load_minueza_tied": km,
        "hbm_read_floor_30MB": floor,
        "c1_single_512x512": c1,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
