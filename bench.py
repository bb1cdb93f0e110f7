"""Benchmark of the affine-quantized decode path on one MI355X.

Default workload (the 7B-shaped decode FFN, batch 1): one step is the
gate+up projection (K=4096 -> N=2*14336) followed by the down projection
(K=14336 -> N=4096), both int4 codes with fp16 scale and bias per group of
64, fp16 activations, fp32 outputs. Sixteen distinct weight sets (1.59 GB,
far above the 256 MB Infinity Cache) are cycled so every step streams its
weights from HBM. Inputs are seeded synthetic data (``synth``) resident in
HBM before timing starts. Steps are replayed from a HIP graph; the timed
region is bracketed by device synchronizations and measured with HIP
events on the launch stream.

Printed: one JSON line with the achieved HBM bandwidth over the K timed
steps (algorithmic bytes over time), each projection timed alone (median of
5 trials of >= 200 launches) against both the 8 TB/s peak and the read-only
stream kernel's rate at the same byte count (the practical ceiling), the
roofline of the dominant kernel, µs per decode MoE layer (the c3 workload,
median of 5 trials of 240 layer calls), and the fp64 CPU oracle timed on a
bounded sample of the same workload, with the host CPU model.

Other workloads (``--config``): c1 (4096x4096 GEMV), c3 (MoE decode layer),
c4 (prefill chunk GEMM), c5 (70B-shaped sweep over batch 1/2/4/8), verify
(the verification GEMM over 16 and 32 drafted tokens on the c4 matrix),
attn (decode attention of one token through 25 sliding-window and 5
full-attention layers).
``--format mirai-m`` / ``mirai-l`` runs c1, c2 and c5 on the Mirai weight
formats of the uzu engine (4-bit codes with bf16 scale and 4-bit zero point
per group of 64; signed 8-bit codes with bf16 scale per group of 64).
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

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "achieved HBM GB/s (% of peak) for int4 g64 GEMV at batch 1; µs/MoE layer"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--config", default="c2",
                   choices=["c1", "c2", "c3", "c4", "c4moe", "c5", "verify", "attn", "stream"])
    p.add_argument("--sets", type=int, default=0, help="weight sets cycled (0 = workload default)")
    p.add_argument("--format", default="affine", choices=["affine", "mirai-m", "mirai-l"],
                   help="weight format of the dense GEMV workloads (c1, c2, c5)")
    p.add_argument("--rht", action="store_true",
                   help="Mirai formats: fuse RMSNorm + the block-32 random Hadamard rotation "
                        "ahead of the GEMV (qgemv_mirai_*_rht)")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-moe", action="store_true",
                   help="c2: leave the decode MoE layer figure out of the line")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--eager", action="store_true",
                   help="launch every step from the host instead of replaying HIP graphs "
                        "(shows the launch overhead the graphs remove)")
    return p.parse_args()


def matrix_bytes(N: int, K: int, bits: int = 4, fmt: str = "affine") -> int:
    """Algorithmic bytes of one packed matrix: codes + per-group parameters
    (affine: fp16 scale + fp16 bias; Mirai-M: bf16 scale + packed 4-bit zero
    points, rows padded to whole words; Mirai-L: bf16 scale)."""
    G = K // 64
    if fmt == "mirai-m":
        return N * K // 2 + 2 * N * G + 4 * N * ((G + 7) // 8)
    if fmt == "mirai-l":
        return N * K + 2 * N * G
    return N * K * bits // 8 + 2 * 2 * N * G


def gemv_bytes(N: int, K: int, batch: int, bits: int = 4, fmt: str = "affine", rht: bool = False) -> int:
    """Per launch: the matrix, fp16 activations in, fp32 outputs; with the
    rotation prologue also the RMSNorm weights (fp16) and the sign bits."""
    extra = K * 2 + K // 8 if rht else 0
    return matrix_bytes(N, K, bits, fmt) + batch * K * 2 + batch * N * 4 + extra


def source_hash(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


GEMV_SOURCES = ["affine_quantized_gemv_qgemv_amd/csrc/gemv.hip",
                "affine_quantized_gemv_qgemv_amd/csrc/gemv_kernel.h",
                "affine_quantized_gemv_qgemv_amd/csrc/gemv_affine4.hip",
                "affine_quantized_gemv_qgemv_amd/csrc/common.h"]


def stored_traffic(name: str, sources):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("source_hash") != source_hash(sources):
        return None
    return d.get("hbm_bytes_per_launch")


EAGER = False   # set from --eager


class Timer:
    """Times a list of step callables replayed from HIP graphs on the current
    stream (or, with --eager, launched one by one from the host)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, step_fns, steps: int, warmup: int):
        torch = self.torch
        # a graph of at least 32 steps, so one replay's launch cost is spread
        # (a short cycle, e.g. one weight set, repeats its steps in order)
        step_fns = list(step_fns) * max(1, -(-32 // len(step_fns)))
        n = len(step_fns)
        for i in range(warmup):
            step_fns[i % n]()
        torch.cuda.synchronize()
        if EAGER:
            start = torch.cuda.Event(enable_timing=True)
            end = torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            start.record()
            for i in range(steps):
                step_fns[i % n]()
            end.record()
            torch.cuda.synchronize()
            return start.elapsed_time(end) / 1e3, time.perf_counter() - t0
        cyc = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cyc):
            for f in step_fns:
                f()
        rem = steps % n
        remg = None
        if rem:
            remg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(remg):
                for f in step_fns[:rem]:
                    f()
        cyc.replay()
        if remg is not None:
            remg.replay()   # every graph replayed once before the timed region
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record()
        for _ in range(steps // n):
            cyc.replay()
        if remg is not None:
            remg.replay()
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return start.elapsed_time(end) / 1e3, wall


TRIALS = 5          # trials per figure (the median is reported)
MIN_CALLS = 200     # calls per trial


def median_time(step_fns, calls: int = MIN_CALLS, trials: int = TRIALS, warmup: int = 8):
    """Median over `trials` timings of `calls` replayed calls (seconds per call),
    each trial bracketed by device synchronizations; also returns every trial."""
    import torch
    timer = Timer(torch)
    calls = max(calls, len(step_fns))
    per = []
    for t in range(trials):
        secs, _ = timer.run(step_fns, calls, warmup if t == 0 else 0)
        per.append(secs / calls)
    return float(np.median(per)), per


def cpu_model() -> str:
    """The host CPU model (from /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stream_ceiling(torch, qd, nbytes: int, min_total: int = 1 << 30):
    """The read-only stream kernel (qd_stream_read) over buffers of nbytes each,
    cycled so that their total exceeds the 256 MB Infinity Cache: median GB/s of
    5 trials of >= 200 reads."""
    nbuf = max(2, -(-min_total // nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    fns = [(lambda b=b: qd.stream_read(b, sink)) for b in bufs]
    t, _ = median_time(fns)
    del bufs
    return nbytes / t / 1e9, t


def cpu_threads():
    try:
        return len(os.sched_getaffinity(0))
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline_gemv(mats, seconds: float, threads: int = 0):
    """The fp64 oracle on the same matrices (one step = every matrix once), repeated
    until `seconds` of CPU time have passed; returns GB/s on the algorithmic bytes.
    threads = 0: every core this process may use."""
    import oracle
    oracle.set_threads(threads or cpu_threads())
    done, nbytes = 0, 0
    t0 = time.perf_counter()
    while True:
        for w, xb, *rot in mats:
            if rot:
                oracle.mirai_gemv_rht(w, xb, "f16", rot[0], rot[1], 1e-6)
                nbytes += gemv_bytes(w.N, w.K, xb.shape[0], fmt="mirai-" + w.fmt.lower(), rht=True)
            elif hasattr(w, "fmt"):
                oracle.mirai_gemv_x(w, xb)
                nbytes += gemv_bytes(w.N, w.K, xb.shape[0], fmt="mirai-" + w.fmt.lower())
            else:
                oracle.gemv_f16(w, xb)
                nbytes += gemv_bytes(w.N, w.K, xb.shape[0], w.bits)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return nbytes / el / 1e9, done, el, oracle.get_threads()


# ---------------------------------------------------------------------------
def to_dev_codes(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).cuda()


def to_dev_half(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.float16)


def to_dev_bf16(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def device_mirai(torch, gen, fmt, shape_nk):
    """Mirai weights with the synth distributions, drawn on the device: uniform
    code (and zero-point) words, scales U[0.002, 0.02] (/16 for Mirai-L)
    rounded to bf16."""
    N, K = shape_nk
    G = K // 64
    bits = 4 if fmt == "mirai-m" else 8
    wq = torch.randint(-2**31, 2**31 - 1, (N, K * bits // 32), dtype=torch.int32, device="cuda",
                       generator=gen)
    su = torch.rand((N, G), device="cuda", generator=gen) * 0.018 + 0.002
    if fmt == "mirai-l":
        su = su / 16.0
    zq = None
    if fmt == "mirai-m":
        zq = torch.randint(-2**31, 2**31 - 1, (N, (G + 7) // 8), dtype=torch.int32, device="cuda",
                           generator=gen)
    return (wq, su.to(torch.bfloat16), zq, None)


def make_sets(torch, shapes, nsets, cfg_id, fmt="affine"):
    """Weight sets cycled by the dense benchmarks. Set 0 comes from the seeded
    host generator (the CPU baseline and the parity tests use the same
    recipe); sets 1.. are drawn on the device with the same distributions
    (device_affine / device_mirai), which keeps the 21 GB of the 70B sweep
    quick to build. Each entry: (codes, scales, biases or zero points or
    None, host weights or None)."""
    import synth
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7919 * cfg_id + 1)
    sets = []
    for s in range(nsets):
        mats = []
        for j, (K, N) in enumerate(shapes):
            if s == 0 and fmt == "affine":
                w = synth.affine_weights(4, N, K, cfg=cfg_id, set_id=s, tensor_base=8 * j)
                mats.append((to_dev_codes(torch, w.wq), to_dev_half(torch, w.scales),
                             to_dev_half(torch, w.biases), w))
            elif s == 0:
                w = synth.mirai_weights("M" if fmt == "mirai-m" else "L", N, K, cfg=cfg_id,
                                        set_id=s, tensor_base=8 * j)
                mats.append((to_dev_codes(torch, w.wq), to_dev_bf16(torch, w.scales),
                             None if w.zeros is None else to_dev_codes(torch, w.zeros), w))
            elif fmt == "affine":
                mats.append(device_affine(torch, gen, 4, (N, K)))
            else:
                mats.append(device_mirai(torch, gen, fmt, (N, K)))
        sets.append(mats)
    return sets


def run_dense(args, torch, qd, shapes, batch, sets, cfg_id, fmt="affine", rht=False):
    import synth
    nsets = len(sets)
    xs, ys, xbits, rots = [], [], [], []
    for j, (K, N) in enumerate(shapes):
        xb = synth.x_f16(batch, K, cfg=cfg_id, set_id=1000 + j)
        xbits.append(xb)
        xs.append(to_dev_half(torch, xb))
        ys.append(torch.empty((batch, N), dtype=torch.float32, device="cuda"))
        if rht:
            sg = synth.rht_signs(K, cfg=cfg_id, set_id=1000 + j)
            gb = synth.rmsnorm_gamma(K, cfg=cfg_id, set_id=1000 + j)
            rots.append((to_dev_codes(torch, sg), to_dev_half(torch, gb), sg, gb))

    def step_fn(s, only=None):
        def f():
            for j in range(len(shapes)):
                if only is not None and j != only:
                    continue
                wq, sc, third = sets[s][j][:3]
                if rht:
                    sg, g = rots[j][:2]
                    if fmt == "mirai-m":
                        qd.qgemv_mirai_m_rht(wq, sc, third, xs[j], sg, g, 1e-6, out=ys[j])
                    else:
                        qd.qgemv_mirai_l_rht(wq, sc, xs[j], sg, g, 1e-6, out=ys[j])
                elif fmt == "affine":
                    qd.qgemv_affine4(wq, sc, third, xs[j], out=ys[j])
                elif fmt == "mirai-m":
                    qd.qgemv_mirai_m(wq, sc, third, xs[j], out=ys[j])
                else:
                    qd.qgemv_mirai_l(wq, sc, xs[j], out=ys[j])
        return f

    timer = Timer(torch)
    steps = args.steps
    secs, wall = timer.run([step_fn(s) for s in range(nsets)], steps, args.warmup)
    step_bytes = sum(gemv_bytes(N, K, batch, fmt=fmt, rht=rht) for K, N in shapes)
    per_shape = []
    for j, (K, N) in enumerate(shapes):
        # each projection alone: median of 5 trials of >= 200 launches
        t, trials = median_time([step_fn(s, j) for s in range(nsets)])
        nb = gemv_bytes(N, K, batch, fmt=fmt, rht=rht)
        per_shape.append(dict(K=K, N=N, us=t * 1e6, gbs=nb / t / 1e9,
                              trials_us=[round(x * 1e6, 3) for x in trials]))
    cpu = [(sets[0][j][3], xbits[j]) + ((rots[j][2], rots[j][3]) if rht else ())
           for j in range(len(shapes))]
    return dict(secs=secs, wall=wall, step_bytes=step_bytes, per_shape=per_shape,
                launches_per_step=len(shapes), cpu_mats=cpu)


def bench_chunk(args, torch, qd):
    """Prefill chunk: M=128 x K=4096 x N=14336 int4 g64 weights, bf16 activations,
    fp32 output; 16 weight sets cycled (528 MB). Beside it the 7B down projection
    over the same chunk (K=14336 -> N=4096, K split across workgroups)."""
    import synth
    M = 128
    nsets = args.sets or 16

    def one(K, N):
        sets = make_sets(torch, [(K, N)], nsets, 4)
        xb = synth.x_bf16(M, K, cfg=4, set_id=1000)
        x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(qd.chunk_workspace_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")

        def step(s):
            def f():
                wq, sc, bi = sets[s][0][:3]
                qd.qgemm_affine4_chunk(wq, sc, bi, x, out=y, workspace=ws)
            return f

        secs, _ = Timer(torch).run([step(s) for s in range(nsets)], args.steps, args.warmup)
        del sets
        return secs / args.steps

    K, N = 4096, 14336
    t = one(K, N)
    td = one(14336, 4096)
    flops = 2.0 * M * N * K
    nbytes = matrix_bytes(N, K) + M * K * 2 + M * N * 4
    tflops = flops / t / 1e12
    return {"metric": "prefill chunk GEMM TFLOP/s (bf16 MFMA, int4 g64 weights)",
            "value": round(tflops, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(t * 1e3, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"c4: prefill chunk M={M} x K={K} x N={N}, int4 g64, "
                                   f"{nsets} weight sets cycled", "us_per_call": round(t * 1e6, 2),
                       "GBps": round(nbytes / t / 1e9, 1),
                       "down_projection": {"K": 14336, "N": 4096, "us_per_call": round(td * 1e6, 2),
                                           "TFLOPs": round(flops / td / 1e12, 1),
                                           "GBps": round((matrix_bytes(4096, 14336) + M * 14336 * 2
                                                          + M * 4096 * 4) / td / 1e9, 1)}},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                         "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)},
            "cpu_baseline": None}


def bench_verify(args, torch, qd):
    """Verification GEMM over M = 16 and 32 drafted tokens, int4 g64 weights of
    the 7B FFN: up projection K=4096 -> N=14336 and down projection K=14336 ->
    N=4096, fp32 output; activations fp16 or bf16 (qgemm_affine4_verify) or
    fp16 quantized per token to int8 on the fly (qgemm_affine4_verify_i8: the
    quantization pass and the int8 GEMM both inside the timed step); 16 weight
    sets cycled per shape (528 MB). Weight-stream bound at these M."""
    import synth
    nsets = args.sets or 16
    rows = []
    for K, N in ((4096, 14336), (14336, 4096)):
        sets = make_sets(torch, [(K, N)], nsets, 4)
        for M in (16, 32):
            ws = torch.empty(max(qd.verify_i8_workspace_bytes(M, K), 16), dtype=torch.uint8, device="cuda")
            vws = torch.empty(max(qd.verify_workspace_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")
            for dt in ("f16", "bf16", "i8"):
                xb = synth.x_bf16(M, K, cfg=4, set_id=2000 + M) if dt == "bf16" else \
                    synth.x_f16(M, K, cfg=4, set_id=2000 + M)
                x = to_dev_bf16(torch, xb) if dt == "bf16" else to_dev_half(torch, xb)
                y = torch.empty((M, N), dtype=torch.float32, device="cuda")

                def step(s, x=x, y=y, dt=dt, ws=ws, vws=vws):
                    def f():
                        wq, sc, bi = sets[s][0][:3]
                        if dt == "i8":
                            qd.qgemm_affine4_verify_i8(wq, sc, bi, x, out=y, workspace=ws)
                        else:
                            qd.qgemm_affine4_verify(wq, sc, bi, x, out=y, workspace=vws)
                    return f

                secs, _ = Timer(torch).run([step(s) for s in range(nsets)], args.steps, args.warmup)
                t = secs / args.steps
                nbytes = matrix_bytes(N, K) + M * K * 2 + M * N * 4
                rows.append(dict(K=K, N=N, M=M, dtype=dt, us=round(t * 1e6, 2),
                                 GBps=round(nbytes / t / 1e9, 1),
                                 TFLOPs=round(2.0 * M * N * K / t / 1e12, 1), bytes=nbytes))
        del sets
    main_row = [r for r in rows if r["M"] == 32 and r["dtype"] == "f16" and r["K"] == 4096][0]
    gbs = main_row["GBps"]
    return {"metric": "verification GEMM achieved HBM GB/s (32 drafted tokens, int4 g64 weights)",
            "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(main_row["us"] / 1e3, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
            "data": "synthetic",
            "config": {"workload": "verify: M drafted tokens x 7B FFN up (K=4096 -> N=14336) and down "
                                   f"(K=14336 -> N=4096) projections, int4 g64, {nsets} weight sets "
                                   "cycled; dtype i8 = fp16 activations quantized per token to int8 "
                                   "inside the step", "runs": rows},
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "qgemm_affine4_verify M=32, fp16 activations, K=4096 -> N=14336",
                         "bytes_per_launch": main_row["bytes"], "avg_launch_us": main_row["us"]},
            "cpu_baseline": None}


def bench_attn(args, torch, qd):
    """Decode attention of one token through a 30-layer stack: 25 sliding-window
    layers (circular KV, window 1024) and 5 full-attention layers (linear KV of
    4096 positions, the cache full), 16 query heads over 8 key/value heads of
    dim 128, fp16 KV. Four such stacks (different sequences) are cycled so the
    756 MB of KV stream from HBM. A step = one token through the 30 layers."""
    Hq, Hkv, D, W, C = 16, 8, 128, 1024, 4096
    nstack = args.sets or 4
    layers = [("sliding", W, W)] * 25 + [("full", C, 0)] * 5
    gen = torch.Generator(device="cuda")
    gen.manual_seed(97)
    stacks = []
    for _ in range(nstack):
        st = []
        for kind, cap, window in layers:
            kc = torch.randn((Hkv, cap, D), device="cuda", generator=gen).half()
            vc = torch.randn((Hkv, cap, D), device="cuda", generator=gen).half()
            st.append((kc, vc, cap, window))
        stacks.append(st)
    q = torch.randn((Hq, D), device="cuda", generator=gen).half()
    kn = torch.randn((Hkv, D), device="cuda", generator=gen).half()
    vn = torch.randn((Hkv, D), device="cuda", generator=gen).half()
    out = torch.empty((Hq, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(qd.qattn_workspace_bytes(Hq, Hkv, D, C), dtype=torch.uint8, device="cuda")
    pos = C - 1

    def step(si, only=None):
        def f():
            for li, (kc, vc, cap, window) in enumerate(stacks[si]):
                if only is not None and layers[li][0] != only:
                    continue
                qd.qattn_decode(q, kn, vn, kc, vc, pos, window, out=out, workspace=ws)
        return f

    def kv_bytes(cap_n):
        return 2 * Hkv * cap_n * D * 2 + (Hq * D * 2 + 2 * Hkv * D * 2 + Hq * D * 4)

    step_bytes = sum(kv_bytes(cap) for _, cap, _ in layers)
    timer = Timer(torch)
    secs, _ = timer.run([step(i) for i in range(nstack)], args.steps, args.warmup)
    t = secs / args.steps
    per = {}
    for kind, cap in (("sliding", W), ("full", C)):
        nl = sum(1 for l in layers if l[0] == kind)
        sk, _ = timer.run([step(i, kind) for i in range(nstack)], args.steps, min(args.warmup, 8))
        us = sk / args.steps / nl * 1e6
        per[kind] = dict(layers=nl, positions=cap, us_per_layer=round(us, 2),
                         GBps=round(kv_bytes(cap) / us / 1e3, 1))
    gbs = step_bytes / t / 1e9
    dom = per["full"]
    return {"metric": "decode attention achieved HBM GB/s (30-layer step, fp16 KV)",
            "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(t * 1e3, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": {"workload": "attn: one decode token through 25 sliding-window (window 1024, "
                                   "circular KV) + 5 full-attention (4096 positions, linear KV) layers, "
                                   f"Hq=16, Hkv=8, D=128, fp16 KV; {nstack} stacks cycled",
                       "step_bytes": step_bytes, "us_per_step": round(t * 1e6, 2), "per_kind": per},
            "roofline": {"bound": "hbm", "achieved": dom["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dom["GBps"] / HBM_PEAK_GBS, 4), "traffic": None,
                         "kernel": "qattn_decode, full-attention layer (4096 positions)",
                         "bytes_per_launch": kv_bytes(C), "avg_launch_us": dom["us_per_layer"]},
            "cpu_baseline": None}


def device_affine(torch, gen, bits, shape_nk, extra=()):
    """Weights with the synth distributions, drawn on the device (fast enough to
    fill 30 MoE layers): uniform code words, scales U[0.002, 0.02] (x 15/255 for
    8-bit), biases -mid*s + N(0, 1e-3) rounded to fp16."""
    N, K = shape_nk
    lead = tuple(extra)
    wq = torch.randint(-2**31, 2**31 - 1, lead + (N, K * bits // 32), dtype=torch.int32,
                       device="cuda", generator=gen)
    su = torch.rand(lead + (N, K // 64), device="cuda", generator=gen) * 0.018 + 0.002
    if bits == 8:
        su = su * (15.0 / 255.0)
    s16 = su.half()
    mid = 8.0 if bits == 4 else 128.0
    b16 = (-mid * s16.float() + torch.randn(lead + (N, K // 64), device="cuda", generator=gen) * 1e-3).half()
    return wq, s16, b16


MOE_SHAPE = dict(E=128, H=2816, I=704, Is=2112, k=8, layers=30)


def build_moe(torch, qd, prefill: bool, nlayers: int):
    """MoE layers with the synth distributions drawn on the device, and the
    activations: decode 16 distinct fp16 tokens, prefill one bf16 chunk of 128."""
    E, H, I, Is = MOE_SHAPE["E"], MOE_SHAPE["H"], MOE_SHAPE["I"], MOE_SHAPE["Is"]
    T = 128 if prefill else 1
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3 if not prefill else 4)
    layers = []
    for _ in range(nlayers):
        rq, rs, rb = device_affine(torch, gen, 8, (E, H))
        guq, gus, gub = device_affine(torch, gen, 4, (2 * I, H), (E,))
        dnq, dns, dnb = device_affine(torch, gen, 4, (H, I), (E,))
        sgq, sgs, sgb = device_affine(torch, gen, 4, (2 * Is, H))
        sdq, sds, sdb = device_affine(torch, gen, 4, (H, Is))
        layers.append(qd.MoeWeights(E, H, I, Is, rq, rs, rb, guq, gus, gub, dnq, dns, dnb,
                                    sgq, sgs, sgb, sdq, sds, sdb))
    ntok = 16 if not prefill else 1
    xdt = torch.bfloat16 if prefill else torch.float16
    xs = [torch.randn((T, H), device="cuda", generator=gen).to(xdt) for _ in range(ntok)]
    return layers, xs, T


def moe_steps(torch, qd, layers, xs, T, prefill: bool):
    """One step per (layer, token) pair (at most 240), and the step's algorithmic
    bytes: router + each distinct selected expert once + shared expert +
    activations in and out."""
    E, H, I, Is, k = (MOE_SHAPE[n] for n in ("E", "H", "I", "Is", "k"))
    ntok = len(xs)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, qd.qmoe_workspace_bytes(layers[0], T, k)), dtype=torch.uint8, device="cuda")

    def step(i):
        lw, x = layers[i % len(layers)], xs[i % ntok]

        def f():
            qd.qmoe_layer(lw, x, k=k, workspace=ws, logits=logits, idx=idx, weights=wts, out=y)
        return f

    ncyc = min(len(layers) * ntok if not prefill else len(layers), 240)
    fns = [step(i) for i in range(ncyc)]
    expert_bytes = matrix_bytes(2 * I, H) + matrix_bytes(H, I)
    shared_bytes = matrix_bytes(2 * Is, H) + matrix_bytes(H, Is)
    router_bytes = matrix_bytes(E, H, 8)
    uniq = []
    for i in range(min(ncyc, 32)):
        fns[i]()
        torch.cuda.synchronize()
        uniq.append(len(set(idx.cpu().numpy().ravel().tolist())))
    mean_uniq = float(np.mean(uniq))
    step_bytes = router_bytes + mean_uniq * expert_bytes + shared_bytes + T * H * (2 + 4)
    return fns, step_bytes, mean_uniq


def moe_decode_figure(torch, qd):
    """µs per decode MoE layer (the c3 workload): median of 5 trials of 240
    layer calls over 30 resident layers (13.2 GB) and 16 tokens."""
    layers, xs, T = build_moe(torch, qd, False, MOE_SHAPE["layers"])
    fns, step_bytes, mean_uniq = moe_steps(torch, qd, layers, xs, T, False)
    t, trials = median_time(fns, calls=240)
    gbs = step_bytes / t / 1e9
    del layers
    torch.cuda.empty_cache()
    return {"workload": "c3: MoE decode layer, batch 1, hidden 2816, 128 experts (int4 g64 "
                        "gate+up 2816->2x704, down 704->2816), int8 router, top-8, shared expert "
                        "2816->2x2112->2816, 30 layers cycled",
            "us_per_layer": round(t * 1e6, 2), "trials_us": [round(x * 1e6, 2) for x in trials],
            "GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "step_bytes": int(step_bytes), "mean_distinct_experts": mean_uniq,
            "launches_per_layer": 3}


def bench_moe(args, torch, qd, prefill: bool):
    """MoE layer (router int8 -> top-8 -> 8 routed + shared expert), 30 layers
    cycled. Decode: batch 1, fp16 activations (16 distinct tokens per layer).
    Prefill: one 128-token chunk of bf16 activations per step."""
    E, H, I, Is, k = (MOE_SHAPE[n] for n in ("E", "H", "I", "Is", "k"))
    layers, xs, T = build_moe(torch, qd, prefill, args.sets or MOE_SHAPE["layers"])
    fns, step_bytes, mean_uniq = moe_steps(torch, qd, layers, xs, T, prefill)
    secs, _ = Timer(torch).run(fns, args.steps, args.warmup)
    t = secs / args.steps
    tm, trials = median_time(fns, calls=max(MIN_CALLS, len(fns)))
    gbs = step_bytes / t / 1e9
    name = "c4 MoE prefill chunk" if prefill else "c3 MoE decode layer"
    return {"metric": "µs per MoE layer" + (" (128-token prefill chunk)" if prefill else " (decode, batch 1)"),
            "value": round(t * 1e6, 2), "unit": "us", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(t * 1e3, 5), "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if prefill else "f16",
            "data": "synthetic",
            "config": {"workload": f"{name}: hidden {H}, {E} experts (int4 g64 gate+up {H}->2x{I}, "
                                   f"down {I}->{H}), router int8, top-{k}, shared expert "
                                   f"{H}->2x{Is}->{H}, {len(layers)} layers cycled, T={T}",
                       "GBps": round(gbs, 1), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                       "median5_us": round(tm * 1e6, 2), "trials_us": [round(x * 1e6, 2) for x in trials],
                       "mean_distinct_experts": mean_uniq, "step_bytes": int(step_bytes),
                       "launches_per_layer": 3 if not prefill else 6},
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
            "cpu_baseline": None}


def bench_stream(args, torch, qd):
    """The read-only stream kernel (qd_stream_read) at the workloads' matrix sizes
    and beyond, each cycled over >= 1 GB of buffers: the practical HBM read
    ceiling. Also torch's device copy and a reduction over 2 GiB buffers (the
    known-size reference used to scale the FETCH_SIZE / WRITE_SIZE counters)."""
    sizes = [("c1 4096x4096", matrix_bytes(4096, 4096)), ("c2 down", matrix_bytes(4096, 14336)),
             ("c2 gate+up", matrix_bytes(28672, 4096)), ("c5 matrix", matrix_bytes(28672, 8192)),
             ("512 MiB", 1 << 29), ("2 GiB", 1 << 31)]
    ceiling = []
    for name, nb in sizes:
        g, t = stream_ceiling(torch, qd, nb)
        ceiling.append({"size": name, "bytes": nb, "GBps": round(g, 1), "us": round(t * 1e6, 3),
                        "frac_of_hbm_peak": round(g / HBM_PEAK_GBS, 4)})
        torch.cuda.empty_cache()
    n = 1 << 29  # fp32 elements = 2 GiB
    src = torch.empty(n, dtype=torch.float32, device="cuda").normal_()
    dst = torch.empty_like(src)
    acc = torch.empty((), dtype=torch.float32, device="cuda")
    reps = max(4, min(args.steps, 50))
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) / 1e3 / reps
    for _ in range(3):
        torch.sum(src, 0, out=acc)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.sum(src, 0, out=acc)
    e1.record()
    torch.cuda.synchronize()
    red_s = e0.elapsed_time(e1) / 1e3 / reps
    nbytes = n * 4
    return {"config": "stream", "read_stream_kernel": ceiling, "bytes_per_buffer": nbytes, "reps": reps,
            "copy_GBps_read_plus_write": round(2 * nbytes / copy_s / 1e9, 1),
            "copy_us": round(copy_s * 1e6, 2),
            "reduce_GBps_read": round(nbytes / red_s / 1e9, 1),
            "reduce_us": round(red_s * 1e6, 2)}


def emit(out):
    """Prints the result line; records whether steps were graph-replayed."""
    if isinstance(out.get("config"), dict):
        out["config"]["launch"] = "eager" if EAGER else "graph"
    print(json.dumps(out), flush=True)


def main():
    global EAGER
    args = parse()
    EAGER = args.eager
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(--gpus {args.gpus} requested). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    import affine_quantized_gemv_qgemv_amd as qd
    qd.lib()  # fail loudly if the HIP library is missing

    if args.config == "stream":
        emit(bench_stream(args, torch, qd))
        return
    if args.config in ("c1", "c2", "c5"):
        if args.config == "c1":
            shapes, batches, nsets, cfg_id = [(4096, 4096)], [1], 64, 1
            wl = "c1: dense int4 g64 GEMV, batch 1, K=4096 -> N=4096; 64 weight sets cycled (604 MB)"
        elif args.config == "c2":
            shapes, batches, nsets, cfg_id = [(4096, 28672), (14336, 4096)], [1], 16, 2
            wl = ("c2: 7B-shaped decode FFN, batch 1: gate+up K=4096 -> N=2x14336 then down "
                  "K=14336 -> N=4096, int4 g64; 16 weight sets cycled (1.59 GB)")
        else:
            shapes, batches, nsets, cfg_id = [(8192, 28672), (28672, 8192)], [1, 2, 4, 8], 80, 5
            wl = ("c5: 70B-shaped decode, K=8192 -> N=28672 and K=28672 -> N=8192, int4 g64, "
                  "80 weight-set pairs cycled (21.1 GB)")
        fmt = args.format
        rht = args.rht
        if rht and fmt == "affine":
            raise SystemExit("--rht applies to the Mirai formats (--format mirai-m or mirai-l)")
        if fmt != "affine":
            # same shapes; the Mirai-L matrices hold twice the code bytes, so
            # half as many sets keep the cycled footprint alike
            if fmt == "mirai-l":
                nsets = max(2, nsets // 2)
            wl = wl.replace("int4 g64", "Mirai-M (int4, bf16 scale, 4-bit zero point, g64)"
                            if fmt == "mirai-m" else "Mirai-L (signed int8, bf16 scale, g64)")
            wl = wl.split(";")[0] + f"; {nsets if not args.sets else args.sets} weight sets cycled"
        if args.sets:
            nsets = args.sets
        sets = make_sets(torch, shapes, nsets, cfg_id, fmt)
        results = []
        for batch in batches:
            r = run_dense(args, torch, qd, shapes, batch, sets, cfg_id, fmt, rht)
            results.append((batch, r))
        batch, r = results[0]
        secs = r["secs"]
        gbs = r["step_bytes"] * args.steps / secs / 1e9
        # dominant kernel: the largest projection of the step, timed on its own
        dom = max(range(len(shapes)), key=lambda j: shapes[j][0] * shapes[j][1])
        dK, dN = shapes[dom]
        bytes_per_launch = gemv_bytes(dN, dK, batch, fmt=fmt, rht=rht)
        launch_s = r["per_shape"][dom]["us"] / 1e6
        achieved = bytes_per_launch / launch_s / 1e9
        kname = {"affine": "qgemv_affine4", "mirai-m": "qgemv_mirai_m",
                 "mirai-l": "qgemv_mirai_l"}[fmt] + ("_rht" if rht else "")
        traffic = stored_traffic(f"{kname}_{args.config}_traffic.json", GEMV_SOURCES)
        metric = METRIC if fmt == "affine" else \
            f"achieved HBM GB/s (% of peak) for {fmt} GEMV at batch 1" + \
            (" with the fused RMSNorm + block-32 Hadamard prologue" if rht else "")
        out = {
            "metric": metric,
            "value": round(gbs, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": round(secs / args.steps * 1e3, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "f16",
            "data": "synthetic",
            "config": {"workload": wl + ("; RMSNorm + block-32 random Hadamard prologue fused"
                                         if rht else ""),
                       "format": fmt, "rht": rht, "batch": batch, "weight_sets": nsets,
                       "step_bytes": r["step_bytes"],
                       "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                       "per_shape": [{k: (round(v, 3) if isinstance(v, float) else v)
                                      for k, v in d.items()} for d in r["per_shape"]]},
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": traffic,
                         "kernel": f"{kname} K={dK} -> N={dN}, batch {batch}",
                         "bytes_per_launch": bytes_per_launch,
                         "avg_launch_us": round(launch_s * 1e6, 3)},
        }
        # the practical ceiling at each projection's size: the read-only stream
        # kernel over buffers of the matrix's bytes, cycled like the weights
        for j, (K, N) in enumerate(shapes):
            cg, _ = stream_ceiling(torch, qd, matrix_bytes(N, K, fmt=fmt))
            ps = out["config"]["per_shape"][j]
            ps["stream_GBps"] = round(cg, 1)
            ps["pct_of_stream"] = round(100 * ps["gbs"] / cg, 1)
            ps["pct_of_hbm_peak"] = round(100 * ps["gbs"] / HBM_PEAK_GBS, 1)
            if j == dom:
                out["roofline"]["stream_ceiling_GBps"] = round(cg, 1)
                out["roofline"]["frac_of_stream"] = round(achieved / cg, 4)
        torch.cuda.empty_cache()
        if args.config == "c2" and fmt == "affine" and not args.no_moe:
            # the metric's second half: µs per decode MoE layer (c3), same run
            out["config"]["moe_decode"] = moe_decode_figure(torch, qd)
        if len(results) > 1:
            out["config"]["batch_sweep"] = [
                {"batch": b, "GBps": round(rr["step_bytes"] * args.steps / rr["secs"] / 1e9, 1),
                 "us_per_step": round(rr["secs"] / args.steps * 1e6, 2)} for b, rr in results]
        if not args.no_cpu:
            v, done, el, thr = cpu_baseline_gemv(r["cpu_mats"], args.cpu_seconds)
            v1, done1, el1, _ = cpu_baseline_gemv(r["cpu_mats"], args.cpu_seconds / 4, threads=1)
            out["cpu_baseline"] = {"value": round(v, 4), "unit": "GB/s", "cores": thr,
                                   "kind": "oracle", "cpu_model": cpu_model(),
                                   "sample": f"{done} full step(s) of weight set 0 "
                                             f"({', '.join(f'{K}->{N}' for K, N in shapes)}, batch {batch}) "
                                             f"in {el:.1f} s, fp64 C oracle",
                                   "value_1thread": round(v1, 4),
                                   "sample_1thread": f"{done1} step(s) in {el1:.1f} s on one thread"}
        else:
            out["cpu_baseline"] = None
        emit(out)
        return
    if args.config == "c4":
        emit(bench_chunk(args, torch, qd))
        return
    if args.config == "verify":
        emit(bench_verify(args, torch, qd))
        return
    if args.config == "attn":
        emit(bench_attn(args, torch, qd))
        return
    if args.config in ("c3", "c4moe"):
        emit(bench_moe(args, torch, qd, prefill=args.config == "c4moe"))
        return
    raise SystemExit(f"config {args.config} is not wired into bench.py yet")


if __name__ == "__main__":
    main()
