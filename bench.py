#!/usr/bin/env python
"""LoftQ initialisation throughput on one AMD Instinct MI355X.

A step is one LoftQ initialisation of the whole workload (all T alternations of
every matrix: NF4 quantize of the residual, double quant, dequant-subtract,
randomized rank-r SVD, objective) with W already resident in HBM.  The default
workload is the 224 matrices of a 32-layer 7B-class decoder (q, k, v, o, gate, up,
down of every layer), initialised by one loftq_init_batch call over several
streams; single-matrix workloads run one loftq_init.  `value` is matrix elements
per second (sum of rows * cols per step).  The JSON line also carries:
  roofline      the dominant streaming kernel: algorithmic bytes per launch over
                its average launch time, timed with HIP events that the library
                records around each launch on its own stream during a separate
                profiled pass over the same steps, less what the events read for
                an empty kernel bracketed the same way (event_overhead_us);
  nf4_quantize  the same for the NF4 quantize kernel (the metric's second part);
  nf4_merge     the adapter merge of the init's own B, A into its Q, timed the same way;
  warm_start_variant  the same init with a warm-started subspace iteration and one
                power iteration fewer (a variant; `value` stays the pages' method);
  lower_bit     the same init with the 3- and 2-bit NormalFloat codebooks;
  qlora_forward the QLoRA forward of the adapted layer on this init's Q, B, A for a
                2048-token (matrix-core bound) and a 16-token (HBM bound) batch;
  cpu_baseline  the CPU oracle on a bounded row sample of the same workload.
For the decoder batch the adapter merge, the variants and the forward run on its
first matrix (layer 0's q projection, 4096 x 4096).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LoftQ init matrix-elements/s (T alternations) + NF4 quantize GB/s vs HBM peak"
HBM_PEAK_GBS = 8000.0   # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores

# HBM bytes per dispatch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE passes (calibrated
# against a 256 MiB device copy), valid while the kernel source is unchanged (sha256 prefix of
# the file the kernel lives in); reported as null otherwise.
MEASURED_TRAFFIC = {
    # the decoder batch: means over the dispatches of a one-layer batch (the same seven shapes in the
    # same proportions), residual formed from W and the codes
    "c4_decoder_batch_224_bf16": {
        "gemm_nn": {"bytes": 87427740, "source": "gemm_kernels.hip", "sha256": "dce7e2597b8eda97"},
        "gemm_tn": {"bytes": 82520401, "source": "gemm_kernels.hip", "sha256": "dce7e2597b8eda97"},
    },
    # the extras of the decoder batch run on its first matrix (layer 0's q projection, 4096 x 4096,
    # r = 16): the QLoRA forward, 2048 tokens (tiled kernel) and 16 tokens (few-token kernel)
    "c4_l0_q_4096x4096_bf16": {
        "nf4_gemm": {"bytes": 123018591, "source": "forward_kernels.hip", "sha256": "816be8351946cd3b"},
        "nf4_gemm_skinny": {"bytes": 10414080, "source": "forward_kernels.hip", "sha256": "816be8351946cd3b"},
    },
    "c2_4096x4096_bf16": {
        "gemm_nn": {"bytes": 77784775, "source": "gemm_kernels.hip", "sha256": "4322c77aea1b6c85"},
        "gemm_tn": {"bytes": 75687250, "source": "gemm_kernels.hip", "sha256": "4322c77aea1b6c85"},
        # the QLoRA forward on this layer: 2048 tokens (tiled kernel), 16 tokens (few-token kernel)
        "nf4_gemm": {"bytes": 122919263, "source": "forward_kernels.hip", "sha256": "59cd1a34f99baaac"},
        "nf4_gemm_skinny": {"bytes": 10397831, "source": "forward_kernels.hip", "sha256": "59cd1a34f99baaac"},
    },
}

# VALU wave-instructions per dispatch from an SQ_INSTS_VALU counter run of this
# command (summary under profiles/), keyed to the kernel source; the adapter merge
# is VALU-bound, so its roofline is this count over its launch time against the
# non-packed VALU peak (256 CUs x 4 SIMDs x 2.4 GHz / 4 cycles per wave64 op).
VALU_PEAK_GWIS = 256 * 4 * 2.4 / 4
MEASURED_VALU = {
    "c4_l0_q_4096x4096_bf16": {
        "nf4_merge": {"valu": 6362099, "source": "quant_kernels.hip", "sha256": "2b26247299f66d83"},
    },
    "c2_4096x4096_bf16": {
        "nf4_merge": {"valu": 5250600, "source": "quant_kernels.hip", "sha256": "471627fbeb92a6bd"},
    },
}


def measured_valu(workload, kernel):
    import hashlib
    rec = MEASURED_VALU.get(workload, {}).get(kernel)
    if rec is None:
        return None
    path = os.path.join(ROOT, "loftq_qlora_initialization_amd", "csrc", rec["source"])
    try:
        with open(path, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()[:16]
    except OSError:
        return None
    return rec["valu"] if sha == rec["sha256"] else None


def measured_traffic(workload, kernel):
    import hashlib
    rec = MEASURED_TRAFFIC.get(workload, {}).get(kernel)
    if rec is None:
        return None
    path = os.path.join(ROOT, "loftq_qlora_initialization_amd", "csrc", rec["source"])
    try:
        with open(path, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()[:16]
    except OSError:
        return None
    return rec["bytes"] if sha == rec["sha256"] else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 3 for c4, else 20)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 1 for c4, else 3)")
    ap.add_argument("--workload", default="c4", help="c4 (the 224-matrix decoder batch), c1, c2, c3 or c5")
    ap.add_argument("--streams", type=int, default=3, help="streams the batched call spreads its matrices over")
    ap.add_argument("--layers", type=int, default=32, help="decoder layers of the c4 batch (fewer: a smaller batch)")
    ap.add_argument("--cpu-rows", type=int, default=None,
                    help="rows of each sampled matrix timed on the CPU oracle (default 1024 for c4, else 4096)")
    ap.add_argument("--skip-cpu", action="store_true", help="omit the CPU oracle leg")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run three device-to-device copies of this many MiB (HBM counter calibration)")
    return ap.parse_args()


def formed_residual(w, cols):
    """Whether loftq_init's products form E from W and the codes (the library's default,
    materialize_residual = 0) rather than read a stored E: randomized SVD, T >= 1, cols % 8 == 0."""
    return (not w.exact_svd) and w.iterative_steps > 0 and cols % 8 == 0


def algorithmic_bytes(name, w, rows, cols):
    """Bytes the method must move per launch of a kernel (inputs read once, outputs written once)."""
    n = rows * cols
    nb = -(-n // 64)
    ng = -(-nb // 256)
    wb = 2 if w.dtype == "bf16" else 4
    l = w.rank + w.oversample
    scales = (nb + 4 * ng) if w.double_quant else 4 * nb
    formed = formed_residual(w, cols)
    # the residual a product streams: a stored fp32 E, or W, the codes and one fp32 scale per block
    e_in = (n * wb + -(-n // 2) + 4 * nb) if formed else 4 * n
    # the dequant-subtract writes E, or (formed, double quant) only the blocks' scales
    e_out = (4 * nb if w.double_quant else 0) if formed else 4 * n
    table = {
        "nf4_quantize": n * wb + -(-n // 2) + 4 * nb,
        "nf4_quantize_fused": n * wb + -(-n // 2) + 4 * nb + 4 * w.rank * (rows + cols),
        "double_quant": 4 * nb + nb + 4 * ng,
        "nf4_dequantize": n * wb + -(-n // 2) + scales + e_out,
        "gemm_nn": e_in + 4 * cols * l + 4 * rows * l,
        "gemm_tn": e_in + 4 * rows * l + 4 * cols * l,
        "sumsq_weight": n * wb,
        # adapter merge: codes and scales in, codes and fp32 absmax out, B and A
        "nf4_merge": -(-n // 2) + scales + -(-n // 2) + 4 * nb + 4 * w.rank * (rows + cols),
        # the quantized weight a forward reads (codes and scales); activations are added per batch
        "qlora_weight": -(-n // 2) + scales,
    }
    return table.get(name)


def cpu_baseline(specs, rows, extrapolated):
    """The oracle's loftq_init on the first `rows` rows of each matrix in `specs`, repeated
    until about 10 s of CPU work (at most 3 passes); elements per second."""
    import numpy as np
    import oracle
    from loftq_qlora_initialization_amd import synth
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:   # threadpoolctl absent: report the interpreter's own thread
        cores = 1
    samples = []
    for w in specs:
        rr = min(rows, w.rows)
        samples.append((w, rr, synth.make_weight(w, rows=rr)[1]))
    reps, dt = 0, 0.0
    while reps < 3 and (reps == 0 or dt < 10.0):
        t0 = time.perf_counter()
        for w, rr, W in samples:
            oracle.loftq_init(W, rank=w.rank, iterative_steps=w.iterative_steps, double_quant_on=w.double_quant,
                              exact=w.exact_svd, oversample=w.oversample, power_iters=w.power_iters,
                              seed=w.sketch_seed)
        dt += time.perf_counter() - t0
        reps += 1
    elems = sum(rr * w.cols for w, rr, _ in samples)
    if len(specs) == 1:
        w, rr, _ = samples[0]
        what = f"{'all' if rr == w.rows else f'first {rr} of'} {w.rows} rows of {w.name}"
    else:
        what = f"the first {rows} rows of each of {len(specs)} matrices ({', '.join(w.name for w in specs)})"
    out = {"value": reps * elems / dt, "unit": "elements/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{what}, same r/p/q/T/double-quant, {reps} pass(es) in {dt:.1f} s"}
    if extrapolated:
        out["sample"] += "; per-element rate extrapolated to the whole batch"
        out["extrapolated"] = True
    return out


def device_weights(specs, workers):
    """Generate every matrix on the host (seeded, threads in parallel) and copy it to the GPU."""
    import concurrent.futures as cf
    import numpy as np
    import torch
    from loftq_qlora_initialization_amd import synth

    def one(w):
        bits, _ = synth.make_weight(w)
        if w.dtype == "bf16":
            return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(bits).cuda()
    if len(specs) == 1:
        return [one(specs[0])]
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(one, specs))


def kernel_table(prof, steps, bytes_per_step, overhead_us=0.0):
    """Per-kernel launches, average launch time, share and algorithmic GB/s from a profiled pass.
    bytes_per_step(name) -> algorithmic bytes all launches of that kernel move in one step, or None.
    overhead_us: what a bracketed launch's events read beyond its kernel (an empty kernel's bracketed
    time, profile_calibrate); avg_us is net of it, event_us the raw event average."""
    kernels = {}
    total = sum(v[1] for v in prof.values())
    for name, (launches, total_ms) in sorted(prof.items(), key=lambda kv: -kv[1][1]):
        event_us = 1e3 * total_ms / launches
        avg_us = max(event_us - overhead_us, 1e-3)
        entry = {"launches_per_step": launches / steps, "avg_us": round(avg_us, 3), "event_us": round(event_us, 3),
                 "share": round(total_ms / total, 4)}
        nbytes = bytes_per_step(name)
        if nbytes is not None:
            entry["GBps"] = round(nbytes * steps / (launches * avg_us * 1e-6) / 1e9, 1)
            entry["bytes_per_launch"] = round(nbytes * steps / launches)
        kernels[name] = entry
    return kernels


def event_overhead_us(lq, torch):
    """Average bracketed time of an empty kernel on the current stream (256 launches)."""
    lq.profile_collect()
    lq.profile_enable(True)
    lq.profile_calibrate(256)
    torch.cuda.synchronize()
    lq.profile_enable(False)
    rec = lq.profile_collect().get("event_overhead")
    return 1e3 * rec[1] / rec[0] if rec else 0.0


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: libloftq has no multi-GPU path (its kernels are what one device runs "
              "on its share of the matrices; run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_mib:
        # a plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it calibrates
        # the counters against true HBM bytes
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_mib": args.copy_mib, "launches": 3}), flush=True)
        return

    import loftq_qlora_initialization_amd as lq
    from loftq_qlora_initialization_amd import synth

    batch = args.workload == "c4"
    if batch:
        specs = synth.c4_matrix_specs()[:7 * max(1, min(32, args.layers))]
        wname = "c4_decoder_batch_224_bf16" if len(specs) == 224 else f"c4_decoder_batch_{len(specs)}_bf16"
    else:
        specs = [synth.workload(args.workload)]
        wname = specs[0].name
    steps = args.steps if args.steps is not None else (3 if batch else 20)
    warmup = args.warmup if args.warmup is not None else (1 if batch else 3)
    w = specs[0]                      # the configuration (shared by every matrix of the batch)
    total_elems = sum(x.numel for x in specs)
    t_gen = time.perf_counter()
    Ws = device_weights(specs, workers=min(16, os.cpu_count() or 1))
    t_gen = time.perf_counter() - t_gen
    cfg = lq.default_config(iterative_steps=w.iterative_steps, rank=w.rank, oversample=w.oversample,
                            power_iters=w.power_iters, double_quant=int(w.double_quant),
                            exact_svd=int(w.exact_svd), seed=w.sketch_seed)
    if batch:
        runner = lq.BatchRunner(Ws, cfg, nstreams=args.streams)
        bufs = runner.buffers[0]

        def step():
            runner.run()
    else:
        bufs = lq.InitBuffers(w.rows, w.cols, cfg)

        def step():
            lq.loftq_init(Ws[0], cfg, buffers=bufs)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / steps
    value = total_elems * steps / elapsed

    # launches per init of each kernel for every distinct shape (one profiled init each), so
    # the batch's algorithmic bytes per kernel can be summed over its matrices
    shapes = {}
    for x, W in zip(specs, Ws):
        shapes.setdefault((x.rows, x.cols), [x, W, 0])[2] += 1
    per_shape = {}
    for key, (x, W, count) in shapes.items():
        sb = lq.InitBuffers(x.rows, x.cols, cfg)
        lq.loftq_init(W, cfg, buffers=sb)
        torch.cuda.synchronize()
        lq.profile_enable(True)
        lq.loftq_init(W, cfg, buffers=sb)
        torch.cuda.synchronize()
        lq.profile_enable(False)
        per_shape[key] = (x, count, {k: v[0] for k, v in lq.profile_collect().items()})
        del sb

    def bytes_per_step(name):
        tot = 0
        for (rows, cols), (x, count, launches) in per_shape.items():
            b = algorithmic_bytes(name, x, rows, cols)
            if b is None:
                return None
            tot += count * launches.get(name, 0) * b
        return tot

    # profiled pass: HIP events around every library launch.  The batch is profiled in one pass
    # on a single stream, so that a launch's events bracket that launch alone (with several
    # streams a launch can sit behind another stream's kernel between its start event and its
    # first wave); a single matrix repeats the timed steps.
    prof_steps = 1 if batch else steps
    if batch:
        prof_runner = lq.BatchRunner(Ws, cfg, nstreams=1)
        prof_runner.run()
        torch.cuda.synchronize()
        prof_step = prof_runner.run
    else:
        prof_step = step
    lq.profile_enable(True)
    for _ in range(prof_steps):
        prof_step()
    torch.cuda.synchronize()
    lq.profile_enable(False)
    prof = lq.profile_collect()
    if batch:
        del prof_runner
    overhead = event_overhead_us(lq, torch)
    kernels = kernel_table(prof, prof_steps, bytes_per_step, overhead)
    for name, e in kernels.items():   # every launch of the batch accounted for by the per-shape counts
        want = sum(c * l.get(name, 0) for _, c, l in per_shape.values())
        if want and abs(e["launches_per_step"] - want) > 1e-9:
            e["launch_count_mismatch"] = want
    streaming = [k for k in kernels if "GBps" in kernels[k]]
    dom = max(streaming, key=lambda k: kernels[k]["share"])
    achieved = kernels[dom]["GBps"]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(wname, dom),
                "bytes_per_launch": kernels[dom]["bytes_per_launch"], "avg_us": kernels[dom]["avg_us"],
                "event_us": kernels[dom]["event_us"], "event_overhead_us": round(overhead, 3)}
    if batch:
        roofline["note"] = ("launch durations from one profiled pass of the whole batch on a single stream "
                            f"(the timed steps run on {args.streams} streams)")
    qname = "nf4_quantize" if "nf4_quantize" in kernels else None
    nf4 = None
    if qname:
        g = kernels[qname]["GBps"]
        nf4 = {"kernel": qname, "achieved": g, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(g / HBM_PEAK_GBS, 4),
               "avg_us": kernels[qname]["avg_us"]}
        if "nf4_quantize_fused" in kernels:
            gf = kernels["nf4_quantize_fused"]["GBps"]
            nf4["fused_residual"] = {"achieved": gf, "frac": round(gf / HBM_PEAK_GBS, 4),
                                     "avg_us": kernels["nf4_quantize_fused"]["avg_us"]}

    obj = bufs.objective.cpu().numpy().tolist()
    Wd = Ws[0]
    if batch:   # the extras below run on the batch's first matrix
        del runner, shapes
        Ws = Ws[:1]
        torch.cuda.empty_cache()

    # adapter merge (the PEFT guide's merge_adapter on NF4: dequantize, add B A,
    # quantize again) of this init's own B, A into its Q, into separate buffers
    merge = None
    if w.rank > 0 and not w.exact_svd and w.cols % 64 == 0:
        dq = bool(w.double_quant)
        nb = (w.numel + 63) // 64
        mout = {"packed": torch.empty_like(bufs.packed), "absmax": torch.empty_like(bufs.absmax)}
        if dq:
            mout.update(qabsmax=torch.empty_like(bufs.qabsmax), dq_scale=torch.empty_like(bufs.dq_scale))
        scales = dict(qabsmax=bufs.qabsmax, dq_scale=bufs.dq_scale) if dq else dict(absmax=bufs.absmax)
        for _ in range(2):
            lq.loftq_nf4_merge(bufs.packed, (w.rows, w.cols), bufs.B, bufs.A, 1.0, **scales, double_quant=dq, out=mout)
        torch.cuda.synchronize()
        lq.profile_enable(True)
        for _ in range(steps):
            lq.loftq_nf4_merge(bufs.packed, (w.rows, w.cols), bufs.B, bufs.A, 1.0, **scales, double_quant=dq, out=mout)
        torch.cuda.synchronize()
        lq.profile_enable(False)
        mprof = lq.profile_collect()
        if "nf4_merge" in mprof:
            launches, total_ms = mprof["nf4_merge"]
            avg_us = max(1e3 * total_ms / launches - overhead, 1e-3)
            gb = algorithmic_bytes("nf4_merge", w, w.rows, w.cols) / (avg_us * 1e-6) / 1e9
            step_us = 1e3 * sum(v[1] for v in mprof.values()) / steps
            valu = measured_valu(w.name, "nf4_merge")
            merge = {"kernel": "nf4_merge", "bound": "alu", "avg_us": round(avg_us, 3),
                     "achieved": None if valu is None else round(valu / (avg_us * 1e-6) / 1e9, 1),
                     "peak": VALU_PEAK_GWIS, "unit": "G VALU wave-instructions/s",
                     "frac": None if valu is None else round(valu / (avg_us * 1e-6) / 1e9 / VALU_PEAK_GWIS, 4),
                     "valu_per_launch": valu,
                     "hbm": {"achieved": round(gb, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(gb / HBM_PEAK_GBS, 4),
                             "bytes_per_launch": algorithmic_bytes("nf4_merge", w, w.rows, w.cols)},
                     "us_per_merge_with_double_quant": round(step_us, 3),
                     "elements_per_s": round(w.numel / (step_us * 1e-6))}
    # the warm-started subspace iteration (a variant the pages do not describe): one
    # power iteration fewer, started from the previous alternation's V
    warm = None
    if not w.exact_svd and w.power_iters >= 1 and w.iterative_steps >= 2:
        wcfg = lq.default_config(iterative_steps=w.iterative_steps, rank=w.rank, oversample=w.oversample,
                                 power_iters=w.power_iters - 1, double_quant=int(w.double_quant), exact_svd=0,
                                 seed=w.sketch_seed, warm_start=1)
        wbufs = lq.InitBuffers(w.rows, w.cols, wcfg)
        for _ in range(max(warmup, 1)):
            lq.loftq_init(Wd, wcfg, buffers=wbufs)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(steps):
            lq.loftq_init(Wd, wcfg, buffers=wbufs)
        torch.cuda.synchronize()
        wel = time.perf_counter() - t1
        wobj = wbufs.objective.cpu().numpy().tolist()
        warm = {"power_iters": w.power_iters - 1, "value": w.numel * steps / wel, "unit": "elements/s",
                "ms_per_step": 1e3 * wel / steps, "final_objective": wobj[-1],
                "cold_final_objective": obj[-1], "cold_power_iters": w.power_iters}
        del wbufs

    # lower-bit LoftQ: the same init with the 3- and 2-bit NormalFloat codebooks
    lower = {}
    for b in (3, 2):
        bcfg = lq.default_config(iterative_steps=w.iterative_steps, rank=w.rank, oversample=w.oversample,
                                 power_iters=w.power_iters, double_quant=int(w.double_quant),
                                 exact_svd=int(w.exact_svd), seed=w.sketch_seed, bits=b)
        bbufs = lq.InitBuffers(w.rows, w.cols, bcfg)
        lq.loftq_init(Wd, bcfg, buffers=bbufs)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(steps):
            lq.loftq_init(Wd, bcfg, buffers=bbufs)
        torch.cuda.synchronize()
        bel = time.perf_counter() - t1
        bobj = bbufs.objective.cpu().numpy().tolist()
        lower[f"nf{b}"] = {"value": w.numel * steps / bel, "unit": "elements/s",
                           "ms_per_step": 1e3 * bel / steps, "objective_plain": bobj[0],
                           "objective_final": bobj[-1]}
        del bbufs

    # QLoRA forward of the adapted layer (the consumer of this init's Q, B, A): a prefill
    # batch, a product for the bf16 matrix cores, and a decode-sized batch, bound by reading Q
    fwd = {}
    if w.rank > 0 and w.cols % 64 == 0:
        dq = bool(w.double_quant)
        scales = dict(qabsmax=bufs.qabsmax, dq_scale=bufs.dq_scale) if dq else dict(absmax=bufs.absmax)
        gx = np.random.Generator(np.random.PCG64(np.random.SeedSequence(2024)))
        for label, ntok in (("prefill", 2048), ("decode", 16)):
            xb = synth.f32_to_bf16_bits(gx.standard_normal((ntok, w.cols)).astype(np.float32))
            X = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
            Y = torch.empty((ntok, w.rows), dtype=torch.float32, device="cuda")
            ws = torch.empty(max(lq.qlora_forward_workspace_bytes(ntok, w.rank), 16), dtype=torch.uint8,
                             device="cuda")

            def call():
                lq.loftq_qlora_forward(X, bufs.packed, (w.rows, w.cols), **scales, B=bufs.B, A=bufs.A, out=Y, ws=ws)
            reps = 10 * steps
            for _ in range(3):
                call()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for _ in range(reps):
                call()
            torch.cuda.synchronize()
            fel = time.perf_counter() - t1
            lq.profile_enable(True)
            for _ in range(reps):
                call()
            torch.cuda.synchronize()
            lq.profile_enable(False)
            fprof = lq.profile_collect()
            gname = "nf4_gemm" if "nf4_gemm" in fprof else "nf4_gemm_skinny"
            gl, gms = fprof[gname]
            g_us = max(1e3 * gms / gl - overhead, 1e-3)
            d_us = max(1e3 * fprof["lora_down"][1] / fprof["lora_down"][0] - overhead, 0.0) if "lora_down" in fprof else 0.0
            flops = 2.0 * ntok * w.rows * w.cols
            lora_flops = 2.0 * ntok * w.rank * (w.rows + w.cols)
            qbytes = algorithmic_bytes("qlora_weight", w, w.rows, w.cols)
            gbytes = qbytes + 2 * ntok * w.cols + 4 * ntok * w.rows + 4 * ntok * w.rank + 4 * w.rank * w.rows
            ent = {"tokens": ntok, "us_per_forward": round(1e6 * fel / reps, 3),
                   "tokens_per_s": round(ntok * reps / fel),
                   "TFLOPs": round((flops + lora_flops) / (fel / reps) / 1e12, 2),
                   "nf4_gemm_us": round(g_us, 3), "lora_down_us": round(d_us, 3)}
            tf = flops / (g_us * 1e-6) / 1e12
            gbs = gbytes / (g_us * 1e-6) / 1e9
            ent["mfma"] = {"achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops_per_launch": flops}
            ent["hbm"] = {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": gbytes,
                          "traffic": measured_traffic(w.name, gname)}
            ent["kernel"] = gname
            ent["bound"] = "mfma" if label == "prefill" else "hbm"
            fwd[label] = ent
            del X, Y, ws

    config = {"workload": wname, "matrices": len(specs), "elements": total_elems, "storage": w.dtype,
              "rank": w.rank, "iterative_steps": w.iterative_steps, "oversample": w.oversample,
              "power_iters": w.power_iters, "double_quant": w.double_quant, "blocksize": 64, "dq_blocksize": 256,
              "residual": "formed in the products from W and the codes"
              if all(formed_residual(x, x.cols) for x in specs) else "stored E"}
    if batch:
        config.update(shapes={f"{r}x{c}": n for (r, c), (_, n, _) in per_shape.items()}, streams=args.streams,
                      call="loftq_init_batch", extras_on=specs[0].name)
    else:
        config.update(rows=w.rows, cols=w.cols, call="loftq_init")
    line = {
        "metric": METRIC, "value": value, "unit": "elements/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": config, "input_generation_s": round(t_gen, 1),
        "roofline": roofline, "nf4_quantize": nf4, "nf4_merge": merge, "warm_start_variant": warm,
        "lower_bit": lower, "qlora_forward": fwd,
        "objective": obj, "kernels": kernels,
    }
    if not args.skip_cpu:
        rows = args.cpu_rows if args.cpu_rows is not None else (1024 if batch else 4096)
        line["cpu_baseline"] = cpu_baseline(specs[:7] if batch else specs, rows, extrapolated=batch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
