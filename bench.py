#!/usr/bin/env python3
"""Throughput of the AVQ-Attention forward pass on one MI355X.

One step = one pass of the whole hot path over one batch, through the C
interface, on synthetic inputs already resident in HBM:
  avq_assign_aggregate_accum  two-level assignment + value sums and counts
                              (Sec. 4.2, Alg. 1, Eq. 3), added into buffers
                              that hold zeros
  avq_attention_prepare       the value sums as fp16 operand fragments, and a
                              copy of the counts
  avq_attention_fwd_prepared  the attention kernel: parent attention,
                              importance, top-P, child correction, output
                              (Sec. 4.3, Alg. 2, Eq. 6-9); it also zero-fills
                              the value sums and counts it no longer reads,
                              for the next step's accumulation (the zero fill
                              of Alg. 1's first step, moved there)
The three calls are issued with their arguments marshalled once (ctypes
argument tuples built before the timed loop), so the timed loop adds no
Python-side checking between launches.  Three input sets are rotated (larger
than the 256 MB Infinity Cache together) so that every step streams from HBM.

Prints one JSON line:
  value            tokens per second of the whole pass, in millions (B*N / step time)
  roofline         the dominant unit (the attention kernel): its algorithmic
                   bytes per launch over its average duration (HIP events on
                   the launch stream around the call, inside the timed
                   region) against MI355X's 8 TB/s HBM peak, and its
                   algorithmic MFMA flops against the 2.5 PFLOP/s dense bf16
                   peak; traffic = counter-measured HBM bytes per launch;
                   traced = the same fractions at the average duration of
                   the committed kernel trace of the same source
  units            the same figures for every unit of the step
  cpu_baseline     the CPU oracle on the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload grid128]
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

METRIC = "AVQ fwd Mtokens/s at N=16384,H=16,d=64,M0=64,C=8,P=16; % HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP32_PEAK_TFLOPS = 157.3
_ATTN_SRC = ["adaptive_vector_quantized_amd/csrc/attention.hip", "adaptive_vector_quantized_amd/csrc/avq_device.h",
             "adaptive_vector_quantized_amd/csrc/avq_launch.h"]
# each timed unit is one C call; the kernels it launches, and their sources
CALLS = {
    "avq_assign_aggregate": ("zero_kernel + assign_aggregate_kernel",
                             ["adaptive_vector_quantized_amd/csrc/assign_aggregate.hip",
                              "adaptive_vector_quantized_amd/csrc/avq_device.h"]),
    "avq_assign_aggregate_accum": ("assign_aggregate_kernel",
                                   ["adaptive_vector_quantized_amd/csrc/assign_aggregate.hip",
                                    "adaptive_vector_quantized_amd/csrc/avq_device.h"]),
    "avq_attention_prepare": ("attention_prep_kernel", _ATTN_SRC),
    "avq_attention_fwd_prepared": ("attention_kernel", _ATTN_SRC),
    "avq_attention_fwd": ("attention_prep_kernel + attention_kernel", _ATTN_SRC),
}


def source_hash(call: str) -> str:
    h = hashlib.sha256()
    for rel in CALLS[call][1]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def attention_launches(cfg, P):
    """(preparation kernels, attention kernel) the attention calls launch on
    this workload, by the launcher's rules in csrc/attention.hip: the value
    fragments come from attention_prep_kernel, after a first pass of
    attention_absmax_kernel when the prep blocks' repeated reads of a head's
    value sums would pass 8 MiB (bf16 only); the pipelined kernel serves bf16,
    d = 64, at most 64 parents (one LDS-resident pass) and P > 0."""
    bf16 = cfg.dtype == "bf16"
    E = 8 if bf16 else 1
    W = 8 if cfg.C <= 8 else 16
    M0p = (cfg.M0 + 63) // 64 * 64
    nF = (M0p // 32) * (16 // E) * 2 * cfg.d + (cfg.M0 * (W // E) * cfg.d if cfg.C > 0 else 0)
    parts = max(8, -(-nF // (512 * 2)))
    head_bytes = cfg.M0 * (1 + cfg.C) * cfg.d * 4
    prep = ("attention_absmax_kernel + attention_prep_kernel" if bf16 and parts * head_bytes > (8 << 20)
            else "attention_prep_kernel")
    kern = "attention_pipe_kernel" if bf16 and cfg.d == 64 and M0p <= 64 and P > 0 else "attention_kernel"
    return prep, kern


def algorithmic(cfg, P):
    """Bytes each unit must move and flops it must do, per launch.

    avq_assign_aggregate: read K and V once, the head codebooks once, write
    the value sums and counts once; flops 2 d (M0 + C) per key (parent and
    child distances).
    avq_assign_aggregate_accum: the same bytes and flops (the aggregates are
    read-modify-written by atomics in L2; counted once, as written).
    avq_attention_prepare: read the value sums (float) once, write them once
    as operands (fp16 for bf16 inputs, float for fp32 inputs).
    avq_attention_fwd_prepared (the attention kernel): read Q once, write Y
    (float32) once, read the codebooks, the counts and the value operands
    once; MFMA flops 4 d (M0 + P C) per query (logits and weighted value sums
    over the M0 + P C codewords a tile uses).
    avq_attention_fwd (both, as one call): Q, Y, codebooks, float value sums
    and counts once, the same flops."""
    es = 2 if cfg.dtype == "bf16" else 4
    BH, N, d, M0, C, Mt = cfg.BH, cfg.N, cfg.d, cfg.M0, cfg.C, cfg.Mt
    cb = cfg.H * Mt * d * es
    aggr = BH * Mt * (d * 4 + 4)
    operands = BH * Mt * d * es
    k1_bytes = 2 * BH * N * d * es + cb + aggr
    k2_bytes = BH * N * d * es + BH * N * d * 4 + cb + aggr
    kern_bytes = BH * N * d * es + BH * N * d * 4 + cb + BH * Mt * 4 + operands
    k1_flops = 2.0 * d * (M0 + C) * BH * N
    k2_flops = 4.0 * d * (M0 + P * C) * BH * N
    return {"avq_assign_aggregate": (k1_bytes, k1_flops),
            "avq_assign_aggregate_accum": (k1_bytes, k1_flops),
            "avq_attention_prepare": (BH * Mt * d * 4 + operands, 0.0),
            "avq_attention_fwd_prepared": (kern_bytes, k2_flops),
            "avq_attention_fwd": (k2_bytes, k2_flops)}


def load_record(call: str, workload: str):
    """The committed rocprofv3 record of a call on a workload (HBM bytes per
    launch from the counter runs; the kernel trace's average duration), if it
    was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{call}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(call):
        return None
    return rec


def load_traffic(call: str, workload: str):
    """HBM bytes per call from the committed counter record, if current."""
    rec = load_record(call, workload)
    return None if rec is None else rec.get("bytes_per_launch")


def traced_fractions(rec, alg_bytes: float, alg_flops: float, mfma_peak: float):
    """The roofline fractions of the dominant kernel at the average duration
    the committed kernel trace of the same source measured (the figure the
    live HIP-event fractions are checked against), or None."""
    if rec is None or not rec.get("trace_avg_us"):
        return None
    t = rec["trace_avg_us"] * 1e-6
    return {"avg_us": rec["trace_avg_us"], "frac": round(alg_bytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(alg_flops / t / 1e12 / mfma_peak, 4), "stats": rec.get("trace_stats")}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, P, runs: int = 3):
    """The oracle as it stands, on the host cores, over the whole workload
    (OpenMP over the B*H heads): the assignment and aggregation, then the
    importance, top-P and substituted-codebook output, each timed separately;
    the median of `runs` passes."""
    import oracle
    from adaptive_vector_quantized_amd import gen
    data = gen.make(cfg)
    o = oracle.Oracle.for_cfg(cfg)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    t_k1, t_k2 = [], []
    for _ in range(runs):
        t0 = time.perf_counter()
        parent, row = o.assign(data["K"], data["codebook"])
        vsum, counts = o.aggregate(data["V"], parent, row)
        t1 = time.perf_counter()
        w = o.importance(data["Q"], data["codebook"], counts, cfg.block_q, cfg.scale)
        sel = o.select(w, P)
        o.attention_substituted(data["Q"], data["codebook"], vsum, counts, sel, P, cfg.block_q, cfg.scale)
        t2 = time.perf_counter()
        t_k1.append(t1 - t0)
        t_k2.append(t2 - t1)
    k1, k2 = float(np.median(t_k1)), float(np.median(t_k2))
    dt = k1 + k2
    return {
        "value": cfg.B * cfg.N / dt / 1e6,
        "unit": "Mtokens/s",
        "cores": min(threads, cfg.BH),
        "kind": "oracle",
        "sample": f"the whole workload ({cfg.B}x{cfg.H} heads x {cfg.N} tokens), plain-C oracle, median of {runs} "
                  f"passes: assign + aggregate {k1:.3f} s, importance + top-P + substituted-codebook output "
                  f"{k2:.3f} s",
        "assign_aggregate_s": round(k1, 4),
        "attention_s": round(k2, 4),
        "cpu_model": _cpu_model(),
        "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
        "nproc": os.cpu_count(),
    }


class Step:
    """The C calls of one pass over one input set (a dict of device tensors:
    K, V, Q, cb, vsum, counts, Y, ws), with their ctypes arguments built once,
    after one checked call of each through the binding.  With approx or qorder
    the pass is avq_assign_aggregate then one call of
    avq_attention_fwd_approx / _ordered (preparation included); otherwise it
    is avq_assign_aggregate_accum, avq_attention_prepare and
    avq_attention_fwd_prepared clearing the set's value sums and counts."""

    def __init__(self, cfg, P, s, stream, approx=False, qorder=None, block_q=None):
        import ctypes
        import torch
        from adaptive_vector_quantized_amd import _lib
        L = _lib.lib()
        bq = block_q or cfg.block_q
        dt = _lib.AVQ_BF16 if s["Q"].dtype == torch.bfloat16 else _lib.AVQ_F32
        ptr = _lib._ptr
        st = ctypes.c_void_p(stream.cuda_stream)
        shp = (cfg.B, cfg.H, cfg.N, cfg.d, cfg.M0, cfg.C, dt)
        # one checked call of each through the binding (shapes, dtypes, devices)
        _lib.assign_aggregate(s["K"], s["V"], s["cb"], cfg.C, vsum=s["vsum"], counts=s["counts"])
        kargs = (ptr(s["K"]), ptr(s["V"]), ptr(s["cb"])) + shp + (ptr(s["vsum"]), ptr(s["counts"]), None, st)
        wsb = s["ws"].numel()
        tail = (P, bq, float(cfg.scale))
        if approx or qorder is not None:
            self.calls = [("avq_assign_aggregate", L.avq_assign_aggregate, kargs)]
            _lib.attention_fwd(s["Q"], s["cb"], s["vsum"], s["counts"], cfg.C, P, bq, cfg.scale, Y=s["Y"],
                               workspace=s["ws"], approx_denominator=approx, query_order=qorder)
            if qorder is not None:
                args = (ptr(s["Q"]), ptr(s["cb"]), ptr(s["vsum"]), ptr(s["counts"])) + shp + tail + (
                    ptr(qorder), 1 if approx else 0, ptr(s["Y"]), None, None, ptr(s["ws"]), wsb, st)
                self.calls.append(("avq_attention_fwd", L.avq_attention_fwd_ordered, args))
            else:
                args = (ptr(s["Q"]), ptr(s["cb"]), ptr(s["vsum"]), ptr(s["counts"])) + shp + tail + (
                    ptr(s["Y"]), None, None, ptr(s["ws"]), wsb, st)
                self.calls.append(("avq_attention_fwd", L.avq_attention_fwd_approx, args))
        else:
            # the checked calls leave the set's value sums and counts zero, as
            # every step does for the next one
            _lib.attention_prepare(s["vsum"], s["counts"], cfg.C, s["Q"].dtype, workspace=s["ws"])
            _lib.attention_fwd_prepared(s["Q"], s["cb"], s["ws"], cfg.C, P, bq, cfg.scale, Y=s["Y"],
                                        clear_vsum=s["vsum"], clear_counts=s["counts"])
            self.calls = [("avq_assign_aggregate_accum", L.avq_assign_aggregate_accum, kargs),
                          ("avq_attention_prepare", L.avq_attention_prepare,
                           (ptr(s["vsum"]), ptr(s["counts"]), cfg.B, cfg.H, cfg.d, cfg.M0, cfg.C, dt, ptr(s["ws"]),
                            wsb, st)),
                          ("avq_attention_fwd_prepared", L.avq_attention_fwd_prepared,
                           (ptr(s["Q"]), ptr(s["cb"])) + shp + tail + (
                               ptr(s["Y"]), None, None, ptr(s["ws"]), wsb, ptr(s["vsum"]), ptr(s["counts"]), st))]
        self.names = [c[0] for c in self.calls]

    def run(self, events=None):
        """Issue the pass; events (one more than the calls) are recorded
        before the first call and after each."""
        if events is not None:
            events[0].record()
        for i, (name, fn, args) in enumerate(self.calls):
            rc = fn(*args)
            if rc != 0:
                raise RuntimeError(f"{name} returned {rc}")
            if events is not None:
                events[i + 1].record()


def timed_steps(steps_by_set, n_steps, warmup, every=4):
    """Warm up, then time n_steps passes rotating over the input sets: wall
    time, per-unit durations (seconds, one row per sampled step) from events
    on the launch stream around every call of every `every`-th step (an event
    pair costs about a microsecond of stream time, so the other steps run
    without them), and the GPU span from the first step's start to the last
    step's end."""
    import torch
    for i in range(warmup):
        steps_by_set[i % len(steps_by_set)].run()
    torch.cuda.synchronize()
    n_units = len(steps_by_set[0].calls)
    sampled = [i for i in range(n_steps) if i % every == 0]
    ev = {i: [torch.cuda.Event(enable_timing=True) for _ in range(n_units + 1)] for i in sampled}
    first = torch.cuda.Event(enable_timing=True)
    last = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    first.record()
    for i in range(n_steps):
        steps_by_set[i % len(steps_by_set)].run(ev.get(i))
    last.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[ev[i][j].elapsed_time(ev[i][j + 1]) for j in range(n_units)] for i in sampled]) * 1e-3
    span = first.elapsed_time(last) * 1e-3
    return wall, per, span


def complexity(args):
    """Both calls over N in {4096, 16384, 65536} (B = 2, H = 16, d = 64, bf16) for flat
    codebooks of M in {64, 128, 256, 512} (P = 0) and a hierarchical one (M0 = 64, C = 8,
    P in {4, 16, 64}; and M0 = 128, P = 16): the median event time of each call over the timed
    steps, against the codewords a key is compared with (M, or M0 + C) and the codewords a query
    attends to (M, or M0 + P C).  Queries and values are seeded N(0, 1) draws on the device; a
    codebook from the generator; keys are a codeword plus noise, one codeword per run of 64
    consecutive tokens (the locality of the image workloads' 8x8 patches), or per token with
    --complexity-order random.  The attention time is avq_attention_prepare plus
    avq_attention_fwd_prepared.  One JSON line with every point and the log-log slopes."""
    import torch
    from adaptive_vector_quantized_amd import _lib, gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B, H, d = 2, 16, 64
    steps = max(20, min(args.steps, 200))
    warm = max(5, min(args.warmup, 50))
    shapes = [("vq", M, 0, 0) for M in (64, 128, 256, 512)] + [("avq", 64, 8, P) for P in (4, 16, 64)] + \
             [("avq", 128, 8, 16)]
    rows = []
    stream = torch.cuda.current_stream(dev)
    for N in (4096, 16384, 65536):
        g = torch.Generator(device=dev)
        g.manual_seed(2000 + N)
        Q, K, V = (torch.randn((B, H, N, d), generator=g, device=dev).to(torch.bfloat16).contiguous()
                   for _ in range(3))
        for kind, M0, C, P in shapes:
            cfg = gen.Config(f"complexity-{kind}", B=B, H=H, N=N, d=d, M0=M0, C=C, P=P, block_q=128, dtype="bf16",
                             grid=None, parents="uniform", seed=3000 + M0 + C)
            cb = torch.from_numpy(gen.make_codebook(3000 + M0 + C, H, M0, C, d)).to(torch.bfloat16).contiguous().to(dev)
            Mt = M0 * (1 + C)
            run = 1 if args.complexity_order == "random" else 64
            idx = torch.randint(0, Mt, (B, H, N // run), generator=g, device=dev).repeat_interleave(run, dim=2)
            Kc = (cb.float()[torch.arange(H, device=dev)[None, :, None], idx] + 0.1 * K.float()).to(torch.bfloat16)
            s = {"K": Kc.contiguous(), "V": V, "Q": Q, "cb": cb,
                 "vsum": torch.empty((B, H, Mt, d), dtype=torch.float32, device=dev),
                 "counts": torch.empty((B, H, Mt), dtype=torch.int32, device=dev),
                 "Y": torch.empty((B, H, N, d), dtype=torch.float32, device=dev),
                 "ws": torch.empty(_lib.workspace_size(B, H, d, M0, C, torch.bfloat16), dtype=torch.uint8,
                                   device=dev)}
            _, per, _ = timed_steps([Step(cfg, P, s, stream)], steps, warm, every=1)
            k1 = float(np.median(per[:, 0])) * 1e6
            k2 = float(np.median(per[:, 1] + per[:, 2])) * 1e6
            rows.append({"N": N, "kind": kind, "M0": M0, "C": C, "P": P, "precompute_codes": M0 + C,
                         "attention_codes": M0 + P * C, "assign_aggregate_us": round(k1, 2),
                         "attention_fwd_us": round(k2, 2)})
            print(f"[bench] {rows[-1]}", file=sys.stderr, flush=True)
            del cb, s, Kc
        del Q, K, V
        torch.cuda.empty_cache()

    def slope(xs, ys):
        return float(np.polyfit(np.log(xs), np.log(ys), 1)[0])
    fits = {}
    for col, codes in (("assign_aggregate_us", "precompute_codes"), ("attention_fwd_us", "attention_codes")):
        keys = sorted({(r["kind"], r["M0"], r["P"]) for r in rows})
        byN = [slope([r["N"] for r in rows if (r["kind"], r["M0"], r["P"]) == key],
                     [r[col] for r in rows if (r["kind"], r["M0"], r["P"]) == key]) for key in keys]
        vq = [r for r in rows if r["kind"] == "vq" and r["N"] == 65536]
        fits[col] = {"slope_in_N": [round(x, 3) for x in sorted(byN)],
                     "slope_in_codes_flat_N65536": round(slope([r[codes] for r in vq], [r[col] for r in vq]), 3)}
        if col == "attention_fwd_us":
            avq = [r for r in rows if r["kind"] == "avq" and r["M0"] == 64 and r["N"] == 65536]
            fits[col]["slope_in_codes_avq_N65536"] = round(slope([r[codes] for r in avq], [r[col] for r in avq]), 3)
    print(json.dumps({"metric": "call time versus N and codewords used (Tab. 1, Fig. 6)", "unit": "us",
                      "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
                      "config": {"workload": "B=2 H=16 d=64 block_q=128, N in {4096, 16384, 65536}; flat M in "
                                             "{64,128,256,512}; M0=64 C=8 P in {4,16,64}; M0=128 C=8 P=16; keys "
                                             + ("drawn per token" if args.complexity_order == "random"
                                                else "drawn per run of 64 tokens")},
                      "steps": steps, "warmup": warm, "points": rows, "fits": fits}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="grid128")
    ap.add_argument("--P", type=int, default=None)
    ap.add_argument("--sets", type=int, default=3, help="input sets rotated through the timed loop")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--approx-denominator", action="store_true",
                    help="time avq_attention_fwd_approx (importances per 64-parent tile, App. B Eq. 13-14)")
    ap.add_argument("--query-order", choices=("raster", "gilbert"), default="raster",
                    help="query tiles in row-major order, or along the Gilbert curve of the token grid "
                         "(avq_attention_fwd_ordered)")
    ap.add_argument("--codebook-update", choices=("none", "fused", "separate"), default="none",
                    help="time the forward pass plus the codebook update of the training recipe (App. A): key sums "
                         "from avq_assign_aggregate_kv (fused) or from a second aggregation call with V = K "
                         "(separate), then avq_codebook_update")
    ap.add_argument("--complexity", action="store_true",
                    help="time both calls over N and the number of codewords used (flat and hierarchical "
                         "codebooks), with log-log slopes: the linear-scaling check of Tab. 1 / Fig. 6")
    ap.add_argument("--complexity-order", choices=("runs", "random"), default="runs",
                    help="key order of the complexity scan: one codeword per run of 64 tokens, or per token")
    ap.add_argument("--sweep", action="store_true",
                    help="time the whole pass at every refinement budget of the workload (e.g. --workload sweep)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: measures one GPU; --gpus {args.gpus} is not supported (the forward pass "
              "would shard over batch*heads, each GPU running both calls on its share with no "
              "communication)", file=sys.stderr)
        sys.exit(2)

    import torch
    from adaptive_vector_quantized_amd import _lib, gen, gilbert

    if args.complexity:
        complexity(args)
        return
    cfg = gen.CONFIGS[args.workload]
    P = cfg.P if args.P is None else args.P
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def dev4(a):
        return torch.from_numpy(a).to(tdt).reshape(cfg.B, cfg.H, cfg.N, cfg.d).contiguous().to(dev)

    sets = []
    for i in range(args.sets):
        d = gen.make(cfg, seed=cfg.seed + 100 * i)
        sets.append({
            "Q": dev4(d["Q"]), "K": dev4(d["K"]), "V": dev4(d["V"]),
            "cb": torch.from_numpy(d["codebook"]).to(tdt).contiguous().to(dev),
            "vsum": torch.empty((cfg.B, cfg.H, cfg.Mt, cfg.d), dtype=torch.float32, device=dev),
            "counts": torch.empty((cfg.B, cfg.H, cfg.Mt), dtype=torch.int32, device=dev),
            "Y": torch.empty((cfg.B, cfg.H, cfg.N, cfg.d), dtype=torch.float32, device=dev),
            "ws": torch.empty(_lib.workspace_size(cfg.B, cfg.H, cfg.d, cfg.M0, cfg.C, tdt), dtype=torch.uint8,
                              device=dev),
        })
        del d
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: {args.sets} input sets resident, warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    qorder = None
    if args.query_order == "gilbert":
        if cfg.grid is None:
            raise SystemExit("--query-order gilbert needs a workload on a token grid")
        qorder = torch.from_numpy(gilbert.query_order(cfg.grid, cfg.grid)).to(dev)

    def steps_at(Ps):
        return [Step(cfg, Ps, s_, stream, approx=args.approx_denominator, qorder=qorder) for s_ in sets]

    if args.codebook_update != "none":
        # forward pass + codebook update: one line with the step rate and per-call times
        fused = args.codebook_update == "fused"
        for s_ in sets:
            s_["ksum"] = torch.empty_like(s_["vsum"])
            s_["S"] = torch.zeros((cfg.H, cfg.Mt, cfg.d), dtype=torch.float32, device=dev)
            s_["Nema"] = torch.zeros((cfg.H, cfg.Mt), dtype=torch.float32, device=dev)
            s_["cb32"] = s_["cb"].float().contiguous()

        def train_step(s_, e=None):
            if e is not None:
                e[0].record(stream)
            if fused:
                _lib.assign_aggregate_kv(s_["K"], s_["V"], s_["cb"], cfg.C, vsum=s_["vsum"], counts=s_["counts"],
                                         ksum=s_["ksum"])
            else:
                _lib.assign_aggregate(s_["K"], s_["V"], s_["cb"], cfg.C, vsum=s_["vsum"], counts=s_["counts"])
            if e is not None:
                e[1].record(stream)
            _lib.attention_fwd(s_["Q"], s_["cb"], s_["vsum"], s_["counts"], cfg.C, P, cfg.block_q, cfg.scale,
                               Y=s_["Y"], workspace=s_["ws"])
            if e is not None:
                e[2].record(stream)
            if not fused:
                _lib.assign_aggregate(s_["K"], s_["K"], s_["cb"], cfg.C, vsum=s_["ksum"], counts=s_["counts"])
            if e is not None:
                e[3].record(stream)
            _lib.codebook_update(s_["ksum"], s_["counts"], s_["S"], s_["Nema"], s_["cb32"], cfg.C, 0.99)
            if e is not None:
                e[4].record(stream)

        for i in range(args.warmup):
            train_step(sets[i % len(sets)])
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            train_step(sets[i % len(sets)], ev[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        seg = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in ev]) * 1e3  # us
        names = ["avq_assign_aggregate_kv" if fused else "avq_assign_aggregate", "avq_attention_fwd",
                 "" if fused else "avq_assign_aggregate (V = K)", "avq_codebook_update"]
        print(json.dumps({
            "metric": "AVQ fwd + codebook update Mtokens/s", "unit": "Mtokens/s",
            "value": round(cfg.B * cfg.N / (wall / args.steps) / 1e6, 3), "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 5), "higher_is_better": True,
            "dtype": cfg.dtype, "data": "synthetic",
            "config": {"workload": f"{cfg.name}: B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} M0={cfg.M0} C={cfg.C} "
                                   f"P={P} block_q={cfg.block_q}; key sums {args.codebook_update}, decay 0.99"},
            "calls_us": {n: round(float(seg[:, j].mean()), 2) for j, n in enumerate(names) if n}}), flush=True)
        return

    if args.sweep:
        # one line: the whole pass at every refinement budget of the workload
        rows = []
        for Ps in (cfg.sweep_P or (P,)):
            st_ = steps_at(Ps)
            wall, per, _ = timed_steps(st_, args.steps, args.warmup)
            row = {"P": Ps, "value": round(cfg.B * cfg.N / (wall / args.steps) / 1e6, 3),
                   "ms_per_step": round(wall / args.steps * 1e3, 5)}
            for j, n in enumerate(st_[0].names):
                row[f"{n}_us"] = round(float(per[:, j].mean()) * 1e6, 2)
            rows.append(row)
            print(f"[bench] P={Ps}: {rows[-1]}", file=sys.stderr, flush=True)
        print(json.dumps({"metric": "AVQ fwd Mtokens/s versus the refinement budget P", "unit": "Mtokens/s",
                          "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                          "dtype": cfg.dtype, "data": "synthetic",
                          "config": {"workload": f"{cfg.name}: B={cfg.B} H={cfg.H} N={cfg.N} d={cfg.d} M0={cfg.M0} "
                                                 f"C={cfg.C} block_q={cfg.block_q}"},
                          "sweep": rows}), flush=True)
        return

    st_ = steps_at(P)
    wall, per, gpu_span = timed_steps(st_, args.steps, args.warmup)

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    ms_per_step = wall / args.steps * 1e3
    tokens = cfg.B * cfg.N
    value = tokens / (wall / args.steps) / 1e6
    alg = algorithmic(cfg, P)
    mfma_peak = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_FP32_PEAK_TFLOPS
    prep_k, attn_k = attention_launches(cfg, P)
    launches = {"avq_attention_prepare": prep_k, "avq_attention_fwd_prepared": attn_k,
                "avq_attention_fwd": f"{prep_k} + {attn_k}"}
    units = {}
    for j, name in enumerate(st_[0].names):
        b, f = alg[name]
        t = per[:, j]
        avg = float(t.mean())
        units[name] = {
            "launches": launches.get(name, CALLS[name][0]),
            "avg_us": avg * 1e6, "median_us": float(np.median(t)) * 1e6,
            "algorithmic_bytes": b, "algorithmic_flops": f,
            "GBps": b / avg / 1e9, "hbm_frac": b / avg / 1e9 / HBM_PEAK_GBS,
            "TFLOPs": f / avg / 1e12, "mfma_frac": f / avg / 1e12 / mfma_peak,
        }
    dom = max(units, key=lambda k: units[k]["avg_us"])
    kd = units[dom]
    rec = load_record(dom, cfg.name) if qorder is None else None
    traffic = None if rec is None else rec.get("bytes_per_launch")
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Mtokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={cfg.B} H={cfg.H} N={cfg.N}"
                        + (f" ({cfg.grid}x{cfg.grid} token grid, 8x8-patch clusters)" if cfg.grid else "")
                        + f" d={cfg.d} M0={cfg.M0} C={cfg.C} P={P} block_q={cfg.block_q}, {cfg.parents} parent occupancy"
                        + (", importance with the approximate tiled denominator" if args.approx_denominator else "")
                        + (", query tiles along the Gilbert curve" if qorder is not None else ""),
            "global_batch": cfg.B, "seq_len": cfg.N, "heads": cfg.H, "parallelism": "single GPU",
        },
        "roofline": {
            "call": dom, "kernel": units[dom]["launches"],
            "bound": "hbm", "achieved": round(kd["GBps"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(kd["hbm_frac"], 4), "traffic": traffic,
            "mfma": {"achieved": round(kd["TFLOPs"], 2), "peak": mfma_peak, "unit": "TFLOP/s",
                     "frac": round(kd["mfma_frac"], 4)},
            "traced": traced_fractions(rec, kd["algorithmic_bytes"], kd["algorithmic_flops"], mfma_peak),
        },
        "units": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                  for k, v in units.items()},
        "gpu_span_ms_per_step": round(gpu_span / args.steps * 1e3, 5),
        "event_sampled_steps": int(per.shape[0]),
        "unit_sum_ms_per_step": round(float(per.sum(axis=1).mean()) * 1e3, 5),
        "Mhead_tokens_per_s": round(cfg.B * cfg.H * cfg.N / (wall / args.steps) / 1e6, 3),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, P)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
