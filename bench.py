#!/usr/bin/env python3
"""Throughput of the speculative-sampling verify step on one MI355X.

One step = one whole verify call over one batch of synthetic input.  The
default workload is ``c5``, the largest: 1024 requests x 5 positions x
256000 bf16 logits, T = 0.7, top-p = 0.95, sampled and with the acceptance
statistics (alpha, Z, Z', accept_prob) of the same call.  Inputs are
resident in HBM before timing starts; the batch is rotated over enough
copies (>= 600 MB in total) that every step reads HBM rather than the 256 MB
Infinity Cache.  Steps are replayed from HIP graphs (one per copy) so the
host's launch cost does not pace the GPU; ``--no-graph`` times plain stream
launches instead.

Printed: one JSON line with verify rows/s (value); ``roofline`` for the
step's dominant kernel (the stage with the longest mean duration, measured
with HIP events that the library attaches to each kernel dispatch), with
every stage's duration and algorithmic bandwidth beside it and the step's
own fraction of the 8 TB/s peak; and the CPU oracle's rows/s on a bounded
sample (``cpu_baseline``: one process, then a process pool over the host's
cores).  Progress goes to stderr.
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verify rows/sec and achieved HBM GB/s (% of peak) at B×(γ+1)×V"
PEAK_GBPS = 8000.0  # MI355X HBM3E

# Kernel stages the library can time (sv_stage in include/specverify.h):
# name, the tag of its counter summaries under profiles/, and the sources
# its kernels are built from (a summary taken on other sources is stale).
STAGES = {
    0: ("row pass", "rowpass", ["sv_device.h", "sv_rowpass.h"]),
    1: ("row finisher", "rowfinal", ["sv_device.h", "sv_rowfinal.h"]),
    2: ("acceptance and draws", "accept", ["sv_device.h", "sv_rowfinal.h", "sv_verify.h"]),
    3: ("full-row draw sums", "draw_partial", ["sv_device.h", "sv_verify.h"]),
    4: ("full-row draw finish", "draw_finish", ["sv_device.h", "sv_verify.h"]),
    5: ("statistics pass", "stats_pass", ["sv_device.h", "sv_verify.h"]),
    6: ("statistics finish", "stats_finish", ["sv_device.h", "sv_verify.h"]),
    7: ("greedy decision", "greedy", ["sv_device.h", "sv_verify.h"]),
    8: ("dense q row sums", "qsum", ["sv_device.h", "sv_verify.h"]),
    9: ("Z' completion", "stats_zqp", ["sv_device.h", "sv_verify.h"]),
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1, help="GPUs (only 1: the step is measured on one GPU)")
    ap.add_argument("--steps", type=int, default=200, help="timed steps")
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before them")
    ap.add_argument("--config", default="c5", choices=["toy", "c2", "c3", "c4", "c5"],
                    help="workload (default c5: sampling plus the acceptance statistics)")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of graph replays")
    ap.add_argument("--draft-logits", action="store_true",
                    help="hand the draft's logits instead of q (the library forms q); sampling workloads only")
    ap.add_argument("--ragged", action="store_true",
                    help="ragged batch: request b keeps gamma_b ~ uniform{0..gamma} drafts (packed inputs; the "
                         "sampling or greedy call only)")
    ap.add_argument("--lenience", type=float, default=None,
                    help="lenient acceptance factor in (0, 1] for the sampling call (dense q, uniform batch)")
    ap.add_argument("--batch", type=int, default=None,
                    help="requests per step (default: the workload's B); the recipe is otherwise unchanged")
    ap.add_argument("--no-z-qp", action="store_true",
                    help="statistics without Z' = sum (q - p)_+ (alpha, Z and accept_prob only)")
    ap.add_argument("--rotate-mb", type=float, default=600.0,
                    help="workloads smaller than this are copied and the timed loop rotates over the copies, so "
                         "that the inputs come from HBM rather than the last-level cache")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU oracle time budget of each of its two legs (0 = skip)")
    ap.add_argument("--copy-calibration-mb", type=float, default=0.0,
                    help="also run one plain device copy of this size (for counter calibration)")
    return ap.parse_args()


def kernel_source_hash(sources):
    h = hashlib.sha256()
    for n in sources:
        with open(os.path.join(ROOT, "speculative_sampling_verification_sample_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(stage, config):
    """HBM bytes per launch of a stage's kernel from the committed counter
    summary, or None when it is missing or was taken on other sources."""
    _, tag, sources = STAGES[stage]
    path = os.path.join(ROOT, "profiles", f"{tag}_{config}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash(sources):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class HipEvents:
    """hipEvent_t pairs through libamdhip64 (the library records them)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipGetLastError.restype = ctypes.c_int

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        """Milliseconds between two recorded events; RuntimeError (with the
        runtime's error state cleared) when they were never recorded."""
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            self.hip.hipGetLastError()
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the verify step is measured on one MI355X "
              "(requests shard across GPUs with no communication; see the design notes). "
              f"Got --gpus {args.gpus}, WORLD_SIZE={world}.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import speculative_sampling_verification_sample_amd as sv
    from workloads import CONFIGS, generate, pack_ragged, ragged_gammas

    cfg = CONFIGS[args.config]
    if args.batch is not None:
        import dataclasses

        if args.batch < 1:
            raise SystemExit("--batch must be at least 1")
        cfg = dataclasses.replace(cfg, B=args.batch)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = sv.load_library()
    log(f"generating {cfg.name}: B={cfg.B} gamma={cfg.gamma} V={cfg.V} {cfg.dtype}")
    w0 = generate(cfg, dev)
    torch.cuda.synchronize()
    G, B, V = cfg.gamma, cfg.B, cfg.V
    rg = args.ragged
    lenient = args.lenience is not None
    if lenient and (rg or args.draft_logits or cfg.mode == "greedy"):
        raise SystemExit("--lenience applies to the uniform sampling call with a dense q")
    gammas = ragged_gammas(B, G, 1000 + B) if rg else None

    def nbytes(t):
        return 0 if t is None else t.numel() * t.element_size()

    def make(w):
        return pack_ragged(w, gammas) if rg else w

    wu = w0  # the uniform batch (the CPU baseline slices its requests)
    w0 = make(w0)
    qsrc = w0.draft_logits if args.draft_logits else w0.q  # what the step reads for q
    per_copy = sum(nbytes(t) for t in (w0.logits, qsrc, w0.ids, w0.u_accept, w0.u_resample))
    R = max(1, math.ceil(args.rotate_mb * 1e6 / per_copy)) if per_copy < args.rotate_mb * 1e6 else 1
    copies = [w0]
    for _ in range(R - 1):
        c = make(generate(cfg, dev))  # same recipe and seed, distinct memory
        copies.append(c)
    torch.cuda.synchronize()
    log(f"{R} resident copies of {per_copy / 1e6:.1f} MB")

    greedy = cfg.mode == "greedy"
    dl = args.draft_logits
    if dl and (greedy or w0.draft_logits is None):
        raise SystemExit("--draft-logits applies to the sampling workloads (toy, c2, c3, c5)")
    n_draft = int(gammas.sum()) if rg else B * G
    rows = n_draft + B  # target rows the step reads
    if dl:
        need = sv.draft_logits_workspace_size(B, G, V, w0.logits.dtype, w0.draft_logits.dtype, cfg.temperature,
                                              cfg.top_k, cfg.top_p)
    else:
        need = sv.workspace_size(B, G, V, w0.logits.dtype, cfg.temperature, cfg.top_k, cfg.top_p)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    outs = (torch.empty((B, G + 1), dtype=torch.int32, device=dev),
            torch.empty((B,), dtype=torch.int32, device=dev),
            torch.empty((B,), dtype=torch.int32, device=dev))
    stats = cfg.stats and not rg  # the statistics call takes uniform batches
    # sampling and statistics in one call (one pass over the logits), except
    # with lenience, whose call has no statistics: then the separate call
    fused = stats and not lenient
    zqp = not args.no_z_qp
    sout = tuple(None if (k == 2 and not zqp) else torch.empty((B, G), dtype=torch.float32, device=dev)
                 for k in range(4)) if stats else None

    def step(i, timers=None):
        """One verify step; `timers` = {stage: (start, stop)} hipEvents the
        library attaches to that stage's kernel dispatch."""
        w = copies[i % R]
        for st, (ta, tb) in (timers or {}).items():
            lib.spec_set_stage_timer(st, ta, tb)
        if rg and dl:
            sv.verify_sample_ragged_draft_logits(w.logits, w.draft_logits, w.ids, w.cu, w.u_accept, w.u_resample, G,
                                                 cfg.temperature, cfg.top_k, cfg.top_p, workspace=ws, out=outs)
        elif rg and greedy:
            sv.verify_greedy_ragged(w.logits, w.ids, w.cu, G, workspace=ws, out=outs)
        elif rg:
            sv.verify_sample_ragged(w.logits, w.q, w.ids, w.cu, w.u_accept, w.u_resample, G, cfg.temperature,
                                    cfg.top_k, cfg.top_p, workspace=ws, out=outs)
        elif greedy:
            sv.verify_greedy(w.logits, w.ids, workspace=ws, out=outs)
        elif fused and dl:
            sv.verify_sample_stats_draft_logits(w.logits, w.draft_logits, w.ids, w.u_accept, w.u_resample,
                                                cfg.temperature, cfg.top_k, cfg.top_p, workspace=ws, out=outs,
                                                stats_out=sout)
        elif fused:
            sv.verify_sample_stats(w.logits, w.q, w.ids, w.u_accept, w.u_resample, cfg.temperature, cfg.top_k,
                                   cfg.top_p, workspace=ws, out=outs, stats_out=sout)
        elif dl:
            sv.verify_sample_draft_logits(w.logits, w.draft_logits, w.ids, w.u_accept, w.u_resample,
                                          cfg.temperature, cfg.top_k, cfg.top_p, workspace=ws, out=outs)
        elif lenient:
            sv.verify_sample_lenient(w.logits, w.q, w.ids, w.u_accept, w.u_resample, cfg.temperature, cfg.top_k,
                                     cfg.top_p, lenience=args.lenience, workspace=ws, out=outs)
        else:
            sv.verify_sample(w.logits, w.q, w.ids, w.u_accept, w.u_resample, cfg.temperature, cfg.top_k,
                             cfg.top_p, workspace=ws, out=outs)
        for st in (timers or {}):
            lib.spec_set_stage_timer(st, None, None)
        if stats and not fused:
            sv.accept_stats(w.logits, w.q, w.ids, cfg.temperature, cfg.top_k, cfg.top_p, workspace=ws,
                            out=sout)

    # ---- reference outputs (eager) and graph capture ----
    step(0)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graphs = None
    if not args.no_graph:
        graphs = []
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s):
                    step(i)
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graphs[0].replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            if not torch.equal(a, b):
                raise RuntimeError("graph replay differs from the eager step")

    def run(i):
        if graphs is not None:
            graphs[i % R].replay()
        else:
            step(i)

    log(f"warmup {args.warmup}")
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()

    # ---- timed region ----
    log(f"timing {args.steps} steps ({'graph' if graphs else 'eager'})")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / args.steps
    value = rows / (ms_step * 1e-3)

    # ---- per-stage kernel durations (HIP events the library attaches to
    #      each stage's kernel dispatch; the separate statistics call of the
    #      lenient workload runs untimed) ----
    log("stage timing")
    hev = HipEvents()
    nk = min(args.steps, 100)
    pairs = [{st: (hev.create(), hev.create()) for st in STAGES} for _ in range(nk)]
    torch.cuda.synchronize()
    for i, tm in enumerate(pairs):
        step(i, timers=tm)
    torch.cuda.synchronize()
    stage_ms = {}
    for st in STAGES:
        try:
            hev.elapsed_ms(pairs[0][st][0], pairs[0][st][1])
        except RuntimeError:  # events never recorded: no such stage in this call
            continue
        stage_ms[st] = float(np.mean([hev.elapsed_ms(tm[st][0], tm[st][1]) for tm in pairs]))
    for tm in pairs:
        for a, b in tm.values():
            hev.destroy(a)
            hev.destroy(b)
    for a, b in zip(outs, ref):
        if R == 1 and not torch.equal(a, b):
            raise RuntimeError("outputs changed between steps")

    # ---- algorithmic bytes: per stage and per step ----
    nacc = ref[1].cpu().numpy()
    untrunc = cfg.top_k == 0 and cfg.top_p >= 1.0
    row_bytes = V * cfg.logit_bytes
    # q bytes per token: dense float32, or the draft's logits
    qb = (w0.draft_logits.element_size() if dl else 4) if not greedy else 0
    rejected = 0 if greedy else int((nacc < (gammas if rg else G)).sum())
    stage_bytes = {0: rows * row_bytes}
    if greedy:
        step_bytes = rows * row_bytes + n_draft * 4 + B * (G + 2) * 4
    else:
        # a full-row draw reads the drawn row, and q's row on a rejection
        draw_bytes = (B * row_bytes + rejected * V * qb) if untrunc else 0
        stage_bytes[2 if G + 1 <= 64 else 3] = draw_bytes
        step_bytes = rows * row_bytes + draw_bytes + n_draft * 12 + rows * 4 + B * (G + 1) * 4 + B * 4
        if dl:
            step_bytes += n_draft * V * qb  # the draft rows' own pass
        if stats:
            # statistics: untruncated rows stream logits and q again;
            # truncated rows read sum(q) of a dense q for Z' (the row sums
            # beside the target's passes), nothing more without Z' or when q
            # comes from the draft's logits
            if untrunc:
                stage_bytes[5] = B * G * V * (cfg.logit_bytes + qb)
            elif zqp and not dl:
                stage_bytes[8] = B * G * V * 4
            step_bytes += stage_bytes.get(5, 0) + stage_bytes.get(8, 0)
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9

    def stage_line(st):
        ms = stage_ms[st]
        by = stage_bytes.get(st, 0)
        gbps = by / (ms * 1e-3) / 1e9 if by else None
        return {"us": ms * 1e3, "alg_bytes": by, "GBps": gbps, "frac": gbps / PEAK_GBPS if by else None}

    stages = {STAGES[st][0]: stage_line(st) for st in sorted(stage_ms)}
    dom = max(stage_ms, key=lambda st: stage_ms[st])
    # the dominant kernel again, with only its own events attached
    solo = [(hev.create(), hev.create()) for _ in range(nk)]
    torch.cuda.synchronize()
    for i, tm in enumerate(solo):
        step(i, timers={dom: tm})
    torch.cuda.synchronize()
    stage_ms[dom] = float(np.mean([hev.elapsed_ms(a, b) for a, b in solo]))
    for a, b in solo:
        hev.destroy(a)
        hev.destroy(b)
    dom_line = stage_line(dom)
    # counters are taken on uniform batches at the workload's own B
    traffic = None if (rg or args.batch is not None or dl or lenient) else read_traffic(dom, cfg.name)
    k1_traffic = None if (rg or args.batch is not None or dl or lenient) else read_traffic(0, cfg.name)
    log(" ".join(f"{n}={v['us']:.1f}us" for n, v in stages.items()))

    # ---- CPU oracle baseline on a bounded sample: one process, then a pool
    #      over the host's cores (at most 16) ----
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        from oracle import pool as opool

        nsamp = min(B, 64)
        lg = wu.logits[:nsamp].detach().cpu()
        lg = oracle.bf16_bits_to_f64(lg.view(torch.int16).numpy()) if lg.dtype == torch.bfloat16 \
            else lg.double().numpy()
        ids = wu.ids[:nsamp].cpu().numpy()
        if not greedy:
            q = wu.q[:nsamp].cpu().numpy()
            ua = wu.u_accept[:nsamp].cpu().numpy()
            ur = wu.u_resample[:nsamp].cpu().numpy()
        if dl:
            dz = wu.draft_logits[:nsamp].detach().cpu()
            dz = oracle.bf16_bits_to_f64(dz.view(torch.int16).numpy()) if dz.dtype == torch.bfloat16 \
                else dz.double().numpy()
        beta = float(np.float32(args.lenience)) if lenient else 1.0
        log(f"cpu oracle baseline, one process (~{args.cpu_seconds:.0f} s)")
        done = 0
        nrows = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:
            b = done % nsamp
            if rg:
                # request b of the ragged batch: the first gammas[b] drafts
                g = int(gammas[b])
                if greedy:
                    oracle.greedy_request(lg[b, : g + 1], ids[b, :g])
                elif dl:
                    oracle.verify_request_draft_logits(lg[b, : g + 1], dz[b, :g], ids[b, :g], ua[b, :g],
                                                       ur[b, : g + 1], cfg.temperature, cfg.top_k, cfg.top_p)
                else:
                    oracle.verify_request(lg[b, : g + 1], q[b, :g], ids[b, :g], ua[b, :g], ur[b, : g + 1],
                                          cfg.temperature, cfg.top_k, cfg.top_p)
                nrows += g + 1
                done += 1
                continue
            nrows += G + 1
            if greedy:
                oracle.greedy_request(lg[b], ids[b])
            elif dl:
                oracle.verify_request_draft_logits(lg[b], dz[b], ids[b], ua[b], ur[b], cfg.temperature, cfg.top_k,
                                                   cfg.top_p)
                if stats:
                    oracle.stats_request_draft_logits(lg[b], dz[b], ids[b], cfg.temperature, cfg.top_k, cfg.top_p)
            else:
                oracle.verify_request(lg[b], q[b], ids[b], ua[b], ur[b], cfg.temperature, cfg.top_k, cfg.top_p,
                                      beta=beta)
                if stats:
                    oracle.stats_request(lg[b], q[b], ids[b], cfg.temperature, cfg.top_k, cfg.top_p)
            done += 1
        el1 = time.perf_counter() - t0
        single = nrows / el1
        cpu = {"value": single, "unit": "rows/s", "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
               "single_process_rows_per_s": single,
               "sample": f"one process: {done} requests ({nrows} rows) cycled over the first {nsamp} requests of "
                         f"the same {cfg.name} batch, {el1:.1f} s"}
        if not rg:
            # the pool: the first n requests of the batch, n sized from the
            # single-process rate to about --cpu-seconds of work per core; a
            # batch smaller than that is passed over again, as many whole
            # times as fit in that time
            workers = opool.default_workers()
            want = max(workers, math.ceil(done / el1 * workers * args.cpu_seconds))
            n = int(min(B, want))
            arrays = dict(logits=(wu.logits[:n].view(torch.int16) if wu.logits.dtype == torch.bfloat16
                                  else wu.logits[:n]).cpu().numpy(), ids=wu.ids[:n].cpu().numpy())
            prm = dict(T=cfg.temperature, top_k=cfg.top_k, top_p=cfg.top_p, beta=beta)
            if greedy:
                kinds = ["greedy"]
            else:
                arrays.update(u_accept=wu.u_accept[:n].cpu().numpy(), u_resample=wu.u_resample[:n].cpu().numpy())
                if dl:
                    d = wu.draft_logits[:n]
                    arrays["draft_logits"] = (d.view(torch.int16) if d.dtype == torch.bfloat16 else d).cpu().numpy()
                    kinds = ["sample_draft_logits"] + (["stats_draft_logits"] if stats else [])
                else:
                    arrays["q"] = wu.q[:n].cpu().numpy()
                    kinds = ["sample"] + (["stats"] if stats else [])
            log(f"cpu oracle baseline, {workers} processes over {n} requests")
            with opool.make_pool(workers) as pl:
                opool.run("greedy", dict(logits=arrays["logits"][:workers], ids=arrays["ids"][:workers]), {},
                          min(workers, n), pool=pl)  # workers started and warm
                need = {"greedy": ("logits", "ids"),
                        "sample": ("logits", "q", "ids", "u_accept", "u_resample"),
                        "stats": ("logits", "q", "ids"),
                        "sample_draft_logits": ("logits", "draft_logits", "ids", "u_accept", "u_resample"),
                        "stats_draft_logits": ("logits", "draft_logits", "ids")}
                # one pass, then as many more (in one go) as fit the time
                def passes(r):
                    for k in kinds:
                        opool.run(k, {a: arrays[a] for a in need[k]}, prm, n, pool=pl, repeat=r)
                t0 = time.perf_counter()
                passes(1)
                el_one = time.perf_counter() - t0
                more = int((args.cpu_seconds - el_one) // el_one) if el_one > 0 else 0
                if more > 0:
                    passes(more)
                rep = 1 + max(0, more)
                el2 = time.perf_counter() - t0
            cpu.update(value=rep * n * (G + 1) / el2, cores=workers,
                       sample=cpu["sample"] + f"; pool: the first {n} requests"
                                              f"{f' {rep} times over' if rep > 1 else ''}, {workers} worker "
                                              f"processes, {el2:.1f} s (value and cores are the pool's)")

    if args.copy_calibration_mb > 0:
        n = int(args.copy_calibration_mb * 1e6) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n * 4} bytes read, {n * 4} bytes written")

    desc = {"c2": "sampling verify, fp32 logits N(0,2^2), draft = target + N(0,0.5^2), T=1, no truncation",
            "c3": "sampling verify, bf16 logits N(0,3^2) with 1% boosted +6, T=0.8, top-k=50",
            "c4": "greedy verify, bf16 logits N(0,2.5^2)",
            "c5": "sampling verify + acceptance statistics, bf16 Zipf-shaped logits, T=0.7, top-p=0.95",
            "toy": "sampling verify, 1e6 rounds of one Dirichlet request, V=5"}[cfg.name]
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w0.logits.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {desc}", "B": B, "gamma": G, "V": V,
                   "logits": cfg.dtype, "temperature": cfg.temperature, "top_k": cfg.top_k, "top_p": cfg.top_p,
                   "q": "formed from the draft's logits" if dl else "dense float32 input",
                   "acceptance": f"lenient, beta = {args.lenience}" if lenient else "lossless",
                   "statistics": ("none" if not stats else
                                  ("combined sampling + statistics call" if fused else "separate statistics call")
                                  + ("" if zqp else ", without Z'")),
                   "batch": (f"ragged: gamma_b uniform on 0..{G}, {n_draft} drafts, packed; sampling / greedy "
                             f"call only" if rg else "uniform"),
                   "rows_per_step": rows, "rotated_copies": R, "graph_replay": graphs is not None,
                   "wall_s_timed": wall, "step_alg_bytes": step_bytes, "step_alg_GBps": step_gbps},
        "roofline": {"bound": "hbm", "kernel": STAGES[dom][0], "achieved": dom_line["GBps"], "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": dom_line["frac"], "traffic": traffic,
                     "alg_bytes_per_launch": dom_line["alg_bytes"], "launch_us": dom_line["us"],
                     "step_frac": step_gbps / PEAK_GBPS, "stages": stages,
                     # the target logits' row pass (K1), with its own measured traffic
                     "row_pass": (dict(stages[STAGES[0][0]], traffic=k1_traffic)
                                  if STAGES[0][0] in stages else None)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
