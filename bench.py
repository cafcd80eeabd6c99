#!/usr/bin/env python3
"""Throughput of the speculative-sampling verify step on one MI355X.

One step = one whole verify call over one batch of synthetic input (for the
default workload ``c2``: the sampling verify of 64 requests x 5 positions x
32000 fp32 logits).  Inputs are resident in HBM before timing starts; the
batch is rotated over enough copies (>= 600 MB in total) that every step
reads HBM rather than the 256 MB Infinity Cache.  Steps are replayed from HIP
graphs (one per copy) so the host's launch cost does not pace the GPU;
``--no-graph`` times plain stream launches instead.

Printed: one JSON line with verify rows/s (value), the row-pass kernel's
achieved algorithmic HBM bandwidth against the 8 TB/s peak (``roofline``,
its duration measured with HIP events recorded by the library around that
kernel), and the CPU oracle's rows/s on a bounded sample (``cpu_baseline``).
Progress goes to stderr.
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
KERNEL_SOURCES = ["sv_device.h", "sv_rowpass.h"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c2", choices=["toy", "c2", "c3", "c4", "c5"])
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
    ap.add_argument("--rotate-mb", type=float, default=600.0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle time budget (0 = skip)")
    ap.add_argument("--copy-calibration-mb", type=float, default=0.0,
                    help="also run one plain device copy of this size (for counter calibration)")
    return ap.parse_args()


def kernel_source_hash():
    h = hashlib.sha256()
    for n in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "speculative_sampling_verification_sample_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(config):
    """HBM bytes per row-pass launch from the committed counter summary,
    or None when it is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"rowpass_{config}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class HipEvents:
    """hipEvent_t pairs through libamdhip64 (the library records them)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
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

    def step(i, timer=None):
        """One verify step; `timer` = (start, stop) hipEvents around the row
        pass of the sampling / greedy call."""
        w = copies[i % R]
        if timer is not None:
            lib.spec_set_rowpass_timer(timer[0], timer[1])
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
        if timer is not None:
            lib.spec_set_rowpass_timer(None, None)
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

    # ---- row-pass kernel duration (HIP events recorded by the library) ----
    log("row-pass kernel timing")
    hev = HipEvents()
    pairs = [(hev.create(), hev.create()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(pairs):
        step(i, timer=(a, b))
    torch.cuda.synchronize()
    durs = [hev.elapsed_ms(a, b) for a, b in pairs]
    for a, b in pairs:
        hev.destroy(a)
        hev.destroy(b)
    for a, b in zip(outs, ref):
        if R == 1 and not torch.equal(a, b):
            raise RuntimeError("outputs changed between steps")
    k_ms = float(np.mean(durs))
    row_bytes = V * cfg.logit_bytes
    alg_launch = rows * row_bytes  # the row pass reads every logit of the batch once
    achieved = alg_launch / (k_ms * 1e-3) / 1e9
    # counters are taken on the uniform batches at the workload's own B
    traffic = None if (rg or args.batch is not None) else read_traffic(cfg.name)

    # ---- whole-step algorithmic bytes ----
    nacc = ref[1].cpu().numpy()
    if greedy:
        step_bytes = rows * row_bytes + n_draft * 4 + B * (G + 2) * 4
    else:
        rejected = int((nacc < (gammas if rg else G)).sum())
        untrunc = cfg.top_k == 0 and cfg.top_p >= 1.0
        # q bytes per token: dense float32, or the draft's logits (read once
        # per call for their statistics, again on a rejected untruncated row)
        qb = w0.draft_logits.element_size() if dl else 4
        q_rows = rejected * V * qb if untrunc else 0
        step_bytes = rows * row_bytes + q_rows + n_draft * 12 + rows * 4 + B * (G + 1) * 4 + B * 4
        if dl:
            step_bytes += n_draft * V * qb
        if stats and not fused:
            # the separate statistics call: the target's gamma rows and q
            step_bytes += B * G * V * (cfg.logit_bytes + qb)
        elif stats:
            # the combined call's statistics: untruncated rows stream logits
            # and q again; truncated rows read sum(q) of a dense q for Z',
            # nothing more without Z' or when q comes from the draft's logits
            step_bytes += B * G * V * (cfg.logit_bytes + qb) if untrunc else (0 if dl or not zqp else B * G * V * 4)
    step_gbps = step_bytes / (ms_step * 1e-3) / 1e9

    # ---- CPU oracle baseline on a bounded sample ----
    cpu = None
    if args.cpu_seconds > 0:
        import oracle

        log(f"cpu oracle baseline (~{args.cpu_seconds:.0f} s)")
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
                if cfg.stats:
                    oracle.stats_request_draft_logits(lg[b], dz[b], ids[b], cfg.temperature, cfg.top_k, cfg.top_p)
            else:
                oracle.verify_request(lg[b], q[b], ids[b], ua[b], ur[b], cfg.temperature, cfg.top_k, cfg.top_p,
                                      beta=float(np.float32(args.lenience)) if lenient else 1.0)
                if cfg.stats:
                    oracle.stats_request(lg[b], q[b], ids[b], cfg.temperature, cfg.top_k, cfg.top_p)
            done += 1
        el = time.perf_counter() - t0
        cpu = {"value": nrows / el, "unit": "rows/s", "cores": 1, "kind": "oracle",
               "sample": f"{done} requests ({nrows} rows) cycled over the first {nsamp} requests of the "
                         f"same {cfg.name} batch, one process, one thread, {el:.1f} s"}

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
        "dtype": "f32",
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
        "roofline": {"bound": "hbm", "kernel": "rowpass (K1)", "achieved": achieved, "peak": PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / PEAK_GBPS, "traffic": traffic,
                     "alg_bytes_per_launch": alg_launch, "launch_us": k_ms * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
