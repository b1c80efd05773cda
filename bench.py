#!/usr/bin/env python3
"""Decode-step benchmark of the ParisKV retrieval path on one MI355X.

One step = for every (batch, KV head) of one layer: append the new decode key
to the index, retrieve the top-k (query prep, vote scan, threshold, compact +
RSQ-IP rerank, exact top-k) and run split-K sparse attention over the
selected rows.  Inputs are synthetic and resident in HBM; `--layers`
independent layer instances are used in rotation so the 256 MB Infinity
Cache cannot hold one layer's bucket ids across consecutive steps.

The K timed steps are captured into one HIP graph and replayed once between
two device synchronisations (so launch overhead of the ctypes binding does
not pace the GPU).  Per-kernel durations come from the steps that follow,
launched with start/stop HIP events that each kernel's own dispatch stamps.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("decode retrieval+sparse-attn µs/step/layer and keys scanned/s "
          "at 128K-1M ctx")
HBM_PEAK_GBPS = 8000.0
# the sources the vote-scan kernel is built from
KERNEL_SRC = [os.path.join(ROOT, "kv_cache_top_srht_amd", "csrc", f)
              for f in ("pariskv_kernels.hip", "pariskv_device.h", "pariskv_internal.h")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="million")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--cpu-steps", type=int, default=2)
    ap.add_argument("--profile-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed steps eagerly instead of as a graph")
    ap.add_argument("--warm-steps", type=int, default=100,
                    help="steps of the warm figure (one layer repeated)")
    ap.add_argument("--drift", action="store_true",
                    help="run the long-generation drift workload instead: recall@k "
                         "and per-step GPU time at checkpoints while keys are appended")
    ap.add_argument("--drift-steps", type=int, default=0,
                    help="decode steps of the drift run (default: the workload's)")
    ap.add_argument("--drift-every", type=int, default=1024)
    ap.add_argument("--rho", type=int, default=0,
                    help="centroids kept per subspace (default: the workload's); "
                         "tiers become rho, rho-1, ..., 1 unless --tiers is given")
    ap.add_argument("--tiers", default="", help="comma-separated tier weights")
    ap.add_argument("--subspaces", type=int, default=0,
                    help="subspaces B (16: 8 coordinates each, 32: 4 each; "
                         "default: the workload's)")
    ap.add_argument("--cand-frac", default="",
                    help="candidate fraction as num/den (default: the workload's)")
    ap.add_argument("--window", default="",
                    help="L,U: sliding-window regions with L local tokens and an "
                         "update buffer of U; the far store is HBM, or pinned host "
                         "memory with --uva kv")
    ap.add_argument("--retrieval-path", default="auto",
                    choices=["auto", "pipeline", "single"],
                    help="retrieval path: the library's choice (auto), the "
                         "multi-kernel pipeline, or the single kernel")
    ap.add_argument("--per-query-head", action="store_true",
                    help="unshared retrieval: every query head selects its own "
                         "top-k with its own query over its KV head's index")
    ap.add_argument("--si", action="store_true",
                    help="the Self-Indexing workload instead: sign-VQ index with "
                         "LUT-GEMV scores over every key, exact top-k, same attention")
    ap.add_argument("--separate", action="store_true",
                    help="run retrieval and attention as separate calls "
                         "(pariskv_retrieve_topk + pariskv_sparse_attn) instead of "
                         "pariskv_retrieve_attend")
    ap.add_argument("--uva", choices=["none", "v", "kv"], default="none",
                    help="keep V (v) or K and V (kv) of every layer in pinned host "
                         "memory, read by the kernels over the host link")
    return ap.parse_args()


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def read_traffic(name: str, launches_bytes: float):
    """HBM traffic per launch from a committed rocprofv3 --pmc summary, or
    None when it is missing or was taken on a different kernel source."""
    p = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        m = re.match(r"^\s*([a-z0-9_]+)\s*:\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("kernel_sha256_16") != kernel_sha():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(the work shards by (batch, KV head) with no exchange between "
              "GPUs).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import kv_cache_top_srht_amd as pk
    from kv_cache_top_srht_amd import synth

    pk.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.drift:
        drift_run(args, pk, synth, np, torch)
        return
    dev = "cuda"
    w = synth.WORKLOADS[args.workload]
    if args.rho:
        w = w.scaled(rho=args.rho, tiers=tuple(range(args.rho, 0, -1)))
    if args.tiers:
        t = tuple(int(x) for x in args.tiers.split(","))
        w = w.scaled(rho=len(t), tiers=t)
    if args.cand_frac:
        num, den = (int(x) for x in args.cand_frac.split("/"))
        w = w.scaled(cand_num=num, cand_den=den)
    if args.subspaces:
        w = w.scaled(B=args.subspaces)
    if args.si and (args.window or args.per_query_head or args.uva != "none"):
        sys.exit("--si runs alone (no --window, --per-query-head or --uva)")
    if args.per_query_head:
        if args.window:
            sys.exit("--per-query-head runs without --window")
        w = w.scaled(per_query_head=True)
    K_steps, W_steps, Lr = args.steps, args.warmup, max(1, args.layers)
    per_layer = math.ceil((K_steps + W_steps + args.profile_steps) / Lr) + 1
    cap = w.N + per_layer + max(0, args.warm_steps) + 1
    BH = w.batch * w.n_kv_heads
    # retrieval units: one per (batch, KV head), or per (batch, query head)
    # in the unshared mode
    U = w.batch * (w.n_q_heads if w.per_query_head else w.n_kv_heads)
    print("[bench] workload=%s layers=%d cap=%d steps=%d warmup=%d" %
          (args.workload, Lr, cap, K_steps, W_steps), file=sys.stderr, flush=True)

    win_L = win_U = 0
    if args.window:
        win_L, win_U = (int(x) for x in args.window.split(","))
        if args.uva == "v":
            sys.exit("--window keeps K and V together: use --uva kv or none")
    layers = []
    for l in range(Lr):
        lay = synth.make_layer(w.scaled(N=cap), dev, layer=l)
        if args.si:
            L = pk.SiLayer(pk.si_config_for(w, capacity=cap), lay["K"], w.N, k=w.k,
                           device=dev)
            layers.append((L, lay))
            torch.cuda.synchronize()
            continue
        cfg = pk.config_for(w, capacity=cap)
        L = pk.Layer(cfg, lay["signs"], lay["K"], w.N - win_L, k=w.k, device=dev)
        L.set_path({"auto": pk.PATH_AUTO, "pipeline": pk.PATH_PIPELINE,
                    "single": pk.PATH_SINGLE}[args.retrieval_path])
        if args.window:
            # near store: sinks, then the ring of local + buffer rows; far store:
            # the layer's own K/V (positions at their rows), moved to pinned
            # host memory with --uva kv
            S, ring = w.sinks, win_L + win_U
            shp = (w.batch, w.n_kv_heads, S + ring, w.d)
            Kn = torch.zeros(shp, dtype=lay["K"].dtype, device=dev)
            Vn = torch.zeros_like(Kn)
            Kn[:, :, :S], Vn[:, :, :S] = lay["K"][:, :, :S], lay["V"][:, :, :S]
            pos = torch.arange(w.N - win_L, w.N, device=dev)
            slots = S + (pos - S) % ring
            Kn[:, :, slots] = lay["K"][:, :, pos]
            Vn[:, :, slots] = lay["V"][:, :, pos]
            lay["Kn"], lay["Vn"] = Kn, Vn
            if args.uva == "kv":
                for name in ("K", "V"):
                    hst = torch.empty(lay[name].shape, dtype=lay[name].dtype,
                                      pin_memory=True)
                    hst.copy_(lay[name])
                    lay[name] = hst
            lay["win"] = pk.pariskv_window_create(L.handle, win_L, win_U, Kn, Vn,
                                                  lay["K"], lay["V"], cap)
            lay["win_ws"] = torch.empty(
                pk.pariskv_window_attn_workspace_bytes(lay["win"], w.k),
                dtype=torch.uint8, device=dev)
        if args.uva != "none" and not args.window:
            # full-precision rows in pinned host memory, mapped into the GPU's
            # address space; the device copies are dropped
            for name in (("V",) if args.uva == "v" else ("K", "V")):
                hst = torch.empty(lay[name].shape, dtype=lay[name].dtype, pin_memory=True)
                hst.copy_(lay[name])
                lay[name] = hst
        layers.append((L, lay))
        torch.cuda.synchronize()
    idx = torch.empty(U, w.k, dtype=torch.int32, device=dev)
    out = torch.empty_like(layers[0][1]["Q"])
    scale = w.d ** -0.5
    dt_code = pk.PARISKV_DTYPE_BF16 if w.dtype == "bf16" else pk.PARISKV_DTYPE_FP32
    E_of = []

    def step(t, ev=None):
        L, lay = layers[t % Lr]
        if args.window:
            n = pk.pariskv_window_state(lay["win"])[0]
            pk.pariskv_window_append(lay["win"], lay["K"][:, :, n:], lay["V"][:, :, n:],
                                     cap)
            E_of.append(L.size - w.sinks)
            if ev is None:
                L.retrieve(lay["Q"], idx)
                pk.pariskv_window_attn(lay["win"], lay["Q"], idx, w.k, scale, out,
                                       lay["win_ws"])
            else:
                pk.pariskv_retrieve_topk_profiled(L.handle, lay["Q"], w.k, idx, None,
                                                  L.ws, ev[0:12])
                pk.pariskv_window_attn_profiled(lay["win"], lay["Q"], idx, w.k, scale,
                                                out, lay["win_ws"], ev[12:16])
            return
        n = L.size
        L.append(lay["K"][:, :, n:], 1, rows_per_head=cap)
        E_of.append(L.size - w.sinks)
        if not args.si and not args.separate:
            # retrieval and attention in one call; ev: the 6 retrieval stages,
            # then the attention split and merge
            if ev is None:
                L.retrieve_attend(lay["Q"], lay["K"], lay["V"], idx, out, scale=scale)
            else:
                pk.pariskv_retrieve_attend_profiled(L.handle, lay["Q"], lay["K"], lay["V"],
                                                    cap, w.k, scale, idx, None, out,
                                                    L.attend_workspace(), ev[0:16])
            return
        if ev is None:
            L.retrieve(lay["Q"], idx)
            L.attend(lay["Q"], lay["K"], lay["V"], idx, out, scale)
        else:
            # ev[0:12]: start/stop of the 6 retrieval kernels, ev[12:16]: of
            # the 2 attention kernels, stamped by the dispatches themselves
            retr = (pk.pariskv_si_retrieve_topk_profiled if args.si
                    else pk.pariskv_retrieve_topk_profiled)
            retr(L.handle, lay["Q"], w.k, idx, None, L.ws, ev[0:12])
            attn = (pk.pariskv_sparse_attn_per_query_head_profiled if w.per_query_head
                    else pk.pariskv_sparse_attn_profiled)
            attn(lay["Q"], lay["K"], lay["V"], cap, idx, w.k, w.batch, w.n_q_heads,
                 w.n_kv_heads, w.d, dt_code, scale, out, L.attn_ws, ev[12:16])

    for t in range(W_steps):
        step(t)
    torch.cuda.synchronize()

    # timed region: exactly K distinct steps, split into R consecutive parts
    # (R = min(10, K), sizes differing by at most one step); each part is
    # captured as one HIP graph, and the graphs are replayed back to back
    # between two synchronisations, with an event recorded between replays
    # (outside the graphs), so that each part's per-step time is known
    E_of.clear()
    mode = "eager" if args.eager else "hip-graph"
    R = max(1, min(10, K_steps))
    part = [K_steps // R + (1 if r < K_steps % R else 0) for r in range(R)]
    graphs = []
    if not args.eager:
        t = W_steps
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=torch.cuda.Stream()):
                for _ in range(part[r]):
                    step(t)
                    t += 1
            graphs.append(g)
        torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t = W_steps
    marks[0].record()
    for r in range(R):
        if graphs:
            graphs[r].replay()
        else:
            for _ in range(part[r]):
                step(t)
                t += 1
        marks[r + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part_us = np.array([marks[r].elapsed_time(marks[r + 1]) * 1e3 / part[r]
                        for r in range(R)])
    E_timed = list(E_of)

    # kernel durations: the next P steps launched with dispatch-stamped
    # start/stop events on every kernel
    P = min(K_steps, args.profile_steps)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(16)]
              for _ in range(P)]
    for row in events:          # torch creates the underlying event lazily
        for e in row:
            e.record()
    E_of.clear()
    torch.cuda.synchronize()
    for t in range(P):
        step(W_steps + K_steps + t, events[t])
    torch.cuda.synchronize()
    E_prof = np.array(E_of, dtype=np.float64)
    kern = np.array([[events[t][2 * i].elapsed_time(events[t][2 * i + 1])
                      for i in range(8)] for t in range(P)]) * 1e3   # us
    names = ["si_lut", "si_scan", "threshold", "si_compact", "topk",
             "topk_second_pass"] if args.si else \
        [pk.pariskv_stage_name(i) for i in range(pk.PARISKV_RETRIEVE_STAGES)]
    names = names + \
        ["attn_split", "attn_merge"]
    stage_us = {n: float(kern[:, i].mean()) for i, n in enumerate(names)}
    step_us = np.array([events[t][0].elapsed_time(events[t][15])
                        for t in range(P)]) * 1e3
    E_of[:] = E_timed
    E = np.array(E_of, dtype=np.float64)
    keys_scanned = float(E.sum() * U)
    value = keys_scanned / wall
    us_per_step = wall / K_steps * 1e6

    # 16 B of ids per key and KV head: in the unshared mode one scan pass
    # serves the G query heads of a KV head (chunks of 512 keys or more)
    scan_bytes = 16.0 * E_prof.mean() * BH
    scan_us = float(kern[:, 1].mean())
    achieved = scan_bytes / (scan_us * 1e-6) / 1e9
    variant = ("_per_query_head" if w.per_query_head else "") + \
        ("_m%d" % w.m if w.m != 8 else "") + ("_si" if args.si else "")
    traffic = read_traffic("vote_scan_%s%s_traffic.txt" % (args.workload, variant),
                           scan_bytes)
    row_bytes = 2 * w.d * (2 if w.dtype == "bf16" else 4) + 4
    attn_bytes = float(U * w.k * row_bytes + 2 * w.batch * w.n_q_heads * w.d *
                       (2 if w.dtype == "bf16" else 4))
    attn_us = float(kern[:, 6].mean())
    if args.si:
        meta = pk.pariskv_si_debug_intermediate(layers[0][0].handle, w.k, layers[0][0].ws,
                                                pk.SI_DEBUG_META, BH,
                                                layers[0][0].size - w.sinks)
        C = int(round(float(meta[:, 3].mean())))   # keys in the threshold bin and above
    else:
        C = pk.pariskv_retrieve_sizes(layers[0][0].handle, w.k)[1]
    # per candidate: 64 B of codes and B fp16 calibration factors
    rerank_bytes = (64.0 + 2 * w.B) * C * U
    rerank_us = float(kern[:, 3].mean())
    # the single-kernel path: its one kernel is stamped as the scan stage and
    # moves the scan's and the rerank's bytes
    single = (not args.si) and \
        pk.pariskv_retrieval_path(layers[0][0].handle, w.k) == pk.PATH_SINGLE
    roof_kernel = "si_scan" if args.si else "vote_scan"
    if single:
        roof_kernel = "retrieve_single"
        scan_bytes = scan_bytes + rerank_bytes
        achieved = scan_bytes / (scan_us * 1e-6) / 1e9
        traffic = read_traffic("retrieve_single_%s%s_traffic.txt" % (args.workload, variant),
                               scan_bytes)

    step_bytes = scan_bytes + (0.0 if (args.si or single) else rerank_bytes) + attn_bytes
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": W_steps,
        "ms_per_step": us_per_step / 1e3,
        "us_per_step_per_layer": us_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (channel-scaled Gaussian keys with outlier "
                "channels, Gaussian values; no model weights)",
        "config": {
            "workload": w.name, "batch": w.batch, "n_kv_heads": w.n_kv_heads,
            "n_q_heads": w.n_q_heads, "head_dim": w.d, "context": w.N,
            "k": w.k, "sinks": w.sinks, "subspaces": w.B, "m": w.m,
            "rho": w.rho, "tiers": list(w.tiers),
            "candidate_fraction": "%d/%d" % (w.cand_num, w.cand_den),
            "candidates_per_head": C, "layers_in_rotation": Lr,
            "retrieval": ("per query head (%d units)" % U if w.per_query_head
                          else "shared by the %d query heads of a KV head" % w.G),
            "method": ("Self-Indexing sign VQ + LUT-GEMV over all keys" if args.si
                       else "ParisKV votes + RSQ-IP rerank"),
            "parallelism": "single GPU", "launch": mode,
            "retrieval_path": ("Self-Indexing kernels" if args.si else
                               "single kernel" if single else "multi-kernel pipeline"),
            "attention": ("pariskv_retrieve_attend (one call)"
                          if not (args.si or args.separate or args.window)
                          else "separate calls"),
            "kv_placement": {"none": "HBM", "v": "V in pinned host memory",
                             "kv": "K and V in pinned host memory"}[args.uva],
            "window": ({"sinks": w.sinks, "local": win_L, "update_buffer": win_U,
                        "far_store": "pinned host memory" if args.uva == "kv" else "HBM"}
                       if args.window else None),
        },
        "roofline": {
            "kernel": roof_kernel,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": scan_bytes,
            "avg_launch_us": scan_us,
        },
        "gather_roofline": {
            "kernel": "attn_split",
            "achieved": attn_bytes / (attn_us * 1e-6) / 1e9,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": attn_bytes / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "algorithmic_bytes_per_launch": attn_bytes,
            "avg_launch_us": attn_us,
        },
        # the whole step against the HBM peak: the bytes the method must move
        # per step (ids of every key, the candidates' records, the selected
        # K/V rows with q and out), over the timed per-step time
        "step_roofline": {
            "algorithmic_bytes_per_step": step_bytes,
            "achieved": step_bytes / (us_per_step * 1e-6) / 1e9,
            "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": step_bytes / (us_per_step * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "floor_us_at_peak": step_bytes / (HBM_PEAK_GBPS * 1e9) * 1e6,
        },
        "rerank_gather": None if (args.si or single) else {
            "kernel": "compact_rerank",
            "achieved": rerank_bytes / (rerank_us * 1e-6) / 1e9,
            "unit": "GB/s", "algorithmic_bytes_per_launch": rerank_bytes,
            "avg_launch_us": rerank_us,
        },
        "timed_step_us": {"parts": R, "steps_per_part": part,
                          "median": float(np.median(part_us)),
                          "p90": float(np.percentile(part_us, 90)),
                          "mean": float(part_us.mean()),
                          "note": "per-step time of each graph-replayed part of the "
                                  "timed region, from events recorded between "
                                  "replays"},
        "stage_us": stage_us,
        "kernel_timing": "%d further steps, each kernel bracketed by start/stop "
                         "events stamped by its own dispatch" % P,
        "profiled_step_us": {"mean": float(step_us.mean()),
                             "p50": float(np.percentile(step_us, 50)),
                             "p90": float(np.percentile(step_us, 90))},
        "kernel_sha256_16": kernel_sha(),
        "gpu": gpu_info(torch),
    }

    # warm figure: the same step repeated on one layer (graph-replayed like the
    # timed region); its bucket ids would fit the 256 MB Infinity Cache, but
    # the scans read them with streaming loads that the cache does not keep
    if args.warm_steps > 0 and not args.eager:
        Lw = layers[0]
        gw = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=torch.cuda.Stream()):
            for t in range(args.warm_steps):
                step(0)     # layer 0 every time
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        gw.replay()
        torch.cuda.synchronize()
        result["warm_us_per_step_per_layer"] = \
            (time.perf_counter() - t0) / args.warm_steps * 1e6
        result["warm_note"] = ("one layer repeated (%d steps); the scans' streaming "
                               "loads do not keep its bucket ids in the Infinity "
                               "Cache" % args.warm_steps)

    result["recall"] = recall_at_k(pk, torch, np, w, layers[0], idx, cap)
    result["stream_copy"] = stream_copy(torch)
    result["roofline"]["frac_of_stream_copy"] = achieved / result["stream_copy"]["gbps"]
    if not args.no_dense and args.uva == "none" and not args.window \
            and not w.per_query_head and not args.si:
        result["dense_attention"] = dense_attention(pk, torch, w, layers[0],
                                                    cap, scale, dt_code)
        result["dense_attention"]["speedup_of_step"] = \
            result["dense_attention"]["us"] / us_per_step
    if not args.no_cpu_baseline and not w.per_query_head and not args.si:
        result["cpu_baseline"] = cpu_baseline(w, layers[0][1], args.cpu_steps)
    print(json.dumps(result), flush=True)


def gpu_info(torch):
    """Name, architecture, compute units and clock of the GPU the run used."""
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1)}
    clk = getattr(p, "clock_rate", None)
    if clk:
        info["clock_mhz"] = clk / 1000.0
    return info


def exact_topk_rows(torch, w, lay, n):
    """Exact top-k' positions in [S, n) of the group-summed logits
    sum_g <q_g, k_i> (fp32, on the GPU) for every (batch, KV head), or of
    each query head's own logits <q_h, k_i> in the unshared mode."""
    S, kp = w.sinks, w.k - w.sinks
    G = w.G
    out = []
    for b in range(w.batch):
        if w.per_query_head:
            for hq in range(w.n_q_heads):
                q = lay["Q"][b, hq].float()
                sc = torch.mv(lay["K"][b, hq // G, S:n].to(q.device).float(), q)
                out.append(torch.topk(sc, kp).indices + S)
            continue
        for h in range(w.n_kv_heads):
            qs = lay["Q"][b, h * G:(h + 1) * G].float().sum(0)
            sc = torch.mv(lay["K"][b, h, S:n].to(qs.device).float(), qs)
            out.append(torch.topk(sc, kp).indices + S)
    return out


def recall_at_k(pk, torch, np, w, layer, idx, cap):
    """recall@k of one retrieval on layer 0 against the exact inner-product
    top-k' (sinks excluded from both sides); reported, not a parity check."""
    L, lay = layer
    L.retrieve(lay["Q"], idx)
    torch.cuda.synchronize()
    exact = exact_topk_rows(torch, w, lay, L.size)
    S, kp = w.sinks, w.k - w.sinks
    # candidate lists of the same retrieval (vote stage), for the ParisKV path
    cand = None
    if isinstance(L, pk.Layer):
        cand = torch.from_numpy(pk.pariskv_debug_intermediate(
            L.handle, L.k, L.ws, pk.DEBUG_CAND, len(exact))).to(idx.device).long()
    rec, crec = [], []
    for bh, ex in enumerate(exact):
        got = idx[bh, S:].long()
        rec.append(float(torch.isin(got, ex).sum().item()) / kp)
        if cand is not None:
            crec.append(float(torch.isin(ex, cand[bh]).sum().item()) / kp)
    stages = None
    if crec:
        # the exact top-k' kept by the vote stage (inside the candidate set),
        # and the share of those the rerank then keeps in the top-k'
        stages = {"candidate_recall_mean": float(np.mean(crec)),
                  "candidate_recall_min": float(np.min(crec)),
                  "rerank_keeps_mean": float(np.mean([r / c if c else 1.0
                                                      for r, c in zip(rec, crec)])),
                  "per_head": [{"recall": r, "candidate_recall": c}
                               for r, c in zip(rec, crec)]}
    return {"k": w.k, "mean": float(np.mean(rec)), "min": float(np.min(rec)),
            "heads": len(rec), "context": int(L.size), "stages": stages,
            "reference": ("exact top-k' of each query head's logits <q_h, k_i>"
                          if w.per_query_head else
                          "exact top-k' of the group-summed logits sum_g <q_g, k_i>")
                         + " over [sinks, N), fp32"}


def drift_run(args, pk, synth, np, torch):
    """Long-generation drift: prefill N0 keys, then append one key per
    (batch, KV head) per step with the drifting distribution; every
    `drift_every` steps report recall@k of that step's retrieval and the GPU
    time of its kernels (dispatch-stamped events)."""
    w = synth.WORKLOADS["drift"]
    T = args.drift_steps or w.decode_steps
    cap = w.N + T
    dev = "cuda"
    BH = w.batch * w.n_kv_heads
    lay = synth.make_layer(w.scaled(N=cap), dev, layer=0)
    lay["K"][:, :, w.N:] = 0
    lay["V"][:, :, w.N:] = 0
    scales = torch.from_numpy(synth.channel_scales(w.n_kv_heads, w.d, w.seed * 1000))
    chans = synth.drift_channels(w)
    cfg = pk.config_for(w, capacity=cap)
    L = pk.Layer(cfg, lay["signs"], lay["K"], w.N, k=w.k, device=dev)
    idx = torch.empty(BH, w.k, dtype=torch.int32, device=dev)
    out = torch.empty_like(lay["Q"])
    scale = w.d ** -0.5
    dt_code = pk.PARISKV_DTYPE_BF16
    events = [torch.cuda.Event(enable_timing=True) for _ in range(16)]
    for e in events:
        e.record()
    points = []
    t_start = time.perf_counter()
    for t in range(1, T + 1):
        knew, Q, v = synth.drift_step(w, t, scales, chans, dev)
        n = L.size
        lay["K"][:, :, n:n + 1] = knew
        lay["V"][:, :, n:n + 1] = v
        lay["Q"] = Q
        L.append(lay["K"][:, :, n:], 1, rows_per_head=cap)
        if t % args.drift_every == 0 or t == T:
            # the checkpoint step is profiled 3 times (the same retrieval and
            # attention: the index does not change between them); per-stage
            # median, since single eager-launched steps are noisy
            reps = []
            for _ in range(3):
                pk.pariskv_retrieve_topk_profiled(L.handle, Q, w.k, idx, None, L.ws,
                                                  events[0:12])
                pk.pariskv_sparse_attn_profiled(Q, lay["K"], lay["V"], cap, idx, w.k,
                                                w.batch, w.n_q_heads, w.n_kv_heads,
                                                w.d, dt_code, scale, out, L.attn_ws,
                                                events[12:16])
                torch.cuda.synchronize()
                reps.append([events[2 * i].elapsed_time(events[2 * i + 1]) * 1e3
                             for i in range(8)])
            st_us = [float(x) for x in np.median(np.array(reps), axis=0)]
            gpu_us = sum(st_us)
            exact = exact_topk_rows(torch, w, lay, L.size)
            rec = [float(torch.isin(idx[bh].long(), ex).sum().item()) / w.k
                   for bh, ex in enumerate(exact)]
            points.append({"step": t, "context": int(L.size),
                           "recall_mean": float(np.mean(rec)),
                           "recall_min": float(np.min(rec)),
                           "kernel_us": gpu_us,
                           "stage_us": [round(x, 2) for x in st_us]})
            print("[drift] step %d N=%d recall %.4f (min %.4f) kernels %.1f us %s" %
                  (t, L.size, points[-1]["recall_mean"], points[-1]["recall_min"],
                   gpu_us, points[-1]["stage_us"]), file=sys.stderr, flush=True)
        else:
            L.retrieve(Q, idx)
            L.attend(Q, lay["K"], lay["V"], idx, out, scale)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    print(json.dumps({
        "metric": "recall@%d and kernel time under distribution drift" % w.k,
        "workload": w.name, "batch": w.batch, "n_kv_heads": w.n_kv_heads,
        "n_q_heads": w.n_q_heads, "prefill": w.N, "decode_steps": T,
        "checkpoint_every": args.drift_every, "points": points,
        "recall_mean_over_points": float(np.mean([p["recall_mean"] for p in points])),
        "wall_s_eager_with_input_generation": wall,
        "kernel_us_median_over_points": float(np.median([p["kernel_us"] for p in points])),
        "note": "kernel_us = sum over the 8 kernels of the median of 3 dispatch-stamped "
                "durations at the checkpoint step; other steps run eagerly "
                "(launch-bound)",
        "data": "synthetic drift: appended keys and queries shifted on 16 channels "
                "per (b, h) by up to 1.5 channel-scale over the decode"}), flush=True)


def stream_copy(torch, nbytes=2 << 30, iters=5):
    """Achievable HBM bandwidth on this machine: a device-to-device copy of
    nbytes (read + write counted), for comparison with the vendor peak."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    del a, b
    return {"bytes": 2 * nbytes, "us": us, "gbps": 2 * nbytes / (us * 1e-6) / 1e9}


def dense_attention(pk, torch, w, layer, cap, scale, dt_code, iters=5):
    """Context: this library's attention kernel over all N rows (k = N)."""
    L, lay = layer
    N = w.N
    BH = w.batch * w.n_kv_heads
    idx = torch.arange(N, dtype=torch.int32, device="cuda").repeat(BH, 1)
    ws = torch.empty(pk.pariskv_attn_workspace_bytes(w.batch, w.n_q_heads, N, w.d),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(lay["Q"])
    run = lambda: pk.pariskv_sparse_attn(lay["Q"], lay["K"], lay["V"], cap, idx, N,
                                         w.batch, w.n_q_heads, w.n_kv_heads, w.d,
                                         dt_code, scale, out, ws)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        run()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    byts = BH * N * 2 * w.d * (2 if w.dtype == "bf16" else 4)
    del idx, ws
    return {"us": us, "gbps": byts / (us * 1e-6) / 1e9, "k": N}


def cpu_baseline(w, lay, steps):
    """The oracle, as it stands, on the host cores: every (batch, KV head) of
    one layer, `steps` decode steps each (append one key, retrieve, attend);
    the prefill encode of the sample is untimed."""
    import numpy as np
    import torch

    import oracle as orc

    BH = w.batch * w.n_kv_heads
    nthreads = max(1, min(BH, os.cpu_count() or 1, 16))
    N0 = w.N
    Kh = lay["K"][:, :, :N0 + steps].float().cpu().numpy().reshape(BH, N0 + steps, w.d)
    Vh = lay["V"][:, :, :N0 + steps].cpu().reshape(BH, N0 + steps, w.d)
    Qh = lay["Q"].float().cpu().numpy()
    signs = lay["signs"]
    B = w.B
    ids = np.zeros((BH, N0 + steps, B), np.uint8)
    nib = np.zeros((BH, N0 + steps, w.d // 2), np.uint8)
    wq = np.zeros((BH, N0 + steps, B), np.uint16)

    def prefill(bh):
        a, b_, c = orc.encode_keys(signs, Kh[bh, :N0], w.m)
        ids[bh, :N0], nib[bh, :N0], wq[bh, :N0] = a, b_, c

    with cf.ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(prefill, range(BH)))

    def one(bh, t):
        n = N0 + t + 1
        a, b_, c = orc.encode_keys(signs, Kh[bh, n - 1:n], w.m)
        ids[bh, n - 1], nib[bh, n - 1], wq[bh, n - 1] = a[0], b_[0], c[0]
        b, h = divmod(bh, w.n_kv_heads)
        Qg = Qh[b, h * w.G:(h + 1) * w.G]
        r = orc.retrieve_head(signs, Qg, ids[bh, :n], nib[bh, :n], wq[bh, :n],
                              m=w.m, rho=w.rho, tiers=w.tiers, S=w.sinks, k=w.k,
                              num=w.cand_num, den=w.cand_den)
        sel = r["idx"]
        Vsel = Vh[bh][torch.from_numpy(sel).long()].float().numpy()
        orc.attention(Qg, Kh[bh][sel], Vsel, np.arange(len(sel), dtype=np.int32),
                      w.d ** -0.5)
        return n - w.sinks

    keys = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(nthreads) as ex:
        for t in range(steps):
            keys += sum(ex.map(lambda bh: one(bh, t), range(BH)))
    dt = time.perf_counter() - t0
    # plain single thread: one (batch, KV head) step, repeated for (b, h) = 0
    t1 = time.perf_counter()
    one(0, 0)
    single = time.perf_counter() - t1
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count() or 1
    return {"value": keys / dt, "unit": "keys/s", "cores": nthreads,
            "threads": nthreads, "host_cores": os.cpu_count() or 1,
            "host_cores_usable": usable,
            "kind": "oracle",
            "us_per_step_per_layer": dt / steps * 1e6,
            "single_thread_us_per_head_step": single * 1e6,
            "sample": "all %d (batch, KV head) pairs of one %s layer, %d decode "
                      "steps (append + retrieve + attention), index prefill "
                      "untimed; a thread per (batch, KV head), at most %d "
                      "threads" % (BH, w.name, steps, nthreads)}


if __name__ == "__main__":
    main()
