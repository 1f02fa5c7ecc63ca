"""Benchmark: one SVG-EAR routed attention call (cluster -> probe -> route ->
hybrid attention) per step, on the Wan2.2-shaped workload (40 heads x 75,600
tokens, d = 128, bf16, Cq = 100, Ck = 500, rho = 0.15) by default.

Prints ONE JSON line: ms per svgear_forward call (the headline), per-stage ms
from a second timed pass through the per-stage entry points, executed and
dense-equivalent TFLOP/s, the roofline of the dominant kernel (hybrid
attention, MFMA-bound) measured live with HIP events on the stream the library
runs on, and the fp64 oracle timed on this host's cores on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_attention_video_flash_amd import svgear as sv  # noqa: E402
from sparse_attention_video_flash_amd.inputs import WORKLOADS, generate_head  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "ms per routed attention call @40h×75.6K tok; executed TFLOP/s vs MFMA peak"
STAGES = ("cluster_q", "cluster_k", "probe", "route", "attention")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def upload(w, torch, device):
    """Seeded inputs for every head, drawn on host threads, stored bf16/fp32 on the GPU."""
    et = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    N, d, H = w.N, w.d, w.H
    Q = torch.empty(H, N, d, dtype=et, device=device)
    K = torch.empty_like(Q)
    V = torch.empty_like(Q)
    iq = torch.empty(H, w.Cq, dtype=torch.int32, device=device)
    ik = torch.empty(H, w.Ck, dtype=torch.int32, device=device)
    workers = min(16, os.cpu_count() or 4)
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for h, (q, k, v, a, b) in enumerate(ex.map(lambda h: generate_head(w, h), range(H))):
            Q[h].copy_(torch.from_numpy(q).to(et))
            K[h].copy_(torch.from_numpy(k).to(et))
            V[h].copy_(torch.from_numpy(v).to(et))
            iq[h].copy_(torch.from_numpy(a))
            ik[h].copy_(torch.from_numpy(b))
    return Q, K, V, iq, ik


def staged_call(shape, rho, Q, K, V, iq, ik, O, im, ws, ev):
    """The five stages of svgear_forward through the per-stage entry points,
    with an event after each stage (ev[0] before the first)."""
    ev[0].record()
    sv.cluster(shape, 0, Q, iq, dict(labels=im["labels_q"], cent=im["qbar"], counts=im["counts_q"],
                                     offsets=im["offsets_q"], perm=im["perm_q"], inv_perm=im["inv_perm_q"],
                                     Xp=im["Qp"]), ws)
    ev[1].record()
    sv.cluster(shape, 1, K, ik, dict(labels=im["labels_k"], cent=im["kbar"], vbar=im["vbar"],
                                     counts=im["counts_k"], offsets=im["offsets_k"], perm=im["perm_k"],
                                     inv_perm=im["inv_perm_k"], Xp=im["Kp"], Vp=im["Vp"]), ws, V=V)
    ev[2].record()
    sv.probe(shape, im["qbar"], im["counts_q"], im["Kp"], im["Vp"], im["kbar"], im["vbar"], im["counts_k"],
             im["offsets_k"], im["log_ratio"], ws)
    ev[3].record()
    sv.route(shape, rho, im["log_ratio"], im["counts_q"], im["counts_k"], im["mask"], im["sel_cost"], ws)
    ev[4].record()
    sv.attention(shape, im["Qp"], im["offsets_q"], im["perm_q"], im["Kp"], im["Vp"], im["kbar"], im["vbar"],
                 im["counts_k"], im["offsets_k"], im["mask"], O, ws)
    ev[5].record()


def work_counts(w, im):
    """Algorithmic flops of the call (from the routing that was actually taken)."""
    d, H = w.d, w.H
    cq = im["counts_q"].cpu().numpy().astype(np.int64)
    ck = im["counts_k"].cpu().numpy().astype(np.int64)
    mask = im["mask"].cpu().numpy().astype(bool)
    sel = im["sel_cost"].cpu().numpy().astype(np.int64)
    exact_pairs = int(sel.sum())
    # compensation: one centroid term per (query, skipped non-empty key cluster)
    comp_pairs = int(sum(((~mask[h]) & (ck[h] > 0)[None, :]).sum(axis=1) @ cq[h] for h in range(H)))
    f_exact = 4.0 * d * exact_pairs
    f_comp = 4.0 * d * comp_pairs
    f_kmeans = w.iters * 2.0 * d * (w.N * w.Cq + w.N * w.Ck) * H
    f_probe = 2.0 * d * w.Cq * (w.N + w.Ck) * H
    dense = 4.0 * w.N * w.N * d * H
    return dict(exact=f_exact, comp=f_comp, kmeans=f_kmeans, probe=f_probe, dense=dense,
                density=exact_pairs / float(w.N * w.N * H))


def stage_rooflines(w, wk, stage_ms, perm_ms):
    """Achieved rate of each stage against its bound, from the event-timed
    stage durations and algorithmic work: k-means against the bf16 MFMA peak
    (10 iterations of 2 d flop per (token, centroid) distance); probe, route and
    permutation against HBM (one read of what they must read, one write of what
    they must write)."""
    eb = 2 if w.dtype == "bf16" else 4
    H, N, d, Cq, Ck = w.H, w.N, w.d, w.Cq, w.Ck
    row = N * d * eb * H                       # one [H, N, d] tensor
    out = {}

    def mf(name, flops, ms):
        a = flops / (ms * 1e-3) / 1e12
        out[name] = {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(a / PEAK_BF16_TFLOPS, 4), "work": flops}

    def bw(name, nbytes, ms):
        a = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(a / PEAK_HBM_GBS, 4), "bytes": nbytes}

    mf("cluster_q (k-means Q)", w.iters * 2.0 * d * N * Cq * H, stage_ms["cluster_q"])
    mf("cluster_k (k-means K)", w.iters * 2.0 * d * N * Ck * H, stage_ms["cluster_k"])
    # probe: K_p and V_p read once, ln r written
    bw("probe", 2 * row + Cq * Ck * 4 * H, stage_ms["probe"])
    # route: ln r read, mask written
    bw("route", Cq * Ck * 5 * H, stage_ms["route"])
    # permutation: X read, X_p written, labels read, perm and inv_perm written (+ V, V_p on the K side)
    bw("permute_q", 2 * row + 12 * N * H, perm_ms["q"])
    bw("permute_k", 4 * row + 12 * N * H, perm_ms["k"])
    return out


def cpu_baseline(w, rho, rows_stride=16):
    """The fp64 oracle on head 0: full k-means (Q and K), probe and route, and the
    hybrid output on every rows_stride-th query; scaled to a whole call."""
    import oracle
    q, k, v, iq, ik = generate_head(w, 0)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    lq, qbar, cq = oracle.kmeans(q, w.Cq, iq, w.iters)
    lk, kbar, ck = oracle.kmeans(k, w.Ck, ik, w.iters)
    oracle.permutation(lq, w.Cq)
    oracle.permutation(lk, w.Ck)
    vbar = oracle.group_means(v, lk, w.Ck)
    ratio = oracle.probe(qbar, cq, k, v, lk, kbar, vbar, ck)
    mask, _ = oracle.route(ratio, cq, ck, rho, w.N, w.N)
    t1 = time.perf_counter()
    rows = np.arange(0, w.N, rows_stride, dtype=np.int32)
    oracle.hybrid(q, k, v, lq, lk, kbar, vbar, ck, mask, rows)
    t2 = time.perf_counter()
    per_head_s = (t1 - t0) + (t2 - t1) * (w.N / float(len(rows)))
    which = "every query row" if rows_stride == 1 else "every %dth query row" % rows_stride
    return dict(value=per_head_s * w.H * 1e3, unit="ms/call", cores=threads, kind="oracle",
                sample="head 0 of %d: full k-means, probe, route; hybrid output on %s (%d rows), "
                       "scaled by rows and heads; %.1f s of CPU work"
                       % (w.H, which, len(rows), t2 - t0))


def code_digest(path):
    """sha256 of a C++/HIP source with its comments and white space removed, so
    that an edit of comments alone does not mark counters taken on the same
    code as stale."""
    import re
    text = open(path, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode("utf-8")).hexdigest()


def traffic_entry(kernel_file, workload):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel code and on this
    workload; else None."""
    path = os.path.join(ROOT, "profiles", "attention_counters.json")
    src = os.path.join(ROOT, "sparse_attention_video_flash_amd", "csrc", kernel_file)
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    rec = json.load(open(path))
    if rec.get("code_sha256") != code_digest(src) or not str(rec.get("workload", "")).startswith(workload + ":"):
        return None
    return rec.get("bytes_per_launch")


def peaks(torch, dev):
    """What this GPU sustains, to set the published peaks (8 TB/s HBM, 2.5 PFLOP/s
    dense bf16) in context: a 4 GiB device copy (bytes read + written per
    second) and a large bf16 GEMM through the vendor library (torch.matmul),
    each the median of several event-timed runs."""
    out = {}
    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ts = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    t = float(np.median(ts[1:])) * 1e-3
    out["hbm_copy"] = {"bytes": 2 * n, "ms": round(t * 1e3, 3), "achieved_GBs": round(2 * n / t / 1e9, 1),
                       "published_GBs": PEAK_HBM_GBS, "frac": round(2 * n / t / 1e9 / PEAK_HBM_GBS, 4)}
    del src, dst
    m = 8192
    a = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    b = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    c = a @ b
    ts = []
    for _ in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) / 10)
    t = float(np.median(ts[1:])) * 1e-3
    fl = 2.0 * m * m * m
    out["bf16_gemm"] = {"m=n=k": m, "ms": round(t * 1e3, 3), "achieved_TFLOPs": round(fl / t / 1e12, 1),
                        "published_TFLOPs": PEAK_BF16_TFLOPS, "frac": round(fl / t / 1e12 / PEAK_BF16_TFLOPS, 4)}
    return out


VARIANTS = (("error", False), ("logit", False), ("score", False), ("error", True), ("score", True))


def quality(w, torch, dev, row_stride):
    """Output error of the routing variants against dense attention at equal
    density: one clustering (svgear_forward), then per variant and rho the
    variant's probe, route and hybrid attention through the per-stage entry
    points.  Dense attention is evaluated in fp32 (torch, on the GPU) on every
    row_stride-th query of every head.  Also times each variant's probe and
    route stages (HIP events on the library's stream)."""
    torch.backends.cuda.matmul.allow_tf32 = False
    Q, K, V, iq, ik = upload(w, torch, dev)
    shape = sv.make_shape(w.H, w.N, w.N, w.d, w.Cq, w.Ck, w.iters, sv.BF16 if w.dtype == "bf16" else sv.F32)
    ws = sv.alloc_workspace(shape, dev)
    im = sv.alloc_intermediates(shape, dev)
    O = torch.empty_like(Q)
    sv.forward(shape, w.rhos[0], Q, K, V, iq, ik, O, ws, im)
    rows = torch.arange(0, w.N, row_stride, device=dev)
    tau = 1.0 / np.sqrt(w.d)
    dense = torch.empty(w.H, rows.numel(), w.d, device=dev)
    for h in range(w.H):
        s = (Q[h, rows].float() @ K[h].float().T.contiguous()) * tau
        dense[h] = torch.softmax(s, dim=1) @ V[h].float()
    torch.cuda.synchronize()
    log("quality: clustering and dense reference ready")
    flags = {"error": 0, "logit": sv.PROBE_LOGIT, "score": sv.PROBE_SCORE}
    head_groups = [("all", list(range(w.H)))]
    if w.name == "stress":
        head_groups += [("mixture heads 0-7", list(range(8))), ("student-t heads 8-15", list(range(8, 16)))]
    table = []
    for mode, per_row in VARIANTS:
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for rho in w.rhos:
            ev[0].record()
            sv.probe(shape, im["qbar"], im["counts_q"], im["Kp"], im["Vp"], im["kbar"], im["vbar"],
                     im["counts_k"], im["offsets_k"], im["log_ratio"], ws, flags=flags[mode])
            ev[1].record()
            (sv.route_rows if per_row else sv.route)(shape, rho, im["log_ratio"], im["counts_q"],
                                                    im["counts_k"], im["mask"], im["sel_cost"], ws)
            ev[2].record()
            sv.attention(shape, im["Qp"], im["offsets_q"], im["perm_q"], im["Kp"], im["Vp"], im["kbar"],
                         im["vbar"], im["counts_k"], im["offsets_k"], im["mask"], O, ws)
            torch.cuda.synchronize()
            diff = (O[:, rows].float() - dense).pow(2).sum(dim=(1, 2))
            ref = dense.pow(2).sum(dim=(1, 2))
            density = float(im["sel_cost"].double().sum()) / (float(w.N) * w.N * w.H)
            entry = {"variant": mode + (" per-row budget" if per_row else ""), "rho": rho,
                     "density": round(density, 5), "probe_ms": round(ev[0].elapsed_time(ev[1]), 4),
                     "route_ms": round(ev[1].elapsed_time(ev[2]), 4)}
            for name, hs in head_groups:
                entry["rel_l2 " + name] = float(np.sqrt(float(diff[hs].sum()) / float(ref[hs].sum())))
            table.append(entry)
            log("quality %s" % json.dumps(entry))
    return {"experiment": "routing quality at equal density vs dense attention",
            "workload": "%s: %d heads x %d tokens, d=%d, Cq=%d, Ck=%d" % (w.name, w.H, w.N, w.d, w.Cq, w.Ck),
            "rows": "every %dth query row of every head (%d per head), dense attention in fp32"
                    % (row_stride, rows.numel()),
            "results": table}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=None, choices=sorted(WORKLOADS),
                    help="default: wan (stress with --quality)")
    ap.add_argument("--rho", type=float, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows-stride", type=int, default=1)
    ap.add_argument("--peaks", action="store_true",
                    help="measure achievable HBM copy bandwidth and bf16 GEMM throughput on this GPU and exit")
    ap.add_argument("--quality", action="store_true",
                    help="compare the routing variants' output error against dense attention and exit")
    ap.add_argument("--quality-row-stride", type=int, default=16)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 3}), flush=True)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (heads would shard across "
              "GPUs without communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    sv.load()
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.workload or "wan"]
    rho = w.rhos[0] if args.rho is None else args.rho
    if args.peaks:
        print(json.dumps(peaks(torch, dev)), flush=True)
        return
    if args.quality:
        wq = WORKLOADS[args.workload or "stress"]
        print(json.dumps(quality(wq, torch, dev, args.quality_row_stride)), flush=True)
        return
    t = time.perf_counter()
    Q, K, V, iq, ik = upload(w, torch, dev)
    torch.cuda.synchronize()
    log("inputs ready in %.1f s" % (time.perf_counter() - t))
    shape = sv.make_shape(w.H, w.N, w.N, w.d, w.Cq, w.Ck, w.iters, sv.BF16 if w.dtype == "bf16" else sv.F32)
    ws = sv.alloc_workspace(shape, dev)
    im = sv.alloc_intermediates(shape, dev)
    O = torch.empty_like(Q)

    for i in range(args.warmup):
        sv.forward(shape, rho, Q, K, V, iq, ik, O, ws, im)
        torch.cuda.synchronize()
        log("warmup %d done" % i)

    # Timed region: K calls of svgear_forward (one call = the whole path; the
    # library clusters Q on a side stream while K is clustered).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        sv.forward(shape, rho, Q, K, V, iq, ik, O, ws, im)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    log("timed %d calls: %.3f ms/call" % (args.steps, ms_per_step))

    # The same call captured once in a HIP graph and replayed (reported beside
    # the headline, which stays the eager call).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sv.forward(shape, rho, Q, K, V, iq, ik, O, ws, im)
    graph.replay()
    torch.cuda.synchronize()
    tg = time.perf_counter()
    for s in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - tg) * 1e3 / args.steps
    del graph
    log("graph replay: %.3f ms/call" % graph_ms)

    # Second timed region: the same path through the per-stage entry points, one
    # after another on one stream, with HIP events between the stages (stage
    # breakdown and the attention kernel's duration for the roofline).
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for s in range(args.steps):
        staged_call(shape, rho, Q, K, V, iq, ik, O, im, ws, evs[s])
    torch.cuda.synchronize()
    staged_ms = (time.perf_counter() - t2) * 1e3 / args.steps
    stage_ms = {st: float(np.mean([evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]))
                for i, st in enumerate(STAGES)}
    log("staged: %.3f ms/call; stages %s" % (staged_ms, {k: round(v, 3) for k, v in stage_ms.items()}))

    # Third timed region: the permutation alone (counting sort, gathers into
    # cluster order, centroid and value means) through svgear_cluster with the
    # labels the forward produced, Q side and K side.
    perm_ms = {}
    for side in (0, 1):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        lab = im["labels_q" if side == 0 else "labels_k"].clone()
        out = (dict(labels=lab, cent=im["qbar"], counts=im["counts_q"], offsets=im["offsets_q"], perm=im["perm_q"],
                    inv_perm=im["inv_perm_q"], Xp=im["Qp"]) if side == 0 else
               dict(labels=lab, cent=im["kbar"], vbar=im["vbar"], counts=im["counts_k"], offsets=im["offsets_k"],
                    perm=im["perm_k"], inv_perm=im["inv_perm_k"], Xp=im["Kp"], Vp=im["Vp"]))
        torch.cuda.synchronize()
        e[0].record()
        for s_ in range(args.steps):
            sv.cluster(shape, side, Q if side == 0 else K, None, out, ws, V=None if side == 0 else V,
                       flags=sv.LABELS_GIVEN)
            e[s_ + 1].record()
        torch.cuda.synchronize()
        perm_ms["q" if side == 0 else "k"] = float(np.mean([e[i].elapsed_time(e[i + 1])
                                                           for i in range(args.steps)]))
    log("permutation: %s ms" % {k: round(v, 3) for k, v in perm_ms.items()})

    wk = work_counts(w, im)
    t_att = stage_ms["attention"] * 1e-3
    att_flops = wk["exact"] + wk["comp"]
    achieved = att_flops / t_att / 1e12
    routing_ms = stage_ms["cluster_q"] + stage_ms["cluster_k"] + stage_ms["probe"] + stage_ms["route"]
    executed = wk["exact"] + wk["comp"] + wk["kmeans"] + wk["probe"]
    result = {
        "metric": METRIC,
        "value": round(ms_per_step, 4),
        "unit": "ms/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Gaussian-mixture Q/K/V on the latent grid)",
        "config": {"workload": "%s: %d heads x %d tokens (%dx%dx%d), d=%d, Cq=%d, Ck=%d, %d k-means iters, rho=%g"
                   % (w.name, w.H, w.N, *w.grid, w.d, w.Cq, w.Ck, w.iters, rho),
                   "heads": w.H, "tokens": w.N, "d": w.d, "Cq": w.Cq, "Ck": w.Ck, "rho": rho,
                   "parallelism": "single GPU"},
        "stage_ms": {k: round(v, 4) for k, v in stage_ms.items()},
        "staged_ms_per_call": round(staged_ms, 4),
        "graph_replay_ms_per_call": round(graph_ms, 4),
        "routing_share": round(routing_ms / sum(stage_ms.values()), 4),
        "realised_density": round(wk["density"], 5),
        "executed_tflops": round(executed / (ms_per_step * 1e-3) / 1e12, 2),
        "dense_equiv_tflops": round(wk["dense"] / (ms_per_step * 1e-3) / 1e12, 2),
        "stage_rooflines": stage_rooflines(w, wk, stage_ms, perm_ms),
        "roofline": {"kernel": "hybrid attention (svgear_attention)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_entry("attn_mfma.hip", w.name)},
    }
    if not args.no_cpu_baseline:
        log("timing the oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline(w, rho, args.cpu_rows_stride)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
