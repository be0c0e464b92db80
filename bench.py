"""Benchmark of the attention-score token-selection path on one MI355X.

One step = the whole path over one batch already resident in HBM:
tsel_lse -> tsel_colscore -> tsel_budget_topk -> tsel_compact (with the
embedding-row gather) -> tsel_mrope_positions, on the 16384-token GQA
decoder-layer workload
(64 query heads / 8 KV heads, head_dim 128, bf16, causal, 15000 vision
tokens in 20 images of 25x30 plus 1384 text tokens, keep 60%, 5120-dim bf16
hidden states gathered).

Prints one JSON line.  ``value`` is score elements per second of the whole
step: visible (head, row, vision-column) pairs divided by the step time.
The ``roofline`` object describes the dominant kernel (timed with HIP events
on the stream it runs on); ``cpu_baseline`` is the fp64 CPU oracle timed on
a bounded sample of the same workload (whole KV groups of 8 query heads,
added until about 10 s of CPU work are done).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6,   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
               "f16": 2516.6,    # same rate for fp16
               "fp8": 5033.2,    # dense fp8 MFMA: twice the bf16 rate
               "f32": 157.3}     # fp32 matrix rate
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def visible_pairs(prob):
    """Visible (head, row, candidate) pairs of the column-score step and
    (head, row, key) pairs of the LSE step, from the layout alone."""
    import numpy as np
    cols = keys = 0
    cu, ci, st, hw = prob.cu_seqlens, prob.cu_images, prob.img_start, prob.img_hw
    for b in range(prob.B):
        lo, hi = int(cu[b]), int(cu[b + 1])
        n = hi - lo
        if prob.mask == "causal":
            keys += n * (n + 1) // 2
            for s in range(ci[b], ci[b + 1]):
                t = np.arange(st[s], st[s] + hw[s, 0] * hw[s, 1]) - lo
                cols += int((n - t).sum())
        elif prob.mask == "full":
            keys += n * n
            cols += n * int(sum(hw[s, 0] * hw[s, 1] for s in range(ci[b], ci[b + 1])))
        else:
            for s in range(ci[b], ci[b + 1]):
                m = int(hw[s, 0] * hw[s, 1])
                keys += m * m
                cols += m * m
    return cols * prob.hq, keys * prob.hq


def kernel_source_digest() -> str:
    """sha256 of the kernel sources, to tie stored counter data to a build."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_score_selection_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when the summary is missing or was taken from other sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return rec.get("bytes_per_launch", {}).get(kernel)


def cpu_baseline(prob, elems_per_head, budget_s=10.0):
    """The oracle as it stands, on whole KV groups of query heads (one group
    at a time, stopping once about budget_s seconds of CPU work are done)."""
    import oracle
    workers = oracle.default_workers()
    hg = prob.hq // prob.hkv
    done, dt = 0, 0.0
    while done < prob.hkv and dt < budget_s:
        heads = list(range(done * hg, (done + 1) * hg))
        t0 = time.perf_counter()
        oracle.attention_stats(prob, heads=heads, workers=workers)
        dt += time.perf_counter() - t0
        done += 1
    elems = elems_per_head * done * hg
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    try:
        visible = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        visible = os.cpu_count() or 1
    return {"value": elems / dt, "unit": "score elements/s", "cores": workers, "kind": "oracle",
            "cores_visible": visible,
            "cores_note": "threads = the cores this process may run on, capped at 16: the host's CPU "
                          "share of one GPU on this machine class",
            "cpu_model": model,
            "sample": f"fp64 LSE + column mass of query heads 0-{done * hg - 1} "
                      f"({done} KV group(s), {elems:.4g} elements) of the same workload, {dt:.1f} s"}


def budget_competition(prob, outs):
    """Kept fraction of the images with dominant keys against the others in
    one global pool (the REDtech article's multi-image budget competition:
    detail-dense images keep more tokens).  Reported, not a target: the
    synthetic populations stand in for the article's image sets."""
    import numpy as np
    if prob.S < 2 or len(prob.dominant) == 0:
        return None
    img_of = np.full(prob.T, -1, np.int64)
    for s in range(prob.S):
        n = int(prob.img_hw[s, 0] * prob.img_hw[s, 1])
        img_of[prob.img_start[s]:prob.img_start[s] + n] = s
    dom_imgs = set(int(x) for x in img_of[prob.dominant] if x >= 0)
    if not dom_imgs or len(dom_imgs) == prob.S:
        return None
    counts = outs["img_counts"][: prob.S].cpu().numpy().astype(np.float64)
    sizes = (prob.img_hw[:, 0] * prob.img_hw[:, 1]).astype(np.float64)
    frac = counts / sizes
    dom = np.array([s in dom_imgs for s in range(prob.S)])
    return {"images_with_dominant_keys": int(dom.sum()), "other_images": int((~dom).sum()),
            "kept_fraction_dominant": float(frac[dom].mean()), "kept_fraction_other": float(frac[~dom].mean())}


def time_forward(tsel, prob, q, k, lay, dev, stream, args, peak, lse_elems):
    """The layer's attention forward (O and LSE) timed with HIP events;
    4*d flops per visible (head, row, key) pair (QK^T and PV)."""
    import torch
    if prob.dtype not in ("bf16", "f16"):
        return {"skipped": "the forward takes bf16/f16 inputs"}
    v = prob.v.to(dev)
    out = torch.empty(q.shape, dtype=q.dtype, device=dev)
    lse = torch.empty((prob.hq, prob.T), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        tsel.tsel_attention_fwd(q, k, v, lay, prob.mask, 0.0, out=out, lse=lse)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.steps):
        tsel.tsel_attention_fwd(q, k, v, lay, prob.mask, 0.0, out=out, lse=lse)
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    t = ev[0].elapsed_time(ev[1]) / 1e3 / args.steps
    flops = 4.0 * prob.d * lse_elems
    return {"ms": t * 1e3, "tflops": flops / t / 1e12, "mfma_frac": flops / t / 1e12 / peak,
            "flops_per_launch": flops}


def time_mass(tsel, prob, score, lay, dev, stream, args):
    """tsel_budget_mass on the step's own scores (target fraction --mass-tau,
    bounds [0, 1]) timed with HIP events; algorithmic bytes 5 per candidate
    (score read, flag written), as for the top-k."""
    import torch
    B = prob.B
    tau, lo, hi = [args.mass_tau] * B, [0.0] * B, [1.0] * B
    keep = torch.empty((prob.N,), dtype=torch.uint8, device=dev)
    kd = torch.empty((max(B, 1),), dtype=torch.int32, device=dev)
    for _ in range(args.warmup):
        tsel.tsel_budget_mass(lay, score, tau, lo, hi, out=keep, k_out=kd)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.steps):
        tsel.tsel_budget_mass(lay, score, tau, lo, hi, out=keep, k_out=kd)
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    t = ev[0].elapsed_time(ev[1]) / 1e3 / args.steps
    ks = [int(x) for x in kd[:B].cpu()]
    return {"ms": t * 1e3, "tau": args.mass_tau, "k": ks if B > 1 else ks[0],
            "kept_fraction": sum(ks) / max(prob.N, 1), "candidates_per_s": prob.N / t,
            "GBps": 5.0 * prob.N / t / 1e9}


def time_gemm(n, dev, stream, args):
    """A dense bf16 n x n x n product through torch.matmul (hipBLASLt) on
    normal random operands, timed with HIP events: a reference for the MFMA
    rate, and the clock it runs at, that a tuned dense kernel reaches here."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    a = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
    for _ in range(max(args.warmup, 3)):
        torch.matmul(a, b, out=c)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    reps = max(args.steps, 10)
    ev[0].record(stream)
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    t = ev[0].elapsed_time(ev[1]) / 1e3 / reps
    tf = 2.0 * n ** 3 / t / 1e12
    return {"n": n, "ms": t * 1e3, "tflops": tf, "frac": tf / PEAK_TFLOPS["bf16"],
            "library": "torch.matmul (hipBLASLt), bf16 in and out, fp32 accumulate"}


def calib_suite(dev):
    """Kernels whose HBM traffic is known, run once each in this order (a
    counter pass lists their dispatches last): device-to-device copies (read
    and write n bytes), a sum (reads 1 GiB), a fill (writes 1 GiB)."""
    import torch
    ops = []
    for mb in (16, 64, 256, 1024):
        n = mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        ops.append({"op": f"copy {mb} MiB", "read": n, "write": n})
        del src, dst
    x = torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize(dev)
    float(x.sum())
    ops.append({"op": "sum 1 GiB fp32", "read": 1 << 30, "write": 0})
    x.fill_(2.0)
    torch.cuda.synchronize(dev)
    ops.append({"op": "fill 1 GiB fp32", "read": 0, "write": 1 << 30})
    del x
    return ops


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30,
                    help="untimed steps before the timed ones (the GPU clock ramps up over the first ~50 ms of a run from idle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB once (counter calibration)")
    ap.add_argument("--calib-suite", action="store_true",
                    help="after timing, run kernels of known traffic once each (device copies of 16, "
                         "64, 256 and 1024 MiB, a 1 GiB read-only sum, a 1 GiB fill), to check how "
                         "the HBM byte counters relate to real traffic")
    ap.add_argument("--calib-gemm", type=int, default=8192,
                    help="after timing, also time a plain n x n x n bf16 matrix product (torch.matmul, "
                         "i.e. the vendor GEMM library) on random data: the MFMA rate a dense library "
                         "kernel sustains on this GPU, for comparison with the kernels' (0: skip)")
    ap.add_argument("--forward", action="store_true",
                    help="also time the attention forward (tsel_attention_fwd) on the same layer")
    ap.add_argument("--cold", action="store_true",
                    help="also time single steps after evicting the caches (median of 3)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed")
    ap.add_argument("--mass-tau", type=float, default=None,
                    help="also time the input-dependent budget (tsel_budget_mass) at this mass fraction")
    ap.add_argument("--config", type=int, choices=(1, 2, 3, 4, 5), default=4,
                    help="named workload (default 4: the 16384-token GQA decoder layer); the others are "
                         "parity workloads, timed here for reference only")
    ap.add_argument("--dtype", choices=("bf16", "fp8"), default="bf16",
                    help="Q/K storage type of the workload (fp8: OCP E4M3 with per-tensor factors)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the selection path "
                                   "has no multi-GPU code",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import attention_score_selection_amd as tsel
    from workloads import make_config

    if args.dtype == "bf16":
        prob = make_config(args.config)
    else:
        prob = make_config(args.config, dtype=args.dtype)
    scale = prob.softmax_scale if prob.softmax_scale is not None else 0.0
    peak = PEAK_TFLOPS[prob.dtype]
    dev = torch.device("cuda:0")
    lay = tsel.Layout.from_problem(prob, dev)
    q, k, emb = prob.q.to(dev), prob.k.to(dev), prob.emb.to(dev)
    ratios = prob.keep_ratio
    col_elems, lse_elems = visible_pairs(prob)
    d = prob.d

    # Preallocated outputs and workspaces: the timed loop allocates nothing.
    lse = torch.empty((prob.hq, prob.T), dtype=torch.float32, device=dev)
    score = torch.empty((prob.N,), dtype=torch.float32, device=dev)
    keep = torch.empty((prob.N,), dtype=torch.uint8, device=dev)
    ws_col = torch.empty((max(16, tsel.tsel_workspace_size(1, lay, q, k, prob.mask, scale)),),
                         dtype=torch.uint8, device=dev)
    ws_cmp = torch.empty((tsel.tsel_workspace_size(3, lay),), dtype=torch.uint8, device=dev)
    ws_lse = torch.empty((max(16, tsel.tsel_workspace_size(0, lay, q, k, prob.mask, scale)),),
                         dtype=torch.uint8, device=dev)
    ws_topk = torch.empty((max(16, tsel.tsel_workspace_size(2, lay)),), dtype=torch.uint8, device=dev)
    _, ks = tsel.tsel_budget_topk(
        lay, tsel.tsel_colscore(q, k, lay, prob.mask, tsel.tsel_lse(q, k, lay, prob.mask, scale), scale),
        ratios, out=keep)
    outs = {}
    tsel.tsel_compact(lay, keep, ks, emb, workspace=ws_cmp, outputs=outs)
    t_out = int(outs["token_idx"].numel())
    pos = torch.empty((t_out, 3), dtype=torch.int32, device=dev)
    ws_rope = torch.empty((max(4, tsel.tsel_workspace_size(4, lay)),), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    # A workload with a supplied LSE (the reuse path) takes it as an input: it
    # is computed once here, outside the timed step.
    tsel.tsel_lse(q, k, lay, prob.mask, scale, out=lse, workspace=ws_lse)

    def step(ev=None):
        if ev: ev[0].record(stream)
        if not prob.lse_supplied:
            tsel.tsel_lse(q, k, lay, prob.mask, scale, out=lse, workspace=ws_lse)
        if ev: ev[1].record(stream)
        tsel.tsel_colscore(q, k, lay, prob.mask, lse, scale, out=score, workspace=ws_col)
        if ev: ev[2].record(stream)
        tsel.tsel_budget_topk(lay, score, ratios, out=keep, workspace=ws_topk)
        if ev: ev[3].record(stream)
        tsel.tsel_compact(lay, keep, ks, emb, workspace=ws_cmp, outputs=outs)
        if ev: ev[4].record(stream)
        tsel.tsel_mrope_positions(lay, outs, out=pos, workspace=ws_rope)
        if ev: ev[5].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    phase = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(5)] for e in events]) / 1e3
    step_median_ms = float(np.median([e[0].elapsed_time(e[5]) for e in events]))
    t_lse, t_col, t_topk, t_cmp, t_rope = phase.mean(axis=0)
    ms_per_step = wall / args.steps * 1e3

    col_flops = 2.0 * d * col_elems
    lse_flops = 2.0 * d * lse_elems
    # The roofline object reports the column score, the kernel the selection
    # step is built around, unless the LSE pass clearly dominates the step
    # (more than 10% longer; the two do nearly the same work per pair).
    dominant = (("tsel_colscore", t_col, col_flops) if (t_lse <= 1.1 * t_col or prob.lse_supplied)
                else ("tsel_lse", t_lse, lse_flops))
    achieved = dominant[2] / dominant[1] / 1e12
    kept = int(np.sum(ks))
    row_bytes = prob.emb_dim * emb.element_size()
    gather_bytes = 2 * t_out * row_bytes + 16 * t_out + prob.N + 4 * prob.N
    result = {
        "metric": "score elements/s (H*Lq*Lk visible pairs) of the whole selection step",
        "value": col_elems / (ms_per_step / 1e3),
        "unit": "score elements/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "step_ms_median": step_median_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": prob.dtype,
        "data": f"synthetic (seeded normal Q/K, std {prob.std:.4g}" +
                (", quantised to fp8 E4M3 with per-tensor factors" if prob.dtype == "fp8" else "") +
                f"; normal {prob.emb_dtype} embeddings)",
        "config": {"workload": prob.name, "tokens": prob.T, "heads_q": prob.hq, "heads_kv": prob.hkv,
                   "head_dim": d, "mask": prob.mask, "vision_candidates": prob.N, "images": prob.S,
                   "keep_ratio": float(ratios[0]) if len(ratios) == 1 else [float(r) for r in ratios],
                   "kept_vision": kept, "tokens_out": t_out,
                   "dense_score_elements": prob.hq * prob.T * prob.N,
                   "emb_dim": prob.emb_dim,
                   "lse": "supplied (not timed)" if prob.lse_supplied else "computed in-library"},
        "phases_ms": {"lse": t_lse * 1e3, "colscore": t_col * 1e3, "budget_topk": t_topk * 1e3,
                      "compact_gather": t_cmp * 1e3, "rope_positions": t_rope * 1e3},
        "colscore_elements_per_s": col_elems / t_col,
        "colscore_mfma_frac": col_flops / t_col / 1e12 / peak,
        "lse_elements_per_s": None if prob.lse_supplied else lse_elems / t_lse,
        "lse_mfma_frac": None if prob.lse_supplied else lse_flops / t_lse / 1e12 / peak,
        "kept_tokens_per_s": kept / (t_topk + t_cmp),
        "select_gather_GBps": gather_bytes / (t_topk + t_cmp) / 1e9,
        "roofline": {"kernel": dominant[0], "bound": "mfma", "achieved": achieved,
                     "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak,
                     "traffic": stored_traffic(prob.name, dominant[0])},
    }
    if args.forward:
        result["attention_forward"] = time_forward(tsel, prob, q, k, lay, dev, stream, args, peak, lse_elems)
    if args.cold:
        # One step after evicting the caches (writing a buffer four times the
        # 256 MB MALL), three times; the median is reported.
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(3):
            flush.fill_(1)
            torch.cuda.synchronize(dev)
            ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ce[0].record(stream)
            step()
            ce[1].record(stream)
            torch.cuda.synchronize(dev)
            cold.append(ce[0].elapsed_time(ce[1]))
        del flush
        result["cold_step_ms"] = float(np.median(cold))
    if args.graph:
        # The same step captured once in a HIP graph and replayed (the library
        # only enqueues kernels, so the whole step is capturable).
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        torch.cuda.synchronize(dev)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step()
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize(dev)
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        gev[0].record(stream)
        for _ in range(args.steps):
            g.replay()
        gev[1].record(stream)
        torch.cuda.synchronize(dev)
        result["graph_replay"] = {"ms_per_step": gev[0].elapsed_time(gev[1]) / args.steps}
    comp = budget_competition(prob, outs)
    if comp is not None:
        result["budget_competition"] = comp
    if args.mass_tau is not None:
        result["budget_mass"] = time_mass(tsel, prob, score, lay, dev, stream, args)
    if args.calib_copy_mb > 0:
        n = args.calib_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        result["calib_copy_bytes"] = n
    if args.calib_suite:
        result["calib_suite"] = calib_suite(dev)
    if args.calib_gemm > 0:
        gm = time_gemm(args.calib_gemm, dev, stream, args)
        # The path's kernels against the library GEMM on the same GPU and run
        # (bf16 products on both sides only when the workload is bf16/f16).
        if prob.dtype in ("bf16", "f16"):
            gm["colscore_rate_vs_gemm"] = col_flops / t_col / 1e12 / gm["tflops"]
            gm["lse_rate_vs_gemm"] = None if prob.lse_supplied else lse_flops / t_lse / 1e12 / gm["tflops"]
        result["calib_gemm"] = gm
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(prob, col_elems / prob.hq)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
