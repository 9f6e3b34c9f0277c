"""Benchmark of one Prism dynamic sparse video self-attention layer on one MI355X.

A step is one pass of the whole layer over the 2K headline workload (latent
grid 32 x 88 x 160 = 450,560 video tokens, 2 heads of 128 channels, bf16,
top-k 16, top-p 0.9, density cap 10%): zone statistics, shape planning,
permutation + pooled block selection, sparse forward and sparse backward.
Inputs are seeded synthetic tensors already resident in HBM.

Prints one JSON line: fwd+bwd milliseconds per head (the whole layer), the
achieved MFMA TFLOP/s of the attention kernels, a roofline entry for the
forward attention kernel (HIP-event timed; its entry point launches it alone
apart from three small scheduling kernels) and one for the backward entry
point (bwd_pre, dQ and dK/dV kernels; the dK/dV kernel is the largest of the
step), the in-house dense flash attention on the same inputs, and the CPU
oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2k]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
PEAK_SCLK_GHZ = 2.4   # the shader clock the published MFMA peak is quoted at

# HBM bytes per launch of attn_fwd_kernel at the 2K workload (both heads):
# FETCH_SIZE x 2.000 + WRITE_SIZE, the factors read from plain 1 GiB copy
# kernels in the same counter runs.  Valid only for the kernel source the
# counters were taken on (hash of attn.hip + prism_device.h without comments);
# reported as null for any other source or workload.
FWD_TRAFFIC = dict(workload="2k", bytes=65_086_028 * 1024,
                   source_sha256="0da91f5fc95d36268f2a2336c12c3162d2fefbd41f7b3c73f8e9baec7412f1a6")


def attn_source_sha256(base: str | None = None) -> str:
    """Hash of the attention kernel source (attn.hip + prism_device.h) with
    // comments and blank space removed, so that only a change of code makes
    the stored counter figures stale."""
    import hashlib
    import re
    h = hashlib.sha256()
    if base is None:
        base = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dynamic_block_sparse_macro_amd", "csrc")
    for f in ("attn.hip", "prism_device.h"):
        with open(os.path.join(base, f), encoding="utf-8") as fh:
            text = fh.read()
        code = "\n".join(" ".join(re.sub(r"//.*", "", line).split()) for line in text.splitlines())
        h.update(re.sub(r"\n+", "\n", code).encode())
    return h.hexdigest()


def log(*a):
    print(f"[bench {time.strftime('%H:%M:%S')}]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="2k")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense flash-attention baseline")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="target seconds of CPU oracle work")
    ap.add_argument("--dump-index", default="", help="write the block index of the last step to this .npz")
    ap.add_argument("--no-infer", action="store_true", help="skip the forward-only inference timing")
    ap.add_argument("--a2v-channels", type=int, default=0,
                    help="channels of the A2V producer timing (default heads * head_dim)")
    ap.add_argument("--dense-reps", type=int, default=5, help="timed dense-baseline runs (median reported)")
    ap.add_argument("--no-kernel-times", action="store_true",
                    help="skip the profiled step that gives per-kernel durations (for runs under rocprofv3)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run one plain 512 MiB device-to-device copy (a known-size kernel for HBM counters)")
    return ap.parse_args()


def selected_pairs(layer) -> list[int]:
    import numpy as np
    out = []
    for ix in layer.index_host():
        sizes = np.diff(ix["blk_start"]) * 64
        rows = np.repeat(np.arange(sizes.size), np.diff(ix["row_ptr"]))
        out.append(int((sizes[rows] * sizes[ix["col_idx"]]).sum()))
    return out


def cpu_baseline(wl, params_o, pairs_per_head, budget_s: float) -> dict:
    """The oracle as it stands, on the host cores, on a bounded sample of the
    same workload, scaled to milliseconds per head of the whole layer."""
    import numpy as np

    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    cores = len(os.sched_getaffinity(0))
    c = wl.cfg
    h = 0
    v = wl.f32("v")[h:h + 1]
    t0 = time.perf_counter()
    zs = O.zone_statistics(v, wl.a, c.T, c.H, c.W, params_o.eps)
    plan = O.plan_shapes(zs["g"], zs["rho"], params_o.tau128, params_o.tau256)
    perm, bs = O.partition(plan["shape_id"][0], c.T, c.H, c.W)
    t_plan = time.perf_counter() - t0
    qp = O.permute_tokens(wl.f32("q")[h], perm)
    kp = O.permute_tokens(wl.f32("k")[h], perm)
    vp = O.permute_tokens(wl.f32("v")[h], perm)
    dop = O.permute_tokens(wl.f32("do")[h], perm)
    nb = bs.size - 1
    rng = np.random.default_rng(0)
    # selection on a row sample
    t0 = time.perf_counter()
    qbar, kbar = O.pool_blocks(qp, bs), O.pool_blocks(kp, bs)
    t_pool = time.perf_counter() - t0
    rows = rng.choice(nb, min(nb, 48), replace=False)
    t0 = time.perf_counter()
    sel = O.select_blocks(qp, kp, bs, params_o, c.N, rows=rows)
    t_sel = time.perf_counter() - t0 - t_pool   # select_blocks pools again
    t_sel_per_row = max(t_sel, 1e-9) / rows.size
    # attention forward + backward on the sampled query blocks, until the budget
    sizes = np.diff(bs) * 64
    t_attn, pairs_done, done = 0.0, 0, 0
    scale = params_o.score_scale(c.head_dim)
    per_block = []   # (seconds, token pairs) of each sampled query block
    for i in rows:
        cols = sel["rows"][int(i)]["cols"]
        rp = np.zeros(nb + 1, np.int64)
        rp[i + 1:] = cols.size
        t0 = time.perf_counter()
        op_, lse = O.sparse_attention_fwd(qp, kp, vp, bs, rp, cols, scale, rows=[int(i)])
        O.sparse_attention_bwd(qp, kp, vp, op_, dop, lse, bs, rp, cols, scale, rows=[int(i)])
        dt = time.perf_counter() - t0
        t_attn += dt
        pairs_done += int(sizes[i] * sizes[cols].sum())
        per_block.append((dt, int(sizes[i] * sizes[cols].sum())))
        done += 1
        if t_attn + t_plan + t_sel > budget_s:
            break
    t_attn_full = t_attn / max(pairs_done, 1) * pairs_per_head
    ms_per_head = 1e3 * (t_plan + t_pool + t_sel_per_row * nb + t_attn_full)
    # uncertainty of the scaling: the spread of the sampled blocks' seconds
    # per token pair (the attention term is nearly all of the estimate)
    rates = np.array([dt / max(pp, 1) for dt, pp in per_block])
    rel_se = float(rates.std(ddof=1) / rates.mean() / np.sqrt(rates.size)) if rates.size > 1 else None
    return dict(value=round(ms_per_head, 1), unit="ms/head", cores=threads, host_cpus=cores, kind="oracle",
                sample=(f"head 0: full zone statistics, shapes and partition; pooled scores and selection of "
                        f"{rows.size} of {nb} query-block rows; float64 forward+backward of {done} query blocks "
                        f"({pairs_done} of {pairs_per_head} token pairs); scaled by rows and pairs"),
                seconds_measured=round(t_plan + t_pool + t_sel + t_attn, 2),
                attention_share=round(t_attn_full * 1e3 / ms_per_head, 4),
                extrapolation_rel_stderr=(round(rel_se, 4) if rel_se is not None else None))


def kernel_figures(step, stream, cfg, pairs: int, args) -> dict:
    """Device durations of the step's kernels from one step under
    torch.profiler (after the timed steps), with the algorithmic HBM bytes of
    the memory-bound kernels and the MFMA work of the attention kernels."""
    import torch
    from torch.profiler import ProfilerActivity, profile
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        step()
        torch.cuda.synchronize()
    times: dict[str, list[float]] = {}
    for e in prof.events():
        if e.device_type.name != "CUDA":
            continue
        name = e.name.replace("prism::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        times.setdefault(name, []).append(float(e.device_time_total) * 1e-3)   # ms
    h, N, D = cfg.heads, cfg.N, cfg.head_dim
    tiles = N // 64
    hbm = {   # algorithmic bytes of all the step's launches of the kernel
        # V once per head and the audio map once
        "zone_stats_kernel<%d>" % D: h * 2 * N * D + 4 * N,
        # q, k and v: each read from THW through perm and written as tiles;
        # the q and k launches also write float64 per-tile channel sums
        "permute_kernel<%d>" % D: 3 * h * (4 * N * D + 4 * N) + 2 * h * tiles * D * 8,
        # dO, O and its low parts, perm and LSE read; dOp, -Delta and lse2 written
        "bwd_pre_kernel<%d>" % D: h * (8 * N * D + 20 * N),
    }
    out = {"profiled": "one step under torch.profiler after the timed steps"}
    for name, b in hbm.items():
        ts = times.get(name)
        if not ts:
            continue
        ms = sum(ts)
        out[name] = dict(launches=len(ts), ms=round(ms, 4), bytes=int(b), gbps=round(b / (ms * 1e-3) / 1e9, 1),
                         frac_hbm=round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
    # MFMA work over the selected token pairs: forward S and PV; dQ pass S,
    # dP and dQ; dK/dV pass S, dP, dV and dK.  The two backward passes
    # execute exactly this; the forward also runs the tiles of its walk that
    # one of its two query tiles does not attend to (masked) and two
    # pipeline-drain iterations per work item: +1.7% at 2K by the MFMA
    # instruction counters
    mfma = {"attn_fwd_kernel<%d, false>" % D: 4, "attn_bwd_dq_kernel<%d, false>" % D: 6,
            "attn_bwd_dkdv_kernel<%d, false>" % D: 8}
    for name, per_pair in mfma.items():
        ts = times.get(name)
        if not ts:
            continue
        ms = sum(ts)
        f = per_pair * D * pairs
        out[name] = dict(ms=round(ms, 4), pair_flops=f, basis=f"{per_pair}*D per selected token pair",
                         tflops=round(f / (ms * 1e-3) / 1e12, 1),
                         frac=round(f / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))
    out["all_kernels_ms"] = round(sum(sum(v) for v in times.values()), 4)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the layer runs on one GPU; head sharding over several GPUs is a design "
                                   "only (no collectives are implemented)", "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    from dynamic_block_sparse_macro_amd import binding as B
    from dynamic_block_sparse_macro_amd.pipeline import DenseAttention, LayerShape, PrismLayer
    from workload import CONFIGS, generate

    B.load_library()
    cfg = CONFIGS[args.workload]
    log("generating", cfg.name, cfg.note)
    wl = generate(cfg)
    shape = LayerShape(cfg.T, cfg.H, cfg.W, cfg.heads, cfg.head_dim)
    par = B.make_params(top_k=cfg.top_k, top_p=cfg.top_p, density_cap=cfg.density_cap)
    dev = torch.device("cuda:0")

    def tdev(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v, do = (tdev(b) for b in (wl.q_bits, wl.k_bits, wl.v_bits, wl.do_bits))
    a = torch.from_numpy(wl.a).to(dev)
    o = torch.empty_like(q)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    layer = PrismLayer(shape, par, device=dev)
    if args.calibrate_copy:
        # plain copy kernels of known size for scaling the HBM byte counters:
        # 1 GiB fill (write only), 1 GiB device copy, 1 GiB float32 negation
        # (read 1 GiB, write 1 GiB); larger than the 256 MB last-level cache
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.neg(src.view(torch.float32), out=dst.view(torch.float32))
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream(dev)

    names = ["zone_stats", "plan_shapes", "select_blocks", "attn_fwd", "attn_bwd"]

    def step(ev=None):
        marks = [None] * 6
        if ev is not None:
            ev[0].record(stream)
        layer.zone_stats(v, a)
        if ev is not None:
            ev[1].record(stream)
        layer.plan_shapes()
        if ev is not None:
            ev[2].record(stream)
        layer.select_blocks(q, k, v)
        if ev is not None:
            ev[3].record(stream)
        layer.attn_fwd(o)
        if ev is not None:
            ev[4].record(stream)
        layer.attn_bwd(o, do, dq, dk, dv)
        if ev is not None:
            ev[5].record(stream)
        return marks

    log("warmup", args.warmup)
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    pairs = selected_pairs(layer)
    if args.dump_index:
        ix = layer.index_host()
        np.savez_compressed(args.dump_index, **{f"{k}_{h}": v for h, d in enumerate(ix) for k, v in d.items()
                                                if k != "perm"})
    nnz = [int(x) for x in layer.nnz]
    nb = [int(x) for x in layer.n_blocks.cpu()]

    log("timing", args.steps, "steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(args.steps):
        step(evs[s])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    stage_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(names)}
    heads, D = cfg.heads, cfg.head_dim
    P = sum(pairs)
    f_fwd, f_bwd = 4 * D * P, 10 * D * P
    fwd_tflops = f_fwd / (stage_ms["attn_fwd"] * 1e-3) / 1e12
    bwd_tflops = f_bwd / (stage_ms["attn_bwd"] * 1e-3) / 1e12
    attn_tflops = (f_fwd + f_bwd) / ((stage_ms["attn_fwd"] + stage_ms["attn_bwd"]) * 1e-3) / 1e12
    density = P / (heads * cfg.N ** 2)
    log(f"step {ms_step:.2f} ms; stages {json.dumps({k: round(v, 3) for k, v in stage_ms.items()})}")
    log(f"density {density:.4f}, attention {attn_tflops:.1f} TFLOP/s (fwd {fwd_tflops:.1f}, bwd {bwd_tflops:.1f})")

    kernels = None
    sclk = None
    if not args.no_kernel_times:
        kernels = kernel_figures(step, stream, cfg, P, args)
        log("kernels", json.dumps(kernels))
        # shader clock under a sustained MFMA stream (median of 3 probes): the
        # peak the kernels can approach is the published one scaled by it
        sclk = float(np.median([B.prism_sclk_probe(stream) for _ in range(3)]))
        log(f"shader clock under MFMA load {sclk:.3f} GHz")

    dense = None
    if not args.no_dense:
        log("dense baseline")
        dn = DenseAttention(shape, par, device=dev)
        od = torch.empty_like(q)
        for _ in range(3):   # warm-ups
            dn.forward(q, k, v, od)
            dn.backward(q, k, v, od, do, dq, dk, dv)
        torch.cuda.synchronize()
        dts = []
        for _ in range(args.dense_reps):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record(stream)
            dn.forward(q, k, v, od)
            e[1].record(stream)
            dn.backward(q, k, v, od, do, dq, dk, dv)
            e[2].record(stream)
            torch.cuda.synchronize()
            dts.append((e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])))
        dfwd = float(np.median([x[0] for x in dts]))
        dbwd = float(np.median([x[1] for x in dts]))
        fdf, fdb = 4 * D * heads * cfg.N ** 2, 10 * D * heads * cfg.N ** 2
        dense = dict(timing=f"median of {args.dense_reps} after 3 warm-ups", fwd_ms=round(dfwd, 2),
                     bwd_ms=round(dbwd, 2), ms_per_head=round((dfwd + dbwd) / heads, 2),
                     tflops=round((fdf + fdb) / ((dfwd + dbwd) * 1e-3) / 1e12, 1),
                     pct_peak=round(100 * (fdf + fdb) / ((dfwd + dbwd) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     fwd_pct_peak=round(100 * fdf / (dfwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     bwd_pct_peak=round(100 * fdb / (dbwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     kernels="the sparse path's attention kernels with every key tile selected")
        log("dense", dense)
        del dn, od
        torch.cuda.empty_cache()

    # audio-to-video norm producer (upstream of the zone statistics, not part
    # of the timed step): HBM-bound read of h-hat
    from dynamic_block_sparse_macro_amd.pipeline import a2v_norms
    from workload import a2v_output
    ch = args.a2v_channels or heads * D
    hh = torch.from_numpy(a2v_output(wl, ch).view(np.int16)).to(dev).view(torch.bfloat16)
    an = torch.empty(cfg.N, dtype=torch.float32, device=dev)
    a2v_norms(hh, an)
    # each repetition after a 512 MiB read (twice the 256 MB last-level cache,
    # clean lines), so h-hat comes from HBM.  float32: torch sums it in place
    # (an int32 sum first writes a 1 GiB int64 copy, whose dirty lines would
    # then be written back during the timed kernel)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    ts = []
    for _ in range(10):
        flush.sum()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        a2v_norms(hh, an)
        e[1].record(stream)
        torch.cuda.synchronize()
        ts.append(e[0].elapsed_time(e[1]))
    del flush
    a2v_ms = float(np.median(ts))
    a2v_bytes = cfg.N * (2 * ch + 4)
    producer = dict(kernel="a2v_norm_kernel", channels=ch, ms=round(a2v_ms, 4), bytes=a2v_bytes,
                    timing="median of 10, each after reading 512 MiB (twice the last-level cache)",
                    gbps=round(a2v_bytes / (a2v_ms * 1e-3) / 1e9, 1),
                    frac_hbm=round(a2v_bytes / (a2v_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4))
    log("a2v producer", producer)
    del hh

    # forward-only inference path: the 720p forward-only clip and this
    # workload, against the training path's device bytes
    infer = None
    if not args.no_infer:
        from dynamic_block_sparse_macro_amd.pipeline import PrismInference, training_path_bytes
        infer = {}
        for wname in ("720p", args.workload):
            if wname in infer:
                continue
            if wname == args.workload:
                wi, qi, ki, vi, ai, lay, nnz_i = wl, q, k, v, a, layer, sum(nnz)
            else:
                wi = generate(CONFIGS[wname])
                qi, ki, vi = (tdev(b) for b in (wi.q_bits, wi.k_bits, wi.v_bits))
                ai = torch.from_numpy(wi.a).to(dev)
                ci = wi.cfg
                pi = B.make_params(top_k=ci.top_k, top_p=ci.top_p, density_cap=ci.density_cap)
                lay = PrismLayer(LayerShape(ci.T, ci.H, ci.W, ci.heads, ci.head_dim), pi, device=dev)
                nnz_i = sum(lay.forward(qi, ki, vi, ai, torch.empty_like(qi)))
            ci = wi.cfg
            inf = PrismInference(lay.shape, lay.params, device=dev)
            oi = torch.empty_like(qi)
            inf.forward(qi, ki, vi, ai, oi)
            torch.cuda.synchronize()
            reps = 5
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(stream)
            for _ in range(reps):
                inf.forward(qi, ki, vi, ai, oi)
            e[1].record(stream)
            torch.cuda.synchronize()
            ms = e[0].elapsed_time(e[1]) / reps
            tr = training_path_bytes(lay, int(nnz_i))
            infer[wname] = dict(tokens=ci.N, heads=ci.heads, ms=round(ms, 3), ms_per_head=round(ms / ci.heads, 3),
                                workspace_bytes=inf.ws_bytes.value, training_path_bytes=tr["total"],
                                memory_saving=round(1 - inf.ws_bytes.value / tr["total"], 4))
            log("inference", wname, infer[wname])
            del inf, oi
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu:
        import oracle as O
        log("cpu oracle sample")
        po = O.Params(top_k=cfg.top_k, top_p=cfg.top_p, density_cap=cfg.density_cap)
        cpu = cpu_baseline(wl, po, pairs[0], args.cpu_budget)
        log("cpu", cpu)

    fwd_ms = stage_ms["attn_fwd"]
    traffic = None
    if args.workload == FWD_TRAFFIC["workload"] and attn_source_sha256() == FWD_TRAFFIC["source_sha256"]:
        traffic = FWD_TRAFFIC["bytes"]
    roof = dict(bound="mfma", kernel="attn_fwd_kernel<128,sparse>", achieved=round(fwd_tflops, 1),
                peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=round(fwd_tflops / PEAK_BF16_TFLOPS, 4), traffic=traffic,
                traffic_unit="bytes per launch", flops_per_launch=f_fwd, launch_ms=round(fwd_ms, 4))
    # the backward entry point: algorithmic F_bwd = 10 D pairs (5 GEMMs); its
    # kernels execute 14 D pairs (dQ pass: S, dP, dQ; dK/dV pass: S, dP, dV, dK)
    bwd_ms = stage_ms["attn_bwd"]
    roof_bwd = dict(bound="mfma", entry_point="prism_attn_bwd",
                    kernels=["bwd_pre_kernel", "attn_bwd_dq_kernel<128,sparse>", "attn_bwd_dkdv_kernel<128,sparse>"],
                    achieved=round(bwd_tflops, 1), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(bwd_tflops / PEAK_BF16_TFLOPS, 4), flops_per_call=f_bwd,
                    executed_flops_per_call=14 * D * P, executed_frac=round(14 * D * P / (bwd_ms * 1e-3) / 1e12
                                                                            / PEAK_BF16_TFLOPS, 4),
                    call_ms=round(bwd_ms, 4))
    if sclk is not None:
        peak_sclk = PEAK_BF16_TFLOPS * sclk / PEAK_SCLK_GHZ
        for r, tf in ((roof, fwd_tflops), (roof_bwd, bwd_tflops)):
            r.update(sclk_ghz=round(sclk, 3), peak_at_sclk=round(peak_sclk, 1), frac_at_sclk=round(tf / peak_sclk, 4))
    line = {
        "metric": "fwd+bwd ms per head at 450K tokens; achieved MFMA TFLOP/s (% of peak)",
        "value": round(ms_step / heads, 3),
        "unit": "ms/head",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generator: static background, directional zone fields, sound blobs)",
        "config": {"workload": f"{cfg.note}: grid {cfg.T}x{cfg.H}x{cfg.W}, {heads} heads, head_dim {D}, "
                               f"top-k {cfg.top_k}, top-p {cfg.top_p}, density cap {cfg.density_cap}",
                   "tokens": cfg.N, "heads": heads, "head_dim": D, "parallelism": "single GPU"},
        "attention_tflops": round(attn_tflops, 1),
        "attention_pct_peak": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(fwd_tflops, 1),
        "bwd_tflops": round(bwd_tflops, 1),
        "stage_ms": {k: round(v, 3) for k, v in stage_ms.items()},
        "selected_density": round(density, 5),
        "n_blocks": nb,
        "nnz_block_pairs": nnz,
        "token_pairs": pairs,
        "roofline": roof,
        "roofline_backward": roof_bwd,
        "kernels": kernels,
        "dense_baseline": dense,
        "speedup_vs_dense": (round(dense["ms_per_head"] / (ms_step / heads), 2) if dense else None),
        "cpu_baseline": cpu,
        "a2v_producer": producer,
        "inference": infer,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
