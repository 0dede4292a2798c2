"""Benchmark: one clustered block-sparse attention layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan|hy|tab|mid]
                    [--natural] [--cold] [--no-cpu-baseline] [--no-dense] [--copy-probe]
                    [--gemm-probe]

Default workload: a Wan-2.1-14B-720p-shaped attention layer (40 heads,
21x45x80 = 75600 tokens, d = 128, bf16; smooth-field + 3D-RoPE queries/keys,
Gaussian values), balanced bisection into 128-token clusters for queries and
keys, mean compensation on, at fixed 10% density (Top-k of 59 of 591 key
clusters per query cluster, Top-p off).  `--workload hy` runs the
HunyuanVideo-720p-shaped layer (24 x 118800 x 128, key subspace clustering,
lookup-table scores, floor of 10% of the keys), `tab` the unstructured
tabular-shaped tokens (6 x 131072 x 64), `mid` the 8 x 10800 x 128 k-means
layer; `--natural` uses the workload's own Top-p (and online Top-k) instead of
the fixed density.

A step is one sa_forward call: cluster Q and K (one bisection problem of 2H
heads when both bisect), permute V, score + select,
block-sparse attention (+ compensation, + unpermute).  Inputs are resident in
HBM before timing starts.  Prints one JSON line: the headline metric
(effective sparse-attention TFLOP/s over the whole step), ms per layer, a
per-stage breakdown, the dense comparison, the attention kernels' roofline
figure (their own duration, from HIP events that each timed call's attention
configuration asks the library to record around them on the launch stream) and the oracle's CPU timing on a bounded sample.
`--copy-probe` finishes with three 1 GiB device copies of known size, the
calibration for hardware byte counters.

Every timed step is also bracketed by stream events: the line carries their
median, minimum and mean.  `--cold` writes a 512 MB scratch buffer before every
step (warm-up and timed), which evicts the 256 MB memory-side cache, so each
step starts from HBM; the fills sit between the events, and in that mode
`ms_per_step` and `value` come from the events' mean.  `--gemm-probe` adds the
rate of torch's bf16 GEMM (hipBLASLt) on 16384^3, a practical ceiling for MFMA
work on the same GPU.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

METRIC = "effective sparse-attn TFLOP/s + ms per layer vs dense at fixed density, 1 MI355X"
BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
FP32_PEAK_TFLOPS = 157.3

WORKLOADS = {
    "wan": (wl.WAN, "wan2.1-14b-720p-shaped attention layer"),
    "hy": (wl.HUNYUAN, "hunyuanvideo-720p-shaped attention layer, key subspace clustering + lookup-table scores"),
    "tab": (wl.TABULAR, "tabular-transformer-shaped tokens, gaussian mixture, no positional structure"),
    "mid": (wl.MID, "mid-size video layer 9x30x40, k-means clusters"),
}


def effective_flops(mask_bits: torch.Tensor, q_off: torch.Tensor, k_off: torch.Tensor, d: int) -> float:
    """sum over heads, query clusters i and selected key clusters j of
    4 |Q_i| |K_j| d (real tokens only)."""
    qs = (q_off[:, 1:] - q_off[:, :-1]).double()          # [H, Cq]
    ks = (k_off[:, 1:] - k_off[:, :-1]).double()          # [H, Ck]
    sel_keys = torch.bmm(mask_bits.double(), ks.unsqueeze(-1)).squeeze(-1)
    return float(4.0 * d * (qs * sel_keys).sum())


def compensation_flops(mask_bits: torch.Tensor, q_off: torch.Tensor, k_off: torch.Tensor, d: int) -> float:
    """4 d per (query token, excluded non-empty key cluster) pair."""
    qs = (q_off[:, 1:] - q_off[:, :-1]).double()
    nonempty = ((k_off[:, 1:] - k_off[:, :-1]) > 0).double()
    excl = nonempty.sum(-1, keepdim=True) - torch.bmm(mask_bits.double(), nonempty.unsqueeze(-1)).squeeze(-1)
    return float(4.0 * d * (qs * excl).sum())


def unpack_bits(words: torch.Tensor, Ck: int) -> torch.Tensor:
    w = words.to(torch.int64) & 0xFFFFFFFF
    shifts = torch.arange(32, device=words.device)
    bits = (w.unsqueeze(-1) >> shifts) & 1
    return bits.reshape(*words.shape[:-1], -1)[..., :Ck]


class Timer:
    def __init__(self):
        self.ev = []

    def start(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.ev.append([e, None])

    def stop(self):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.ev[-1][1] = e

    def ms(self):
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in self.ev]


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(w, q, k, v, budget_s=10.0):
    """The fp64 oracle on whole heads of the same inputs, one head after the
    other until `budget_s` seconds have passed, scaled to the metric's unit
    (effective TFLOP/s of those heads)."""
    import oracle
    qc, kc = (oracle.ClusterCfg(method=c.method, clusters=c.clusters, leaf=c.leaf, iters=c.iters,
                                sub_dims=tuple(c.sub_dims), sub_clusters=c.clusters) for c in (w.q, w.k))
    sc = oracle.SelectCfg(top_p=w.top_p, floor=w.floor, online_topk=w.online_topk, size_weighted=w.size_weighted)
    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    while heads < w.heads and time.perf_counter() - t0 < budget_s:
        h = heads
        qs, ks, vs = (t[h].double().cpu().numpy() for t in (q, k, v))
        r = oracle.forward_head(qs, ks, vs, qc, kc, sc, compensate=w.compensate)
        qsz = np.diff(r.q["offsets"]).astype(np.float64)
        ksz = np.diff(r.k["offsets"]).astype(np.float64)
        flops += 4.0 * w.d * float((qsz[:, None] * r.mask * ksz[None, :]).sum())
        heads += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpus_in_affinity": len(os.sched_getaffinity(0)),
            "sample": f"{heads} of {w.heads} heads of the same layer and inputs (fp64 NumPy oracle: clustering, "
                      f"selection, attention{' with compensation' if w.compensate else ''}), {dt:.1f} s"}


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "attention_traffic_wan720p.json")


def stored_traffic(workload: str):
    """HBM bytes per attention launch from the committed counter measurement
    (FETCH_SIZE + WRITE_SIZE, calibrated on device copies of known size), or
    None when it was taken on another workload or another version of the
    attention kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    from clustered_block_sparse_amd.profiling import source_hash
    if rec.get("source_sha256") != source_hash() or rec.get("workload") != workload:
        return None
    return rec.get("bytes_per_launch")


def describe(name, w, natural, density):
    base = WORKLOADS[name][1]
    rule = ""
    if w.domain != "row":
        rule += f", {w.domain} competition domain" + (f" (groups of {w.group}, entropy < {w.max_entropy})"
                                                      if w.domain == "group" else "")
    if w.rule == "stat":
        rule += f", statistical threshold mean + {w.stat_lambda} std"
        return f"{base}{rule}, floor {w.floor}" + (", online per-head top-k" if w.online_topk else "")
    if natural:
        return f"{base}, top-p {w.top_p}" + (", online per-head top-k" if w.online_topk else "") + rule
    return f"{base}, fixed {100 * density:g}% density" + rule


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default="wan")
    ap.add_argument("--natural", action="store_true", help="the workload's own top-p instead of fixed density")
    ap.add_argument("--cold", action="store_true", help="evict the memory-side cache before every step")
    ap.add_argument("--density", type=float, default=0.1)
    ap.add_argument("--heads", type=int, default=0, help="override the head count")
    ap.add_argument("--domain", choices=["row", "head", "group"], default=None,
                    help="selection competition domain (EG-Sparse groups, VMoBA head-global)")
    ap.add_argument("--group", type=int, default=4, help="heads per group (--domain group)")
    ap.add_argument("--max-entropy", type=float, default=1.0, help="heads below it are pooled (--domain group)")
    ap.add_argument("--stat-lambda", type=float, default=None,
                    help="BSA statistical threshold (mean + lambda std) in place of Top-p")
    ap.add_argument("--raster", type=str, default=None,
                    help="clustering-free raster blocks bt,bh,bw for queries and keys (VMoBA 1D/2D/3D)")
    ap.add_argument("--quality", action="store_true",
                    help="relative error of O against dense fp32 attention on sampled query rows")
    ap.add_argument("--backward", action="store_true",
                    help="also time the block-sparse attention backward (compensation off)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--gemm-probe", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported here (every step is per head, so "
              f"heads shard across GPUs with no exchange inside the layer)", file=sys.stderr)
        sys.exit(2)
    dev = "cuda"
    base = WORKLOADS[args.workload][0]
    w = base if args.natural else base.forced_density(args.density)
    if args.heads:
        w = w.with_heads(args.heads)
    if args.domain is not None:
        from dataclasses import replace
        w = replace(w, domain=args.domain, group=args.group, max_entropy=args.max_entropy)
    if args.raster is not None:
        from dataclasses import replace
        ext = tuple(int(x) for x in args.raster.split(","))
        spec = wl.ClusterSpec("raster", sub_dims=ext)
        w = replace(w, q=spec, k=spec)
        if not args.natural:
            w = w.forced_density(args.density)
    if args.stat_lambda is not None:
        from dataclasses import replace
        w = replace(w, rule="stat", stat_lambda=args.stat_lambda, floor=max(1, w.floor))
    if args.backward:
        from dataclasses import replace
        w = replace(w, compensate=False)
    L.load()
    t_gen = time.perf_counter()
    q, k, v = wl.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    print(f"# {w.name}: inputs {tuple(q.shape)} {q.dtype} generated in {time.perf_counter() - t_gen:.1f}s",
          file=sys.stderr, flush=True)

    p, qc, kc, sc, ac = api.cfgs(w)
    ws = L.workspace(L.sa_workspace_size(p, qc, kc, sc, ac), dev)
    Cq, Ck = L.sa_num_clusters(p, qc), L.sa_num_clusters(p, kc)
    o = torch.empty_like(q)
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=dev)

    def step():
        L.sa_forward(p, qc, kc, sc, ac, q, k, v, o, mask, ws)

    # 512 MB written before each step in --cold mode: twice the memory-side cache
    scratch = torch.empty(256 << 20, dtype=torch.bfloat16, device=dev) if args.cold else None

    def evict(i):
        if scratch is not None:
            scratch.fill_(float(i % 7))

    for i in range(args.warmup):
        evict(i)
        step()
    # each timed step records its own pair of events around the attention
    # kernels (passed in that step's attention configuration)
    probes = [(L.HipEvent(), L.HipEvent()) for _ in range(args.steps)]
    timed_ac = [L.attn_cfg(ac.compensate, ac.scale, events=pr) for pr in probes]
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evict(i)
        step_ev[i][0].record()
        L.sa_forward(p, qc, kc, sc, timed_ac[i], q, k, v, o, mask, ws)
        step_ev[i][1].record()
    torch.cuda.synchronize()
    ms_wall = (time.perf_counter() - t0) * 1e3 / args.steps
    attn_kernel_ms = [a.elapsed_ms(b) for a, b in probes]
    step_ms = [a.elapsed_time(b) for a, b in step_ev]
    ms_step = float(np.mean(step_ms)) if args.cold else ms_wall
    del scratch
    print(f"# sa_forward {ms_step:.3f} ms/layer, attention kernels {np.mean(attn_kernel_ms):.3f} ms",
          file=sys.stderr, flush=True)

    # --- per-stage breakdown with the component calls (same kernels, same launch configs)
    qt = L.alloc_clusters(p, qc, dev, q.dtype)
    kt = L.alloc_clusters(p, kc, dev, k.dtype)
    v_perm = torch.empty_like(v)
    vbar = torch.empty(w.heads, Ck, w.d, dtype=torch.float32, device=dev) if w.compensate else None
    counts = torch.empty(w.heads, Cq, dtype=torch.int32, device=dev)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=dev)
    mask2 = torch.empty_like(mask)
    o2 = torch.empty_like(o)
    stages = {"cluster_qk": lambda: L.sa_cluster_qk(p, qc, kc, q, k, qt, kt, ws),
              "permute_v": lambda: L.sa_permute(p, kt, v, v_perm, vbar),
              "select": lambda: L.sa_select(p, sc, qt, kt, mask2, counts, None, ktop, ws),
              "attention": lambda: L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, vbar, mask2, o2, ws)}
    for fn in stages.values():
        fn()
    timers = {n: Timer() for n in stages}
    reps = max(3, min(args.steps, 10))
    for _ in range(reps):
        for n, fn in stages.items():
            timers[n].start()
            fn()
            timers[n].stop()
    stage_ms = {n: float(np.mean(t.ms())) for n, t in timers.items()}
    torch.cuda.synchronize()
    same = bool(torch.equal(o2, o) and torch.equal(mask2, mask))

    bits = unpack_bits(mask2, Ck)
    eff = effective_flops(bits, qt.offsets, kt.offsets, w.d)
    comp = compensation_flops(bits, qt.offsets, kt.offsets, w.d) if w.compensate else 0.0
    dense_flops = 4.0 * w.d * w.n * w.n * w.heads
    density = eff / dense_flops
    del bits
    attn_ms = float(np.mean(attn_kernel_ms))
    attn_tf = eff / (attn_ms * 1e-3) / 1e12
    fp32 = w.dtype == "f32"

    # --- dense comparisons
    dense_own = dense_sdpa = None
    if not args.no_dense:
        full = torch.full_like(mask2, -1)
        if Ck % 32:
            full[..., -1] = (1 << (Ck % 32)) - 1
        ac0 = L.attn_cfg(False)
        L.sa_block_sparse_attn(p, ac0, qt, kt, v_perm, None, full, o2, ws)
        t = Timer()
        for _ in range(3):
            t.start()
            L.sa_block_sparse_attn(p, ac0, qt, kt, v_perm, None, full, o2, ws)
            t.stop()
        dense_own = float(np.mean(t.ms()))
        del full
        try:
            sdpa = torch.nn.functional.scaled_dot_product_attention
            qq, kk, vv = q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0)
            sdpa(qq, kk, vv)
            t = Timer()
            for _ in range(3):
                t.start()
                sdpa(qq, kk, vv)
                t.stop()
            dense_sdpa = float(np.mean(t.ms()))
        except Exception as e:  # pragma: no cover
            print(f"# sdpa unavailable: {e}", file=sys.stderr)
    dense_list = [x for x in (dense_own, dense_sdpa) if x is not None]
    dense_best = min(dense_list) if dense_list else None

    backward = None
    if args.backward:
        # gradients of the selected-block attention for a random dO, given
        # the forward's clusters, mask and output
        gen = torch.Generator(device="cpu").manual_seed(2)
        d_o = torch.randn(q.shape, generator=gen).to(q.dtype).to(dev)
        wsb = L.workspace(L.sa_block_sparse_attn_bwd_workspace_size(p, Cq, Ck), dev)
        grads = [torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3)]
        # the forward's log-sum-exp, which the backward then takes instead of
        # recomputing it
        lse = torch.empty(w.heads, w.n, dtype=torch.float32, device=dev)
        L.sa_block_sparse_attn(p, L.attn_cfg(False, ac.scale, lse=lse), qt, kt, v_perm, None, mask2, o2, ws)
        timed = {}
        for name, given in (("lse_given", lse), ("lse_recomputed", None)):
            bwd = lambda: L.sa_block_sparse_attn_bwd(p, ac, qt, kt, v_perm, mask2, o2, d_o, *grads, wsb, lse=given)
            bwd()
            t = Timer()
            for _ in range(reps):
                t.start()
                bwd()
                t.stop()
            timed[name] = float(np.mean(t.ms()))
        bms = timed["lse_given"]
        # 10 d flops per selected (query, key) pair: S, dP, dV, dQ, dK
        bflops = 2.5 * eff
        backward = {"ms": bms, "algorithmic_flops": bflops, "tflops": bflops / (bms * 1e-3) / 1e12,
                    "ms_lse_recomputed": timed["lse_recomputed"],
                    "flops_rule": "10 d per selected (query, key) pair (S, dP, dV, dQ, dK); the forward's "
                                  "log-sum-exp given"}
        print(f"# backward {bms:.3f} ms, {backward['tflops']:.1f} TFLOP/s", file=sys.stderr, flush=True)
        del wsb, grads, d_o, lse

    quality = None
    if args.quality:
        # O of sampled query rows against softmax(q k^T / sqrt(d)) v in fp32
        gen = torch.Generator(device="cpu").manual_seed(1)
        errs = []
        for h in (0, w.heads - 1):
            rows = torch.randperm(w.n, generator=gen)[:2048].to(dev)
            qh = q[h, rows].float()
            s_ = (qh @ k[h].float().T) / math.sqrt(w.d)
            ref = torch.softmax(s_, dim=-1) @ v[h].float()
            got = o[h, rows].float()
            errs.append(float((got - ref).norm() / ref.norm()))
            del s_, ref
        quality = {"rel_l2_error_vs_dense": float(np.mean(errs)), "rows": 2 * 2048,
                   "heads": [0, w.heads - 1]}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q, k, v)

    if args.copy_probe:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# copy probe: 3 copies of {src.numel() * 2} bytes", file=sys.stderr, flush=True)

    gemm = None
    if args.gemm_probe:
        n = 16384
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
        for _ in range(2):
            c = a @ b
        t = Timer()
        for _ in range(5):
            t.start()
            c = a @ b
            t.stop()
        gms = float(np.median(t.ms()))
        gemm = {"shape": [n, n, n], "ms": gms, "tflops": 2.0 * n ** 3 / (gms * 1e-3) / 1e12}
        del a, b, c

    cfg = {"workload": describe(args.workload, w, args.natural, args.density),
           "heads": w.heads, "n": w.n, "d": w.d, "grid": [w.frames, w.height, w.width],
           "clustering": f"q {w.q.method} / k {w.k.method}" + (f" {tuple(w.q.sub_dims)}" if w.q.method == "raster" else ""),
           "query_clusters": Cq, "key_clusters": Ck,
           "top_p": w.top_p, "topk_floor": w.floor, "online_topk": w.online_topk,
           "compensation": w.compensate, "density": density,
           "selection_domain": w.domain, "selection_rule": w.rule}
    line = {
        "metric": METRIC,
        "value": eff / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if fp32 else "bf16",
        "data": "synthetic",
        "config": cfg,
        "ms_per_layer": ms_step,
        "cache": "cold: 512 MB written before every step" if args.cold else "warm",
        "step_ms_events": {"median": float(np.median(step_ms)), "min": float(np.min(step_ms)),
                           "mean": float(np.mean(step_ms))},
        "effective_flops": eff,
        "compensation_flops": comp,
        "stage_ms": stage_ms,
        "attention_kernel_ms": attn_ms,
        "attention_kernel_ms_median_min": [float(np.median(attn_kernel_ms)), float(np.min(attn_kernel_ms))],
        "attention_tflops": attn_tf,
        "dense_ms_own_kernel": dense_own,
        "dense_ms_torch_sdpa": dense_sdpa,
        "speedup_vs_dense": (dense_best / ms_step) if dense_best else None,
        "dense_equiv_tflops": dense_flops / (ms_step * 1e-3) / 1e12,
        "forward_matches_components": same,
        "roofline": {"bound": "mfma", "achieved": attn_tf,
                     "peak": FP32_PEAK_TFLOPS if fp32 else BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tf / (FP32_PEAK_TFLOPS if fp32 else BF16_PEAK_TFLOPS),
                     "traffic": stored_traffic(cfg["workload"]),
                     "kernel": "attention kernels (attn_mfma aligned + general instantiations), selected-block "
                               "flops over their event-timed duration per launch; traffic: HBM bytes per launch "
                               "of the aligned instantiation (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"},
        "cpu_baseline": cpu,
    }
    if gemm is not None:
        line["gemm_probe_bf16"] = gemm
    if quality is not None:
        line["quality"] = quality
    if backward is not None:
        line["backward"] = backward
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
