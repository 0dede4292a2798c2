"""Shared helpers of the GPU parity tests: small workloads, oracle <-> GPU
conversions, comparison rules.  Test infrastructure only."""

from __future__ import annotations

import math
import sys
from dataclasses import replace

import numpy as np
import torch

import oracle
from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

DEV = "cuda"

# Reduced-size workloads the oracle finishes in seconds, each spanning several
# query tiles and key tiles with a ragged last cluster.
TINY = wl.TINY
MID_S = replace(wl.MID, name="mid_small", heads=2, frames=5)                       # N = 6000
WAN_S = replace(wl.WAN, name="wan_small", heads=2, frames=5, height=24, width=40)  # N = 4800, 38 leaves
TAB_S = replace(wl.TABULAR, name="tab_small", heads=2, width=8292)                # N = 8292, d = 64


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().to("cpu", torch.float64).numpy() if t.is_floating_point() else t.cpu().numpy()


def ocfg(spec, n):
    return oracle.ClusterCfg(method=spec.method, clusters=spec.clusters, leaf=spec.leaf, iters=spec.iters,
                             sub_dims=spec.sub_dims, sub_clusters=spec.clusters)


def oracle_clusters(x, spec):
    """Per-head oracle clustering of x [H, N, d] (torch, any device)."""
    xs = to_np(x)
    return [oracle.cluster_head(xs[h], ocfg(spec, xs.shape[1])) for h in range(xs.shape[0])]


def clusters_to_gpu(p, x_gpu, rl, method, centroids=None):
    """ClusterTensors holding the oracle's perm/offsets/labels and fp32 means,
    with x_perm gathered on the GPU."""
    C = rl[0]["C"]
    ct = L.ClusterTensors(
        labels=torch.tensor(np.stack([r["labels"] for r in rl]), dtype=torch.int32, device=DEV),
        perm=torch.tensor(np.stack([r["perm"] for r in rl]), dtype=torch.int32, device=DEV),
        offsets=torch.tensor(np.stack([r["offsets"] for r in rl]), dtype=torch.int32, device=DEV),
        centroids=torch.tensor(np.stack([r["means"] for r in rl]) if centroids is None else centroids,
                               dtype=torch.float32, device=DEV),
        x_perm=torch.empty_like(x_gpu), num_clusters=C, method=L.METHODS[method])
    L.sa_permute(p, ct, x_gpu, ct.x_perm)
    return ct


def pack_mask(mask_bool):
    """bool [..., Ck] -> int32 words [..., ceil(Ck/32)], bit j LSB first."""
    m = np.asarray(mask_bool, dtype=bool)
    Ck = m.shape[-1]
    W = (Ck + 31) // 32
    pad = np.zeros(m.shape[:-1] + (W * 32,), dtype=bool)
    pad[..., :Ck] = m
    by = np.packbits(pad, axis=-1, bitorder="little")
    return by.view("<u4").astype(np.uint32).view(np.int32)


def unpack_mask(words, Ck):
    w = np.ascontiguousarray(words.cpu().numpy()).view(np.uint32)
    by = w.view(np.uint8)
    bits = np.unpackbits(by, axis=-1, bitorder="little")
    return bits[..., :Ck].astype(bool)


def workspace_for(p, qc=None, kc=None, sc=None, ac=None):
    return L.workspace(L.sa_workspace_size(p, qc, kc, sc, ac), DEV)


BF16_HALF_ULP_REL = 2.0 ** -8  # bf16 keeps 8 significant bits


def assert_attn_close(O_gpu, O_ref, dtype, what=""):
    """fp32 outputs: max-abs <= 1e-4.  bf16 outputs: mean-abs <= 1e-3 and,
    elementwise, |err| <= 1e-2 + 2^-8 |O_ref|.  The second term is the bf16
    representation error of the output value itself (half an ulp), which any
    kernel that returns bf16 carries; with peaked attention |O| reaches ~4 for
    unit-scale V, where half an ulp alone is 0.0156."""
    got = to_np(O_gpu)
    err = np.abs(got - O_ref)
    mx, mean = float(err.max()), float(err.mean())
    if dtype == torch.float32:
        say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e}")
        assert mx <= 1e-4, (what, mx)
        return
    ref_bf = torch.tensor(O_ref).to(torch.bfloat16).double().numpy()
    excess = float((err - BF16_HALF_ULP_REL * np.abs(O_ref)).max())
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} max|O| {np.abs(O_ref).max():.2f} "
        f"max-abs beyond output rounding {excess:.3e} vs bf16(ref): max {np.abs(got - ref_bf).max():.3e} "
        f"mean {np.abs(got - ref_bf).mean():.3e}")
    assert mean <= 1e-3, (what, mean)
    assert excess <= 1e-2, (what, excess)


def inputs(w, device=DEV):
    q, k, v = wl.make_inputs(w, device="cpu")
    return q.to(device), k.to(device), v.to(device)


def scale_of(w):
    return 1.0 / math.sqrt(w.d)
