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


def assert_attn_close(O_gpu, O_ref, dtype, what=""):
    """Attention given identical clusters, mask and means, for unit-scale V:
    fp32 outputs max-abs <= 1e-4; bf16 outputs max-abs <= 1e-2 and mean-abs
    <= 1e-3, element by element against the fp64 oracle."""
    got = to_np(O_gpu)
    err = np.abs(got - O_ref)
    mx, mean = float(err.max()), float(err.mean())
    say(f"  {what}: max-abs {mx:.3e} mean-abs {mean:.3e} max|O| {np.abs(O_ref).max():.2f}")
    if dtype == torch.float32:
        assert mx <= 1e-4, (what, mx)
        return
    assert mx <= 1e-2, (what, mx)
    assert mean <= 1e-3, (what, mean)


def check_selection_head(gm_h, counts_h, init_h, ktop_h, s, redo, qsizes, N, online, what=""):
    """One head's selection against the oracle's (`s`, from oracle.select on
    the same logits), given identical centroids and sizes.

    Rows the oracle does not flag must agree exactly: mask, final count and
    initial count.  A flagged row may differ only on the units whose rank or
    crossing sits inside the flag: the GPU's set must contain the oracle's
    first cut_lo ranked units and lie within its first cut_hi, its initial
    count within the counts of the first init_lo .. init_hi units.  k_h must
    equal ceil(sum |Q_i| n_i / N) over the GPU's own initial counts, and the
    oracle's k_h unless a flagged row's initial count differs; then every row
    is checked again against the oracle's selection given the GPU's k_h
    (`redo(k_h)`)."""
    Cq = gm_h.shape[0]
    flagged = np.asarray(s["near_tie"], dtype=bool)
    if init_h is not None:
        assert int(ktop_h) == (-(-int((qsizes * init_h).sum()) // N) if online else 0), \
            f"{what}: k_h is not the weighted mean of the GPU's own initial counts"
        d_init = np.nonzero(init_h != s["n_init"])[0]
        assert all(flagged[d_init]), f"{what}: initial counts differ on unflagged rows {d_init[:10]}"
    if online and int(ktop_h) != s["k_h"]:
        assert init_h is not None and len(d_init) > 0, f"{what}: k_h differs with identical initial counts"
        say(f"  {what}: k_h gpu {int(ktop_h)} oracle {s['k_h']} (flagged rows' initial counts differ): "
            f"rows checked given the GPU's k_h")
        s = redo(int(ktop_h))
        flagged = np.asarray(s["near_tie"], dtype=bool)
    un = ~flagged
    bad = np.nonzero((gm_h[un] != s["mask"][un]).any(axis=1))[0]
    assert len(bad) == 0, f"{what}: unflagged rows differ {np.nonzero(un)[0][bad][:10]}"
    assert np.array_equal(counts_h[un], s["n_final"][un]), f"{what}: final counts of unflagged rows"
    if init_h is not None:
        assert np.array_equal(init_h[un], s["n_init"][un]), f"{what}: initial counts of unflagged rows"
    ndiff = 0
    Ck = gm_h.shape[1]
    for i in np.nonzero(flagged)[0]:
        order = s["orders"][i]
        lo, hi = int(s["cut_lo"][i]), int(s["cut_hi"][i])
        must = np.zeros(Ck, dtype=bool)
        must[order[:lo]] = True
        may = np.zeros(Ck, dtype=bool)
        may[order[:hi]] = True
        g = gm_h[i]
        assert not (must & ~g).any() and not (g & ~may).any(), \
            f"{what}: flagged row {i} differs outside its flagged units (cut {s['t_final'][i]}, range {lo}..{hi})"
        ndiff += int((g != s["mask"][i]).any())
        if init_h is not None:
            cu = s["cum_units"][i]
            a, b = int(s["init_lo"][i]), int(s["init_hi"][i])
            n_lo = cu[a - 1] if a > 0 else 0
            n_hi = cu[b - 1] if b > 0 else 0
            assert n_lo <= init_h[i] <= n_hi, f"{what}: flagged row {i} initial count"
    say(f"  {what}: {Cq} rows, {int(flagged.sum())} flagged near ties ({ndiff} differ inside their flags), "
        f"k_h {int(ktop_h)}")
    return s


def inputs(w, device=DEV):
    q, k, v = wl.make_inputs(w, device="cpu")
    return q.to(device), k.to(device), v.to(device)


def scale_of(w):
    return 1.0 / math.sqrt(w.d)
