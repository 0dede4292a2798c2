"""GPU: addressing past 2^31 elements and past 2 GiB inside one head.

A Wan-shaped field of 33 x 512 x 512 tokens (N = 8,650,752, two heads, d =
128, bf16): one head's rows of a tensor span 2.2 GB (more than 2^31 bytes, so
byte offsets inside a head need 32 unsigned bits), and the second head ends at
element 2.2e9 (past 2^31, so element offsets need 64 bits).  Two layouts go
through the component calls and sa_forward:

* aligned: raster blocks of 33 x 64 x 64 tokens for Q and K (64 blocks, every
  range 64-aligned: the whole-block attention path);
* gather: k-means with 64 clusters for Q and raster blocks of 33 x 61 x 63
  for K (81 blocks of sizes that are no multiple of 64: the row-gather path),
  clustered side by side.

Each checks, against the oracle: raster labels, order and offsets exactly
(k-means: order and offsets from its labels); the rows in cluster order (all
of them, on the device); cluster and V means of the first, a middle and the
last cluster of every head; the selection given the GPU's means; and the
output rows of sampled tokens of the first, a middle and the last query
cluster of every head (including each cluster's last member, whose original
index is the cluster's largest), each computed by the oracle's attention over
the selected keys and the compensation terms; sa_forward's output and mask
equal the component calls'.  Selection is the fixed floor of two key clusters
(Top-p 0), compensation on."""

from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import DEV, assert_attn_close, check_selection_head, say, scale_of, unpack_mask, workspace_for

pytestmark = pytest.mark.gpu

BIG = replace(wl.WAN, name="wan_bigindex", heads=2, frames=33, height=512, width=512, top_p=0.0, floor=2,
              compensate=True)
CASES = {
    "aligned": replace(BIG, q=wl.ClusterSpec("raster", sub_dims=(33, 64, 64)),
                       k=wl.ClusterSpec("raster", sub_dims=(33, 64, 64))),
    "gather": replace(BIG, q=wl.ClusterSpec("kmeans", 64, iters=5, sub_dims=(32, 48, 48)),
                      k=wl.ClusterSpec("raster", sub_dims=(33, 61, 63))),
}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def picks(C):
    return sorted({0, C // 2, C - 1})


def check_order(w, name, x, t, spec):
    """perm / offsets against the oracle, rows in cluster order on the device."""
    C = t.num_clusters
    if spec.method == "raster":
        labels, Co = oracle.raster_blocks(w.frames, w.height, w.width, *spec.sub_dims)
        assert Co == C
        perm_o, off_o = oracle.permute(labels, C)
    for h in range(w.heads):
        lab = t.labels[h].cpu().numpy()
        if spec.method == "raster":
            assert np.array_equal(lab, labels), f"{name} head {h}: raster labels"
        else:
            assert lab.min() >= 0 and lab.max() < C
            perm_o, off_o = oracle.permute(lab, C)
        assert np.array_equal(t.perm[h].cpu().numpy(), perm_o), f"{name} head {h}: order"
        assert np.array_equal(t.offsets[h].cpu().numpy(), off_o), f"{name} head {h}: offsets"
        assert torch.equal(t.x_perm[h], x[h][t.perm[h].long()]), f"{name} head {h}: rows in cluster order"
    sz = np.diff(t.offsets[-1].cpu().numpy())
    say(f"  {name}: {C} clusters of {sz.min()}..{sz.max()} tokens: order, offsets and rows exact")


def check_means(w, name, x, t, means):
    """Means of the first, a middle and the last cluster of every head, to
    1e-6 of the rows' magnitude (the gate of the smaller tests; one row
    missing from a cluster of 135 k would already move the mean by ~7e-6)."""
    worst = 0.0
    for h in range(w.heads):
        off = t.offsets[h].cpu().numpy()
        for j in picks(t.num_clusters):
            a, b = int(off[j]), int(off[j + 1])
            if b == a:
                continue
            rows = f64(x[h][t.perm[h][a:b].long()])
            ref = oracle.cluster_means(rows, np.arange(b - a), np.array([0, b - a]))[0]
            got = means[h][j].double().cpu().numpy()
            err = np.abs(got - ref).max() / max(1.0, np.abs(rows).max())
            worst = max(worst, err)
            assert err <= 1e-6, f"{name} head {h} cluster {j} ({b - a} rows): {err:.3e}"
    say(f"  {name}: largest error {worst:.2e} of the rows' magnitude")


def check_rows(w, q, k, v, qt, kt, vbar, gm, o, per=16):
    """Output rows of sampled tokens against the oracle's attention over the
    selected keys (gathered into a compact array: the oracle reads keys only
    through k_perm, so the unselected clusters' entries stay unused)."""
    for h in range(w.heads):
        qoff, koff = qt.offsets[h].cpu().numpy(), kt.offsets[h].cpu().numpy()
        kbar, vb = f64(kt.centroids[h]), f64(vbar[h])
        for i in picks(qt.num_clusters):
            a, b = int(qoff[i]), int(qoff[i + 1])
            if b == a:
                continue
            pos = np.unique(np.r_[np.linspace(a, b - 1, per).astype(np.int64), b - 1])
            rows = qt.perm[h][torch.tensor(pos, device=DEV)].long()
            sel = np.nonzero(gm[h][i])[0]
            kpos = np.concatenate([np.arange(koff[j], koff[j + 1]) for j in sel])
            keys = kt.perm[h][torch.tensor(kpos, device=DEV)].long()
            k_perm = np.zeros(w.n, dtype=np.int64)
            k_perm[kpos] = np.arange(len(kpos))
            ref = oracle.attention(f64(q[h][rows]), f64(k[h][keys]), f64(v[h][keys]), np.arange(len(pos)),
                                   np.array([0, len(pos)]), k_perm, koff, gm[h][i:i + 1], scale_of(w),
                                   w.compensate, kbar, vb)
            assert_attn_close(o[h][rows], ref, q.dtype,
                              f"head {h} query cluster {i}: {len(pos)} rows (largest token "
                              f"{int(rows.max())}), {len(sel)} key clusters, {len(kpos)} keys")


@pytest.mark.parametrize("case", list(CASES))
def test_past_32bit_offsets(case):
    w = CASES[case]
    say(f"[bigindex] {case}: H={w.heads} grid {w.frames}x{w.height}x{w.width} (N={w.n}) d={w.d} "
        f"Q {w.q.method}{w.q.sub_dims if w.q.method == 'raster' else w.q.clusters} "
        f"K {w.k.method}{w.k.sub_dims if w.k.method == 'raster' else w.k.clusters} floor {w.floor}")
    assert w.n * w.d * 2 > 2 ** 31 and w.heads * w.n * w.d > 2 ** 31
    q, k, v = wl.make_inputs(w, device=DEV)
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, qc, kc, sc, ac)
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster_qk(p, qc, kc, q, k, qt, kt, ws)
    Cq, Ck = qt.num_clusters, kt.num_clusters
    v_perm = torch.empty_like(v)
    vbar = torch.empty(w.heads, Ck, w.d, dtype=torch.float32, device=DEV)
    L.sa_permute(p, kt, v, v_perm, vbar)
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, Cq, dtype=torch.int32, device=DEV)
    init = torch.empty_like(counts)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, init, ktop, ws)
    o = torch.full_like(q, float("nan"))
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, vbar, mask, o, ws)
    torch.cuda.synchronize()
    say("  component calls done")
    assert not torch.isnan(o).any(), "an output row was not written"

    check_order(w, "Q", q, qt, w.q)
    check_order(w, "K", k, kt, w.k)
    assert torch.equal(v_perm, torch.stack([v[h][kt.perm[h].long()] for h in range(w.heads)])), "V in key order"
    check_means(w, "Q means", q, qt, qt.centroids)
    check_means(w, "K means", k, kt, kt.centroids)
    check_means(w, "V means", v, kt, vbar)

    gm = unpack_mask(mask, Ck)
    qs = np.stack([np.diff(qt.offsets[h].cpu().numpy()) for h in range(w.heads)])
    ks = np.diff(kt.offsets[0].cpu().numpy())
    units = np.ones(Ck, np.int64)
    for h in range(w.heads):
        lg = oracle.cluster_logits(f64(qt.centroids[h]), f64(kt.centroids[h]), np.diff(kt.offsets[h].cpu().numpy()),
                                   scale_of(w), w.size_weighted)
        s = oracle.select(lg, units, qs[h], w.top_p, w.floor, w.online_topk)

        def redo(kh, lg=lg, h=h):
            return oracle.select(lg, units, qs[h], w.top_p, w.floor, w.online_topk, k_h=kh)

        check_selection_head(gm[h], counts[h].cpu().numpy(), init[h].cpu().numpy(), ktop[h], s, redo, qs[h], w.n,
                             w.online_topk, f"head {h}")
    assert ks.sum() == w.n

    check_rows(w, q, k, v, qt, kt, vbar, gm, o)
    del v_perm, vbar, qt, kt
    o2, mask2 = api.forward(q, k, v, w, ws)
    torch.cuda.synchronize()
    assert torch.equal(mask2, mask) and torch.equal(o2, o), "sa_forward differs from its component calls"
    say("  sa_forward equals the component calls")
