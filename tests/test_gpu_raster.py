"""GPU parity of the clustering-free raster blocks (VMoBA 1D-2D-3D block
partition) against the fp64 oracle: block labels, order and offsets exact,
block means to fp32 accuracy, the cumulative-similarity selection (Top-p over
block proxy scores, also head-global) given the GPU's block means, and the
block-sparse attention over the GPU's blocks and mask, end to end through
sa_forward."""

from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import (DEV, TAB_S, WAN_S, assert_attn_close, check_selection_head, inputs, say, scale_of, to_np,
                         unpack_mask, workspace_for)

pytestmark = pytest.mark.gpu


def raster(w, ext, name, **kw):
    spec = wl.ClusterSpec("raster", sub_dims=ext)
    return replace(w, name=name, q=spec, k=spec, **kw)


CASES = [
    raster(WAN_S, (1, 8, 16), "wan_small_raster3d"),                       # 45 blocks, edge blocks of 64
    raster(WAN_S, (5, 6, 8), "wan_small_raster2d", top_p=0.8),             # spatial tiles through all frames
    raster(WAN_S, (1, 24, 40), "wan_small_raster1d", top_p=0.7, floor=2),  # one frame per block
    raster(WAN_S, (2, 7, 9), "wan_small_raster3d_head_global", domain="head", top_p=0.85),
    raster(WAN_S, (1, 8, 16), "wan_small_raster3d_fixed", top_p=0.0, floor=5, compensate=True),
    # d = 64 on an unstructured 1 x 1 x N grid: runs of 128 consecutive tokens (65 blocks, the last of 100)
    raster(TAB_S, (1, 1, 128), "tab_small_raster_runs", top_p=0.9, floor=2, compensate=True),
]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_raster_blocks(w):
    ext = w.q.sub_dims
    say(f"[raster] {w.name} H={w.heads} grid {w.frames}x{w.height}x{w.width} blocks {ext} P={w.top_p} "
        f"floor={w.floor} domain={w.domain} comp={w.compensate}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, qc, kc, sc, ac)
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster_qk(p, qc, kc, q, k, qt, kt, ws)
    labels, C = oracle.raster_blocks(w.frames, w.height, w.width, *ext)
    perm_o, off_o = oracle.permute(labels, C)
    assert qt.num_clusters == kt.num_clusters == C
    torch.cuda.synchronize()
    for x, t in ((q, qt), (k, kt)):
        xs = to_np(x)
        for h in range(w.heads):
            assert np.array_equal(t.labels[h].cpu().numpy(), labels)
            assert np.array_equal(t.perm[h].cpu().numpy(), perm_o)
            assert np.array_equal(t.offsets[h].cpu().numpy(), off_o)
            means = oracle.cluster_means(xs[h], perm_o, off_o)
            got = t.centroids[h].double().cpu().numpy()
            assert np.abs(got - means).max() <= 1e-6 * max(1.0, np.abs(means).max())
        assert torch.equal(t.x_perm, x[:, torch.tensor(perm_o, device=DEV)])
    say(f"  {C} blocks of {np.diff(off_o).min()}..{np.diff(off_o).max()} tokens: labels, order, offsets exact")
    v_perm = torch.empty_like(v)
    vbar = torch.empty(w.heads, C, w.d, dtype=torch.float32, device=DEV)
    L.sa_permute(p, kt, v, v_perm, vbar)
    mask = torch.empty(w.heads, C, L.mask_words(C), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, C, dtype=torch.int32, device=DEV)
    init = torch.empty_like(counts)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, init, ktop, ws)
    o = torch.full_like(q, float("nan"))
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, vbar if w.compensate else None, mask, o, ws)
    o2, mask2 = api.forward(q, k, v, w)
    torch.cuda.synchronize()
    assert torch.equal(mask, mask2) and torch.equal(o, o2), "sa_forward differs from its component calls"
    gm = unpack_mask(mask, C)
    lg = np.stack([oracle.cluster_logits(qt.centroids[h].double().cpu().numpy(), kt.centroids[h].double().cpu().numpy(),
                                         np.diff(off_o), scale_of(w), w.size_weighted) for h in range(w.heads)])
    qs = np.stack([np.diff(off_o)] * w.heads)
    units = np.ones(C, np.int64)
    dom = {"row": oracle.DOMAIN_ROW, "head": oracle.DOMAIN_HEAD}[w.domain]
    r = oracle.select_domains(lg, units, qs, w.top_p, w.floor, w.online_topk, dom)
    pooled = {}
    for pl in r["pools"]:
        pooled.update(oracle.pool_counts(lg, qs, pl, w.top_p))
    qsv, ksv, vsv = to_np(q), to_np(k), to_np(v)
    for h in range(w.heads):
        def redo(kh, h=h):
            return oracle.select(lg[h], units, qs[h], w.top_p, w.floor, w.online_topk, k_h=kh, pool=pooled.get(h))

        check_selection_head(gm[h], counts[h].cpu().numpy(), init[h].cpu().numpy(), ktop[h], r["heads"][h], redo,
                             qs[h], w.n, w.online_topk, f"head {h}")
        ref = oracle.attention(qsv[h], ksv[h], vsv[h], perm_o, off_o, perm_o, off_o, gm[h], scale_of(w), w.compensate,
                               kt.centroids[h].double().cpu().numpy(), vbar[h].double().cpu().numpy())
        assert_attn_close(o[h], ref, q.dtype, f"attention head {h}, density {gm[h].mean():.3f}")
