"""The step variants at the full Wan-shaped size (40 x 75600 x 128 bf16), in
the launch configuration the bench times: VMoBA's head-global selection,
BSA's statistical threshold, and raster blocks (3D boxes of 2 x 8 x 8 tokens
with ragged edge boxes) at fixed 10% density with compensation.  The oracle
replays the whole selection of the first and last head given the GPU's
clusters (the rules of the staged tests: bit-exact except flagged near
ties), raster labels, order and offsets are checked exactly on every head, and
the attention of sampled query blocks against the oracle given the GPU's
blocks, mask and means."""

from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import DEV, assert_attn_close, check_selection_head, say, scale_of, to_np, unpack_mask, workspace_for
from test_gpu_domains import check as check_domains
from test_gpu_domains import oracle_logits, run_select

pytestmark = pytest.mark.gpu

EDGE_HEADS = [0, 39]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def test_head_global_full_size():
    w = replace(wl.WAN, name="wan720p_head_global", domain="head", top_p=0.9)
    say(f"[variants] {w.name} H={w.heads} N={w.n} P={w.top_p}")
    q, k, v = wl.make_inputs(w, device=DEV)
    res = run_select(w, q, k)
    for h in EDGE_HEADS:
        r = check_domains(w, *res[:7], [h])
        assert r["pools"] == [[0]]
    del q, k, v, res
    torch.cuda.empty_cache()


def test_stat_threshold_full_size():
    w = replace(wl.WAN, name="wan720p_stat1", rule="stat", stat_lambda=1.0, floor=1)
    say(f"[variants] {w.name} H={w.heads} N={w.n} lambda={w.stat_lambda}")
    q, k, v = wl.make_inputs(w, device=DEV)
    qt, kt, mask, counts, init, ktop, ent, ws = run_select(w, q, k)
    lg, qs = oracle_logits(w, qt, kt, EDGE_HEADS)
    Ck = kt.num_clusters
    units = np.ones(Ck, np.int64)
    gm = unpack_mask(mask, Ck)
    for x, h in enumerate(EDGE_HEADS):
        def redo(kh, x=x):
            return oracle.select(lg[x], units, qs[x], w.top_p, w.floor, w.online_topk, k_h=kh,
                                 stat_lambda=w.stat_lambda)

        s = oracle.select(lg[x], units, qs[x], w.top_p, w.floor, w.online_topk, stat_lambda=w.stat_lambda)
        check_selection_head(gm[h], counts[h].cpu().numpy(), init[h].cpu().numpy(), ktop[h], s, redo, qs[x], w.n,
                             w.online_topk, f"head {h}")
        say(f"    mean clusters/row {s['n_final'].mean():.1f} of {Ck}")
    del q, k, v, qt, kt, ws
    torch.cuda.empty_cache()


def test_raster_full_size():
    ext = (2, 8, 8)
    spec = wl.ClusterSpec("raster", sub_dims=ext)
    w = replace(wl.WAN, name="wan720p_raster3d", q=spec, k=spec).forced_density(0.1)
    say(f"[variants] {w.name} H={w.heads} N={w.n} blocks {ext} floor={w.floor} comp={w.compensate}")
    q, k, v = wl.make_inputs(w, device=DEV)
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, qc, kc, sc, ac)
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster_qk(p, qc, kc, q, k, qt, kt, ws)
    labels, C = oracle.raster_blocks(w.frames, w.height, w.width, *ext)
    perm_o, off_o = oracle.permute(labels, C)
    assert qt.num_clusters == kt.num_clusters == C
    lab_t = torch.tensor(labels, device=DEV, dtype=torch.int32)
    perm_t = torch.tensor(perm_o, device=DEV, dtype=torch.int32)
    off_t = torch.tensor(off_o, device=DEV, dtype=torch.int32)
    for t in (qt, kt):
        assert torch.equal(t.labels, lab_t.expand_as(t.labels)), "labels"
        assert torch.equal(t.perm, perm_t.expand_as(t.perm)), "order"
        assert torch.equal(t.offsets, off_t.expand_as(t.offsets)), "offsets"
    sizes = np.diff(off_o)
    say(f"  {C} blocks of {sizes.min()}..{sizes.max()} tokens: labels, order, offsets exact on every head")
    v_perm = torch.empty_like(v)
    vbar = torch.empty(w.heads, C, w.d, dtype=torch.float32, device=DEV)
    L.sa_permute(p, kt, v, v_perm, vbar)
    mask = torch.empty(w.heads, C, L.mask_words(C), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, C, dtype=torch.int32, device=DEV)
    init = torch.empty_like(counts)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, init, ktop, ws)
    o = torch.full_like(q, float("nan"))
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, vbar, mask, o, ws)
    o2 = torch.empty_like(q)
    mask2 = torch.empty_like(mask)
    L.sa_forward(p, qc, kc, sc, ac, q, k, v, o2, mask2, ws)
    torch.cuda.synchronize()
    assert torch.equal(mask, mask2) and torch.equal(o, o2), "sa_forward differs from its component calls"
    assert bool(torch.isfinite(o).all())
    gm = unpack_mask(mask, C)
    pc = gm.sum(-1)
    assert np.all(pc == w.floor), "forced density: every row selects exactly the floor"
    units = np.ones(C, np.int64)
    rng = np.random.default_rng(0)
    for h in EDGE_HEADS:
        xs, ks, vs = to_np(q[h]), to_np(k[h]), to_np(v[h])
        qbar = oracle.cluster_means(xs, perm_o, off_o)
        kbar = oracle.cluster_means(ks, perm_o, off_o)
        vb = oracle.cluster_means(vs, perm_o, off_o)
        for name, got, want in (("Q", qt.centroids[h], qbar), ("K", kt.centroids[h], kbar), ("V", vbar[h], vb)):
            err = float(np.abs(got.double().cpu().numpy() - want).max())
            assert err <= 1e-6 * max(1.0, float(np.abs(want).max())), (name, err)
        lg = oracle.cluster_logits(qt.centroids[h].double().cpu().numpy(), kt.centroids[h].double().cpu().numpy(),
                                   sizes, scale_of(w), w.size_weighted)

        def redo(kh, lg=lg):
            return oracle.select(lg, units, sizes, w.top_p, w.floor, w.online_topk, k_h=kh)

        s = oracle.select(lg, units, sizes, w.top_p, w.floor, w.online_topk)
        check_selection_head(gm[h], counts[h].cpu().numpy(), init[h].cpu().numpy(), ktop[h], s, redo, sizes, w.n,
                             w.online_topk, f"select head {h}")
        pick = np.unique(np.concatenate([[0, C - 1], rng.choice(C, size=6, replace=False)]))
        rows = np.concatenate([perm_o[off_o[i]:off_o[i + 1]] for i in pick])
        sub_off = np.concatenate([[0], np.cumsum(sizes[pick])])
        ref = oracle.attention(xs, ks, vs, rows, sub_off, perm_o, off_o, gm[h][pick], scale_of(w), True,
                               kt.centroids[h].double().cpu().numpy(), vbar[h].double().cpu().numpy())
        assert_attn_close(o[h, torch.tensor(rows, device=DEV)], ref[rows], q.dtype,
                          f"attention head {h}, {len(pick)} query blocks, {len(rows)} rows")
    del q, k, v, qt, kt, v_perm, o, o2, ws
    torch.cuda.empty_cache()
