"""GPU parity of libsa against the fp64 oracle, stage by stage.

Stages (each fed identical inputs):
  A/B  k-means assignment + update from given centroids
  C    full k-means and balanced bisection
  D    permutation (perm/offsets consistent with labels)
  E    selection from identical centroids: bit-exact except flagged near ties
  F    attention from identical perm/offsets/mask/means: bf16 max-abs <= 1e-2,
       mean-abs <= 1e-3 (unit-scale V); fp32 <= 1e-4
  G    sa_forward end to end: identical to the component calls; its O matches
       the oracle's attention over the GPU's own clusters and mask
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import (DEV, MID_S, TAB_S, TINY, WAN_S, assert_attn_close, check_selection_head, clusters_to_gpu,
                         inputs, oracle_clusters, pack_mask, say, scale_of, to_np, unpack_mask, workspace_for)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def structs(w):
    p, qc, kc, sc, ac = api.cfgs(w)
    return p, qc, kc, sc, ac


def oracle_select(w, rq, rk, qbar=None, kbar=None):
    out = []
    for h in range(len(rq)):
        qb = rq[h]["means"] if qbar is None else qbar[h]
        kb = rk[h]["means"] if kbar is None else kbar[h]
        lg = oracle.cluster_logits(qb, kb, rk[h]["sizes"], scale_of(w), w.size_weighted)
        out.append(oracle.select(lg, np.ones(rk[h]["C"], np.int64), rq[h]["sizes"], w.top_p, w.floor,
                                 w.online_topk))
    return out


# fp32 inputs (the one-thread-per-row path) at d = 128 and 64, several tiles,
# compensation on
F32_CASES = [replace(WAN_S, dtype="f32", name="wan_small_f32"), replace(TAB_S, dtype="f32", name="tab_small_f32")]
ATTN_CASES = [TINY, MID_S, WAN_S, TAB_S, WAN_S.forced_density(0.1), TAB_S.forced_density(0.1),
              replace(WAN_S, compensate=False, name="wan_small_nocomp")] + F32_CASES


@pytest.mark.parametrize("w", ATTN_CASES, ids=lambda w: f"{w.name}-P{w.top_p}-k{w.floor}")
def test_stage_F_attention(w):
    say(f"[stage F] {w.name} H={w.heads} N={w.n} d={w.d} {w.dtype} comp={w.compensate}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = structs(w)
    rq = oracle_clusters(q, w.q)
    rk = oracle_clusters(k, w.k)
    sel = oracle_select(w, rq, rk)
    vs = to_np(v)
    kbar32 = np.stack([r["means"] for r in rk]).astype(np.float32)
    vbar32 = np.stack([oracle.cluster_means(vs[h], rk[h]["perm"], rk[h]["offsets"])
                       for h in range(w.heads)]).astype(np.float32)
    qt = clusters_to_gpu(p, q, rq, w.q.method)
    kt = clusters_to_gpu(p, k, rk, w.k.method, centroids=kbar32)
    v_perm = torch.empty_like(v)
    L.sa_permute(p, kt, v, v_perm)
    mask = torch.tensor(pack_mask(np.stack([s["mask"] for s in sel])), device=DEV)
    o = torch.full_like(q, float("nan"))
    ws = workspace_for(p, qc, kc, sc, ac)
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, torch.tensor(vbar32, device=DEV) if w.compensate else None,
                           mask, o, ws)
    torch.cuda.synchronize()
    qs, ks = to_np(q), to_np(k)
    ref = np.stack([oracle.attention(qs[h], ks[h], vs[h], rq[h]["perm"], rq[h]["offsets"], rk[h]["perm"],
                                     rk[h]["offsets"], sel[h]["mask"], scale_of(w), w.compensate,
                                     kbar32[h].astype(np.float64), vbar32[h].astype(np.float64))
                    for h in range(w.heads)])
    assert not torch.isnan(o).any()
    assert_attn_close(o, ref, q.dtype, w.name)


SEL_CASES = [TINY, MID_S, WAN_S, TAB_S, WAN_S.forced_density(0.1), MID_S.forced_density(0.1),
             replace(MID_S, size_weighted=False, name="mid_small_unweighted")]


@pytest.mark.parametrize("w", SEL_CASES, ids=lambda w: f"{w.name}-P{w.top_p}-k{w.floor}")
def test_stage_E_select(w):
    say(f"[stage E] {w.name}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = structs(w)
    rq = oracle_clusters(q, w.q)
    rk = oracle_clusters(k, w.k)
    qbar32 = np.stack([r["means"] for r in rq]).astype(np.float32)
    kbar32 = np.stack([r["means"] for r in rk]).astype(np.float32)
    qt = clusters_to_gpu(p, q, rq, w.q.method, centroids=qbar32)
    kt = clusters_to_gpu(p, k, rk, w.k.method, centroids=kbar32)
    Cq, Ck = qt.num_clusters, kt.num_clusters
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, Cq, dtype=torch.int32, device=DEV)
    init = torch.empty_like(counts)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, init, ktop, workspace_for(p, qc, kc, sc, ac))
    torch.cuda.synchronize()
    gm = unpack_mask(mask, Ck)
    for h in range(w.heads):
        lg = oracle.cluster_logits(qbar32[h].astype(np.float64), kbar32[h].astype(np.float64), rk[h]["sizes"],
                                   scale_of(w), w.size_weighted)
        units = np.ones(Ck, np.int64)

        def redo(kh, lg=lg, h=h):
            return oracle.select(lg, units, rq[h]["sizes"], w.top_p, w.floor, w.online_topk, k_h=kh)

        s = oracle.select(lg, units, rq[h]["sizes"], w.top_p, w.floor, w.online_topk)
        check_selection_head(gm[h], counts[h].cpu().numpy(), init[h].cpu().numpy(), ktop[h], s, redo,
                             rq[h]["sizes"], w.n, w.online_topk, f"head {h}")


# cluster counts that are not multiples of 32 (padded centroid blocks of the
# matrix-core step) at d = 128 and d = 64
MID_ODD = replace(MID_S, name="mid_small_odd_c", q=replace(MID_S.q, clusters=50), k=replace(MID_S.k, clusters=77))
TAB_KM = replace(TAB_S, name="tab_small_kmeans", q=wl.ClusterSpec("kmeans", 40, iters=5),
                 k=wl.ClusterSpec("kmeans", 100, iters=5))
# more than 128 clusters: the assignment on the vector ALUs and the separate
# member-mean pass, up to the largest supported count (1024)
MID_BIG_C = replace(MID_S, name="mid_small_c300_c1024", q=replace(MID_S.q, clusters=300),
                    k=replace(MID_S.k, clusters=1024))


@pytest.mark.parametrize("w", [TINY, MID_S, MID_ODD, TAB_KM, MID_BIG_C], ids=lambda w: w.name)
def test_stage_AB_kmeans_step(w):
    """One assignment + update from given centroids."""
    say(f"[stage A/B] {w.name}")
    q, k, v = inputs(w)
    p = structs(w)[0]
    for x, spec in ((q, w.q), (k, w.k)):
        xs = to_np(x)
        C = spec.clusters
        c0 = np.stack([oracle.kmeans(xs[h], C, 2)["centroids"] for h in range(w.heads)]).astype(np.float32)
        cfg = L.cluster_cfg("kmeans", clusters=C, iters=1, init=L.SA_INIT_GIVEN)
        out = L.alloc_clusters(p, cfg, DEV, x.dtype)
        out.centroids.copy_(torch.tensor(c0))
        L.sa_cluster(p, cfg, x, out, workspace_for(p, cfg))
        torch.cuda.synchronize()
        for h in range(w.heads):
            lab_o, _, _, near = oracle.kmeans_assign(xs[h], c0[h].astype(np.float64))
            lab_g = out.labels[h].cpu().numpy()
            diff = np.nonzero(lab_g != lab_o)[0]
            say(f"  C={C} head {h}: label mismatches {len(diff)}, near ties {int(near.sum())}")
            assert all(near[diff])
            # D: perm/offsets are the stable counting sort of the GPU labels
            perm_o, off_o = oracle.permute(lab_g, C)
            assert np.array_equal(out.perm[h].cpu().numpy(), perm_o)
            assert np.array_equal(out.offsets[h].cpu().numpy(), off_o)
            # B: update from the GPU labels (empty clusters keep their centroid)
            cu, sizes = oracle.kmeans_update(xs[h], lab_g, c0[h].astype(np.float64))
            got = out.centroids[h].cpu().numpy().astype(np.float64)
            rel = np.abs(got - cu).max() / max(1e-30, np.abs(cu).max())
            say(f"    centroid rel err {rel:.2e}")
            assert rel <= 1e-6
            # x_perm is the gather of x by perm
            assert torch.equal(out.x_perm[h], x[h][out.perm[h].long()])


def test_stage_C_kmeans_gmm_exact():
    """Full first-k k-means on well-separated mixture data matches exactly."""
    w = replace(wl.TABULAR, heads=2, width=4096,
                q=wl.ClusterSpec("kmeans", 64, iters=5), k=wl.ClusterSpec("kmeans", 64, iters=5))
    say(f"[stage C] kmeans gmm N={w.n}")
    q, k, v = inputs(w)
    p = structs(w)[0]
    cfg = L.cluster_cfg("kmeans", clusters=64, iters=5)
    out = L.alloc_clusters(p, cfg, DEV, q.dtype)
    L.sa_cluster(p, cfg, q, out, workspace_for(p, cfg))
    torch.cuda.synchronize()
    qs = to_np(q)
    for h in range(w.heads):
        r = oracle.kmeans(qs[h], 64, 5)
        assert np.array_equal(out.labels[h].cpu().numpy(), r["labels"])
        np.testing.assert_allclose(out.centroids[h].cpu().numpy(), r["centroids"], rtol=1e-5, atol=1e-5)


def kmeans_traced(x, w, C, iters, what):
    """Full first-k k-means on the GPU, and the same run as `iters` one-step
    calls from given centroids (bit-identical to it).  Every step's labels are
    compared with the oracle's assignment from the GPU's centroids of the step
    before: each disagreement must be an oracle near tie (stage A), and the
    step's centroids must be the oracle's update of the GPU's labels (stage
    B).  Returns the agreement of the final labels with the oracle's own
    k-means run."""
    p = structs(w)[0]
    full_cfg = L.cluster_cfg("kmeans", clusters=C, iters=iters)
    full = L.alloc_clusters(p, full_cfg, DEV, x.dtype)
    L.sa_cluster(p, full_cfg, x, full, workspace_for(p, full_cfg))
    step_cfg = L.cluster_cfg("kmeans", clusters=C, iters=1, init=L.SA_INIT_GIVEN)
    step = L.alloc_clusters(p, step_cfg, DEV, x.dtype)
    ws = workspace_for(p, step_cfg)
    xs = to_np(x)
    c = np.stack([xs[h][:C] for h in range(w.heads)]).astype(np.float32)  # first-k seeds (exact)
    traced = 0
    for it in range(iters):
        step.centroids.copy_(torch.tensor(c))
        L.sa_cluster(p, step_cfg, x, step, ws)
        torch.cuda.synchronize()
        for h in range(w.heads):
            lab_o, _, _, near = oracle.kmeans_assign(xs[h], c[h].astype(np.float64))
            lab_g = step.labels[h].cpu().numpy()
            diff = np.nonzero(lab_g != lab_o)[0]
            assert all(near[diff]), f"{what} step {it} head {h}: label differences off a near tie {diff[:10]}"
            traced += len(diff)
            cu, _ = oracle.kmeans_update(xs[h], lab_g, c[h].astype(np.float64))
            got = step.centroids[h].cpu().numpy().astype(np.float64)
            assert np.abs(got - cu).max() / max(1e-30, np.abs(cu).max()) <= 1e-6
        c = step.centroids.cpu().numpy()
    for f in ("labels", "perm", "offsets", "centroids", "x_perm"):
        assert torch.equal(getattr(step, f), getattr(full, f)), f"{what}: chained steps differ from one call ({f})"
    agree = [float((full.labels[h].cpu().numpy() == oracle.kmeans(xs[h], C, iters)["labels"]).mean())
             for h in range(w.heads)]
    say(f"  {what}: {iters} steps, {traced} label differences, each at an oracle near tie; final agreement "
        f"with the oracle's own run {', '.join(f'{a:.5f}' for a in agree)}")
    return agree


def test_stage_C_kmeans_smooth_traced():
    """Full k-means on smooth fields, traced step by step: a label differs from
    the oracle's only at an assignment near tie of that step."""
    w = MID_S
    say(f"[stage C] kmeans smooth {w.name}")
    q, k, v = inputs(w)
    kmeans_traced(k, w, 128, 5, "K, C=128")
    kmeans_traced(q, w, 64, 5, "Q, C=64")


def test_stage_C_bisect_gmm_exact():
    w = replace(wl.TABULAR, heads=2, width=4096 + 77)
    say(f"[stage C] bisect gmm N={w.n}")
    q, k, v = inputs(w)
    p = structs(w)[0]
    cfg = L.cluster_cfg("bisect", leaf=128, iters=5)
    out = L.alloc_clusters(p, cfg, DEV, q.dtype)
    L.sa_cluster(p, cfg, q, out, workspace_for(p, cfg))
    torch.cuda.synchronize()
    qs = to_np(q)
    for h in range(w.heads):
        r = oracle.bisect(qs[h], 128, 5)
        assert np.array_equal(out.perm[h].cpu().numpy(), r["perm"])
        assert np.array_equal(out.offsets[h].cpu().numpy(), r["offsets"])
        assert np.array_equal(out.labels[h].cpu().numpy(), r["labels"])
        means = oracle.cluster_means(qs[h], r["perm"], r["offsets"])
        np.testing.assert_allclose(out.centroids[h].cpu().numpy(), means, rtol=1e-5, atol=1e-5)


# Three levels of device-wide top-phase splits (segments above 2560 tokens),
# so the children's first rounds formed during their parents' last rounds are
# exercised at two levels: a smooth field and a Gaussian mixture.
WAN_M = replace(wl.WAN, name="wan_mid", heads=2, frames=10, height=30, width=40)  # N = 12000
TAB_M = replace(wl.TABULAR, name="tab_mid", heads=2, width=20000 + 77)             # N = 20077, d = 64


@pytest.mark.parametrize("w", [WAN_S, replace(WAN_S, d=64, name="wan_small_d64"), WAN_M, TAB_M,
                               replace(WAN_M, dtype="f32", name="wan_mid_f32"),
                               replace(TAB_S, dtype="f32", name="tab_small_f32")],
                         ids=lambda w: w.name)
def test_stage_C_bisect_smooth(w):
    """Smooth fields have near-tie medians.  Walking the oracle's tree from
    the root: every node whose ancestors' splits all agreed must hold the same
    token set on the GPU, and its split must agree unless the oracle flags it
    as a near tie (relative median gap <= 1e-5, the fp32 evaluation of delta);
    the size law and the leaf order hold exactly."""
    say(f"[stage C] bisect smooth {w.name}")
    q, k, v = inputs(w)
    p = structs(w)[0]
    cfg = L.cluster_cfg("bisect", leaf=128, iters=5)
    out = L.alloc_clusters(p, cfg, DEV, q.dtype)
    L.sa_cluster(p, cfg, q, out, workspace_for(p, cfg))
    torch.cuda.synchronize()
    qs = to_np(q)
    N, C = w.n, -(-w.n // 128)
    for h in range(w.heads):
        perm = out.perm[h].cpu().numpy()
        off = out.offsets[h].cpu().numpy()
        assert sorted(perm.tolist()) == list(range(N))
        assert off.tolist() == [min(c * 128, N) for c in range(C + 1)]
        for c in range(C):
            assert np.all(np.diff(perm[off[c]:off[c + 1]]) > 0)
        r = oracle.bisect(qs[h], 128, 5)
        # nodes come in depth-first order; a node is reachable when every
        # split above it agreed (then the GPU's segment holds the same tokens)
        differs = []  # (start, n) of nodes whose split differs
        reach = agree = flagged = 0
        for nd in r["nodes"]:
            if any(s0 <= nd.start < s0 + n0 for s0, n0 in differs):
                continue
            reach += 1
            assert set(perm[nd.start:nd.start + nd.n].tolist()) == set(nd.members.tolist()), \
                f"node start={nd.start} n={nd.n} holds other tokens although every split above it agreed"
            if set(perm[nd.start:nd.start + nd.n_left].tolist()) == set(nd.left.tolist()):
                agree += 1
            else:
                say(f"    split differs at node start={nd.start} n={nd.n}: oracle min rel gap {nd.min_rel_gap:.2e}")
                assert nd.min_rel_gap <= oracle.NEAR_TIE_REL
                flagged += 1
                differs.append((nd.start, nd.n))
        say(f"  head {h}: nodes {len(r['nodes'])}, reachable {reach}, same split {agree}, near-tie splits "
            f"{flagged}, leaf agreement {(out.labels[h].cpu().numpy() == r['labels']).mean():.4f}")
        if not differs:
            assert reach == len(r["nodes"])
            assert np.array_equal(perm, r["perm"])


FWD_CASES = [TINY, MID_S, WAN_S, TAB_S, WAN_S.forced_density(0.1)] + F32_CASES


@pytest.mark.parametrize("w", FWD_CASES, ids=lambda w: f"{w.name}-P{w.top_p}")
def test_stage_G_forward(w):
    say(f"[stage G] {w.name}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = structs(w)
    ws = workspace_for(p, qc, kc, sc, ac)
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster(p, qc, q, qt, ws)
    L.sa_cluster(p, kc, k, kt, ws)
    # both tensors in one call (one problem of 2H heads when both bisect):
    # identical to the two separate calls
    qt2 = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt2 = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster_qk(p, qc, kc, q, k, qt2, kt2, ws)
    torch.cuda.synchronize()
    for a, b in ((qt, qt2), (kt, kt2)):
        assert a.num_clusters == b.num_clusters
        for f in ("labels", "perm", "offsets", "centroids", "x_perm"):
            assert torch.equal(getattr(a, f), getattr(b, f)), f
    del qt2, kt2
    v_perm = torch.empty_like(v)
    vbar = torch.empty(w.heads, kt.num_clusters, w.d, dtype=torch.float32, device=DEV)
    L.sa_permute(p, kt, v, v_perm, vbar)
    Cq, Ck = qt.num_clusters, kt.num_clusters
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, Cq, dtype=torch.int32, device=DEV)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, None, ktop, ws)
    o = torch.empty_like(q)
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, vbar if w.compensate else None, mask, o, ws)
    o2, mask2 = api.forward(q, k, v, w)
    torch.cuda.synchronize()
    assert torch.equal(mask, mask2)
    assert torch.equal(o, o2)
    # oracle attention over the GPU's own clusters, mask and means
    qs, ks, vs = to_np(q), to_np(k), to_np(v)
    gm = unpack_mask(mask, Ck)
    ref = np.stack([
        oracle.attention(qs[h], ks[h], vs[h], qt.perm[h].cpu().numpy(), qt.offsets[h].cpu().numpy(),
                         kt.perm[h].cpu().numpy(), kt.offsets[h].cpu().numpy(), gm[h], scale_of(w), w.compensate,
                         kt.centroids[h].cpu().double().numpy(), vbar[h].cpu().double().numpy())
        for h in range(w.heads)])
    assert_attn_close(o, ref, q.dtype, w.name)
    dens = gm.sum() / gm.size
    say(f"  cluster density {dens:.4f}")


def test_determinism():
    w = WAN_S
    say("[determinism]")
    q, k, v = inputs(w)
    o1, m1 = api.forward(q, k, v, w)
    o2, m2 = api.forward(q, k, v, w)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(m1, m2)
