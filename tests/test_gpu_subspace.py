"""GPU parity of the SCOPE key-subspace path (HunyuanVideo-shaped workload at
reduced size) against the fp64 oracle: subspace k-means and combo order,
lookup-table selection in keys with online per-head Top-k, gather attention
over the selected combos, and the whole forward pass."""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import (DEV, assert_attn_close, check_selection_head, clusters_to_gpu, inputs, oracle_clusters,
                         pack_mask, say, scale_of, to_np, unpack_mask, workspace_for)

pytestmark = pytest.mark.gpu

HY_S = replace(wl.HUNYUAN, name="hy_small", heads=2, frames=5, height=16, width=24)   # N = 1920, 32^3 combos
HY_S8 = replace(HY_S, name="hy_small_cs8", k=replace(wl.HUNYUAN.k, clusters=8))
HY_CASES = [HY_S, HY_S8, HY_S.forced_density(0.1), replace(HY_S8, online_topk=False, top_p=0.7, floor=40)]
# fp32 inputs: each slice's k-means on the vector ALUs, the attention one
# thread per query row
HY_F32 = replace(HY_S, name="hy_small_f32", dtype="f32")


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def expanded(sub_cent, dims, d):
    """[3*Cs, d] slice centroids, zeros outside their slice (the ABI layout)."""
    Cs = sub_cent[0].shape[0]
    out = np.zeros((3 * Cs, d))
    off = 0
    for s, ds in enumerate(dims):
        out[s * Cs:(s + 1) * Cs, off:off + ds] = sub_cent[s]
        off += ds
    return out


def slices(cent_expanded, dims, Cs):
    """[3*Cs, d] expanded slice centroids -> the three [Cs, d_s] blocks."""
    out, c0 = [], 0
    for s, ds in enumerate(dims):
        out.append(cent_expanded[s * Cs:(s + 1) * Cs, c0:c0 + ds])
        c0 += ds
    return out


def slice_labels(combo, Cs):
    """combo ids g = (a_t Cs + a_h) Cs + a_w -> (a_t, a_h, a_w)."""
    return [combo // (Cs * Cs), (combo // Cs) % Cs, combo % Cs]


def subspace_step(p, w, x, start, ws):
    """One Lloyd step of every slice from the given slice centroids (expanded
    layout), through sa_cluster with SA_INIT_GIVEN."""
    cfg = L.cluster_cfg("subspace", clusters=w.k.clusters, iters=1, init=L.SA_INIT_GIVEN, sub_dims=w.k.sub_dims)
    out = L.alloc_clusters(p, cfg, DEV, x.dtype)
    out.centroids.copy_(torch.tensor(start, dtype=torch.float32))
    L.sa_cluster(p, cfg, x, out, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("w", [HY_S, HY_S8, HY_F32], ids=lambda w: w.name)
def test_subspace_stage_A_slices(w):
    """One step of each slice's k-means from given centroids (the 32- and
    48-column slices at d = 128): slice labels bit-exact except oracle near
    ties, updated slice centroids the oracle's update of the GPU's labels."""
    say(f"[subspace stage A/B] {w.name} dims={w.k.sub_dims} Cs={w.k.clusters}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = api.cfgs(w)
    ks = to_np(k)
    Cs, dims = w.k.clusters, w.k.sub_dims
    # starting centroids: two oracle Lloyd rounds of each slice, in fp32
    start = np.zeros((w.heads, 3 * Cs, w.d), dtype=np.float32)
    c0 = 0
    for s_, ds in enumerate(dims):
        for h in range(w.heads):
            start[h, s_ * Cs:(s_ + 1) * Cs, c0:c0 + ds] = oracle.kmeans(ks[h][:, c0:c0 + ds], Cs, 2)["centroids"]
        c0 += ds
    out = subspace_step(p, w, k, start, workspace_for(p, kc))
    for h in range(w.heads):
        lab = slice_labels(out.labels[h].cpu().numpy(), Cs)
        got = slices(out.centroids[h].cpu().numpy().astype(np.float64), dims, Cs)
        given = slices(start[h].astype(np.float64), dims, Cs)
        c0 = 0
        for s_, ds in enumerate(dims):
            xs = ks[h][:, c0:c0 + ds]
            lab_o, _, _, near = oracle.kmeans_assign(xs, given[s_])
            diff = np.nonzero(lab[s_] != lab_o)[0]
            assert all(near[diff]), f"head {h} slice {s_}: label differences off a near tie"
            cu, sizes = oracle.kmeans_update(xs, lab[s_], given[s_])
            rel = np.abs(got[s_] - cu).max() / max(1e-30, np.abs(cu).max())
            say(f"  head {h} slice {s_} ({ds} columns): label mismatches {len(diff)} (near ties {int(near.sum())}), "
                f"centroid rel err {rel:.2e}")
            assert rel <= 1e-6
            c0 += ds


@pytest.mark.parametrize("w", [HY_S, HY_S8], ids=lambda w: w.name)
def test_subspace_cluster(w):
    """The whole subspace clustering (first-k seeds, iters steps), and the same
    run as one-step calls from given centroids (bit-identical): every step's
    slice labels differ from the oracle's assignment (from the GPU's centroids
    of the step before) only at near ties, and the centroids are the oracle's
    update of the GPU's labels.  Combo order, offsets and x_perm follow the
    GPU's labels exactly."""
    say(f"[subspace cluster] {w.name} N={w.n} Cs={w.k.clusters}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, kc)
    out = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster(p, kc, k, out, ws)
    torch.cuda.synchronize()
    ks = to_np(k)
    Cs, dims = w.k.clusters, w.k.sub_dims
    cur = np.zeros((w.heads, 3 * Cs, w.d), dtype=np.float32)
    c0 = 0
    for s_, ds in enumerate(dims):
        cur[:, s_ * Cs:(s_ + 1) * Cs, c0:c0 + ds] = ks[:, :Cs, c0:c0 + ds]  # first-k seeds (exact in fp32)
        c0 += ds
    traced = 0
    for it in range(w.k.iters):
        step = subspace_step(p, w, k, cur, ws)
        for h in range(w.heads):
            lab = slice_labels(step.labels[h].cpu().numpy(), Cs)
            given = slices(cur[h].astype(np.float64), dims, Cs)
            got = slices(step.centroids[h].cpu().numpy().astype(np.float64), dims, Cs)
            c0 = 0
            for s_, ds in enumerate(dims):
                xs = ks[h][:, c0:c0 + ds]
                lab_o, _, _, near = oracle.kmeans_assign(xs, given[s_])
                diff = np.nonzero(lab[s_] != lab_o)[0]
                assert all(near[diff]), f"step {it} head {h} slice {s_}: label differences off a near tie"
                traced += len(diff)
                cu, _ = oracle.kmeans_update(xs, lab[s_], given[s_])
                assert np.abs(got[s_] - cu).max() / max(1e-30, np.abs(cu).max()) <= 1e-6
                c0 += ds
        cur = step.centroids.cpu().numpy()
    for f in ("labels", "perm", "offsets", "centroids", "x_perm"):
        assert torch.equal(getattr(step, f), getattr(out, f)), f"chained steps differ from one call ({f})"
    for h in range(w.heads):
        lab = out.labels[h].cpu().numpy()
        r = oracle.subspace_cluster(ks[h], dims, Cs, w.k.iters)
        perm_o, off_o = oracle.permute(lab, Cs ** 3)
        assert np.array_equal(out.perm[h].cpu().numpy(), perm_o)
        assert np.array_equal(out.offsets[h].cpu().numpy(), off_o)
        assert torch.equal(out.x_perm[h], k[h][out.perm[h].long()])
        say(f"  head {h}: combo agreement with the oracle's own run {float((lab == r['labels']).mean()):.5f}, "
            f"non-empty combos {(np.diff(off_o) > 0).sum()}")
    say(f"  {w.k.iters} steps traced: {traced} slice-label differences, each at an oracle near tie")


def subspace_setup(w, q, k):
    rq = oracle_clusters(q, w.q)
    ks = to_np(k)
    rk = []
    for h in range(w.heads):
        r = oracle.subspace_cluster(ks[h], w.k.sub_dims, w.k.clusters, w.k.iters)
        perm, off = oracle.permute(r["labels"], w.k.clusters ** 3)
        r.update(perm=perm, offsets=off, sizes=np.diff(off), C=w.k.clusters ** 3)
        rk.append(r)
    return rq, rk


@pytest.mark.parametrize("w", HY_CASES, ids=lambda w: f"{w.name}-P{w.top_p}-k{w.floor}-o{int(w.online_topk)}")
def test_subspace_select(w):
    say(f"[subspace select] {w.name} P={w.top_p} floor={w.floor} online={w.online_topk}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = api.cfgs(w)
    rq, rk = subspace_setup(w, q, k)
    qbar32 = np.stack([r["means"] for r in rq]).astype(np.float32)
    sub32 = [[c.astype(np.float32) for c in r["sub_centroids"]] for r in rk]
    qt = clusters_to_gpu(p, q, rq, w.q.method, centroids=qbar32)
    kt = clusters_to_gpu(p, k, rk, "subspace",
                         centroids=np.stack([expanded(s, w.k.sub_dims, w.d) for s in sub32]).astype(np.float32))
    kt.sub_clusters = w.k.clusters
    kt.sub_dims = tuple(w.k.sub_dims)
    Cq, Ck = qt.num_clusters, kt.num_clusters
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, Cq, dtype=torch.int32, device=DEV)
    init = torch.empty_like(counts)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, init, ktop, workspace_for(p, qc, kc, sc, ac))
    torch.cuda.synchronize()
    gm = unpack_mask(mask, Ck)
    for h in range(w.heads):
        lg = oracle.subspace_logits(qbar32[h].astype(np.float64), [c.astype(np.float64) for c in sub32[h]],
                                    w.k.sub_dims, rk[h]["sizes"], scale_of(w), w.size_weighted)

        def redo(kh, lg=lg, h=h):
            return oracle.select(lg, rk[h]["sizes"], rq[h]["sizes"], w.top_p, w.floor, w.online_topk, k_h=kh)

        s = oracle.select(lg, rk[h]["sizes"], rq[h]["sizes"], w.top_p, w.floor, w.online_topk)
        s = check_selection_head(gm[h], counts[h].cpu().numpy(), init[h].cpu().numpy(), ktop[h], s, redo,
                                 rq[h]["sizes"], w.n, w.online_topk, f"head {h}")
        say(f"    mean keys/row {s['n_final'].mean():.1f}")


@pytest.mark.parametrize("w", [HY_S, HY_S.forced_density(0.1)], ids=lambda w: f"{w.name}-P{w.top_p}")
def test_subspace_attention(w):
    say(f"[subspace attention] {w.name}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = api.cfgs(w)
    rq, rk = subspace_setup(w, q, k)
    qt = clusters_to_gpu(p, q, rq, w.q.method)
    kt = clusters_to_gpu(p, k, rk, "subspace",
                         centroids=np.stack([expanded(r["sub_centroids"], w.k.sub_dims, w.d) for r in rk]))
    kt.sub_clusters = w.k.clusters
    kt.sub_dims = tuple(w.k.sub_dims)
    masks = []
    for h in range(w.heads):
        lg = oracle.subspace_logits(rq[h]["means"], rk[h]["sub_centroids"], w.k.sub_dims, rk[h]["sizes"],
                                    scale_of(w), w.size_weighted)
        masks.append(oracle.select(lg, rk[h]["sizes"], rq[h]["sizes"], w.top_p, w.floor, w.online_topk)["mask"])
    v_perm = torch.empty_like(v)
    L.sa_permute(p, kt, v, v_perm)
    o = torch.full_like(q, float("nan"))
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, None, torch.tensor(pack_mask(np.stack(masks)), device=DEV), o,
                           workspace_for(p, qc, kc, sc, ac))
    torch.cuda.synchronize()
    qs, ks, vs = to_np(q), to_np(k), to_np(v)
    ref = np.stack([oracle.attention(qs[h], ks[h], vs[h], rq[h]["perm"], rq[h]["offsets"], rk[h]["perm"],
                                     rk[h]["offsets"], masks[h], scale_of(w)) for h in range(w.heads)])
    assert not torch.isnan(o).any()
    assert_attn_close(o, ref, q.dtype, w.name)


@pytest.mark.parametrize("w", [HY_S, HY_S8.forced_density(0.1), HY_F32], ids=lambda w: f"{w.name}-P{w.top_p}")
def test_subspace_forward(w):
    say(f"[subspace forward] {w.name}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, qc, kc, sc, ac)
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster(p, qc, q, qt, ws)
    L.sa_cluster(p, kc, k, kt, ws)
    v_perm = torch.empty_like(v)
    L.sa_permute(p, kt, v, v_perm)
    Cq, Ck = qt.num_clusters, kt.num_clusters
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, Cq, dtype=torch.int32, device=DEV)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, None, ktop, ws)
    o = torch.empty_like(q)
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, None, mask, o, ws)
    o2, mask2 = api.forward(q, k, v, w)
    torch.cuda.synchronize()
    assert torch.equal(mask, mask2) and torch.equal(o, o2)
    qs, ks, vs = to_np(q), to_np(k), to_np(v)
    gm = unpack_mask(mask, Ck)
    ref = np.stack([oracle.attention(qs[h], ks[h], vs[h], qt.perm[h].cpu().numpy(), qt.offsets[h].cpu().numpy(),
                                     kt.perm[h].cpu().numpy(), kt.offsets[h].cpu().numpy(), gm[h], scale_of(w))
                    for h in range(w.heads)])
    assert_attn_close(o, ref, q.dtype, w.name)
    # selected keys per row agree with the reported counts
    sizes = np.diff(kt.offsets.cpu().numpy(), axis=1)
    keys = (gm * sizes[:, None, :]).sum(-1)
    assert np.array_equal(keys, counts.cpu().numpy())
    qsizes = np.diff(qt.offsets.cpu().numpy(), axis=1)
    say(f"  attended fraction of the score matrix {(qsizes * keys).sum() / (w.heads * w.n * w.n):.4f}")
