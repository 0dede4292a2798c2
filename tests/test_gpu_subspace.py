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

from gpu_helpers import (DEV, assert_attn_close, clusters_to_gpu, inputs, oracle_clusters, pack_mask, say,
                         scale_of, to_np, unpack_mask, workspace_for)

pytestmark = pytest.mark.gpu

HY_S = replace(wl.HUNYUAN, name="hy_small", heads=2, frames=5, height=16, width=24)   # N = 1920, 32^3 combos
HY_S8 = replace(HY_S, name="hy_small_cs8", k=replace(wl.HUNYUAN.k, clusters=8))
HY_CASES = [HY_S, HY_S8, HY_S.forced_density(0.1), replace(HY_S8, online_topk=False, top_p=0.7, floor=40)]


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


@pytest.mark.parametrize("w", [HY_S, HY_S8], ids=lambda w: w.name)
def test_subspace_cluster(w):
    say(f"[subspace cluster] {w.name} N={w.n} Cs={w.k.clusters}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = api.cfgs(w)
    out = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster(p, kc, k, out, workspace_for(p, kc))
    torch.cuda.synchronize()
    ks = to_np(k)
    Cs = w.k.clusters
    for h in range(w.heads):
        r = oracle.subspace_cluster(ks[h], w.k.sub_dims, Cs, w.k.iters)
        lab = out.labels[h].cpu().numpy()
        agree = float((lab == r["labels"]).mean())
        say(f"  head {h}: combo agreement {agree:.5f}, non-empty combos {(r['combo_sizes'] > 0).sum()}")
        assert agree >= 0.99
        perm_o, off_o = oracle.permute(lab, Cs ** 3)
        assert np.array_equal(out.perm[h].cpu().numpy(), perm_o)
        assert np.array_equal(out.offsets[h].cpu().numpy(), off_o)
        if agree == 1.0:
            np.testing.assert_allclose(out.centroids[h].cpu().numpy(),
                                       expanded(r["sub_centroids"], w.k.sub_dims, w.d), rtol=1e-5, atol=1e-5)
        assert torch.equal(out.x_perm[h], k[h][out.perm[h].long()])


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
        s = oracle.select(lg, rk[h]["sizes"], rq[h]["sizes"], w.top_p, w.floor, w.online_topk)
        bad = np.nonzero((gm[h] != s["mask"]).any(axis=1))[0]
        say(f"  head {h}: rows differing {len(bad)} (flagged {int(s['near_tie'].sum())}), k_h gpu {int(ktop[h])} "
            f"oracle {s['k_h']}, mean keys/row {s['n_final'].mean():.1f}")
        assert all(s["near_tie"][i] for i in bad), bad
        if not s["near_tie"].any():
            assert np.array_equal(gm[h], s["mask"])
            assert int(ktop[h]) == s["k_h"]
            assert np.array_equal(counts[h].cpu().numpy(), s["n_final"])
            assert np.array_equal(init[h].cpu().numpy(), s["n_init"])


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


@pytest.mark.parametrize("w", [HY_S, HY_S8.forced_density(0.1)], ids=lambda w: f"{w.name}-P{w.top_p}")
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
