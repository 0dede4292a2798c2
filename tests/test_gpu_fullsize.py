"""GPU parity at the configurations' full sizes, in the launch configuration
the bench times: the component calls (sa_cluster_qk, sa_permute, sa_select,
sa_block_sparse_attn) and sa_forward, with one workspace of
sa_workspace_size() bytes.

The oracle cannot run whole layers of these sizes, so the checks are
  * properties that hold at any size, on every head: perms are bijections,
    clusters are contiguous and ascending inside, labels and offsets agree,
    x_perm holds the rows in cluster order, centroids are member means, the
    forced-density rows select exactly the floor, sa_forward equals the
    component calls bit for bit;
  * outputs the oracle computes one by one on a sample: the root split of a
    head's bisection (from the same seeds, over all N tokens), the selection
    of every row of two heads given the GPU's centroids and sizes, and the
    attention output of sampled query clusters given the GPU's clusters,
    mask, K means and V means.
Selection and split differences are accepted only where the oracle flags a
near tie (the rules of the staged tests)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import DEV, assert_attn_close, check_selection_head, say, scale_of, to_np, unpack_mask, workspace_for

pytestmark = pytest.mark.gpu

FULL = [wl.WAN.forced_density(0.1), wl.WAN, wl.TABULAR.forced_density(0.1), wl.TABULAR, wl.MID,
        wl.HUNYUAN.forced_density(0.1), wl.HUNYUAN]


def ids(w):
    return f"{w.name}-P{w.top_p}-k{w.floor}"


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def check_clusters(x, t, spec, N, what):
    """Invariants of one tensor's clustering on every head."""
    H = x.shape[0]
    perm, off, lab = t.perm.long(), t.offsets.long(), t.labels.long()
    C = t.num_clusters
    ar = torch.arange(N, device=DEV)
    assert torch.equal(torch.sort(perm, dim=1).values, ar.expand(H, N)), f"{what}: perm is not a bijection"
    assert torch.all(off[:, 0] == 0) and torch.all(off[:, -1] == N) and torch.all(off[:, 1:] >= off[:, :-1])
    if spec.method == "bisect":
        law = torch.clamp(torch.arange(C + 1, device=DEV) * spec.leaf, max=N)
        assert torch.equal(off, law.expand(H, C + 1)), f"{what}: leaf sizes"
    # cluster of every position, from the offsets
    pos_c = torch.searchsorted(off[:, 1:].contiguous(), ar.expand(H, N).contiguous(), right=True)
    assert torch.equal(lab.gather(1, perm), pos_c), f"{what}: labels disagree with perm/offsets"
    same = pos_c[:, 1:] == pos_c[:, :-1]
    assert torch.all((perm[:, 1:] > perm[:, :-1]) | ~same), f"{what}: order inside a cluster"
    assert torch.equal(t.x_perm, x.gather(1, perm.unsqueeze(-1).expand(-1, -1, x.shape[2]))), f"{what}: x_perm"
    if spec.method in ("bisect", "kmeans"):
        # centroid = member mean (fp64 sums of the rows in cluster order)
        xs = t.x_perm.double()
        cum = torch.zeros(H, N + 1, x.shape[2], dtype=torch.float64, device=DEV)
        cum[:, 1:] = torch.cumsum(xs, dim=1)  # cum[p] = sum of the first p rows
        at = cum.gather(1, off.unsqueeze(-1).expand(-1, -1, x.shape[2]))
        sums = at[:, 1:] - at[:, :-1]
        sizes = (off[:, 1:] - off[:, :-1]).double()
        nonempty = sizes > 0
        means = sums / sizes.clamp(min=1).unsqueeze(-1)
        err = (t.centroids.double() - means).abs()[nonempty]
        tol = 1e-5 * (1.0 + means.abs()[nonempty])
        assert torch.all(err <= tol), f"{what}: centroids, worst {float((err - tol).max()):.3e}"
    say(f"  {what}: {C} clusters, invariants hold on {H} heads")


def check_root_split(x, t, spec, h, what):
    """The root node of head h's bisection, replayed by the oracle over all N
    tokens from the same seeds: the GPU's first n_left positions must be the
    oracle's left set unless the oracle flags the split as a near tie."""
    xs = to_np(x[h])
    N = xs.shape[0]
    C = -(-N // spec.leaf)
    n_left = spec.leaf * (-(-C // 2))
    members = np.arange(N)
    left, _, _, gap = oracle.bisect_split(xs, members, n_left, xs[0].copy(), xs[1].copy(), spec.iters)
    gpu_left = np.sort(t.perm[h, :n_left].cpu().numpy())
    same = np.array_equal(gpu_left, members[left])
    say(f"  {what}: root split of head {h} over {N} tokens, n_left {n_left}: "
        f"{'same' if same else 'different'} (oracle min rel gap {gap:.2e})")
    assert same or gap <= oracle.NEAR_TIE_REL


def oracle_selection(w, qt, kt, h):
    """The oracle's selection of head h given the GPU's centroids and sizes,
    and a function giving it again for a given k_h."""
    qbar = qt.centroids[h].double().cpu().numpy()
    qsz = np.diff(qt.offsets[h].cpu().numpy())
    ksz = np.diff(kt.offsets[h].cpu().numpy())
    if w.k.method == "subspace":
        Cs, dims = w.k.clusters, w.k.sub_dims
        cen = kt.centroids[h].double().cpu().numpy()
        subs, c0 = [], 0
        for s, ds in enumerate(dims):
            subs.append(cen[s * Cs:(s + 1) * Cs, c0:c0 + ds])
            c0 += ds
        lg = oracle.subspace_logits(qbar, subs, dims, ksz, scale_of(w), w.size_weighted)
        units = ksz
    else:
        lg = oracle.cluster_logits(qbar, kt.centroids[h].double().cpu().numpy(), ksz, scale_of(w), w.size_weighted)
        units = np.ones(len(ksz), np.int64)

    def redo(kh):
        return oracle.select(lg, units, qsz, w.top_p, w.floor, w.online_topk, k_h=kh)

    return oracle.select(lg, units, qsz, w.top_p, w.floor, w.online_topk), redo, qsz


@pytest.mark.parametrize("w", FULL, ids=ids)
def test_full_size(w):
    say(f"[full size] {w.name} H={w.heads} N={w.n} d={w.d} {w.dtype} P={w.top_p} floor={w.floor} "
        f"online={w.online_topk} comp={w.compensate}")
    q, k, v = wl.make_inputs(w, device=DEV)
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, qc, kc, sc, ac)
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster_qk(p, qc, kc, q, k, qt, kt, ws)
    Cq, Ck = qt.num_clusters, kt.num_clusters
    v_perm = torch.empty_like(v)
    vbar = torch.empty(w.heads, Ck, w.d, dtype=torch.float32, device=DEV) if w.compensate else None
    L.sa_permute(p, kt, v, v_perm, vbar)
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, Cq, dtype=torch.int32, device=DEV)
    init = torch.empty_like(counts)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, init, ktop, ws)
    o = torch.full_like(q, float("nan"))
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, vbar, mask, o, ws)
    o2 = torch.empty_like(q)
    mask2 = torch.empty_like(mask)
    L.sa_forward(p, qc, kc, sc, ac, q, k, v, o2, mask2, ws)
    torch.cuda.synchronize()
    say("  ran the component calls and sa_forward")
    assert torch.equal(mask, mask2) and torch.equal(o, o2), "sa_forward differs from its component calls"
    assert bool(torch.isfinite(o).all())

    check_clusters(q, qt, w.q, w.n, "Q")
    check_clusters(k, kt, w.k, w.n, "K")
    if w.q.method == "bisect":
        check_root_split(q, qt, w.q, 0, "Q")
    if w.k.method == "bisect":
        check_root_split(k, kt, w.k, w.heads - 1, "K")
    if vbar is not None:
        # V means of sampled clusters against the oracle's member means of
        # the same rows (fp64, original V)
        for h in (0, w.heads - 1):
            off = kt.offsets[h].cpu().numpy()
            perm = kt.perm[h].cpu().numpy()
            pick = np.array(sorted({0, Ck // 3, Ck // 2, Ck - 1}))
            sub_off = np.concatenate([[0], np.cumsum(off[pick + 1] - off[pick])])
            rows = np.concatenate([perm[off[j]:off[j + 1]] for j in pick])
            ref = oracle.cluster_means(to_np(v[h]), rows, sub_off)
            got = vbar[h, torch.tensor(pick, device=DEV)].double().cpu().numpy()
            assert np.all(np.abs(got - ref) <= 1e-6 * (1.0 + np.abs(ref))), "V means"

    gm = unpack_mask(mask, Ck)
    if w.top_p <= 0 and not w.online_topk and w.k.method != "subspace":
        pc = gm.sum(-1)
        qsz = np.diff(qt.offsets.cpu().numpy(), axis=1)
        assert np.all(pc[qsz > 0] == w.floor), "forced density: rows must select exactly the floor"

    # selection of every row of two heads, given the GPU's centroids and sizes
    for h in (0, w.heads - 1):
        s, redo, qsz = oracle_selection(w, qt, kt, h)
        check_selection_head(gm[h], counts[h].cpu().numpy(), init[h].cpu().numpy(), ktop[h], s, redo, qsz, w.n,
                             w.online_topk, f"select head {h}")

    # attention of sampled query clusters, given the GPU's clusters, mask and means
    rng = np.random.default_rng(0)
    for h in (0, w.heads - 1):
        qoff = qt.offsets[h].cpu().numpy()
        nonempty = np.nonzero(np.diff(qoff) > 0)[0]
        pick = np.unique(np.concatenate([nonempty[:1], nonempty[-1:], rng.choice(nonempty, size=4, replace=False)]))
        qperm = qt.perm[h].cpu().numpy()
        rows = [qperm[qoff[i]:qoff[i + 1]] for i in pick]
        sub_off = np.concatenate([[0], np.cumsum([len(r) for r in rows])])
        qs, ks, vs = to_np(q[h]), to_np(k[h]), to_np(v[h])
        kb = kt.centroids[h].double().cpu().numpy() if w.compensate else None
        vb = vbar[h].double().cpu().numpy() if w.compensate else None
        ref = oracle.attention(qs, ks, vs, np.concatenate(rows), sub_off, kt.perm[h].cpu().numpy(),
                               kt.offsets[h].cpu().numpy(), gm[h][pick], scale_of(w), w.compensate, kb, vb)
        tok = np.concatenate(rows)
        got = o[h, torch.tensor(tok, device=DEV)]
        assert_attn_close(got, ref[tok], q.dtype, f"attention head {h}, {len(pick)} query clusters, {len(tok)} rows")
    del q, k, v, qt, kt, v_perm, o, o2, ws
    torch.cuda.empty_cache()
