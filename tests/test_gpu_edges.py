"""GPU parity on degenerate shapes and selections, end to end through the C
ABI: the component calls and sa_forward (which must agree bit for bit), the
selection against the oracle's given the GPU's centroids and sizes, the
attention against the oracle's given the GPU's clusters, mask and means, and,
where every cluster is selected, against plain softmax attention computed in
fp64.

Cases:
  * fewer tokens than one leaf (one cluster per tensor, 100 tokens, one head);
  * one leaf plus one token (a last cluster of a single token);
  * Top-p = 1 (every cluster selected: dense attention; compensation has
    nothing to add);
  * a fixed floor above the number of key clusters (every cluster selected);
  * Top-p = 0 with a floor of one cluster (the sparsest selection)."""

from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import (DEV, WAN_S, assert_attn_close, check_selection_head, inputs, say, scale_of, to_np,
                         unpack_mask, workspace_for)

pytestmark = pytest.mark.gpu

ONE_LEAF = replace(wl.WAN, name="wan_one_leaf", heads=1, frames=1, height=10, width=10)       # N = 100
LEAF_PLUS_ONE = replace(wl.WAN, name="wan_leaf_plus_one", heads=2, frames=1, height=1, width=129)
ALL_TOP_P = replace(WAN_S, name="wan_small_top_p_1", top_p=1.0)
FLOOR_ABOVE = replace(WAN_S, name="wan_small_floor_above", top_p=0.0, floor=WAN_S.key_clusters() + 5)
SPARSEST = replace(WAN_S, name="wan_small_floor_1", top_p=0.0, floor=1)
CASES = [ONE_LEAF, LEAF_PLUS_ONE, ALL_TOP_P, FLOOR_ABOVE, SPARSEST]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def dense_attention(q, k, v, scale):
    """softmax(q k^T scale) v in fp64, one head."""
    s = (q @ k.T) * scale
    s -= s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e @ v) / e.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_edge_case(w):
    say(f"[edges] {w.name} H={w.heads} N={w.n} P={w.top_p} floor={w.floor} comp={w.compensate}")
    q, k, v = inputs(w)
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
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, None, ktop, ws)
    o = torch.full_like(q, float("nan"))
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, vbar if w.compensate else None, mask, o, ws)
    o2, mask2 = api.forward(q, k, v, w)
    torch.cuda.synchronize()
    assert torch.equal(mask, mask2) and torch.equal(o, o2), "sa_forward differs from its component calls"
    assert bool(torch.isfinite(o).all())

    n = w.n
    law = [min(c * 128, n) for c in range(-(-n // 128) + 1)]
    for t in (qt, kt):
        assert t.num_clusters == -(-n // 128)
        assert (t.offsets.cpu().numpy() == np.array(law)).all()
        assert torch.equal(torch.sort(t.perm, dim=1).values.cpu(), torch.arange(n).expand(w.heads, n).to(torch.int32))

    gm = unpack_mask(mask, Ck)
    qs, ks, vs = to_np(q), to_np(k), to_np(v)
    every = True
    for h in range(w.heads):
        qbar = qt.centroids[h].double().cpu().numpy()
        ksz = np.diff(kt.offsets[h].cpu().numpy())
        qsz = np.diff(qt.offsets[h].cpu().numpy())
        lg = oracle.cluster_logits(qbar, kt.centroids[h].double().cpu().numpy(), ksz, scale_of(w), w.size_weighted)
        units = np.ones(Ck, np.int64)

        def redo(kh, lg=lg, qsz=qsz):
            return oracle.select(lg, units, qsz, w.top_p, w.floor, w.online_topk, k_h=kh)

        s = oracle.select(lg, units, qsz, w.top_p, w.floor, w.online_topk)
        say(f"  head {h}: {Cq} x {Ck} clusters, selected {int(gm[h].sum())}")
        check_selection_head(gm[h], counts[h].cpu().numpy(), None, ktop[h], s, redo, qsz, w.n, w.online_topk,
                             f"{w.name} head {h}")
        every &= bool(gm[h].all())
        ref = oracle.attention(qs[h], ks[h], vs[h], qt.perm[h].cpu().numpy(), qt.offsets[h].cpu().numpy(),
                               kt.perm[h].cpu().numpy(), kt.offsets[h].cpu().numpy(), gm[h], scale_of(w),
                               w.compensate, kt.centroids[h].cpu().double().numpy(),
                               vbar[h].cpu().double().numpy())
        assert_attn_close(o[h], ref, q.dtype, f"{w.name} head {h} vs oracle")
        if gm[h].all():
            assert_attn_close(o[h], dense_attention(qs[h], ks[h], vs[h], scale_of(w)), q.dtype,
                              f"{w.name} head {h} vs dense softmax")
    if w in (ONE_LEAF, ALL_TOP_P, FLOOR_ABOVE):
        assert every, "every cluster must be selected"
    if w is SPARSEST:
        assert (counts.cpu().numpy() == 1).all()
