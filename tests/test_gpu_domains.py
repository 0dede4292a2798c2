"""GPU parity of the selection's competition domains against the fp64 oracle
(oracle.select_domains), given the GPU's own clusters (identical centroids and
sizes on both sides): VMoBA's head-global block selection and EG-Sparse's
entropy-gated grouped cross-head pools, with and without SCOPE's online
Top-k, at reduced sizes and on one group of the full Wan-shaped layer.

Head entropies must agree to 1e-12; every head's mask, counts, initial counts
and k_h follow the selection rules of the staged tests (bit-exact except
flagged near ties, which may differ only inside their flags).  sa_forward with
the same configuration must equal the component calls."""

from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import (DEV, MID_S, WAN_S, check_selection_head, inputs, say, scale_of, unpack_mask,
                         workspace_for)

pytestmark = pytest.mark.gpu

DOMAIN = {"row": oracle.DOMAIN_ROW, "head": oracle.DOMAIN_HEAD, "group": oracle.DOMAIN_GROUP}


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def run_select(w, q, k, ws=None):
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, qc, kc, sc, ac) if ws is None else ws
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster_qk(p, qc, kc, q, k, qt, kt, ws)
    Cq, Ck = qt.num_clusters, kt.num_clusters
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, Cq, dtype=torch.int32, device=DEV)
    init = torch.empty_like(counts)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    ent = torch.full((w.heads,), float("nan"), dtype=torch.float64, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, init, ktop, ws, head_entropy=ent)
    torch.cuda.synchronize()
    return qt, kt, mask, counts, init, ktop, ent, ws


def oracle_logits(w, qt, kt, heads):
    lg, qs = [], []
    for h in heads:
        ksz = np.diff(kt.offsets[h].cpu().numpy())
        lg.append(oracle.cluster_logits(qt.centroids[h].double().cpu().numpy(), kt.centroids[h].double().cpu().numpy(),
                                        ksz, scale_of(w), w.size_weighted))
        qs.append(np.diff(qt.offsets[h].cpu().numpy()))
    return np.stack(lg), np.stack(qs)


def check(w, qt, kt, mask, counts, init, ktop, ent, heads):
    """Oracle selection of `heads` (whole groups) given the GPU's clusters."""
    lg, qs = oracle_logits(w, qt, kt, heads)
    Ck = kt.num_clusters
    units = np.ones(Ck, np.int64)
    h0 = heads[0]
    group = w.group if w.domain == "group" else 1
    r = oracle.select_domains(lg, units, qs, w.top_p, w.floor, w.online_topk, DOMAIN[w.domain], group,
                              w.max_entropy)
    ge = ent.cpu().numpy()[heads]
    say(f"  entropies gpu {np.round(ge, 6).tolist()} pools {[[h0 + x for x in pl] for pl in r['pools']]}")
    assert np.all(np.abs(ge - r["entropy"]) <= 1e-12), (ge, r["entropy"])
    pooled = {}
    for pl in r["pools"]:
        pooled.update(oracle.pool_counts(lg, qs, pl, w.top_p))
    gm = unpack_mask(mask, Ck)
    for x, h in enumerate(heads):
        pc = pooled.get(x)

        def redo(kh, x=x, pc=pc):
            return oracle.select(lg[x], units, qs[x], w.top_p, w.floor, w.online_topk, k_h=kh, pool=pc)

        check_selection_head(gm[h], counts[h].cpu().numpy(), init[h].cpu().numpy(), ktop[h], r["heads"][x], redo,
                             qs[x], w.n, w.online_topk, f"head {h} ({'pooled' if pc else 'per row'})")
    return r


WAN6 = replace(WAN_S, name="wan_small6", heads=6)
MID4 = replace(MID_S, name="mid_small4", heads=4)


@pytest.mark.parametrize("w", [
    replace(WAN6, name="wan6_head_global", domain="head"),
    replace(WAN6, name="wan6_head_global_p05", domain="head", top_p=0.5, floor=2),
    replace(MID4, name="mid4_head_global_online", domain="head"),
    replace(WAN6, name="wan6_groups3_all", domain="group", group=3, max_entropy=2.0, top_p=0.6),
], ids=lambda w: w.name)
def test_domains_fixed_routing(w):
    say(f"[domains] {w.name} H={w.heads} N={w.n} P={w.top_p} floor={w.floor} online={w.online_topk} "
        f"domain={w.domain} group={w.group} max_entropy={w.max_entropy}")
    q, k, v = inputs(w)
    res = run_select(w, q, k)
    r = check(w, *res[:7], list(range(w.heads)))
    if w.domain == "head":
        assert r["pools"] == [[h] for h in range(w.heads)]


@pytest.mark.parametrize("base", [WAN6, MID4], ids=lambda w: w.name)
def test_domains_entropy_gated_groups(base):
    """EG-Sparse routing with a threshold between the heads' entropies, so
    each group of two holds pooled and per-row heads (or pools of two)."""
    q, k, v = inputs(base)
    # entropies from a first call, then a threshold at their median
    probe = replace(base, domain="group", group=2, max_entropy=-1.0)
    res0 = run_select(probe, q, k)
    e = np.sort(res0[6].cpu().numpy())
    tau = float(0.5 * (e[len(e) // 2 - 1] + e[len(e) // 2]))
    w = replace(base, name=base.name + "_gated", domain="group", group=2, max_entropy=tau)
    say(f"[domains] {w.name} H={w.heads} P={w.top_p} online={w.online_topk} groups of 2, max_entropy {tau:.6f}")
    res = run_select(w, q, k, ws=res0[7])
    r = check(w, *res[:7], list(range(w.heads)))
    assert 0 < sum(len(p) for p in r["pools"]) < w.heads
    # with no head below the threshold the rule is the per-row one, bit for bit
    row = run_select(replace(base, domain="row"), q, k, ws=res0[7])
    assert torch.equal(res0[2], row[2]) and torch.equal(res0[3], row[3]) and torch.equal(res0[5], row[5])


def test_domains_forward_matches_components():
    w = replace(WAN6, name="wan6_gated_fwd", domain="group", group=3, max_entropy=0.97, top_p=0.8)
    q, k, v = inputs(w)
    qt, kt, mask, counts, init, ktop, ent, ws = run_select(w, q, k)
    p, qc, kc, sc, ac = api.cfgs(w)
    v_perm = torch.empty_like(v)
    vbar = torch.empty(w.heads, kt.num_clusters, w.d, dtype=torch.float32, device=DEV)
    L.sa_permute(p, kt, v, v_perm, vbar)
    o = torch.empty_like(q)
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, vbar, mask, o, ws)
    o2, mask2 = api.forward(q, k, v, w)
    torch.cuda.synchronize()
    assert torch.equal(mask, mask2) and torch.equal(o, o2)


def test_domains_full_size_group():
    """The Wan-shaped layer (40 x 75600 x 128) with EG-Sparse groups of four
    heads: the oracle replays the first group (heads 0-3) in full."""
    # a threshold between the first group's entropies (0.99623, 0.99602, 0.99619, 0.99610):
    # heads 1 and 3 share a pool, heads 0 and 2 select per row
    w = replace(wl.WAN, name="wan720p_groups4", domain="group", group=4, max_entropy=0.99615, top_p=0.9)
    say(f"[domains] {w.name} H={w.heads} N={w.n} groups of 4, max_entropy {w.max_entropy}")
    q, k, v = wl.make_inputs(w, device=DEV)
    res = run_select(w, q, k)
    say(f"  head entropies (first 8) {np.round(res[6].cpu().numpy()[:8], 5).tolist()}")
    r = check(w, *res[:7], [0, 1, 2, 3])
    assert r["pools"] == [[1, 3]]
    del q, k, v, res
    torch.cuda.empty_cache()


@pytest.mark.parametrize("w", [
    replace(WAN6, name="wan6_stat1", rule="stat", stat_lambda=1.0),
    replace(WAN6, name="wan6_stat0_floor3", rule="stat", stat_lambda=0.0, floor=3),
    replace(MID4, name="mid4_stat05_online", rule="stat", stat_lambda=0.5),
    replace(wl.TABULAR, name="tab_small_stat2", heads=2, width=8292, rule="stat", stat_lambda=2.0),
], ids=lambda w: w.name)
def test_stat_threshold_rule(w):
    """BSA's statistical dynamic threshold in place of Top-p: every row keeps
    the units whose proxy probability reaches mean + lambda * std of its row."""
    say(f"[stat rule] {w.name} H={w.heads} N={w.n} lambda={w.stat_lambda} floor={w.floor} online={w.online_topk}")
    q, k, v = inputs(w)
    qt, kt, mask, counts, init, ktop, ent, ws = run_select(w, q, k)
    lg, qs = oracle_logits(w, qt, kt, list(range(w.heads)))
    Ck = kt.num_clusters
    units = np.ones(Ck, np.int64)
    gm = unpack_mask(mask, Ck)
    for h in range(w.heads):
        def redo(kh, h=h):
            return oracle.select(lg[h], units, qs[h], w.top_p, w.floor, w.online_topk, k_h=kh,
                                 stat_lambda=w.stat_lambda)

        s = oracle.select(lg[h], units, qs[h], w.top_p, w.floor, w.online_topk, stat_lambda=w.stat_lambda)
        check_selection_head(gm[h], counts[h].cpu().numpy(), init[h].cpu().numpy(), ktop[h], s, redo, qs[h], w.n,
                             w.online_topk, f"head {h}")
        say(f"    mean clusters/row {s['n_final'].mean():.1f} of {Ck}")
    o2, mask2 = api.forward(q, k, v, w)
    torch.cuda.synchronize()
    assert torch.equal(mask, mask2)
