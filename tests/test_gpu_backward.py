"""GPU parity of the block-sparse attention backward (sa_block_sparse_attn_bwd)
against the fp64 oracle (oracle.attention_backward) given the GPU's own
clusters, selection and forward output: bisection (a partial last leaf), k-means
(uneven clusters) and d = 64, at fixed density and with the natural Top-p.

Tolerance (bf16 inputs, fp32 gradients): the kernels round P and dS to bf16 for
the matrix cores (2^-9 relative each) and take D_n = <dO_n, O_n> from the
forward's bf16 output.  The rows of dS sum to zero, so dQ and dK are sums with
cancellation: an emulation of these roundings in fp64 on the small Wan case
gives dq errors of 0.55% of its mean magnitude (0.9% of its largest), dk 0.19%
(0.34%), dv 0.16% (0.13%).  The bounds are about twice that: dq and dk mean-abs
<= 1.2e-2 of the mean reference magnitude and max-abs <= 3e-2 of the largest,
dv 4e-3 and 1.5e-2.  A dropped term (D, a selected cluster, the scale) moves
the mean error by whole percents."""

from __future__ import annotations

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import DEV, MID_S, TAB_S, WAN_S, inputs, pack_mask, say, scale_of, to_np, unpack_mask, workspace_for

pytestmark = pytest.mark.gpu

TOL = {"dq": (3e-2, 1.2e-2), "dk": (3e-2, 1.2e-2), "dv": (1.5e-2, 4e-3)}  # (max, mean), relative

CASES = [replace(WAN_S.forced_density(0.1), compensate=False, name="wan_small_fixed"),
         replace(WAN_S, compensate=False, name="wan_small_p09"),
         replace(MID_S, compensate=False, name="mid_small_kmeans"),
         replace(TAB_S.forced_density(0.1), compensate=False, name="tab_small_d64")]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


@pytest.mark.parametrize("w", CASES, ids=lambda w: w.name)
def test_backward(w):
    say(f"[backward] {w.name} H={w.heads} N={w.n} d={w.d} P={w.top_p} floor={w.floor}")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, qc, kc, sc, ac)
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster_qk(p, qc, kc, q, k, qt, kt, ws)
    Cq, Ck = qt.num_clusters, kt.num_clusters
    v_perm = torch.empty_like(v)
    L.sa_permute(p, kt, v, v_perm, None)
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, Cq, dtype=torch.int32, device=DEV)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, None, ktop, ws)
    o = torch.empty_like(q)
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, None, mask, o, ws)
    g = torch.Generator(device="cpu").manual_seed(7)
    d_o = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
    wsb = L.workspace(L.sa_block_sparse_attn_bwd_workspace_size(p, Cq, Ck), DEV)
    grads = [torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV) for _ in range(3)]
    L.sa_block_sparse_attn_bwd(p, ac, qt, kt, v_perm, mask, o, d_o, *grads, wsb)
    again = [torch.empty_like(x) for x in grads]
    L.sa_block_sparse_attn_bwd(p, ac, qt, kt, v_perm, mask, o, d_o, *again, wsb)
    torch.cuda.synchronize()
    for a_, b_ in zip(grads, again):
        assert torch.equal(a_, b_), "backward is not deterministic"
    gm = unpack_mask(mask, Ck)
    qs, ks, vs, gs = to_np(q), to_np(k), to_np(v), to_np(d_o)
    bad = []
    for h in range(w.heads):
        ref = oracle.attention_backward(qs[h], ks[h], vs[h], qt.perm[h].cpu().numpy(), qt.offsets[h].cpu().numpy(),
                                        kt.perm[h].cpu().numpy(), kt.offsets[h].cpu().numpy(), gm[h], scale_of(w),
                                        gs[h])
        for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
            got = got[h].double().cpu().numpy()
            assert np.isfinite(got).all(), name
            err = np.abs(got - want)
            mx, mean = float(err.max()), float(err.mean())
            rmax, rmean = float(np.abs(want).max()), float(np.abs(want).mean())
            say(f"  head {h} {name}: max-abs {mx:.3e} ({mx / rmax:.2e} of max {rmax:.3e}), "
                f"mean-abs {mean:.3e} ({mean / rmean:.2e} of mean {rmean:.3e})")
            tol_max, tol_mean = TOL[name]
            if not (mx <= tol_max * rmax and mean <= tol_mean * rmean):
                bad.append((h, name, mx / rmax, mean / rmean))
    assert not bad, bad


def test_backward_full_size():
    """The Wan 720p layer at full size in the configuration the backward bench
    times (fixed 10% density, compensation off; natural Top-p is covered by
    the smaller cases): the oracle recomputes, for sampled key clusters of the
    first and last head, every query cluster that selected them; dK and dV of
    the key cluster's rows and dQ of those query clusters' rows are then
    complete and compared element by element (the same bounds)."""
    w = replace(wl.WAN.forced_density(0.1), compensate=False)
    say(f"[backward full size] {w.name} H={w.heads} N={w.n} d={w.d} P={w.top_p}")
    q, k, v = wl.make_inputs(w, device=DEV)
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, qc, kc, sc, ac)
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster_qk(p, qc, kc, q, k, qt, kt, ws)
    Cq, Ck = qt.num_clusters, kt.num_clusters
    v_perm = torch.empty_like(v)
    L.sa_permute(p, kt, v, v_perm, None)
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, Cq, dtype=torch.int32, device=DEV)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, None, ktop, ws)
    o = torch.empty_like(q)
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, None, mask, o, ws)
    del ws
    g = torch.Generator(device="cpu").manual_seed(11)
    d_o = torch.randn(q.shape, generator=g).to(torch.bfloat16).to(DEV)
    wsb = L.workspace(L.sa_block_sparse_attn_bwd_workspace_size(p, Cq, Ck), DEV)
    grads = [torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV) for _ in range(3)]
    L.sa_block_sparse_attn_bwd(p, ac, qt, kt, v_perm, mask, o, d_o, *grads, wsb)
    torch.cuda.synchronize()
    say("  ran the forward and the backward")
    for x in grads:
        assert bool(torch.isfinite(x).all()), "every gradient row is written"
    gm = unpack_mask(mask, Ck)
    rng = np.random.default_rng(3)
    bad = []
    for h in (0, w.heads - 1):
        qs, ks, vs, gs = to_np(q[h]), to_np(k[h]), to_np(v[h]), to_np(d_o[h])
        qperm, qoff = qt.perm[h].cpu().numpy(), qt.offsets[h].cpu().numpy()
        kperm, koff = kt.perm[h].cpu().numpy(), kt.offsets[h].cpu().numpy()
        sel_by = gm[h].sum(0)  # query clusters selecting each key cluster
        cand = np.nonzero(sel_by > 0)[0]
        cand = cand[np.argsort(sel_by[cand], kind="stable")]
        # the least selected key cluster and one from the less selected half
        picks = np.unique([cand[0], rng.choice(cand[:max(1, len(cand) // 2)])])
        for j in picks:
            I = np.nonzero(gm[h][:, j])[0]
            rows = np.concatenate([qperm[qoff[i]:qoff[i + 1]] for i in I])
            sub_off = np.concatenate([[0], np.cumsum(qoff[I + 1] - qoff[I])])
            ref = oracle.attention_backward(qs, ks, vs, rows, sub_off, kperm, koff, gm[h][I], scale_of(w), gs)
            keys = kperm[koff[j]:koff[j + 1]]
            for name, got, want, idx in zip(("dq", "dk", "dv"), grads, ref, (rows, keys, keys)):
                got = got[h, torch.tensor(idx, device=DEV)].double().cpu().numpy()
                want = want[idx]
                err = np.abs(got - want)
                mx, mean = float(err.max()), float(err.mean())
                rmax, rmean = float(np.abs(want).max()), float(np.abs(want).mean())
                say(f"  head {h} key cluster {j} ({len(I)} query clusters) {name}: max {mx / rmax:.2e} of max, "
                    f"mean {mean / rmean:.2e} of mean")
                tol_max, tol_mean = TOL[name]
                if not (mx <= tol_max * rmax and mean <= tol_mean * rmean):
                    bad.append((h, int(j), name, mx / rmax, mean / rmean))
    assert not bad, bad


def test_backward_given_mask_edges():
    """A hand-made mask over the GPU's clusters: rows with no selected key
    cluster (their queries get dQ = 0 and give nothing to any key), key
    clusters no row selects (their keys get dK = dV = 0), a row selecting
    every cluster, and single selections; element by element against the
    oracle, zeros exactly."""
    w = replace(WAN_S.forced_density(0.1), compensate=False, name="wan_small_edges")
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, qc, kc, sc, ac)
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster_qk(p, qc, kc, q, k, qt, kt, ws)
    Cq, Ck = qt.num_clusters, kt.num_clusters
    v_perm = torch.empty_like(v)
    L.sa_permute(p, kt, v, v_perm, None)
    rng = np.random.default_rng(5)
    gm = rng.random((w.heads, Cq, Ck)) < 0.15
    gm[:, ::7, :] = False          # rows with no key
    gm[:, :, ::5] = False          # key clusters nobody selects
    gm[:, 3, :] = True             # a row with every cluster
    gm[:, 3, ::5] = False
    gm[:, 5, :] = False
    gm[:, 5, 1] = True             # a single selection
    mask = torch.tensor(pack_mask(gm), device=DEV)
    o = torch.empty_like(q)
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, None, mask, o, ws)
    d_o = torch.randn(q.shape, generator=torch.Generator(device="cpu").manual_seed(3)).to(torch.bfloat16).to(DEV)
    wsb = L.workspace(L.sa_block_sparse_attn_bwd_workspace_size(p, Cq, Ck), DEV)
    grads = [torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV) for _ in range(3)]
    L.sa_block_sparse_attn_bwd(p, ac, qt, kt, v_perm, mask, o, d_o, *grads, wsb)
    torch.cuda.synchronize()
    qs, ks, vs, gs = to_np(q), to_np(k), to_np(v), to_np(d_o)
    bad = []
    for h in range(w.heads):
        qperm, qoff = qt.perm[h].cpu().numpy(), qt.offsets[h].cpu().numpy()
        kperm, koff = kt.perm[h].cpu().numpy(), kt.offsets[h].cpu().numpy()
        ref = oracle.attention_backward(qs[h], ks[h], vs[h], qperm, qoff, kperm, koff, gm[h], scale_of(w), gs[h])
        empty_rows = np.concatenate([qperm[qoff[i]:qoff[i + 1]] for i in range(Cq) if not gm[h, i].any()])
        unused = np.concatenate([kperm[koff[j]:koff[j + 1]] for j in range(Ck) if not gm[h, :, j].any()])
        got = [x[h].double().cpu().numpy() for x in grads]
        assert np.all(got[0][empty_rows] == 0.0), "dQ of queries with no key"
        assert np.all(got[1][unused] == 0.0) and np.all(got[2][unused] == 0.0), "dK, dV of unselected keys"
        for name, g_, want in zip(("dq", "dk", "dv"), got, ref):
            assert np.isfinite(g_).all(), name
            err = np.abs(g_ - want)
            mx, mean = float(err.max()), float(err.mean())
            rmax, rmean = float(np.abs(want).max()), float(np.abs(want).mean())
            say(f"  head {h} {name}: max {mx / rmax:.2e} of max, mean {mean / rmean:.2e} of mean")
            tol_max, tol_mean = TOL[name]
            if not (mx <= tol_max * rmax and mean <= tol_mean * rmean):
                bad.append((h, name, mx / rmax, mean / rmean))
    assert not bad, bad


LSE_CASES = [replace(wl.TINY, name="tiny_f32"),
             replace(wl.TINY, compensate=True, name="tiny_f32_comp"),
             replace(WAN_S.forced_density(0.1), compensate=False, name="wan_small_fixed"),
             replace(WAN_S.forced_density(0.1), name="wan_small_fixed_comp"),
             replace(TAB_S.forced_density(0.1), name="tab_small_d64_comp"),
             replace(WAN_S, compensate=False, name="wan_small_p09")]


@pytest.mark.parametrize("w", LSE_CASES, ids=lambda w: w.name)
def test_forward_lse_and_backward_given_lse(w):
    """The forward's log-sum-exp output against oracle.attention_lse given the
    GPU's clusters, mask and means (absolute, in the log domain: the kernel's
    denominator adds bf16-rounded probabilities, up to 2^-9 relative each, so
    at most 2^-8 ~ 4e-3 on any query, and 2^-10 ~ 1e-3 on average, the mean
    rounding error when one key dominates the sum); then, without compensation,
    the backward taking it in place of its own pass: the oracle bounds of the
    other cases, and the recomputing backward within the same bounds.  The
    fp32 path (no rounded probabilities) to 1e-5."""
    say(f"[lse] {w.name} H={w.heads} N={w.n} d={w.d} comp={w.compensate}")
    q, k, v = inputs(w)
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
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, None, ktop, ws)
    o = torch.empty_like(q)
    lse = torch.full((w.heads, w.n), float("nan"), dtype=torch.float32, device=DEV)
    L.sa_block_sparse_attn(p, L.attn_cfg(w.compensate, 0.0, lse=lse), qt, kt, v_perm, vbar, mask, o, ws)
    o_plain = torch.empty_like(q)
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, vbar, mask, o_plain, ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain), "the log-sum-exp output changes nothing else"
    gm = unpack_mask(mask, Ck)
    qs, ks = to_np(q), to_np(k)
    for h in range(w.heads):
        kb = kt.centroids[h].double().cpu().numpy() if w.compensate else None
        ref = oracle.attention_lse(qs[h], ks[h], qt.perm[h].cpu().numpy(), qt.offsets[h].cpu().numpy(),
                                   kt.perm[h].cpu().numpy(), kt.offsets[h].cpu().numpy(), gm[h], scale_of(w),
                                   w.compensate, kb)
        got = lse[h].double().cpu().numpy()
        err = np.abs(got - ref)
        say(f"  head {h}: lse max-abs {err.max():.2e} mean-abs {err.mean():.2e} (range {ref.min():.2f}..{ref.max():.2f})")
        if w.dtype == "f32":  # fp32 path: no rounding of the probabilities
            assert np.isfinite(got).all() and err.max() <= 1e-5
        else:
            assert np.isfinite(got).all() and err.max() <= 4e-3 and err.mean() <= 1e-3
    if w.compensate or w.dtype != "bf16":  # the backward is bf16 without compensation
        return
    d_o = torch.randn(q.shape, generator=torch.Generator(device="cpu").manual_seed(9)).to(torch.bfloat16).to(DEV)
    wsb = L.workspace(L.sa_block_sparse_attn_bwd_workspace_size(p, Cq, Ck), DEV)
    given = [torch.full(q.shape, float("nan"), dtype=torch.float32, device=DEV) for _ in range(3)]
    L.sa_block_sparse_attn_bwd(p, ac, qt, kt, v_perm, mask, o, d_o, *given, wsb, lse=lse)
    recomp = [torch.empty_like(x) for x in given]
    L.sa_block_sparse_attn_bwd(p, ac, qt, kt, v_perm, mask, o, d_o, *recomp, wsb)
    torch.cuda.synchronize()
    vs, gs = to_np(v), to_np(d_o)
    bad = []
    for h in range(w.heads):
        ref = oracle.attention_backward(qs[h], ks[h], vs[h], qt.perm[h].cpu().numpy(), qt.offsets[h].cpu().numpy(),
                                        kt.perm[h].cpu().numpy(), kt.offsets[h].cpu().numpy(), gm[h], scale_of(w),
                                        gs[h])
        for name, g_, r_, want in zip(("dq", "dk", "dv"), given, recomp, ref):
            g_ = g_[h].double().cpu().numpy()
            r_ = r_[h].double().cpu().numpy()
            assert np.isfinite(g_).all(), name
            rmax, rmean = float(np.abs(want).max()), float(np.abs(want).mean())
            tol_max, tol_mean = TOL[name]
            for label, x in (("oracle", want), ("recomputing backward", r_)):
                err = np.abs(g_ - x)
                mx, mean = float(err.max()), float(err.mean())
                say(f"  head {h} {name} vs {label}: max {mx / rmax:.2e} of max, mean {mean / rmean:.2e} of mean")
                if not (mx <= tol_max * rmax and mean <= tol_mean * rmean):
                    bad.append((h, name, label, mx / rmax, mean / rmean))
    assert not bad, bad
