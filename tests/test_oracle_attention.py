"""Pins of the oracle's attention step and of the whole per-head path (CPU).

Pinned to scalar brute force of softmax attention, to the token-mask form of
block sparsity, to the sparse-attention error identity, and to the exactness
conditions of mean compensation."""

import math

import numpy as np
import pytest

import oracle


def brute_attention(q, k, v, scale, allowed=None):
    """Scalar loops: softmax over the allowed keys of each query."""
    N = len(q)
    out = np.zeros((N, v.shape[1]))
    for n in range(N):
        keys = range(len(k)) if allowed is None else allowed[n]
        s = [scale * sum(q[n][t] * k[m][t] for t in range(q.shape[1])) for m in keys]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        z = sum(w)
        for wi, m in zip(w, keys):
            out[n] += wi / z * v[m]
    return out


def setup(rng, N=40, M=36, d=4, Cq=4, Ck=6):
    q = rng.normal(size=(N, d))
    k = rng.normal(size=(M, d))
    v = rng.normal(size=(M, d))
    ql = rng.integers(0, Cq, size=N)
    kl = rng.integers(0, Ck, size=M)
    kl[kl == 2] = 3  # key cluster 2 empty
    qp, qo = oracle.permute(ql, Cq)
    kp, ko = oracle.permute(kl, Ck)
    return q, k, v, ql, kl, qp, qo, kp, ko


def test_all_selected_is_dense(rng):
    q, k, v, ql, kl, qp, qo, kp, ko = setup(rng)
    mask = np.ones((4, 6), dtype=bool)
    O = oracle.attention(q, k, v, qp, qo, kp, ko, mask, 0.4)
    np.testing.assert_allclose(O, brute_attention(q, k, v, 0.4), atol=1e-12)


def test_mask_equals_token_mask(rng):
    q, k, v, ql, kl, qp, qo, kp, ko = setup(rng)
    mask = rng.random((4, 6)) < 0.5
    mask[:, 0] = True
    O = oracle.attention(q, k, v, qp, qo, kp, ko, mask, 0.4)
    allowed = [[m for m in range(len(k)) if mask[ql[n], kl[m]]] for n in range(len(q))]
    np.testing.assert_allclose(O, brute_attention(q, k, v, 0.4, allowed), atol=1e-12)


def test_sparse_error_identity(rng):
    """O_sparse - O_dense = (1 - m) (O_sel - O_excl), m = true attention mass
    on the selected keys (derived for the ClusterAttention error analysis)."""
    q, k, v, ql, kl, qp, qo, kp, ko = setup(rng)
    mask = rng.random((4, 6)) < 0.5
    mask[:, 1] = True
    mask[:, 4] = False
    scale = 0.4
    Os = oracle.attention(q, k, v, qp, qo, kp, ko, mask, scale)
    Od = oracle.dense_attention(q, k, v, scale)
    Oe = oracle.attention(q, k, v, qp, qo, kp, ko, ~mask, scale)
    s = q @ k.T * scale
    for n in range(len(q)):
        w = np.exp(s[n] - s[n].max())
        w /= w.sum()
        sel = mask[ql[n], kl]
        m = w[sel].sum()
        np.testing.assert_allclose(Os[n] - Od[n], (1 - m) * (Os[n] - Oe[n]), atol=1e-12)


def test_compensation_exact_for_identical_keys(rng):
    """An excluded cluster whose keys are all equal is reproduced exactly by
    |K_j| copies of (kbar_j, vbar_j), whatever its values."""
    q, k, v, ql, kl, qp, qo, kp, ko = setup(rng)
    for j in range(6):
        members = kp[ko[j]:ko[j + 1]]
        if len(members):
            k[members] = rng.normal(size=4)
    mask = rng.random((4, 6)) < 0.4
    mask[:, 0] = True
    kbar = oracle.cluster_means(k, kp, ko)
    vbar = oracle.cluster_means(v, kp, ko)
    O = oracle.attention(q, k, v, qp, qo, kp, ko, mask, 0.4, True, kbar, vbar)
    np.testing.assert_allclose(O, oracle.dense_attention(q, k, v, 0.4), atol=1e-12)


def test_compensation_jensen_and_noop(rng):
    q, k, v, ql, kl, qp, qo, kp, ko = setup(rng)
    scale = 0.6
    kbar = oracle.cluster_means(k, kp, ko)
    vbar = oracle.cluster_means(v, kp, ko)
    # nothing excluded: compensation changes nothing (empty cluster aside)
    full = np.ones((4, 6), dtype=bool)
    np.testing.assert_allclose(
        oracle.attention(q, k, v, qp, qo, kp, ko, full, scale, True, kbar, vbar),
        oracle.attention(q, k, v, qp, qo, kp, ko, full, scale), atol=1e-14)
    # Jensen: |K_j| e^{<q, kbar_j>} <= sum_{m in K_j} e^{<q, k_m>}
    for j in range(6):
        members = kp[ko[j]:ko[j + 1]]
        if len(members) == 0:
            continue
        for n in range(len(q)):
            comp = len(members) * math.exp(scale * q[n] @ kbar[j])
            true = sum(math.exp(scale * q[n] @ k[m]) for m in members)
            assert comp <= true * (1 + 1e-12)


@pytest.mark.parametrize("method", ["kmeans", "bisect"])
def test_forward_all_selected_is_dense(rng, method):
    """The whole path with every cluster selected is dense attention, whatever
    the clustering (the permutations and unpermute are exact)."""
    N, d = 96, 8
    q = rng.normal(size=(N, d))
    k = rng.normal(size=(N, d))
    v = rng.normal(size=(N, d))
    cfg = oracle.ClusterCfg(method=method, clusters=5, leaf=16, iters=3)
    r = oracle.forward_head(q, k, v, cfg, cfg, oracle.SelectCfg(top_p=1.0, floor=0))
    np.testing.assert_allclose(r.O, oracle.dense_attention(q, k, v, 1 / math.sqrt(d)), atol=1e-12)


def test_forward_subspace_all_selected_is_dense(rng):
    N, d = 80, 8
    q = rng.normal(size=(N, d))
    k = rng.normal(size=(N, d))
    v = rng.normal(size=(N, d))
    qc = oracle.ClusterCfg(method="bisect", leaf=16, iters=2)
    kc = oracle.ClusterCfg(method="subspace", iters=2, sub_dims=(2, 3, 3), sub_clusters=3)
    r = oracle.forward_head(q, k, v, qc, kc, oracle.SelectCfg(top_p=1.0, floor=0))
    np.testing.assert_allclose(r.O, oracle.dense_attention(q, k, v, 1 / math.sqrt(d)), atol=1e-12)


def brute_lse(q, k, scale, allowed, extra=None):
    """Scalar loops: log of the sum of exp(score) over the allowed keys of
    each query, plus the given (log-weight) extra terms."""
    out = []
    for n in range(len(q)):
        terms = [scale * sum(q[n][t] * k[m][t] for t in range(q.shape[1])) for m in allowed[n]]
        if extra is not None:
            terms += list(extra[n])
        if not terms:
            out.append(-math.inf)
            continue
        mx = max(terms)
        out.append(mx + math.log(sum(math.exp(x - mx) for x in terms)))
    return np.array(out)


def test_lse_brute_force(rng):
    """Without compensation: the log-sum-exp over each query's selected keys,
    by scalar loops; a query cluster with no selection gets -inf."""
    q, k, v, ql, kl, qp, qo, kp, ko = setup(rng)
    mask = rng.random((4, 6)) < 0.5
    mask[1] = False
    allowed = [[m for m in range(len(k)) if mask[ql[n], kl[m]]] for n in range(len(q))]
    got = oracle.attention_lse(q, k, qp, qo, kp, ko, mask, 0.7)
    want = brute_lse(q, k, 0.7, allowed)
    assert np.all(np.isneginf(got[ql == 1])) and np.all(np.isneginf(want[ql == 1]))
    fin = ql != 1
    assert np.allclose(got[fin], want[fin], rtol=0, atol=1e-12)


def test_lse_compensated_brute_force(rng):
    """With compensation: each excluded non-empty key cluster adds
    log|K_j| + <q, kbar_j> scale as one term (empty clusters add nothing)."""
    q, k, v, ql, kl, qp, qo, kp, ko = setup(rng)
    mask = rng.random((4, 6)) < 0.4
    mask[2] = False  # a row with every cluster excluded: compensation terms only
    kbar = oracle.cluster_means(k, kp, ko)
    ksz = np.diff(ko)
    allowed = [[m for m in range(len(k)) if mask[ql[n], kl[m]]] for n in range(len(q))]
    extra = [[math.log(ksz[j]) + 0.5 * float(np.dot(q[n], kbar[j])) for j in range(6)
              if not mask[ql[n], j] and ksz[j] > 0] for n in range(len(q))]
    got = oracle.attention_lse(q, k, qp, qo, kp, ko, mask, 0.5, True, kbar)
    assert np.allclose(got, brute_lse(q, k, 0.5, allowed, extra), rtol=0, atol=1e-12)


def test_lse_weights_reproduce_attention(rng):
    """The weights e^{s - lse} (and |K_j| e^{<q,kbar_j> scale - lse} for the
    compensated clusters) sum to one and give the attention output."""
    q, k, v, ql, kl, qp, qo, kp, ko = setup(rng)
    mask = rng.random((4, 6)) < 0.5
    mask[:, 0] = True
    kbar, vbar = oracle.cluster_means(k, kp, ko), oracle.cluster_means(v, kp, ko)
    ksz = np.diff(ko)
    for comp in (False, True):
        lse = oracle.attention_lse(q, k, qp, qo, kp, ko, mask, 0.6, comp, kbar)
        O = oracle.attention(q, k, v, qp, qo, kp, ko, mask, 0.6, comp, kbar, vbar)
        for n in range(len(q)):
            sel = [m for m in range(len(k)) if mask[ql[n], kl[m]]]
            w = np.exp(0.6 * (k[sel] @ q[n]) - lse[n])
            tot, acc = w.sum(), w @ v[sel]
            if comp:
                ex = [j for j in range(6) if not mask[ql[n], j] and ksz[j] > 0]
                wc = ksz[ex] * np.exp(0.6 * (kbar[ex] @ q[n]) - lse[n])
                tot, acc = tot + wc.sum(), acc + wc @ vbar[ex]
            assert abs(tot - 1.0) <= 1e-12
            assert np.allclose(acc, O[n], rtol=0, atol=1e-12)
