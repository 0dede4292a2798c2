"""Pins of the oracle's proxy scores and selection (CPU only).

Top-p / floor are pinned to brute force over all subsets; the online per-head
Top-k to closed forms and a hand-derived worked example stored in
tests/golden/; the centroid scores to bilinearity (pairwise brute force) and
to the per-key proxy softmax they stand for; the lookup table to the direct
dot product with the concatenated representative."""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_min_size_reaching(p, P):
    """Smallest t such that some t-subset has mass >= P, and that max mass."""
    Ck = len(p)
    for t in range(0, Ck + 1):
        best = max((sum(p[list(S)]) for S in itertools.combinations(range(Ck), t)), default=0.0)
        if best >= P:
            return t, best
    return Ck, sum(p)


@pytest.mark.parametrize("seed", range(12))
def test_top_p_floor_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    Ck = int(rng.integers(2, 11))
    logits = rng.normal(size=(3, Ck)) * rng.uniform(0.5, 3)
    P = float(rng.uniform(0.05, 0.99))
    floor = int(rng.integers(0, Ck + 1))
    r = oracle.select(logits, np.ones(Ck, np.int64), np.array([5, 3, 2]), P, floor, False)
    for i in range(3):
        p = np.exp(logits[i] - logits[i].max())
        p /= p.sum()
        t_star, best = brute_min_size_reaching(p, P)
        t = max(t_star, floor)
        assert r["n_init"][i] == t == r["mask"][i].sum()
        sel_mass = p[r["mask"][i]].sum()
        if t == t_star:
            assert abs(sel_mass - best) < 1e-12
        # invariants: mass >= P, count >= floor, minimality
        assert sel_mass >= P - 1e-12 and r["mask"][i].sum() >= floor
        if t > max(floor, 1):
            # dropping the lowest-ranked selected unit loses the mass target
            low = min(np.nonzero(r["mask"][i])[0], key=lambda j: (p[j], -j))
            assert sel_mass - p[low] < P


def test_top_p_edges():
    logits = np.log(np.array([[0.5, 0.25, 0.125, 0.125]]))
    one = np.ones(4, np.int64)
    assert oracle.select(logits, one, [4], 1.0, 0, False)["mask"].sum() == 4
    assert oracle.select(logits, one, [4], 0.0, 3, False)["mask"].sum() == 3
    with pytest.raises(ValueError):
        oracle.select(logits, one, [4], 0.0, 0, False)
    # empty unit never selected even at P = 1
    lg = logits.copy()
    lg[0, 2] = -np.inf
    m = oracle.select(lg, one, [4], 1.0, 0, False)["mask"]
    assert m.sum() == 3 and not m[0, 2]


def test_empty_query_cluster_selects_nothing():
    logits = np.log(np.array([[0.5, 0.3, 0.2], [0.2, 0.3, 0.5]]))
    r = oracle.select(logits, np.ones(3, np.int64), [0, 7], 0.6, 1, True)
    assert r["mask"][0].sum() == 0 and r["n_final"][0] == 0
    assert r["mask"][1].tolist() == [False, True, True] and r["k_h"] == 2


def test_ties_rank_lower_index_first():
    logits = np.zeros((1, 5))
    r = oracle.select(logits, np.ones(5, np.int64), [1], 0.39, 0, False)
    assert r["mask"][0].tolist() == [True, True, False, False, False]
    assert r["near_tie"][0]


def test_golden_worked_example():
    with open(os.path.join(GOLDEN, "select_worked_example.json")) as f:
        g = json.load(f)
    logits = np.log(np.array(g["masses"], dtype=np.float64))
    for case in g["cases"]:
        r = oracle.select(logits, np.array(g["units"]), np.array(case["query_cluster_sizes"]),
                          g["top_p"], case["floor"], True)
        assert r["n_init"].tolist() == case["expected_initial_counts"]
        assert r["k_h"] == case["expected_head_topk"]
        assert r["n_final"].tolist() == case["expected_final_counts"]
        assert r["mask"].astype(int).tolist() == case["expected_mask"]


def test_online_topk_closed_forms(rng):
    Cq, Ck = 6, 9
    logits = rng.normal(size=(Cq, Ck)) * 2
    qs = rng.integers(1, 50, size=Cq)
    one = np.ones(Ck, np.int64)
    r0 = oracle.select(logits, one, qs, 0.6, 1, False)
    r1 = oracle.select(logits, one, qs, 0.6, 1, True)
    A = int((qs * r0["n_init"]).sum())
    assert r1["k_h"] == math.ceil(A / qs.sum())
    for i in range(Cq):
        if r0["n_init"][i] >= r1["k_h"]:
            assert np.array_equal(r1["mask"][i], r0["mask"][i])
        else:
            assert r1["n_final"][i] == r1["k_h"]
            assert np.all(r1["mask"][i] >= r0["mask"][i])  # extension keeps the initial set
    # equal initial counts: k_h equals them and nothing changes
    eq = np.tile(np.log(np.array([0.7, 0.2, 0.1])), (4, 1))
    r2 = oracle.select(eq, np.ones(3, np.int64), [3, 1, 4, 1], 0.65, 0, True)
    assert r2["k_h"] == 1 and np.array_equal(r2["n_final"], r2["n_init"])


def test_subspace_units_count_keys():
    # units are keys per combo: floor counted in keys, Top-k in keys
    logits = np.log(np.array([[0.4, 0.3, 0.2, 0.1]]))
    units = np.array([1, 5, 2, 7])
    r = oracle.select(logits, units, [10], 0.3, 4, False)
    # mass reaches 0.3 after 1 unit (1 key), floor of 4 keys needs unit 1 too (6 keys)
    assert r["n_init"][0] == 6 and r["mask"][0].tolist() == [True, True, False, False]


# --------------------------------------------------------------------------
# proxy scores
# --------------------------------------------------------------------------

def test_centroid_score_is_mean_pairwise_dot(rng):
    """<qbar_i, kbar_j> equals the mean of <q_a, k_b> over all member pairs."""
    q = rng.normal(size=(30, 5))
    k = rng.normal(size=(40, 5))
    ql = rng.integers(0, 3, size=30)
    kl = rng.integers(0, 4, size=40)
    qp, qo = oracle.permute(ql, 3)
    kp, ko = oracle.permute(kl, 4)
    qbar = oracle.cluster_means(q, qp, qo)
    kbar = oracle.cluster_means(k, kp, ko)
    scale = 0.37
    s = oracle.cluster_logits(qbar, kbar, np.diff(ko), scale, size_weighted=False)
    for i in range(3):
        for j in range(4):
            pairs = [float(np.dot(q[a], k[b])) for a in np.nonzero(ql == i)[0] for b in np.nonzero(kl == j)[0]]
            assert abs(s[i, j] - scale * np.mean(pairs)) < 1e-12


def test_size_weighted_softmax_is_per_key_softmax(rng):
    """softmax_j(l_ij) with l = s + ln|K_j| equals the softmax over per-key
    proxy scores (each key carrying its cluster's score), summed per cluster."""
    qbar = rng.normal(size=(2, 4))
    kbar = rng.normal(size=(5, 4))
    sizes = np.array([3, 1, 0, 7, 2])
    lw = oracle.cluster_logits(qbar, kbar, sizes, 0.5, True)
    lu = oracle.cluster_logits(qbar, kbar, sizes, 0.5, False)
    for i in range(2):
        per_key = np.concatenate([[lu[i, j]] * sizes[j] for j in range(5)])
        owner = np.concatenate([[j] * sizes[j] for j in range(5)])
        pk = np.exp(per_key - per_key.max())
        pk /= pk.sum()
        agg = np.array([pk[owner == j].sum() for j in range(5)])
        valid = np.isfinite(lw[i])
        pw = np.zeros(5)
        pw[valid] = np.exp(lw[i, valid] - lw[i, valid].max())
        pw /= pw.sum()
        np.testing.assert_allclose(pw, agg, atol=1e-14)
        assert not np.isfinite(lw[i, 2])


def test_lut_equals_concatenated_representative(rng):
    dims = (2, 3, 3)
    Cs = 3
    sub = [rng.normal(size=(Cs, ds)) for ds in dims]
    qbar = rng.normal(size=(4, 8))
    sizes = rng.integers(0, 3, size=Cs ** 3)
    lut = oracle.subspace_logits(qbar, sub, dims, sizes, 0.25, True)
    for g in range(Cs ** 3):
        a_t, a_h, a_w = g // (Cs * Cs), (g // Cs) % Cs, g % Cs
        rep = np.concatenate([sub[0][a_t], sub[1][a_h], sub[2][a_w]])
        for i in range(4):
            if sizes[g] == 0:
                assert lut[i, g] == -np.inf
            else:
                assert abs(lut[i, g] - (0.25 * np.dot(qbar[i], rep) + math.log(sizes[g]))) < 1e-12


def test_near_tie_cut_ranges():
    """A cut inside a run of equal logits is flagged and its range covers
    every equal unit; a cut with a clear gap is exact (range = the cut)."""
    one = np.ones(5, np.int64)
    # units 1 and 3 share a logit across the floor-2 cut: either may be second
    lg = np.log(np.array([[0.4, 0.2, 0.1, 0.2, 0.1]]))
    r = oracle.select(lg, one, [3], 0.0, 2, False)
    assert r["near_tie"][0] and r["t_final"][0] == 2
    assert r["cut_lo"][0] == 1 and r["cut_hi"][0] == 3
    assert set(r["orders"][0][:3].tolist()) == {0, 1, 3}
    # a clear gap at the cut
    lg2 = np.log(np.array([[0.4, 0.3, 0.1, 0.15, 0.05]]))
    r2 = oracle.select(lg2, one, [3], 0.0, 2, False)
    assert not r2["near_tie"][0] and r2["cut_lo"][0] == r2["cut_hi"][0] == 2
    # Top-p crossing exactly at a prefix mass (0.4 + 0.3 = 0.7 with P = 0.7):
    # an evaluation in another order may need one unit more
    r3 = oracle.select(np.log(np.array([[0.4, 0.3, 0.2, 0.1]])), np.ones(4, np.int64), [3], 0.7, 1, False)
    assert r3["near_tie"][0] and r3["t_final"][0] == 2 and (r3["cut_lo"][0], r3["cut_hi"][0]) == (2, 3)


def test_given_head_topk():
    """select(..., k_h=k) runs the online extension with k instead of its own
    estimate: rows below k extend to k, the others are unchanged."""
    rng = np.random.default_rng(5)
    lg = rng.normal(size=(6, 12))
    qs = np.array([5, 9, 3, 7, 2, 8])
    own = oracle.select(lg, np.ones(12, np.int64), qs, 0.5, 1, True)
    for k in (own["k_h"], own["k_h"] + 2, 1):
        r = oracle.select(lg, np.ones(12, np.int64), qs, 0.5, 1, True, k_h=k)
        assert r["k_h"] == k
        assert np.array_equal(r["n_init"], own["n_init"])
        assert np.array_equal(r["n_final"], np.maximum(own["n_init"], k))


def test_stat_threshold_worked_example():
    """Hand-derived: p = (1/2, 1/4, 1/8, 1/8) has mean 1/4 and population
    variance ((1/4)^2 + 0 + 2 (1/8)^2) / 4 = 3/128, std 0.1530931...; the
    threshold keeps p >= 1/4 + lam * 0.1530931: lam = 1 -> 0.4031 -> 1 unit,
    lam = 0 -> 1/4 -> 2 units (1/4 itself is kept), lam = -1 -> 0.0969 ->
    4 units; a floor of 3 raises the first to 3."""
    p = np.array([0.5, 0.25, 0.125, 0.125])
    lg = np.log(p)[None]
    one = np.ones(4, np.int64)
    assert math.isclose(oracle.stat_threshold(p, 1.0), 0.25 + math.sqrt(3 / 128), rel_tol=1e-15)
    for lam, want in ((1.0, 1), (-1.0, 4), (2.0, 1)):
        r = oracle.select(lg, one, [5], 0.9, 1, False, stat_lambda=lam)
        assert r["n_init"][0] == want and not r["near_tie"][0]
    r0 = oracle.select(lg, one, [5], 0.9, 1, False, stat_lambda=0.0)
    # 1/4 sits exactly on the threshold: kept, and flagged as a tie at the cut
    assert r0["n_init"][0] == 2 and r0["near_tie"][0] and (r0["cut_lo"][0], r0["cut_hi"][0]) == (1, 2)
    assert oracle.select(lg, one, [5], 0.9, 3, False, stat_lambda=1.0)["n_init"][0] == 3
    # a uniform row: every unit equals the mean, the std is 0 -> all kept
    assert oracle.select(np.zeros((1, 6)), np.ones(6, np.int64), [2], 0.9, 1, False, stat_lambda=1.0)["n_init"][0] == 6


def test_stat_threshold_keeps_an_upper_set(rng):
    """The kept units are exactly those at or above the threshold, which is a
    prefix of the probability ranking; the threshold ignores top_p; online
    Top-k extends the rows below k_h as with Top-p."""
    for trial in range(10):
        Ck = int(rng.integers(3, 30))
        lg = rng.normal(size=(4, Ck)) * rng.uniform(0.5, 3)
        lg[rng.random(size=lg.shape) < 0.1] = -np.inf
        lg[:, 0] = 0.0
        lam = float(rng.uniform(-1, 2))
        qs = rng.integers(1, 9, size=4)
        r = oracle.select(lg, np.ones(Ck, np.int64), qs, float(rng.uniform(0.1, 0.9)), 1, True, stat_lambda=lam)
        r2 = oracle.select(lg, np.ones(Ck, np.int64), qs, 0.5, 1, True, stat_lambda=lam)
        assert np.array_equal(r["mask"], r2["mask"])
        for i in range(4):
            v = np.isfinite(lg[i])
            p = np.zeros(Ck)
            e = np.exp(lg[i][v] - lg[i][v].max())
            p[v] = e / e.sum()
            th = p[v].mean() + lam * p[v].std()
            kept = max(int((p[v] >= th).sum()), 1)
            assert r["n_init"][i] == kept
            assert r["n_final"][i] == max(kept, min(r["k_h"], int(v.sum())))
