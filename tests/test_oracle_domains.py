"""Pins of the oracle's competition domains (CPU only): the entropy that
gates heads, pooled Top-p over a head or a group of heads (VMoBA global
block selection, EG-Sparse grouped cross-head pools) and the routing of heads
to pools.

Pinned by a hand-derived worked example (tests/golden/domains_worked_example.json),
closed forms of the entropy, brute-force optimality of the pooled cut on
equal query clusters (the largest probabilities first reach a mass target
with the fewest pairs), reductions to the per-row rule (a pool of one row;
no low-entropy head) and invariants (mass reached, minimality, an upper set
of the ranking, a prefix of every row's own ranking)."""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example():
    with open(os.path.join(GOLDEN, "domains_worked_example.json")) as f:
        g = json.load(f)
    lg = np.log(np.array(g["probs"]))
    qs = np.array(g["query_cluster_sizes"])
    ones = np.ones(lg.shape[1], np.int64)
    assert math.isclose(oracle.head_entropy(lg, qs), g["expected_head_entropy"], rel_tol=0, abs_tol=1e-14)
    for r, want in enumerate(g["expected_row_entropies"]):
        assert math.isclose(oracle.head_entropy(lg[r:r + 1], [1]), want, rel_tol=0, abs_tol=1e-14)
    for case in g["cases"]:
        pc = oracle.pool_counts(lg[None], qs[None], [0], case["top_p"])[0]
        assert pc["count"].tolist() == case["expected_counts"]
        r = oracle.select_domains(lg[None], ones, qs[None], case["top_p"], 1, False, oracle.DOMAIN_HEAD)
        assert r["heads"][0]["mask"].astype(int).tolist() == case["expected_mask"]
        local = oracle.select(lg, ones, qs, case["top_p"], 1, False)
        assert local["n_init"].tolist() == case["per_row_counts"]


def test_entropy_closed_forms():
    # uniform rows: 1; a single non-empty unit: 0; a two-point law
    assert math.isclose(oracle.head_entropy(np.zeros((3, 7)), [1, 2, 3]), 1.0, abs_tol=1e-15)
    one = np.full((2, 4), -np.inf)
    one[:, 2] = 0.0
    assert oracle.head_entropy(one, [5, 5]) == 0.0
    p = 0.75
    want = -(p * math.log(p) + (1 - p) * math.log(1 - p)) / math.log(2)
    assert math.isclose(oracle.head_entropy(np.log([[p, 1 - p]]), [4]), want, abs_tol=1e-15)
    # query-size weighting: an empty query cluster does not count
    lg = np.log(np.array([[0.5, 0.5], [0.9, 0.1]]))
    assert math.isclose(oracle.head_entropy(lg, [3, 0]), 1.0, abs_tol=1e-15)


def test_pool_of_one_row_is_the_row_rule(rng):
    for _ in range(10):
        Ck = int(rng.integers(2, 9))
        lg = rng.normal(size=(1, Ck)) * 2
        P = float(rng.uniform(0.1, 0.99))
        pc = oracle.pool_counts(lg[None], np.array([[7]]), [0], P)[0]
        local = oracle.select(lg, np.ones(Ck, np.int64), [7], P, 0 if P > 0 else 1, False)
        assert pc["count"][0] == local["t_init"][0]


@pytest.mark.parametrize("seed", range(8))
def test_pooled_cut_is_a_minimum_cardinality_set(seed):
    """With equal query clusters the pair masses are proportional to p, and
    taking the largest first reaches a mass target with the fewest pairs:
    brute force over every subset of a pool of two heads of 2 x 3 pairs."""
    rng = np.random.default_rng(40 + seed)
    lg = rng.normal(size=(2, 2, 3)) * 1.5
    qs = np.full((2, 2), 4)
    P = float(rng.uniform(0.2, 0.95))
    pc = oracle.pool_counts(lg, qs, [0, 1], P)
    got = sum(int(pc[h]["count"].sum()) for h in (0, 1))
    probs = np.stack([oracle.proxy_probs(lg[h]) for h in (0, 1)])
    mass = (probs * 4 / 8).reshape(-1)  # |Q_i| p / N per pair, N = 8 per head
    target = P * 2
    best = min(len(S) for t in range(0, 13) for S in itertools.combinations(range(12), t)
               if mass[list(S)].sum() >= target - 1e-12)
    assert got == best


def test_pool_invariants(rng):
    for _ in range(20):
        H, Cq, Ck = 3, int(rng.integers(1, 5)), int(rng.integers(2, 7))
        lg = rng.normal(size=(H, Cq, Ck)) * 2
        lg[rng.random(size=lg.shape) < 0.15] = -np.inf
        lg[:, :, 0] = np.where(np.isfinite(lg[:, :, 0]), lg[:, :, 0], 0.0)  # a non-empty unit per row
        qs = rng.integers(0, 6, size=(H, Cq))
        qs[:, 0] = np.maximum(qs[:, 0], 1)
        P = float(rng.uniform(0.05, 0.99))
        heads = [0, 2]
        pc = oracle.pool_counts(lg, qs, heads, P)
        sel, rest, mass = [], [], 0.0
        for h in heads:
            pr = oracle.proxy_probs(lg[h])
            N = qs[h].sum()
            for i in range(Cq):
                order = np.lexsort((np.arange(Ck), -pr[i]))
                order = order[pr[i][order] > 0]
                c = pc[h]["count"][i]
                assert c == 0 or qs[h][i] > 0
                for k, j in enumerate(order):
                    if qs[h][i] == 0:
                        continue
                    (sel if k < c else rest).append((pr[i, j], qs[h][i] * pr[i, j] / N))
        mass = sum(m for _, m in sel)
        assert mass >= P * len(heads) - 1e-12                      # reaches the target
        if sel:
            low = min(p for p, _ in sel)
            assert all(p <= low + 1e-15 for p, _ in rest)            # an upper set of the ranking
            drop = min(sel, key=lambda t: t[0])
            assert mass - drop[1] < P * len(heads) + 1e-12           # minimal


def test_domain_routing_reductions(rng):
    H, Cq, Ck = 4, 5, 6
    lg = rng.normal(size=(H, Cq, Ck)) * np.array([0.3, 3.0, 0.5, 4.0])[:, None, None]
    qs = rng.integers(1, 9, size=(H, Cq))
    one = np.ones(Ck, np.int64)
    row = oracle.select_domains(lg, one, qs, 0.8, 1, False, oracle.DOMAIN_ROW)
    # no head below the threshold: every head selects per row
    none = oracle.select_domains(lg, one, qs, 0.8, 1, False, oracle.DOMAIN_GROUP, 2, 0.0)
    assert none["pools"] == []
    for h in range(H):
        assert np.array_equal(row["heads"][h]["mask"], none["heads"][h]["mask"])
        assert np.array_equal(row["heads"][h]["mask"], oracle.select(lg[h], one, qs[h], 0.8, 1, False)["mask"])
    # every head below the threshold, groups of one: the head-global rule
    glob = oracle.select_domains(lg, one, qs, 0.8, 1, False, oracle.DOMAIN_HEAD)
    g1 = oracle.select_domains(lg, one, qs, 0.8, 1, False, oracle.DOMAIN_GROUP, 1, 2.0)
    assert glob["pools"] == g1["pools"] == [[0], [1], [2], [3]]
    for h in range(H):
        assert np.array_equal(glob["heads"][h]["mask"], g1["heads"][h]["mask"])
    # groups of two with a threshold between the heads' entropies: the
    # low-entropy heads of each group share a pool, the others select per row
    ent = row["entropy"]
    tau = float(np.sort(ent)[2])
    grp = oracle.select_domains(lg, one, qs, 0.8, 1, False, oracle.DOMAIN_GROUP, 2, tau)
    want = [[h for h in g if ent[h] < tau] for g in ([0, 1], [2, 3])]
    assert grp["pools"] == [p for p in want if p]
    pooled = {h for p in grp["pools"] for h in p}
    for h in range(H):
        if h not in pooled:
            assert np.array_equal(grp["heads"][h]["mask"], row["heads"][h]["mask"])
    # the floor still holds in pooled rows, and rows stay prefixes of their ranking
    fl = oracle.select_domains(lg, one, qs, 0.3, 3, False, oracle.DOMAIN_HEAD)
    for h in range(H):
        r = fl["heads"][h]
        assert np.all(r["n_final"] >= 3)
        for i in range(Cq):
            assert set(np.nonzero(r["mask"][i])[0]) == set(r["orders"][i][:r["t_final"][i]].tolist())


def test_pooled_ties_across_rows_go_to_the_lower_row():
    """Hand-derived: two rows of one head with p = (1/2, 1/2) and |Q| = 1
    each (N = 2) give four pairs of mass 1/4 that all tie on p.  In (row,
    unit) order the cumulative masses are 1/4, 1/2, 3/4, 1, so P = 0.6 keeps
    three pairs: both units of row 0 and the first of row 1.  A pool of two
    such heads has the target 0.6 * 2 = 1.2; head 0's four pairs come first
    (cumulative 1/4 .. 1) and the fifth pair, head 1's (row 0, unit 0),
    reaches 5/4: head 0 keeps 2 and 2 units, head 1 keeps 1 and 0."""
    lg = np.log(np.full((2, 2), 0.5))
    qs = np.array([1, 1])
    pc = oracle.pool_counts(lg[None], qs[None], [0], 0.6)[0]
    assert pc["count"].tolist() == [2, 1]
    pc2 = oracle.pool_counts(np.stack([lg, lg]), np.stack([qs, qs]), [0, 1], 0.6)
    assert pc2[0]["count"].tolist() == [2, 2] and pc2[1]["count"].tolist() == [1, 0]
