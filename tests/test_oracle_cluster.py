"""Pins of the oracle's clustering steps (CPU only).

k-means is pinned to SciPy's Lloyd implementation (an independent library
routine with the same first-k / keep-empty semantics) and to invariants; the
balanced bisection to its size law, to separated blobs and to a brute-force
optimum of the balanced split; the permutation to bijection/stability laws."""

import itertools
import json
import os

import numpy as np
import pytest
import scipy.cluster.vq as vq

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def smooth_points(rng, n, d):
    t = np.linspace(0, 6, n)[:, None]
    return np.sin(t * rng.uniform(0.5, 2, size=(1, d)) + rng.uniform(0, 6, size=(1, d))) + 0.05 * rng.normal(size=(n, d))


def test_kmeans_matches_scipy_lloyd(rng):
    for trial in range(5):
        x = smooth_points(rng, 300, 6) if trial % 2 else rng.normal(size=(300, 6))
        C, T = 9, 5
        r = oracle.kmeans(x, C, T)
        code, label = vq.kmeans2(x.copy(), x[:C].copy(), iter=T, minit="matrix", missing="warn")
        assert np.array_equal(r["labels"], label)
        np.testing.assert_allclose(r["centroids"], code, rtol=0, atol=1e-12)


def test_kmeans_assign_ties_go_to_smallest_index():
    x = np.array([[0.0, 0.0], [1.0, 0.0]])
    c = np.array([[1.0, 1.0], [-1.0, 0.0], [1.0, -1.0], [0.5, 0.0]])
    labels, dmin, gap, near = oracle.kmeans_assign(x, c)
    # token 0: centroids 0 and 2 are at distance 2, centroid 1 at 1, 3 at 0.25
    assert labels[0] == 3
    # token 1: centroids 0, 2 at distance 1, centroid 3 at 0.25 -> 3; drop 3 to force the tie
    labels2, _, gap2, near2 = oracle.kmeans_assign(x, c[:3])
    assert labels2[1] == 0 and gap2[1] == 0 and near2[1]
    assert labels2[0] == 1


def test_kmeans_invariants(rng):
    x = smooth_points(rng, 400, 8)
    C = 12
    c = x[:C].copy()
    prev = np.inf
    for _ in range(6):
        labels, dmin, _, _ = oracle.kmeans_assign(x, c)
        obj = dmin.sum()
        assert obj <= prev + 1e-9
        prev = obj
        c, sizes = oracle.kmeans_update(x, labels, c)
        assert sizes.sum() == len(x)
        for j in range(C):
            if sizes[j]:
                np.testing.assert_allclose(c[j], x[labels == j].mean(0), atol=1e-12)


def test_kmeans_empty_cluster_keeps_centroid():
    # duplicate first tokens: centroid 1 equals centroid 0 and loses every tie
    x = np.array([[0.0, 0.0], [0.0, 0.0], [5.0, 5.0], [5.1, 5.0], [0.1, 0.0]])
    r = oracle.kmeans(x, 3, 1)
    assert r["sizes"].tolist() == [3, 0, 2]
    np.testing.assert_array_equal(r["centroids"][1], [0.0, 0.0])
    # next round: the kept centroid (0,0) is nearer to the two duplicates than
    # the moved centroid 0 (0.033, 0), so cluster 1 wins them back
    r2 = oracle.kmeans(x, 3, 2)
    assert r2["sizes"].tolist() == [1, 2, 2]


def test_kmeans_empty_cluster_keeps_nonzero_centroid():
    """An empty cluster keeps its previous (non-zero) centroid, so it can win
    tokens back in the next round.  Hand derivation (first-k seeding):
    round 1: c = (1,1), (1,1), (5,5); every tie goes to the lower index, so
    cluster 1 is empty and keeps (1,1); c0 = mean of (1,1),(1,1),(1.5,1) =
    (7/6, 1), c2 = (5.25, 5).  Round 2: the two (1,1) tokens are at 0 from c1
    and 1/36 from c0, so they move to cluster 1; (1.5,1) is 1/9 from c0 and
    1/4 from c1 and stays.  A centroid reset to the origin instead would be 2
    away from (1,1) and cluster 1 would stay empty."""
    x = np.array([[1.0, 1.0], [1.0, 1.0], [5.0, 5.0], [5.5, 5.0], [1.5, 1.0]])
    r = oracle.kmeans(x, 3, 1)
    assert r["labels"].tolist() == [0, 0, 2, 2, 0] and r["sizes"].tolist() == [3, 0, 2]
    np.testing.assert_array_equal(r["centroids"][1], [1.0, 1.0])
    np.testing.assert_allclose(r["centroids"][0], [7.0 / 6.0, 1.0], rtol=0, atol=1e-15)
    r2 = oracle.kmeans(x, 3, 2)
    assert r2["labels"].tolist() == [1, 1, 2, 2, 0] and r2["sizes"].tolist() == [1, 2, 2]
    np.testing.assert_array_equal(r2["centroids"], [[1.5, 1.0], [1.0, 1.0], [5.25, 5.0]])


# --------------------------------------------------------------------------
# bisection
# --------------------------------------------------------------------------

def test_bisect_worked_example():
    """Hand-derived two-round bisection on six integer points
    (tests/golden/bisect_worked_example.json): an odd leaf count at the root,
    a delta tie across the cut in the last round (a duplicated point) and a
    second round whose split differs from the first."""
    with open(os.path.join(GOLDEN, "bisect_worked_example.json")) as f:
        g = json.load(f)
    x = np.array(g["points"], dtype=np.float64)
    r = oracle.bisect(x, g["leaf"], g["iters"])
    leaves = [r["perm"][r["offsets"][j]:r["offsets"][j + 1]].tolist() for j in range(len(r["offsets"]) - 1)]
    assert leaves == g["expected_leaves"]
    assert r["labels"].tolist() == g["expected_labels"]
    assert r["offsets"].tolist() == g["expected_offsets"]
    assert len(r["nodes"]) == len(g["expected_nodes"])
    for node, want in zip(r["nodes"], g["expected_nodes"]):
        assert node.members.tolist() == want["members"]
        assert node.n_left == want["n_left"]
        assert node.left.tolist() == want["left"]
        np.testing.assert_array_equal(node.c1, want["c1"])
        np.testing.assert_array_equal(node.c2, want["c2"])
    # the first round alone, from the seeds x[0], x[1]
    r1 = g["expected_root_round1"]
    left, c1, c2, _ = oracle.bisect_split(x, np.arange(len(x)), 4, x[0].copy(), x[1].copy(), 1)
    assert np.nonzero(left)[0].tolist() == r1["left"]
    np.testing.assert_array_equal(c1, r1["c1"])
    np.testing.assert_array_equal(c2, r1["c2"])


def test_bisect_split_rounds_compose(rng):
    """T rounds of the split rule = T-1 rounds followed by one round from the
    means they return; the returned means are the means of the returned
    sides; every round's split is a minimum-cost balanced assignment for the
    means it started from (brute force)."""
    for trial in range(12):
        n = int(rng.integers(5, 12))
        n_left = int(rng.integers(1, n))
        x = rng.normal(size=(n, 3))
        x[int(rng.integers(0, n))] = x[0]  # a duplicate: a delta tie every round
        members = np.arange(n)
        c1, c2 = x[0].copy(), x[1].copy()
        for T in range(1, 5):
            left_T, a_T, b_T, _ = oracle.bisect_split(x, members, n_left, x[0].copy(), x[1].copy(), T)
            np.testing.assert_allclose(a_T, x[left_T].mean(0), rtol=0, atol=1e-14)
            np.testing.assert_allclose(b_T, x[~left_T].mean(0), rtol=0, atol=1e-14)
            one, a1, b1, _ = oracle.bisect_split(x, members, n_left, c1.copy(), c2.copy(), 1)
            assert np.array_equal(one, left_T)
            d1 = ((x - c1) ** 2).sum(1)
            d2 = ((x - c2) ** 2).sum(1)
            best = min(d1[list(S)].sum() + d2.sum() - d2[list(S)].sum()
                       for S in itertools.combinations(range(n), n_left))
            assert d1[one].sum() + d2[~one].sum() <= best + 1e-12
            c1, c2 = a1, b1


def test_bisect_left_child_takes_the_larger_half():
    """The root's left child takes L*ceil(c/2) tokens, the larger half for an
    odd leaf count c: N = 5L (c = 5) sends 3L left, N = 5L + 3 (c = 6) 3L,
    N = 3L + 1 (c = 4) 2L."""
    rng = np.random.default_rng(7)
    for N, L in [(5 * 8 + 3, 8), (5 * 8, 8), (3 * 16 + 1, 16)]:
        x = rng.normal(size=(N, 4))
        r = oracle.bisect(x, L, 2)
        c = -(-N // L)
        assert r["nodes"][0].n_left == L * ((c + 1) // 2)
        assert r["nodes"][0].start == 0 and r["nodes"][0].n == N

@pytest.mark.parametrize("N,L", [(1000, 128), (256, 128), (300, 64), (129, 128), (128, 128), (77, 8)])
def test_bisect_size_law(rng, N, L):
    x = rng.normal(size=(N, 5))
    r = oracle.bisect(x, L, 3)
    C = -(-N // L)
    sizes = np.diff(r["offsets"])
    assert len(sizes) == C
    assert np.all(sizes[:-1] == L) and sizes[-1] == N - (C - 1) * L
    assert sorted(r["perm"].tolist()) == list(range(N))
    for j in range(C):
        seg = r["perm"][r["offsets"][j]:r["offsets"][j + 1]]
        assert np.all(np.diff(seg) > 0)  # ascending original index in a leaf
        assert np.all(r["labels"][seg] == j)


def test_bisect_recovers_separated_blobs(rng):
    L, k = 16, 3
    centres = rng.normal(size=(2 ** k, 4)) * 50
    pts = np.concatenate([c + rng.normal(size=(L, 4)) for c in centres])
    blob = np.repeat(np.arange(2 ** k), L)
    sh = rng.permutation(len(pts))
    pts, blob = pts[sh], blob[sh]
    r = oracle.bisect(pts, L, 5)
    for j in range(2 ** k):
        seg = r["perm"][r["offsets"][j]:r["offsets"][j + 1]]
        assert len(set(blob[seg].tolist())) == 1
    assert len(set(blob[r["perm"][r["offsets"][j]:r["offsets"][j + 1]]][0] for j in range(2 ** k))) == 2 ** k


def test_bisect_split_is_optimal_balanced_assignment(rng):
    """For fixed (c1, c2), the (delta, index) rule is the balanced assignment
    minimising sum_left ||x-c1||^2 + sum_right ||x-c2||^2 (brute force)."""
    for trial in range(20):
        n = int(rng.integers(4, 13))
        n_left = int(rng.integers(1, n))
        x = rng.normal(size=(n, 3))
        c1, c2 = rng.normal(size=3), rng.normal(size=3)
        members = np.arange(n)
        left, _, _, _ = oracle.bisect_split(x, members, n_left, c1.copy(), c2.copy(), 1)
        d1 = ((x - c1) ** 2).sum(1)
        d2 = ((x - c2) ** 2).sum(1)
        best = min(sum(d1[list(S)]) + d2.sum() - sum(d2[list(S)])
                   for S in itertools.combinations(range(n), n_left))
        got = d1[left].sum() + d2[~left].sum()
        assert left.sum() == n_left
        assert got <= best + 1e-12


def test_bisect_sides_follow_nearest_mean():
    # two groups: the group near x[0] must go left (sign of delta)
    x = np.array([[0.0], [10.0], [0.2], [10.2], [0.1], [9.9], [0.3], [10.1]])
    r = oracle.bisect(x, 4, 2)
    left = r["perm"][:4]
    assert set(left.tolist()) == {0, 2, 4, 6}


# --------------------------------------------------------------------------
# permutation, subspace combos
# --------------------------------------------------------------------------

def test_permute_laws(rng):
    labels = rng.integers(0, 7, size=200)
    labels[labels == 3] = 2  # cluster 3 empty
    perm, off = oracle.permute(labels, 7)
    assert sorted(perm.tolist()) == list(range(200))
    assert off[0] == 0 and off[-1] == 200 and off[4] - off[3] == 0
    x = rng.normal(size=(200, 3))
    xp = x[perm]
    back = np.empty_like(xp)
    back[perm] = xp
    np.testing.assert_array_equal(back, x)
    for j in range(7):
        seg = perm[off[j]:off[j + 1]]
        assert np.all(labels[seg] == j) and np.all(np.diff(seg) > 0)


def test_subspace_combo_ids(rng):
    k = smooth_points(rng, 500, 8)
    dims = (2, 3, 3)
    r = oracle.subspace_cluster(k, dims, 4, 3)
    off = 0
    for s, ds in enumerate(dims):
        rs = oracle.kmeans(k[:, off:off + ds], 4, 3)
        assert np.array_equal(rs["labels"], r["sub_labels"][s])
        off += ds
    a_t, a_h, a_w = r["sub_labels"]
    assert np.array_equal(r["labels"], a_t * 16 + a_h * 4 + a_w)
    assert r["combo_sizes"].sum() == 500
