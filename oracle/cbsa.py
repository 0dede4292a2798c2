"""Plain fp64 CPU oracle of centroid-guided clustered block-sparse attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library (clustered_block_sparse_amd/,
its HIP sources or its C ABI) imports, links or runs this module, and this
module imports nothing from the library.  Only tests/, __graft_entry__.smoke()
and bench.py's cpu_baseline leg use it.

Every step follows the pages' description in their order, written out plainly
in float64 NumPy (library primitives used as steps: matmul, argmin, stable
sort, cumsum).  Pages cited:

* "SCOPE: Subspace Clustering with Online Per-Head Top-K Estimation for Sparse
  Video Attention" (arXiv 2608.12780), English abstract and the method
  sections (technical framework, key design).
* "ClusterAttention: A training-free speedup of bidirectional attention"
  (arXiv 2608.26965), English abstract and Chinese abstract.

Where the pages leave a step open, the reading taken is stated in the function
docstring (the same readings are listed in the design notes of the repo).

Parity pins: every function here is pinned by tests/test_oracle_*.py against
brute force, closed forms or invariants; none is "parity unpinned".
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Near-tie tolerance of decisions taken on fp32 evaluations (k-means
# assignments and bisection splits), relative to the magnitude of the compared
# quantities: a distance gap below 1e-5 relative may flip under fp32 rounding.
NEAR_TIE_REL = 1e-5
# Near-tie tolerances of the selection.  Its logits and masses are evaluated
# in fp64 on both sides from identical centroids, so only the order of fp64
# operations separates them: logit gaps below 1e-11 relative (to max(1, |l|))
# and cumulative masses within 1e-10 of top_p (32768 fp64 or 2^-52
# fixed-point terms) are the decisions rounding order can change.
SELECT_TIE_LOGIT_REL = 1e-11
SELECT_TIE_MASS = 1e-10


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# k-means (Lloyd), first-k initialisation
# --------------------------------------------------------------------------

def sq_dists(x, c, chunk=2048):
    """||x_n - c_j||^2 for all n, j, evaluated as the sum of squared
    differences (no expansion), in float64.  x: [N, d], c: [C, d] -> [N, C]."""
    x = _f64(x)
    c = _f64(c)
    out = np.empty((x.shape[0], c.shape[0]), dtype=np.float64)
    for s in range(0, x.shape[0], chunk):
        diff = x[s:s + chunk, None, :] - c[None, :, :]
        out[s:s + chunk] = np.einsum("ncd,ncd->nc", diff, diff)
    return out


def kmeans_assign(x, c):
    """Assignment step: a_n = argmin_j ||x_n - c_j||^2, ties to the smallest j.

    Returns (labels int64 [N], dmin [N], gap [N], near_tie bool [N]) where gap is
    the distance to the second-nearest centroid minus the nearest one and a
    token is a near tie when gap <= 1e-5 * (||x_n||^2 + ||c_a||^2) (the scale an
    fp32 evaluation is accurate to)."""
    x = _f64(x)
    c = _f64(c)
    D = sq_dists(x, c)
    labels = np.argmin(D, axis=1)  # first minimum -> smallest index on ties
    dmin = D[np.arange(len(x)), labels]
    if c.shape[0] > 1:
        D2 = D.copy()
        D2[np.arange(len(x)), labels] = np.inf
        gap = D2.min(axis=1) - dmin
    else:
        gap = np.full(len(x), np.inf)
    scale = (x * x).sum(1) + (c[labels] * c[labels]).sum(1)
    near = gap <= NEAR_TIE_REL * scale
    return labels, dmin, gap, near


def kmeans_update(x, labels, c_prev):
    """Update step: c_j <- mean of the members of cluster j.  An empty cluster
    keeps its previous centroid and has size 0.  Returns (centroids, sizes)."""
    x = _f64(x)
    C = c_prev.shape[0]
    sizes = np.bincount(labels, minlength=C).astype(np.int64)
    sums = np.zeros((C, x.shape[1]), dtype=np.float64)
    np.add.at(sums, labels, x)
    c = _f64(c_prev).copy()
    nz = sizes > 0
    c[nz] = sums[nz] / sizes[nz, None]
    return c, sizes


def kmeans(x, C, iters, init=None):
    """Plain Lloyd k-means on the rows of x (one head).

    Reading (the pages give only "k-means"; the tiny workload fixes first-k
    seeding and 5 iterations): initial centroids are the first C tokens in
    raster order (or `init`), then `iters` rounds of assignment followed by
    update, so the returned centroids are the member means of the returned
    assignment.  Returns a dict with labels, centroids, sizes and the near-tie
    flags of the last assignment."""
    x = _f64(x)
    if init is None:
        if C > x.shape[0]:
            raise ValueError("more clusters than tokens")
        c = x[:C].copy()
    else:
        c = _f64(init).copy()
    if iters < 1:
        raise ValueError("iters must be >= 1")
    for _ in range(iters):
        labels, dmin, gap, near = kmeans_assign(x, c)
        c, sizes = kmeans_update(x, labels, c)
    return dict(labels=labels, centroids=c, sizes=sizes, gap=gap, near_tie=near,
                objective=float(dmin.sum()))


# --------------------------------------------------------------------------
# Balanced recursive 2-means bisection to power-of-two sized leaves
# (ClusterAttention, English abstract: fast recursive clustering giving
# power-of-two cluster sizes)
# --------------------------------------------------------------------------

@dataclass
class BisectNode:
    start: int          # first position of the node in the final leaf order
    n: int              # tokens in the node
    n_left: int         # tokens sent to the left child
    members: np.ndarray  # ascending original token indices
    left: np.ndarray    # ascending original indices sent left
    c1: np.ndarray      # final left mean
    c2: np.ndarray      # final right mean
    min_rel_gap: float  # smallest relative boundary gap over the iterations


def bisect_split(x, members, n_left, c1, c2, iters):
    """The split rule of one node, `iters` rounds starting from (c1, c2).

    Each round: delta_n = ||x_n - c1||^2 - ||x_n - c2||^2 for the node's tokens;
    the n_left tokens first in (delta ascending, original index ascending)
    order go left; c1, c2 <- means of the two sides.  Returns (left mask over
    `members`, c1, c2, smallest relative gap between the n_left-th and the
    (n_left+1)-th delta over the rounds)."""
    xs = _f64(x)[members]
    min_rel = math.inf
    left = None
    for _ in range(iters):
        d1 = ((xs - c1) ** 2).sum(1)
        d2 = ((xs - c2) ** 2).sum(1)
        delta = d1 - d2
        order = np.lexsort((members, delta))  # primary delta, then index
        left = np.zeros(len(members), dtype=bool)
        left[order[:n_left]] = True
        a, b = order[n_left - 1], order[n_left]
        scale = max((xs[a] ** 2).sum(), (xs[b] ** 2).sum()) + max((c1 ** 2).sum(), (c2 ** 2).sum())
        min_rel = min(min_rel, (delta[b] - delta[a]) / scale)
        c1 = xs[left].mean(0)
        c2 = xs[~left].mean(0)
    return left, c1, c2, min_rel


def bisect(x, leaf, iters):
    """Balanced recursive bisection of one head's rows into C = ceil(N/leaf)
    leaves, all of `leaf` tokens except the last.

    Reading (ClusterAttention gives no procedure beyond "recursive",
    "attention-aware" and power-of-two sizes): a node of n tokens needing
    c = ceil(n/leaf) leaves is a leaf when c == 1; otherwise its left child gets
    leaf*ceil(c/2) tokens, the two means start at the node's first two tokens
    (ascending original index), `iters` rounds of `bisect_split` run, the node
    is split stably and the left child is processed before the right one.
    Leaves are numbered in that depth-first order.

    Returns dict(labels [N], perm [N], offsets [C+1], nodes [BisectNode])."""
    x = _f64(x)
    N = x.shape[0]
    if iters < 1:
        raise ValueError("iters must be >= 1")
    leaves: list[np.ndarray] = []
    nodes: list[BisectNode] = []

    def rec(members, start):
        n = len(members)
        c = -(-n // leaf)
        if c <= 1:
            leaves.append(members)
            return
        n_left = leaf * (-(-c // 2))
        c1 = x[members[0]].copy()
        c2 = x[members[1]].copy()
        left, c1, c2, rel = bisect_split(x, members, n_left, c1, c2, iters)
        nodes.append(BisectNode(start, n, n_left, members, members[left], c1, c2, rel))
        rec(members[left], start)
        rec(members[~left], start + n_left)

    rec(np.arange(N), 0)
    C = len(leaves)
    labels = np.empty(N, dtype=np.int64)
    for j, m in enumerate(leaves):
        labels[m] = j
    perm = np.concatenate(leaves)
    offsets = np.zeros(C + 1, dtype=np.int64)
    offsets[1:] = np.cumsum([len(m) for m in leaves])
    return dict(labels=labels, perm=perm, offsets=offsets, nodes=nodes)


# --------------------------------------------------------------------------
# SCOPE key subspace clustering: t / h / w slices clustered independently,
# key combo id g = (a_t*Cs + a_h)*Cs + a_w
# --------------------------------------------------------------------------

def subspace_cluster(k, dims, Cs, iters):
    """SCOPE technical framework: post-RoPE keys split into the temporal,
    height and width RoPE subspaces (column slices of widths `dims`), each
    clustered independently (k-means, Cs centroids).  A key's combo is
    g = (a_t*Cs + a_h)*Cs + a_w.  Returns dict(labels (combo ids), sub_labels
    [3, N], sub_centroids list of [Cs, d_s], combo_sizes [Cs^3])."""
    k = _f64(k)
    if sum(dims) != k.shape[1]:
        raise ValueError("subspace dims must sum to d")
    off = 0
    sub_labels, sub_cent = [], []
    for ds in dims:
        r = kmeans(k[:, off:off + ds], Cs, iters)
        sub_labels.append(r["labels"])
        sub_cent.append(r["centroids"])
        off += ds
    a_t, a_h, a_w = sub_labels
    combo = (a_t * Cs + a_h) * Cs + a_w
    sizes = np.bincount(combo, minlength=Cs ** 3).astype(np.int64)
    return dict(labels=combo, sub_labels=np.stack(sub_labels), sub_centroids=sub_cent,
                combo_sizes=sizes)


# --------------------------------------------------------------------------
# Clustering-free raster blocks (VMoBA, English abstract, item (1): a
# layer-wise recurrent 1D-2D-3D block partition)
# --------------------------------------------------------------------------

def raster_blocks(frames, height, width, bt, bh, bw):
    """Block label of every token of an F x H x W grid (token n = (t*H + h)*W
    + w) for blocks of bt x bh x bw tokens.

    Reading (VMoBA gives the 1D-2D-3D scheme, not the block shapes): a block
    partition along one axis (1D: bt consecutive frames, (bt, H, W)), two
    (2D: spatial tiles through all frames, (F, bh, bw)) or three (3D: cubes);
    edge blocks keep what remains; blocks are numbered in raster order of
    their (t, h, w) block coordinates.  Returns (labels [N], C)."""
    nt, nh, nw = -(-frames // bt), -(-height // bh), -(-width // bw)
    labels = np.empty(frames * height * width, dtype=np.int64)
    for t in range(frames):
        for h in range(height):
            for w in range(width):
                labels[(t * height + h) * width + w] = ((t // bt) * nh + h // bh) * nw + w // bw
    return labels, nt * nh * nw


# --------------------------------------------------------------------------
# Permutation into cluster order and cluster means
# --------------------------------------------------------------------------

def permute(labels, C):
    """perm = tokens ordered by (cluster id, original index); offsets =
    exclusive prefix sum of the cluster sizes.  perm[p] is the original index
    of the token at cluster-order position p."""
    labels = np.asarray(labels)
    perm = np.argsort(labels, kind="stable")
    sizes = np.bincount(labels, minlength=C)
    offsets = np.zeros(C + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(sizes)
    return perm.astype(np.int64), offsets


def cluster_means(x, perm, offsets):
    """Member mean of every cluster (zero vector for an empty cluster)."""
    x = _f64(x)
    C = len(offsets) - 1
    out = np.zeros((C, x.shape[1]), dtype=np.float64)
    for j in range(C):
        a, b = offsets[j], offsets[j + 1]
        if b > a:
            out[j] = x[perm[a:b]].mean(0)
    return out


# --------------------------------------------------------------------------
# Centroid proxy scores (SCOPE: cluster-level proxy scores; LUT aggregation)
# --------------------------------------------------------------------------

def cluster_logits(qbar, kbar, ksizes, scale, size_weighted=True):
    """l_ij = <qbar_i, kbar_j> * scale (+ ln|K_j| when size-weighted); empty key
    clusters get -inf and are never selectable.

    Reading: the proxy softmax over clusters is weighted by cluster size, which
    equals the softmax over per-key proxy scores (every key carrying its
    cluster's score) summed per cluster (SCOPE, English abstract: per key proxy
    scores)."""
    s = (_f64(qbar) @ _f64(kbar).T) * scale
    ksizes = np.asarray(ksizes)
    if size_weighted:
        with np.errstate(divide="ignore"):
            s = s + np.log(ksizes.astype(np.float64))[None, :]
    s = np.where(ksizes[None, :] > 0, s, -np.inf)
    return s


def subspace_logits(qbar, sub_centroids, dims, combo_sizes, scale, size_weighted=True):
    """SCOPE lookup-table aggregation: T_s[i, c] = <qbar_i|_s, kbar^s_c> * scale
    per subspace s; the score of combo g = (a_t, a_h, a_w) is
    T_t[i, a_t] + T_h[i, a_h] + T_w[i, a_w] (+ ln|g|); empty combos -inf."""
    qbar = _f64(qbar)
    off = 0
    T = []
    for s, ds in enumerate(dims):
        T.append((qbar[:, off:off + ds] @ _f64(sub_centroids[s]).T) * scale)
        off += ds
    Cs = T[0].shape[1]
    lut = T[0][:, :, None, None] + T[1][:, None, :, None] + T[2][:, None, None, :]
    s = lut.reshape(qbar.shape[0], Cs ** 3)
    combo_sizes = np.asarray(combo_sizes)
    if size_weighted:
        with np.errstate(divide="ignore"):
            s = s + np.log(combo_sizes.astype(np.float64))[None, :]
    return np.where(combo_sizes[None, :] > 0, s, -np.inf)


# --------------------------------------------------------------------------
# Hybrid Top-p / fixed Top-k selection and SCOPE's online per-head Top-k
# --------------------------------------------------------------------------

def _first_reaching(cum, target):
    """Smallest prefix length t >= 1 with cum[t-1] >= target, or len(cum) if
    none."""
    idx = np.nonzero(cum >= target)[0]
    return int(idx[0]) + 1 if len(idx) else len(cum)


def _tie_run(sl, cut):
    """Ranked positions [a, b) around the boundary before position `cut`
    whose order is uncertain: the maximal run of consecutive logit gaps within
    SELECT_TIE_LOGIT_REL that contains the gap at the cut ([cut, cut) if that
    gap is wide)."""
    def close(k):  # gap between ranked positions k - 1 and k
        a, b = sl[k - 1], sl[k]
        return a - b <= SELECT_TIE_LOGIT_REL * max(1.0, abs(a), abs(b))
    if not (0 < cut < len(sl)) or not close(cut):
        return cut, cut
    a, b = cut - 1, cut + 1
    while a > 0 and close(a):
        a -= 1
    while b < len(sl) and close(b):
        b += 1
    return a, b


def stat_threshold(p, lam):
    """BSA's statistical dynamic threshold of one row ("Bidirectional Sparse
    Attention for Faster Video Diffusion Training", abstract: KV blocks are
    kept by a statistical dynamic threshold).  Reading: the mean plus `lam`
    population standard deviations of the row's proxy probabilities over its
    non-empty units; a unit is kept when its probability is at least that."""
    p = _f64(p)
    mu = p.mean()
    return mu + lam * math.sqrt(((p - mu) ** 2).mean())


def select(logits, units, qsizes, top_p, floor, online_topk, k_h=None, pool=None, stat_lambda=None):
    """Per-row selection over one head.

    logits [Cq, Ck] (-inf = empty unit), units [Ck] count of each unit
    (1 per cluster; keys per combo in subspace mode), qsizes [Cq] query cluster
    sizes.

    Steps (SCOPE, English abstract and key design section):
      1. p_ij = softmax_j l_ij over the non-empty units.
      2. Rank units by (p descending, j ascending).
      3. Top-p: the shortest prefix whose mass reaches top_p (>= top_p);
         top_p >= 1 takes every non-empty unit, top_p <= 0 the empty prefix.
      4. Fixed Top-k floor: the initial prefix is the shortest one that meets
         both the mass and `floor` counted units; n_i = its unit count.
      5. Online per-head Top-k (if enabled): A = sum_i |Q_i| n_i,
         k_h = ceil(A / sum_i |Q_i|) in exact integers; rows with n_i < k_h
         extend their prefix along the same ranking until the count reaches
         k_h (capped at every non-empty unit); other rows are unchanged.
         `k_h` given: step 5 runs with that value (a staged comparison, given
         the other side's k_h).

    `pool` (from pool_counts): rows of a head that competes in a pooled
    domain take their Top-p count from the pool instead of step 3, with the
    pool's range of counts under near ties; the floor and the online Top-k
    then apply as above.

    `stat_lambda` given: step 3 keeps instead the units whose probability
    reaches the row's statistical threshold (stat_threshold), a prefix of the
    ranking; a unit within SELECT_TIE_LOGIT_REL of the threshold flags the row.

    An empty query cluster (|Q_i| = 0) has no query to serve: it selects
    nothing and counts 0 (reading; it does not enter k_h either way).

    Returns a dict with mask [Cq, Ck] bool, n_init, n_final, k_h, prefix
    lengths t_init / t_final, the ranking, and per-row near-tie flags with the
    range of prefix lengths an evaluation in another fp64 operation order may
    take: [init_lo, init_hi] for the initial prefix, [cut_lo, cut_hi] for the
    final one (both equal to the prefix length on unflagged rows).  A row is
    flagged when its Top-p crossing sits within SELECT_TIE_MASS of top_p, or a
    cut falls inside a run of logits within SELECT_TIE_LOGIT_REL."""
    logits = _f64(logits)
    units = np.asarray(units, dtype=np.int64)
    qsizes = np.asarray(qsizes, dtype=np.int64)
    Cq, Ck = logits.shape
    if top_p <= 0 and floor <= 0:
        raise ValueError("top_p <= 0 with floor <= 0 selects nothing")
    orders, cum_mass, cum_units, sorted_l = [], [], [], []
    t_init = np.zeros(Cq, dtype=np.int64)
    n_init = np.zeros(Cq, dtype=np.int64)
    init_lo = np.zeros(Cq, dtype=np.int64)
    init_hi = np.zeros(Cq, dtype=np.int64)
    near = np.zeros(Cq, dtype=bool)
    for i in range(Cq):
        row = logits[i]
        valid = np.isfinite(row)
        js = np.nonzero(valid)[0]
        m = row[js].max() if len(js) else 0.0
        e = np.exp(row[js] - m)
        p = e / e.sum() if len(js) else e
        o = np.lexsort((js, -p))  # p descending, then j ascending
        order = js[o]
        cm = np.cumsum(p[o])
        cu = np.cumsum(units[order])
        sl = row[order]
        tp_lo = tp_hi = 0
        if top_p >= 1:
            tp = len(order)
        elif top_p <= 0:
            tp = 0
        else:
            tp = _first_reaching(cm, top_p)
            tp_lo = tp_hi = tp
            # a neighbouring prefix mass within tolerance of top_p: the
            # crossing may move by one position either way
            if tp >= 2 and abs(cm[tp - 2] - top_p) <= SELECT_TIE_MASS:
                tp_lo = tp - 1
            if abs(cm[tp - 1] - top_p) <= SELECT_TIE_MASS and tp < len(cm):
                tp_hi = tp + 1
        stat = stat_lambda is not None
        if stat:
            ps = p[o]
            th = stat_threshold(ps, stat_lambda) if len(ps) else 0.0
            tp = int((ps >= th).sum())
            tol = SELECT_TIE_LOGIT_REL * max(th, 1e-300)
            tp_lo = int((ps >= th + tol).sum())
            tp_hi = int((ps >= th - tol).sum())
        if pool is not None and pool["count"][i] >= 0:
            tp = int(pool["count"][i])
            tp_lo, tp_hi = int(pool["lo"][i]), int(pool["hi"][i])
        tf = _first_reaching(cu, floor) if floor > 0 else 0
        if qsizes[i] > 0:
            t = max(tp, tf)
            lo, hi = t, t
            pooled = pool is not None and pool["count"][i] >= 0
            if (0 < top_p < 1 or pooled or stat) and tp >= tf:  # the mass or threshold decides the cut
                lo, hi = max(tp_lo, tf), max(tp_hi, tf)
            # units tied in logit with the ones at a candidate cut
            a0, _ = _tie_run(sl, lo)
            _, b1 = _tie_run(sl, hi)
            lo, hi = min(lo, a0), max(hi, b1)
        else:
            t = lo = hi = 0
        t_init[i], init_lo[i], init_hi[i] = t, lo, hi
        n_init[i] = cu[t - 1] if t > 0 else 0
        near[i] = (lo, hi) != (t, t)
        orders.append(order)
        cum_mass.append(cm)
        cum_units.append(cu)
        sorted_l.append(sl)
    # online per-head Top-k
    total = int(qsizes.sum())
    if online_topk:
        if k_h is None:
            A = int((qsizes * n_init).sum())
            k_h = -(-A // total) if total > 0 else 0
        k_h = int(k_h)
    else:
        k_h = 0
    t_final = t_init.copy()
    cut_lo = init_lo.copy()
    cut_hi = init_hi.copy()
    for i in range(Cq):
        if online_topk and n_init[i] < k_h and qsizes[i] > 0:
            tk = _first_reaching(cum_units[i], k_h)
            t_final[i] = max(t_init[i], tk)
            # another evaluation's initial prefix may lie anywhere in
            # [init_lo, init_hi]; each is extended to tk (whole units) unless
            # it already reaches k_h
            a, b = _tie_run(sorted_l[i], tk)
            lo = max(init_lo[i], min(tk, a))
            hi = max(init_hi[i], b if b > tk else tk)
            cut_lo[i], cut_hi[i] = lo, hi
            near[i] = near[i] or (lo, hi) != (t_final[i], t_final[i])
    mask = np.zeros((Cq, Ck), dtype=bool)
    n_final = np.zeros(Cq, dtype=np.int64)
    for i in range(Cq):
        t = t_final[i]
        mask[i, orders[i][:t]] = True
        n_final[i] = cum_units[i][t - 1] if t > 0 else 0
    return dict(mask=mask, n_init=n_init, n_final=n_final, k_h=k_h, t_init=t_init,
                t_final=t_final, near_tie=near, orders=orders, init_lo=init_lo, init_hi=init_hi,
                cut_lo=cut_lo, cut_hi=cut_hi, cum_units=cum_units)


# --------------------------------------------------------------------------
# Competition domains (EG-Sparse: entropy-gated grouped cross-head pools;
# VMoBA: global block selection over a whole head)
# --------------------------------------------------------------------------

def proxy_probs(logits):
    """Row-wise softmax of proxy logits (-inf = empty unit -> 0)."""
    logits = _f64(logits)
    out = np.zeros_like(logits)
    for i in range(logits.shape[0]):
        v = np.isfinite(logits[i])
        if v.any():
            e = np.exp(logits[i][v] - logits[i][v].max())
            out[i][v] = e / e.sum()
    return out


def head_entropy(logits, qsizes):
    """Entropy of one head's proxy attention (EG-Sparse, abstract: heads are
    routed by entropy, from scores the sparse pipeline already has).

    Reading: the Shannon entropy of each row's proxy distribution, divided by
    the log of its number of non-empty units (1 -> 0), so that it lies in
    [0, 1]; the head's entropy is their mean weighted by query-cluster size
    (the expected normalised entropy of a query's proxy attention)."""
    P = proxy_probs(logits)
    units = np.isfinite(_f64(logits)).sum(axis=1)
    qsizes = np.asarray(qsizes, dtype=np.float64)
    ent = np.zeros(len(P))
    for i in range(len(P)):
        p = P[i][P[i] > 0]
        if units[i] > 1:
            ent[i] = -(p * np.log(p)).sum() / math.log(units[i])
    total = qsizes.sum()
    return float((qsizes * ent).sum() / total) if total > 0 else 0.0


DOMAIN_ROW, DOMAIN_HEAD, DOMAIN_GROUP = 0, 1, 2


def domains(entropies, domain, group, max_entropy):
    """Pools of heads.  ROW: every head selects per row (no pool).  HEAD
    (VMoBA global block selection): every head is a pool of its own.  GROUP
    (EG-Sparse): heads are cut into groups of `group` consecutive heads; the
    heads of a group whose entropy is below `max_entropy` form one pool, the
    others select per row.  Returns a list of pools (lists of head indices)."""
    H = len(entropies)
    if domain == DOMAIN_ROW:
        return []
    if domain == DOMAIN_HEAD:
        return [[h] for h in range(H)]
    pools = []
    for g0 in range(0, H, group):
        low = [h for h in range(g0, min(g0 + group, H)) if entropies[h] < max_entropy]
        if low:
            pools.append(low)
    return pools


def pool_counts(logits, qsizes, heads, top_p):
    """Pooled Top-p over the (head, row, unit) pairs of the heads in `heads`.

    Reading (VMoBA, abstract (2): the most salient query-key block
    interactions are chosen across a whole head; EG-Sparse, abstract: a grouped
    cross-head pool): every pair of a non-empty query cluster and a non-empty
    unit competes by its proxy probability p_ij (descending; ties by head,
    row, unit ascending), carrying the mass |Q_i| p_ij / N, so that a head's
    pairs sum to 1 and a pool of m heads to m; the pool takes the shortest
    prefix whose mass reaches top_p * m (top_p >= 1: every pair; top_p <= 0:
    none).  A row's pooled pairs are then the first ones of its own ranking,
    and their number is the row's Top-p count.

    Returns {h: dict(count, lo, hi)} with per-row counts and their range
    under near ties (a crossing within SELECT_TIE_MASS of the target, or a cut
    inside a run of probabilities within SELECT_TIE_LOGIT_REL relative)."""
    pairs = []   # (p, h, i, j, mass)
    for h in heads:
        P = proxy_probs(logits[h])
        N = float(np.sum(qsizes[h]))
        for i in range(P.shape[0]):
            if qsizes[h][i] <= 0:
                continue
            for j in np.nonzero(P[i] > 0)[0]:
                pairs.append((P[i, j], h, i, int(j), qsizes[h][i] * P[i, j] / N))
    pairs.sort(key=lambda t: (-t[0], t[1], t[2], t[3]))
    m = len(heads)
    cm = np.cumsum([t[4] for t in pairs]) if pairs else np.zeros(0)
    if top_p >= 1:
        cut = lo = hi = len(pairs)
    elif top_p <= 0:
        cut = lo = hi = 0
    else:
        target = top_p * m
        cut = _first_reaching(cm, target)
        lo = hi = cut
        if cut >= 2 and abs(cm[cut - 2] - target) <= SELECT_TIE_MASS * m:
            lo = cut - 1
        if abs(cm[cut - 1] - target) <= SELECT_TIE_MASS * m and cut < len(pairs):
            hi = cut + 1
        pv = np.array([t[0] for t in pairs])

        def close(k):
            a, b = pv[k - 1], pv[k]
            return a - b <= SELECT_TIE_LOGIT_REL * max(a, b)
        while 0 < lo < len(pairs) and close(lo):
            lo -= 1
        while 0 < hi < len(pairs) and close(hi):
            hi += 1
    out = {}
    for h in heads:
        Cq = logits[h].shape[0]
        out[h] = dict(count=np.zeros(Cq, np.int64), lo=np.zeros(Cq, np.int64), hi=np.zeros(Cq, np.int64))
    for k, (_, h, i, _, _) in enumerate(pairs):
        if k < cut:
            out[h]["count"][i] += 1
        if k < lo:
            out[h]["lo"][i] += 1
        if k < hi:
            out[h]["hi"][i] += 1
    return out


def select_domains(logits, units, qsizes, top_p, floor, online_topk, domain=DOMAIN_ROW, group=1,
                   max_entropy=0.0):
    """Selection of every head under a competition rule (EG-Sparse, VMoBA).

    logits [H, Cq, Ck], qsizes [H, Cq], units [Ck] (clusters: ones).  Steps:
    head entropies; pools from the rule (`domains`); each pool's Top-p counts
    (`pool_counts`); then every head's selection as `select`, with its rows'
    Top-p counts taken from its pool when it has one.  Returns dict(heads =
    per-head select() results, entropy [H], pools)."""
    H = len(logits)
    ent = np.array([head_entropy(logits[h], qsizes[h]) for h in range(H)])
    pools = domains(ent, domain, group, max_entropy)
    pooled = {}
    for pl in pools:
        pooled.update(pool_counts(logits, qsizes, pl, top_p))
    res = []
    for h in range(H):
        pc = pooled.get(h)
        res.append(select(logits[h], units, qsizes[h], top_p, floor, online_topk, pool=pc))
    return dict(heads=res, entropy=ent, pools=pools)


# --------------------------------------------------------------------------
# Block-sparse attention with optional mean compensation (closed form)
# --------------------------------------------------------------------------

def attention(q, k, v, q_perm, q_off, k_perm, k_off, mask, scale,
              compensate=False, kbar=None, vbar=None):
    """Sparse attention of every query token over the original keys/values of
    the key clusters its query cluster selected (SCOPE: attention over the
    selected original keys and values), with optional compensation of each
    excluded non-empty key cluster through its mean (ClusterAttention: the
    excluded cluster enters as |K_j| copies of (kbar_j, vbar_j)):

      O_n = [sum_{m in sel} e^{s_nm} v_m + c sum_{j excl} |K_j| e^{<q_n,kbar_j> scale} vbar_j]
          / [sum_{m in sel} e^{s_nm}     + c sum_{j excl} |K_j| e^{<q_n,kbar_j> scale}]

    with s_nm = <q_n, k_m> * scale, evaluated with the row maximum subtracted.
    Output rows are in original token order."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    N, d = q.shape
    O = np.zeros((N, v.shape[1]), dtype=np.float64)
    Cq = len(q_off) - 1
    Ck = len(k_off) - 1
    ksz = np.diff(np.asarray(k_off))
    for i in range(Cq):
        rows = q_perm[q_off[i]:q_off[i + 1]]
        if len(rows) == 0:
            continue
        sel = np.nonzero(mask[i])[0]
        keys = np.concatenate([k_perm[k_off[j]:k_off[j + 1]] for j in sel]) if len(sel) else np.zeros(0, np.int64)
        s = (q[rows] @ k[keys].T) * scale
        vals = v[keys]
        if compensate:
            excl = np.array([j for j in range(Ck) if not mask[i, j] and ksz[j] > 0], dtype=np.int64)
            if len(excl):
                sc = (q[rows] @ _f64(kbar)[excl].T) * scale + np.log(ksz[excl].astype(np.float64))[None, :]
                s = np.concatenate([s, sc], axis=1)
                vals = np.concatenate([vals, _f64(vbar)[excl]], axis=0)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        O[rows] = (e @ vals) / e.sum(axis=1, keepdims=True)
    return O


def attention_lse(q, k, q_perm, q_off, k_perm, k_off, mask, scale, compensate=False, kbar=None):
    """Natural-log normaliser of the sparse attention of every query token:
    lse_n = log( sum_{m in sel} e^{s_nm} + c sum_{j excl} |K_j| e^{<q_n,kbar_j> scale} ),
    the log of the denominator of `attention` (same terms, same notation), so
    its weights are e^{s_nm - lse_n}.  -inf for a query with nothing to attend
    (no selected key and no compensated cluster).  Original token order."""
    q, k = _f64(q), _f64(k)
    N = q.shape[0]
    out = np.full(N, -np.inf)
    Ck = len(k_off) - 1
    ksz = np.diff(np.asarray(k_off))
    for i in range(len(q_off) - 1):
        rows = q_perm[q_off[i]:q_off[i + 1]]
        if len(rows) == 0:
            continue
        sel = np.nonzero(mask[i])[0]
        keys = np.concatenate([k_perm[k_off[j]:k_off[j + 1]] for j in sel]) if len(sel) else np.zeros(0, np.int64)
        s = (q[rows] @ k[keys].T) * scale
        if compensate:
            excl = np.array([j for j in range(Ck) if not mask[i, j] and ksz[j] > 0], dtype=np.int64)
            if len(excl):
                sc = (q[rows] @ _f64(kbar)[excl].T) * scale + np.log(ksz[excl].astype(np.float64))[None, :]
                s = np.concatenate([s, sc], axis=1)
        if s.shape[1] == 0:
            continue
        m = s.max(axis=1)
        out[rows] = m + np.log(np.exp(s - m[:, None]).sum(axis=1))
    return out


def attention_backward(q, k, v, q_perm, q_off, k_perm, k_off, mask, scale, dO):
    """Gradients of the block-sparse attention without compensation (the
    trainable use of block-sparse attention: "Bidirectional Sparse Attention
    for Faster Video Diffusion Training", abstract; VMoBA, English abstract)
    with respect to q, k and v, given the output gradient dO (original token
    order).  For a query n of query cluster i over the keys of its selected
    clusters: P_nm = softmax_m(s_nm), s_nm = <q_n, k_m> scale, and

      dV_m += P_nm dO_n,   dP_nm = <dO_n, v_m>,   D_n = sum_m P_nm dP_nm,
      dS_nm = P_nm (dP_nm - D_n),   dQ_n = scale sum_m dS_nm k_m,
      dK_m += scale dS_nm q_n.

    Returns (dq, dk, dv) in original token order."""
    q, k, v, dO = _f64(q), _f64(k), _f64(v), _f64(dO)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for i in range(len(q_off) - 1):
        rows = q_perm[q_off[i]:q_off[i + 1]]
        sel = np.nonzero(mask[i])[0]
        if len(rows) == 0 or len(sel) == 0:
            continue
        keys = np.concatenate([k_perm[k_off[j]:k_off[j + 1]] for j in sel])
        s = (q[rows] @ k[keys].T) * scale
        P = np.exp(s - s.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dv[keys] += P.T @ dO[rows]
        dP = dO[rows] @ v[keys].T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dq[rows] += scale * (dS @ k[keys])
        dk[keys] += scale * (dS.T @ q[rows])
    return dq, dk, dv


def dense_attention(q, k, v, scale):
    """softmax(q k^T * scale) v for one head."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    s = (q @ k.T) * scale
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    return (e @ v) / e.sum(axis=1, keepdims=True)


# --------------------------------------------------------------------------
# The whole path for one head
# --------------------------------------------------------------------------

@dataclass
class ClusterCfg:
    method: str = "kmeans"      # "kmeans" | "bisect" | "subspace" (keys only) | "raster"
    clusters: int = 8           # kmeans clusters; bisect derives ceil(N/leaf)
    leaf: int = 128             # bisect leaf size
    iters: int = 5
    sub_dims: tuple = (16, 24, 24)   # subspace: t/h/w column widths; raster: block extents
    sub_clusters: int = 32
    grid: tuple = (0, 0, 0)          # raster: frames, height, width of the token grid


@dataclass
class SelectCfg:
    top_p: float = 0.9
    floor: int = 1
    online_topk: bool = False
    size_weighted: bool = True


@dataclass
class HeadResult:
    O: np.ndarray
    mask: np.ndarray
    q: dict = field(default_factory=dict)
    k: dict = field(default_factory=dict)
    sel: dict = field(default_factory=dict)


def cluster_head(x, cfg: ClusterCfg):
    """Cluster one head's rows per cfg; returns labels, perm, offsets, member
    means (fp64) and sizes, plus the method's own diagnostics."""
    x = _f64(x)
    if cfg.method == "kmeans":
        r = kmeans(x, cfg.clusters, cfg.iters)
        C = cfg.clusters
    elif cfg.method == "bisect":
        r = bisect(x, cfg.leaf, cfg.iters)
        C = len(r["offsets"]) - 1
    elif cfg.method == "subspace":
        r = subspace_cluster(x, cfg.sub_dims, cfg.sub_clusters, cfg.iters)
        C = cfg.sub_clusters ** 3
    elif cfg.method == "raster":
        labels, C = raster_blocks(*cfg.grid, *cfg.sub_dims)
        r = dict(labels=labels)
    else:
        raise ValueError(cfg.method)
    perm, offsets = permute(r["labels"], C)
    if cfg.method == "bisect":
        assert np.array_equal(perm, r["perm"]) and np.array_equal(offsets, r["offsets"])
    r.update(perm=perm, offsets=offsets, sizes=np.diff(offsets), means=cluster_means(x, perm, offsets), C=C)
    return r


def forward_head(q, k, v, qcfg: ClusterCfg, kcfg: ClusterCfg, scfg: SelectCfg,
                 compensate=False, scale=None):
    """The whole path on one head: cluster Q and K, score, select, attend."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    d = q.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    rq = cluster_head(q, qcfg)
    rk = cluster_head(k, kcfg)
    if kcfg.method == "subspace":
        logits = subspace_logits(rq["means"], rk["sub_centroids"], kcfg.sub_dims, rk["sizes"], scale,
                                 scfg.size_weighted)
        units = rk["sizes"]
    else:
        logits = cluster_logits(rq["means"], rk["means"], rk["sizes"], scale, scfg.size_weighted)
        units = np.ones(rk["C"], dtype=np.int64)
    sel = select(logits, units, rq["sizes"], scfg.top_p, scfg.floor, scfg.online_topk)
    vbar = cluster_means(v, rk["perm"], rk["offsets"]) if compensate else None
    O = attention(q, k, v, rq["perm"], rq["offsets"], rk["perm"], rk["offsets"], sel["mask"], scale,
                  compensate, rk["means"], vbar)
    return HeadResult(O=O, mask=sel["mask"], q=rq, k=rk, sel=sel)
