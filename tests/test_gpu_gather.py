"""GPU parity of the gathered attention path on rows with many short ranges.

Key clusters of 1 to 5 keys in a random order, and per query cluster either
every other key cluster (half the rows) or a random half of them, so a row
walks more than 512 merged ranges: several chunks of staged ranges, the
software pipeline over many whole tiles per chunk, and a partial last tile
in each chunk.  Clusters, mask and means are given; the output is compared
element by element with the oracle's attention given the same clusters and
mask, with and without compensation."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from clustered_block_sparse_amd import _lib as L

from gpu_helpers import DEV, assert_attn_close, pack_mask, say

pytestmark = pytest.mark.gpu

H, N, D = 2, 4096, 128
QC = 128  # query cluster size


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def key_clusters(rng):
    sizes = []
    while sum(sizes) < N:
        sizes.append(int(rng.integers(1, 6)))
    sizes[-1] -= sum(sizes) - N
    if sizes[-1] == 0:
        sizes.pop()
    perm = rng.permutation(N)
    off = np.concatenate([[0], np.cumsum(sizes)])
    labels = np.empty(N, np.int64)
    for j in range(len(sizes)):
        labels[perm[off[j]:off[j + 1]]] = j
    return perm, off, labels


@pytest.mark.parametrize("comp", [False, True], ids=["nocomp", "comp"])
def test_gathered_many_ranges(comp):
    rng = np.random.default_rng(7)
    g = torch.Generator().manual_seed(7)
    q = (0.5 * torch.randn(H, N, D, generator=g)).to(torch.bfloat16)
    k = torch.randn(H, N, D, generator=g).to(torch.bfloat16)
    v = torch.randn(H, N, D, generator=g).to(torch.bfloat16)
    qs, ks, vs = (t.double().numpy() for t in (q, k, v))

    Cq = N // QC
    qperm = np.arange(N)
    qoff = np.arange(0, N + 1, QC)
    qlab = qperm // QC
    kp, ko, kl = zip(*[key_clusters(rng) for _ in range(H)])
    Ck = min(len(o) - 1 for o in ko)
    # equal cluster counts across heads: merge any extra trailing clusters
    kp, ko, kl = list(kp), [o[:Ck + 1].copy() for o in ko], list(kl)
    for h in range(H):
        ko[h][-1] = N
        kl[h] = np.minimum(kl[h], Ck - 1)
    masks = np.zeros((H, Cq, Ck), bool)
    for h in range(H):
        for i in range(Cq):
            m = (np.arange(Ck) + i) % 2 == 0 if i % 2 == 0 else rng.random(Ck) < 0.5
            m[rng.integers(Ck)] = True
            masks[h, i] = m
    nr = [int((np.diff(np.concatenate([[0], masks[h, i].astype(np.int8), [0]])) == 1).sum())
          for h in range(H) for i in range(Cq)]
    say(f"[gather] H={H} N={N} Ck={Ck} comp={comp}: ranges per row {min(nr)}..{max(nr)}")
    assert max(nr) > 512

    qbar = np.stack([np.stack([qs[h][qperm[qoff[i]:qoff[i + 1]]].mean(0) for i in range(Cq)]) for h in range(H)])
    kbar = np.stack([np.stack([ks[h][kp[h][ko[h][j]:ko[h][j + 1]]].mean(0) for j in range(Ck)]) for h in range(H)])
    vbar = np.stack([oracle.cluster_means(vs[h], kp[h], ko[h]) for h in range(H)])

    p = L.problem(H, N, D, 1, 1, N, torch.bfloat16)
    ac = L.attn_cfg(compensate=comp)
    ws = L.workspace(256 << 20, DEV)  # the call checks that it is large enough
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)

    def tensors(x, perm, off, lab, cen, C):
        t = L.ClusterTensors(
            labels=torch.tensor(np.stack(lab), dtype=torch.int32, device=DEV),
            perm=torch.tensor(np.stack(perm), dtype=torch.int32, device=DEV),
            offsets=torch.tensor(np.stack(off), dtype=torch.int32, device=DEV),
            centroids=torch.tensor(cen, dtype=torch.float32, device=DEV),
            x_perm=torch.empty_like(x), num_clusters=C, method=L.METHODS["kmeans"])
        L.sa_permute(p, t, x, t.x_perm)
        return t

    qt = tensors(qd, [qperm] * H, [qoff] * H, [qlab] * H, qbar, Cq)
    kt = tensors(kd, kp, ko, kl, kbar, Ck)
    v_perm = torch.empty_like(vd)
    L.sa_permute(p, kt, vd, v_perm)
    mask = torch.tensor(pack_mask(masks), device=DEV)
    o = torch.full_like(qd, float("nan"))
    L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, torch.tensor(vbar, dtype=torch.float32, device=DEV) if comp else None,
                           mask, o, ws)
    torch.cuda.synchronize()
    assert not torch.isnan(o).any()
    kbar32 = kt.centroids.cpu().double().numpy()
    ref = np.stack([oracle.attention(qs[h], ks[h], vs[h], qperm, qoff, kp[h], ko[h], masks[h], 1.0 / math.sqrt(D),
                                     comp, kbar32[h], vbar[h].astype(np.float32).astype(np.float64))
                    for h in range(H)])
    assert_attn_close(o, ref, torch.bfloat16, f"gather many ranges comp={comp}")
