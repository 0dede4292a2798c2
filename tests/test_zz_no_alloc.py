"""GPU check of sa_block_sparse_attn_noalloc, the attention entry point that
allocates nothing (its scratch is the library's own per-GPU array): through
the C ABI it must reproduce sa_block_sparse_attn (same kernels) bit for bit,
on two calls in a row, the second on a smaller problem, so the array keeps
the first call's contents when the second one runs."""

from __future__ import annotations

from dataclasses import replace

import pytest
import torch

from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import DEV, inputs, say, workspace_for

pytestmark = pytest.mark.gpu

BIG = replace(wl.WAN, name="wan_noalloc_big", heads=3, frames=5, height=24, width=40)    # N = 4800, 38 clusters
SMALL = replace(wl.WAN, name="wan_noalloc_small", heads=1, frames=3, height=16, width=24,
                compensate=False)                                                           # N = 1152, 9 clusters


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def prepared(w):
    """Clusters, permuted V, V means and a selection of a workload, from the
    component calls with a caller workspace."""
    q, k, v = inputs(w)
    p, qc, kc, sc, ac = api.cfgs(w)
    ws = workspace_for(p, qc, kc, sc, ac)
    qt = L.alloc_clusters(p, qc, DEV, q.dtype)
    kt = L.alloc_clusters(p, kc, DEV, k.dtype)
    L.sa_cluster_qk(p, qc, kc, q, k, qt, kt, ws)
    v_perm = torch.empty_like(v)
    vbar = torch.empty(w.heads, kt.num_clusters, w.d, dtype=torch.float32, device=DEV)
    L.sa_permute(p, kt, v, v_perm, vbar)
    mask = torch.empty(w.heads, qt.num_clusters, L.mask_words(kt.num_clusters), dtype=torch.int32, device=DEV)
    counts = torch.empty(w.heads, qt.num_clusters, dtype=torch.int32, device=DEV)
    ktop = torch.empty(w.heads, dtype=torch.int32, device=DEV)
    L.sa_select(p, sc, qt, kt, mask, counts, None, ktop, ws)
    return p, ac, qt, kt, v_perm, (vbar if w.compensate else None), mask, ws, q


def test_noalloc_matches_workspace_entry_point_twice():
    runs = [prepared(BIG), prepared(SMALL)]
    for w, (p, ac, qt, kt, v_perm, vbar, mask, ws, q) in zip((BIG, SMALL), runs):
        say(f"[noalloc] {w.name} H={w.heads} N={w.n} comp={w.compensate}")
        ref = torch.full_like(q, float("nan"))
        L.sa_block_sparse_attn(p, ac, qt, kt, v_perm, vbar, mask, ref, ws)
        got = torch.full_like(q, float("nan"))
        L.sa_block_sparse_attn_noalloc(p, ac, qt, kt, v_perm, vbar, mask, got)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(ref).all())
        assert torch.equal(got, ref), f"{w.name}: the allocation-free call differs from sa_block_sparse_attn"


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    """A problem whose attention scratch exceeds the library's array is
    refused before any work (SA_ERR_WORKSPACE); pointers are never touched."""
    p = L.problem(2000, 75600, 128, 21, 45, 80, "bf16")
    fake = torch.empty(1, dtype=torch.int32, device=DEV)
    ct = L.ClusterTensors(labels=fake, perm=fake, offsets=fake, centroids=fake.float(), x_perm=fake,
                          num_clusters=591, method=L.SA_BISECT)
    with pytest.raises(L.SAError) as e:
        L.sa_block_sparse_attn_noalloc(p, L.attn_cfg(True), ct, ct, fake, fake.float(), fake, fake)
    assert e.value.status == "SA_ERR_WORKSPACE"
