"""GPU: the query tile size is tiling only.

`sa_cluster_cfg.tile_cap` bounds the query rows of an attention tile; each
query row's softmax runs over the same key ranges in the same order whatever
tile holds it, so sa_forward's output and mask must be bit-identical for
every cap.  Checked on the bisection and k-means layers (k-means clusters
have sizes that no cap divides), with caps of 32, 48, 64 and the default
128, compensation on and off."""

from __future__ import annotations

from dataclasses import replace

import pytest
import torch

from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api

from gpu_helpers import DEV, MID_S, WAN_S, inputs, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


@pytest.mark.parametrize("w", [WAN_S, replace(WAN_S, name="wan_small_nocomp", compensate=False), MID_S],
                         ids=lambda w: w.name)
def test_tile_cap_changes_nothing(w):
    q, k, v = inputs(w)
    ref_o, ref_m = api.forward(q, k, v, w)
    torch.cuda.synchronize()
    for cap in (32, 48, 64):
        wc = replace(w, q=replace(w.q, tile_cap=cap))
        o, m = api.forward(q, k, v, wc)
        torch.cuda.synchronize()
        assert torch.equal(m, ref_m), f"tile cap {cap}: mask differs"
        assert torch.equal(o, ref_o), f"tile cap {cap}: output differs"
    say(f"[tiling] {w.name}: caps 32, 48, 64 equal the default tiles bit for bit")
