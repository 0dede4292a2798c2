"""GPU: sa_forward under HIP graph capture and on a caller's own stream.

The library allocates nothing and synchronises nothing inside a call, so a
caller can capture sa_forward into a graph (torch.cuda.CUDAGraph) and replay
it.  With Q and K clustered by different settings (the mid layer's k-means
with 64 and 128 clusters), K's clustering runs on the library's second
stream, forked from the captured stream and joined back by events, so the
capture must take both.  Each case replays the graph several times, with
eager work and synchronisations between replays, once on new inputs written
into the captured tensors, and compares every replay bit for bit with an
eager call on the same inputs.  A call on a caller-created stream is checked
the same way after synchronising only that stream."""

from __future__ import annotations

from dataclasses import replace

import pytest
import torch

from clustered_block_sparse_amd import _lib as L
from clustered_block_sparse_amd import api
from clustered_block_sparse_amd import workloads as wl

from gpu_helpers import DEV, MID_S, WAN_S, say, workspace_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def setup(w):
    p, qc, kc, sc, ac = api.cfgs(w)
    Cq, Ck = L.sa_num_clusters(p, qc), L.sa_num_clusters(p, kc)
    q, k, v = wl.make_inputs(w, device=DEV)
    o = torch.empty_like(q)
    mask = torch.empty(w.heads, Cq, L.mask_words(Ck), dtype=torch.int32, device=DEV)
    return (p, qc, kc, sc, ac), (q, k, v), o, mask, workspace_for(p, qc, kc, sc, ac)


def eager(cf, qkv, ws):
    o = torch.empty_like(qkv[0])
    p, qc, kc, sc, ac = cf
    Ck = L.sa_num_clusters(p, kc)
    mask = torch.empty(p.heads, L.sa_num_clusters(p, qc), L.mask_words(Ck), dtype=torch.int32, device=DEV)
    L.sa_forward(*cf, *qkv, o, mask, ws)
    torch.cuda.synchronize()
    return o, mask


@pytest.mark.parametrize("w", [MID_S, WAN_S], ids=lambda w: w.name)
def test_forward_graph_replays(w):
    say(f"[graph] {w.name}: Q {w.q.method} K {w.k.method}")
    cf, qkv, o, mask, ws = setup(w)
    ws_eager = workspace_for(*cf)
    ref_o, ref_m = eager(cf, qkv, ws_eager)  # also sets up the second stream outside the capture
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.sa_forward(*cf, *qkv, o, mask, ws)
    torch.cuda.synchronize()
    for r in range(3):
        o.fill_(float("nan"))
        mask.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(mask, ref_m), f"replay {r} differs from the eager call"
        eager(cf, qkv, ws_eager)  # eager work between replays, on its own workspace
    # new inputs written into the captured tensors
    w2 = replace(w, seed=w.seed + 1)
    for dst, src in zip(qkv, wl.make_inputs(w2, device=DEV)):
        dst.copy_(src)
    ref2_o, ref2_m = eager(cf, qkv, ws_eager)
    assert not torch.equal(ref2_o, ref_o)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(o, ref2_o) and torch.equal(mask, ref2_m), "replay on new inputs differs"
    say("  3 replays and one on new inputs equal the eager calls")


@pytest.mark.parametrize("w", [MID_S, WAN_S], ids=lambda w: w.name)
def test_forward_on_caller_stream(w):
    cf, qkv, o, mask, ws = setup(w)
    ref_o, ref_m = eager(cf, qkv, workspace_for(*cf))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o.fill_(float("nan"))
        L.sa_forward(*cf, *qkv, o, mask, ws)
    s.synchronize()  # only the caller's stream: the second stream was joined into it
    assert torch.equal(o, ref_o) and torch.equal(mask, ref_m)
