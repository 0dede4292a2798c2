"""Configuration presets -> C structs, and a one-call forward.

Argument marshalling only: every step runs in libsa's kernels.
"""

from __future__ import annotations

import torch

from . import _lib as L
from .workloads import Workload


def cfgs(w: Workload):
    """(problem, qcfg, kcfg, scfg, acfg) C structs of a workload preset."""
    p = L.problem(w.heads, w.n, w.d, w.frames, w.height, w.width, w.dtype)

    def cc(spec):
        return L.cluster_cfg(spec.method, spec.clusters, spec.leaf, spec.tile_cap, spec.iters,
                             L.SA_INIT_FIRST, spec.sub_dims)

    return (p, cc(w.q), cc(w.k),
            L.select_cfg(w.top_p, w.floor, w.online_topk, w.size_weighted, w.domain, w.group, w.max_entropy,
                         w.rule, w.stat_lambda),
            L.attn_cfg(w.compensate))


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, w: Workload, ws: torch.Tensor | None = None):
    """sa_forward on [H, N, d] tensors with the workload's configuration.
    Returns (o, mask)."""
    p, qc, kc, sc, ac = cfgs(w)
    p.heads = q.shape[0]
    need = L.sa_workspace_size(p, qc, kc, sc, ac)
    if ws is None or ws.numel() < need:
        ws = L.workspace(need, q.device)
    Cq = L.sa_num_clusters(p, qc)
    Ck = L.sa_num_clusters(p, kc)
    o = torch.empty_like(q)
    mask = torch.empty(q.shape[0], Cq, L.mask_words(Ck), dtype=torch.int32, device=q.device)
    L.sa_forward(p, qc, kc, sc, ac, q, k, v, o, mask, ws)
    return o, mask
