"""ctypes binding of libsa (include/sa.h): argument marshalling only.

Each function has the name of the C entry point it calls.  Tensors are torch
tensors on the GPU; the binding passes their data pointers and the current
torch stream.  Output and workspace tensors are allocated with torch (device
memory plumbing); no step of the method runs here.  If libsa.so is missing
the first call raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsa.so")

SA_F32, SA_BF16 = 0, 1
SA_KMEANS, SA_BISECT, SA_SUBSPACE, SA_RASTER = 0, 1, 2, 3
SA_INIT_FIRST, SA_INIT_GIVEN = 0, 1
STATUS = {0: "SA_OK", 1: "SA_ERR_INVALID_ARG", 2: "SA_ERR_SHAPE", 3: "SA_ERR_DTYPE",
          4: "SA_ERR_WORKSPACE", 5: "SA_ERR_UNSUPPORTED", 6: "SA_ERR_HIP"}
METHODS = {"kmeans": SA_KMEANS, "bisect": SA_BISECT, "subspace": SA_SUBSPACE, "raster": SA_RASTER}

I32 = ctypes.c_int32


class Problem(ctypes.Structure):
    _fields_ = [("heads", I32), ("n", I32), ("d", I32), ("frames", I32), ("height", I32),
                ("width", I32), ("dtype", I32)]


class ClusterCfg(ctypes.Structure):
    _fields_ = [("method", I32), ("clusters", I32), ("leaf", I32), ("tile_cap", I32),
                ("iters", I32), ("init", I32), ("sub_dims", I32 * 3)]


class SelectCfg(ctypes.Structure):
    _fields_ = [("top_p", ctypes.c_double), ("topk_floor", I32), ("online_topk", I32),
                ("size_weighted", I32), ("domain", I32), ("group", I32), ("max_entropy", ctypes.c_double),
                ("rule", I32), ("stat_lambda", ctypes.c_double)]


class AttnCfg(ctypes.Structure):
    _fields_ = [("compensate", I32), ("scale", ctypes.c_float), ("ev_start", ctypes.c_void_p),
                ("ev_stop", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


class Clusters(ctypes.Structure):
    _fields_ = [("labels", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("centroids", ctypes.c_void_p), ("x_perm", ctypes.c_void_p), ("num_clusters", I32),
                ("method", I32), ("sub_clusters", I32), ("sub_dims", I32 * 3)]


class SAError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code
        self.status = STATUS.get(code, str(code))


_lib = None


def load():
    """Load libsa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m clustered_block_sparse_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.sa_num_clusters.argtypes = [P(Problem), P(ClusterCfg)]
    lib.sa_num_clusters.restype = I32
    lib.sa_workspace_size.argtypes = [P(Problem), P(ClusterCfg), P(ClusterCfg), P(SelectCfg), P(AttnCfg),
                                      P(ctypes.c_size_t)]
    lib.sa_cluster.argtypes = [P(Problem), P(ClusterCfg), vp, P(Clusters), vp, ctypes.c_size_t, vp]
    lib.sa_cluster_qk.argtypes = [P(Problem), P(ClusterCfg), P(ClusterCfg), vp, vp, P(Clusters), P(Clusters),
                                  vp, ctypes.c_size_t, vp]
    lib.sa_permute.argtypes = [P(Problem), P(Clusters), vp, vp, vp, vp]
    lib.sa_select.argtypes = [P(Problem), P(SelectCfg), P(Clusters), P(Clusters), vp, vp, vp, vp, vp, vp,
                              ctypes.c_size_t, vp]
    lib.sa_block_sparse_attn.argtypes = [P(Problem), P(AttnCfg), P(Clusters), P(Clusters), vp, vp, vp, vp,
                                         vp, ctypes.c_size_t, vp]
    lib.sa_block_sparse_attn_noalloc.argtypes = [P(Problem), P(AttnCfg), P(Clusters), P(Clusters), vp, vp, vp,
                                                 vp, vp]
    lib.sa_block_sparse_attn_bwd_workspace_size.argtypes = [P(Problem), I32, I32, P(ctypes.c_size_t)]
    lib.sa_block_sparse_attn_bwd.argtypes = [P(Problem), P(AttnCfg), P(Clusters), P(Clusters), vp, vp, vp, vp, vp,
                                             vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sa_forward.argtypes = [P(Problem), P(ClusterCfg), P(ClusterCfg), P(SelectCfg), P(AttnCfg), vp, vp,
                               vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sa_status_string.argtypes = [I32]
    lib.sa_status_string.restype = ctypes.c_char_p
    for fn in ("sa_workspace_size", "sa_cluster", "sa_cluster_qk", "sa_permute", "sa_select",
               "sa_block_sparse_attn", "sa_block_sparse_attn_noalloc", "sa_forward",
               "sa_block_sparse_attn_bwd_workspace_size", "sa_block_sparse_attn_bwd"):
        getattr(lib, fn).restype = I32
    _lib = lib
    return lib


# --------------------------------------------------------------------------
# struct builders
# --------------------------------------------------------------------------

def problem(heads, n, d, frames, height, width, dtype) -> Problem:
    dt = dtype if isinstance(dtype, int) else (SA_F32 if dtype in (torch.float32, "f32") else SA_BF16)
    return Problem(heads, n, d, frames, height, width, dt)


def problem_of(x: torch.Tensor, frames, height, width) -> Problem:
    H, N, d = x.shape
    return problem(H, N, d, frames, height, width, x.dtype)


def cluster_cfg(method="kmeans", clusters=0, leaf=128, tile_cap=0, iters=5, init=SA_INIT_FIRST,
                sub_dims=(0, 0, 0)) -> ClusterCfg:
    m = METHODS[method] if isinstance(method, str) else method
    return ClusterCfg(m, clusters, leaf, tile_cap, iters, init, (I32 * 3)(*sub_dims))


SA_DOMAIN_ROW, SA_DOMAIN_HEAD, SA_DOMAIN_GROUP = 0, 1, 2
DOMAINS = {"row": SA_DOMAIN_ROW, "head": SA_DOMAIN_HEAD, "group": SA_DOMAIN_GROUP}


SA_RULE_TOP_P, SA_RULE_STAT = 0, 1
RULES = {"top_p": SA_RULE_TOP_P, "stat": SA_RULE_STAT}


def select_cfg(top_p=0.9, topk_floor=1, online_topk=False, size_weighted=True, domain="row", group=1,
               max_entropy=0.0, rule="top_p", stat_lambda=0.0) -> SelectCfg:
    d = DOMAINS[domain] if isinstance(domain, str) else int(domain)
    r = RULES[rule] if isinstance(rule, str) else int(rule)
    return SelectCfg(float(top_p), int(topk_floor), int(bool(online_topk)), int(bool(size_weighted)), d,
                     int(group), float(max_entropy), r, float(stat_lambda))


def attn_cfg(compensate=False, scale=0.0, events=None, lse=None) -> AttnCfg:
    """events: optional (start, stop) HipEvent pair recorded around the
    attention kernels of the calls made with this configuration; lse:
    optional float32 [H, n] tensor that receives each query's log-sum-exp."""
    start, stop = events if events is not None else (None, None)
    return AttnCfg(int(bool(compensate)), float(scale), start.handle if start else None,
                   stop.handle if stop else None, None if lse is None else lse.data_ptr())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(fn, code):
    if code != 0:
        raise SAError(fn, code)


@dataclass
class ClusterTensors:
    """Caller-owned outputs of sa_cluster (torch tensors)."""
    labels: torch.Tensor
    perm: torch.Tensor
    offsets: torch.Tensor
    centroids: torch.Tensor
    x_perm: torch.Tensor
    num_clusters: int = 0
    method: int = 0
    sub_clusters: int = 0
    sub_dims: tuple = (0, 0, 0)

    def struct(self) -> Clusters:
        return Clusters(_ptr(self.labels), _ptr(self.perm), _ptr(self.offsets), _ptr(self.centroids),
                        _ptr(self.x_perm), self.num_clusters, self.method, self.sub_clusters,
                        (I32 * 3)(*self.sub_dims))


def sa_num_clusters(p: Problem, cfg: ClusterCfg) -> int:
    return int(load().sa_num_clusters(ctypes.byref(p), ctypes.byref(cfg)))


def sa_workspace_size(p: Problem, qcfg=None, kcfg=None, scfg=None, acfg=None) -> int:
    out = ctypes.c_size_t(0)
    r = lambda s: ctypes.byref(s) if s is not None else None  # noqa: E731
    _check("sa_workspace_size", load().sa_workspace_size(ctypes.byref(p), r(qcfg), r(kcfg), r(scfg), r(acfg),
                                                         ctypes.byref(out)))
    return int(out.value)


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def alloc_clusters(p: Problem, cfg: ClusterCfg, device, dtype) -> ClusterTensors:
    C = sa_num_clusters(p, cfg)
    if C < 0:
        raise SAError("sa_num_clusters", 1)
    rows = 3 * cfg.clusters if cfg.method == SA_SUBSPACE else C
    H, N, d = p.heads, p.n, p.d
    return ClusterTensors(
        labels=torch.empty(H, N, dtype=torch.int32, device=device),
        perm=torch.empty(H, N, dtype=torch.int32, device=device),
        offsets=torch.empty(H, C + 1, dtype=torch.int32, device=device),
        centroids=torch.zeros(H, rows, d, dtype=torch.float32, device=device),
        x_perm=torch.empty(H, N, d, dtype=dtype, device=device),
        num_clusters=C, method=cfg.method,
        sub_clusters=cfg.clusters if cfg.method == SA_SUBSPACE else 0,
        sub_dims=tuple(cfg.sub_dims) if cfg.method == SA_SUBSPACE else (0, 0, 0))


def sa_cluster(p: Problem, cfg: ClusterCfg, x: torch.Tensor, out: ClusterTensors, ws: torch.Tensor):
    s = out.struct()
    _check("sa_cluster", load().sa_cluster(ctypes.byref(p), ctypes.byref(cfg), _ptr(x), ctypes.byref(s),
                                           _ptr(ws), ws.numel(), _stream()))
    out.num_clusters, out.method, out.sub_clusters = s.num_clusters, s.method, s.sub_clusters
    out.sub_dims = tuple(s.sub_dims)
    return out


def sa_cluster_qk(p: Problem, qcfg: ClusterCfg, kcfg: ClusterCfg, q: torch.Tensor, k: torch.Tensor,
                  qout: ClusterTensors, kout: ClusterTensors, ws: torch.Tensor):
    sq, sk = qout.struct(), kout.struct()
    _check("sa_cluster_qk", load().sa_cluster_qk(ctypes.byref(p), ctypes.byref(qcfg), ctypes.byref(kcfg), _ptr(q),
                                                 _ptr(k), ctypes.byref(sq), ctypes.byref(sk), _ptr(ws), ws.numel(),
                                                 _stream()))
    for out, s in ((qout, sq), (kout, sk)):
        out.num_clusters, out.method, out.sub_clusters = s.num_clusters, s.method, s.sub_clusters
        out.sub_dims = tuple(s.sub_dims)
    return qout, kout


def sa_permute(p: Problem, c: ClusterTensors, x: torch.Tensor, x_perm: torch.Tensor, means=None):
    s = c.struct()
    _check("sa_permute", load().sa_permute(ctypes.byref(p), ctypes.byref(s), _ptr(x), _ptr(x_perm),
                                           _ptr(means), _stream()))


def sa_select(p: Problem, cfg: SelectCfg, q: ClusterTensors, k: ClusterTensors, mask, counts, init_counts,
              head_topk, ws, head_entropy=None):
    _check("sa_select", load().sa_select(ctypes.byref(p), ctypes.byref(cfg), ctypes.byref(q.struct()),
                                         ctypes.byref(k.struct()), _ptr(mask), _ptr(counts), _ptr(init_counts),
                                         _ptr(head_topk), _ptr(head_entropy), _ptr(ws), ws.numel(), _stream()))


def sa_block_sparse_attn(p: Problem, cfg: AttnCfg, q: ClusterTensors, k: ClusterTensors, v_perm, v_means,
                         mask, o, ws):
    _check("sa_block_sparse_attn",
           load().sa_block_sparse_attn(ctypes.byref(p), ctypes.byref(cfg), ctypes.byref(q.struct()),
                                       ctypes.byref(k.struct()), _ptr(v_perm), _ptr(v_means), _ptr(mask),
                                       _ptr(o), _ptr(ws), ws.numel(), _stream()))


def sa_block_sparse_attn_noalloc(p: Problem, cfg: AttnCfg, q: ClusterTensors, k: ClusterTensors, v_perm, v_means,
                                 mask, o):
    _check("sa_block_sparse_attn_noalloc",
           load().sa_block_sparse_attn_noalloc(ctypes.byref(p), ctypes.byref(cfg), ctypes.byref(q.struct()),
                                               ctypes.byref(k.struct()), _ptr(v_perm), _ptr(v_means), _ptr(mask),
                                               _ptr(o), _stream()))


def sa_block_sparse_attn_bwd_workspace_size(p: Problem, q_clusters: int, k_clusters: int) -> int:
    out = ctypes.c_size_t(0)
    _check("sa_block_sparse_attn_bwd_workspace_size",
           load().sa_block_sparse_attn_bwd_workspace_size(ctypes.byref(p), q_clusters, k_clusters, ctypes.byref(out)))
    return int(out.value)


def sa_block_sparse_attn_bwd(p: Problem, cfg: AttnCfg, q: ClusterTensors, k: ClusterTensors, v_perm, mask, o, d_o,
                             dq, dk, dv, ws, lse=None):
    _check("sa_block_sparse_attn_bwd",
           load().sa_block_sparse_attn_bwd(ctypes.byref(p), ctypes.byref(cfg), ctypes.byref(q.struct()),
                                           ctypes.byref(k.struct()), _ptr(v_perm), _ptr(mask), _ptr(o), _ptr(d_o),
                                           _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                                           _stream()))


def sa_forward(p: Problem, qcfg: ClusterCfg, kcfg: ClusterCfg, scfg: SelectCfg, acfg: AttnCfg, q, k, v, o,
               mask, ws):
    _check("sa_forward", load().sa_forward(ctypes.byref(p), ctypes.byref(qcfg), ctypes.byref(kcfg),
                                           ctypes.byref(scfg), ctypes.byref(acfg), _ptr(q), _ptr(k), _ptr(v),
                                           _ptr(o), _ptr(mask), _ptr(ws), ws.numel(), _stream()))


class HipEvent:
    """A raw hipEvent_t of the HIP runtime this process already runs (the one
    libsa.so and torch share), for the timing events of attn_cfg."""

    _hip = None

    def __init__(self):
        if HipEvent._hip is None:
            load()
            HipEvent._hip = ctypes.CDLL("libamdhip64.so.7")
            HipEvent._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                          ctypes.c_void_p]
            HipEvent._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            HipEvent._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h = ctypes.c_void_p()
        err = HipEvent._hip.hipEventCreate(ctypes.byref(h))
        if err != 0:
            raise RuntimeError(f"hipEventCreate failed ({err})")
        self.handle = h

    def elapsed_ms(self, stop: "HipEvent") -> float:
        """Milliseconds from this event to `stop` (waits for `stop`)."""
        hip = HipEvent._hip
        if hip.hipEventSynchronize(stop.handle) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        err = hip.hipEventElapsedTime(ctypes.byref(ms), self.handle, stop.handle)
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({err})")
        return float(ms.value)

    def __del__(self):
        # type(self): the module's globals may already be gone at interpreter exit
        hip = getattr(type(self), "_hip", None)
        if hip is not None and getattr(self, "handle", None):
            hip.hipEventDestroy(self.handle)


def mask_words(num_key_clusters: int) -> int:
    return (num_key_clusters + 31) // 32


def sa_status_string(code: int) -> str:
    return load().sa_status_string(code).decode()
