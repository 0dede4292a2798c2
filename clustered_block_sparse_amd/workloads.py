"""Seeded synthetic inputs shaped like the pages' workloads, and the presets.

This module holds input generation only: none of the method's arithmetic.
Both sides of every comparison (the HIP library and the fp64 oracle) consume
the tensors it returns; it imports neither of them.

Inputs are post-RoPE Q and K and a value tensor V, all [heads, N, d] with
token n = (t * height + h) * width + w (raster order over frames x height x
width), as the attention of a video diffusion transformer sees them after its
3D rotary embedding (SCOPE, technical framework: clustering runs on post-RoPE
keys).  Recipes:

* Smooth video-like tokens: one field z [N, d] per head, every channel a 3D
  Gaussian random field of covariance exp(-r^2 / (2 l^2)) (white noise filtered
  by a separable Gaussian of std l/sqrt(2), truncated at 4 std, evaluated on
  the interior of a padded grid, taps scaled so the field has unit variance).
  Q = RoPE(z + 0.1 e_q), K = RoPE(z + 0.1 e_k), V ~ N(0, 1).  Q and K share z
  so that attention has query/key structure.
* Unstructured tabular-like tokens: per head 512 Gaussian mixture means
  mu_c ~ N(0, I_d); each token draws one component c_n (uniform) shared by its
  query and key, q = mu_c + 0.3 e_q, k = mu_c + 0.3 e_k; no RoPE; V ~ N(0, 1).
* RoPE: base 10000, d split over (t, h, w) as d/4, 3d/8, 3d/8 columns,
  interleaved pairs inside each slice, integer grid positions.
* bf16 tensors are the fp32 samples rounded to nearest even.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

# --------------------------------------------------------------------------
# presets
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class ClusterSpec:
    method: str = "kmeans"       # kmeans | bisect | subspace
    clusters: int = 8            # kmeans: C; bisect: derived ceil(N/leaf); subspace: Cs per slice
    leaf: int = 128
    tile_cap: int = 128
    iters: int = 5
    sub_dims: tuple = (16, 24, 24)


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    frames: int
    height: int
    width: int
    d: int
    dtype: str                   # "f32" | "bf16"
    tokens: str                  # "grf" | "gmm"
    q: ClusterSpec = field(default_factory=ClusterSpec)
    k: ClusterSpec = field(default_factory=ClusterSpec)
    top_p: float = 0.9
    floor: int = 1
    online_topk: bool = False
    compensate: bool = False
    size_weighted: bool = True
    seed: int = 0
    domain: str = "row"          # selection competition domain: row | head | group
    group: int = 1               # heads per group (domain "group")
    max_entropy: float = 0.0     # heads below it are pooled (domain "group")
    rule: str = "top_p"          # initial selection: top_p | stat (statistical threshold)
    stat_lambda: float = 0.0     # rule "stat": standard deviations above the mean

    @property
    def n(self) -> int:
        return self.frames * self.height * self.width

    def _clusters(self, spec: ClusterSpec) -> int:
        if spec.method == "bisect":
            return -(-self.n // spec.leaf)
        if spec.method == "subspace":
            return spec.clusters ** 3
        if spec.method == "raster":
            bt, bh, bw = spec.sub_dims
            return -(-self.frames // bt) * -(-self.height // bh) * -(-self.width // bw)
        return spec.clusters

    def key_clusters(self) -> int:
        return self._clusters(self.k)

    def query_clusters(self) -> int:
        return self._clusters(self.q)

    def forced_density(self, rho: float = 0.1) -> "Workload":
        """Fixed-density variant: Top-p off, floor = round(rho * units), online
        Top-k off (units are clusters, or keys in subspace mode)."""
        units = self.n if self.k.method == "subspace" else self.key_clusters()
        return replace(self, top_p=0.0, floor=max(1, int(round(rho * units))), online_topk=False)

    def with_heads(self, heads: int) -> "Workload":
        return replace(self, heads=heads)


TINY = Workload("tiny", 1, 4, 8, 8, 64, "f32", "grf",
                q=ClusterSpec("kmeans", 8, iters=5, sub_dims=(16, 24, 24)),
                k=ClusterSpec("kmeans", 8, iters=5, sub_dims=(16, 24, 24)),
                top_p=0.9, floor=2)
MID = Workload("mid", 8, 9, 30, 40, 128, "bf16", "grf",
               q=ClusterSpec("kmeans", 64, tile_cap=256, iters=5, sub_dims=(32, 48, 48)),
               k=ClusterSpec("kmeans", 128, iters=5, sub_dims=(32, 48, 48)),
               top_p=0.95, floor=1, online_topk=True)
WAN = Workload("wan720p", 40, 21, 45, 80, 128, "bf16", "grf",
               q=ClusterSpec("bisect", leaf=128, iters=5, sub_dims=(32, 48, 48)),
               k=ClusterSpec("bisect", leaf=128, iters=5, sub_dims=(32, 48, 48)),
               top_p=0.9, floor=1, compensate=True)
HUNYUAN = Workload("hunyuan720p", 24, 33, 45, 80, 128, "bf16", "grf",
                   q=ClusterSpec("bisect", leaf=128, iters=5, sub_dims=(32, 48, 48)),
                   k=ClusterSpec("subspace", 32, iters=5, sub_dims=(32, 48, 48)),
                   top_p=0.9, floor=1, online_topk=True)
TABULAR = Workload("tabular", 6, 1, 1, 131072, 64, "bf16", "gmm",
                   q=ClusterSpec("bisect", leaf=128, iters=5, sub_dims=(16, 24, 24)),
                   k=ClusterSpec("bisect", leaf=128, iters=5, sub_dims=(16, 24, 24)),
                   top_p=0.99, floor=1, compensate=True)

PRESETS = {w.name: w for w in (TINY, MID, WAN, HUNYUAN, TABULAR)}


# --------------------------------------------------------------------------
# generators
# --------------------------------------------------------------------------

_STREAM_FIELD, _STREAM_EQ, _STREAM_EK, _STREAM_V, _STREAM_MU, _STREAM_C = range(6)


def _gen(seed: int, stream: int, head: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + stream * 10_007 + head) % (2 ** 62))
    return g


def gaussian_taps(ell: float) -> torch.Tensor:
    """Taps of the separable smoothing filter: Gaussian of std ell/sqrt(2),
    truncated at 4 std, scaled to unit sum of squares (unit output variance
    for unit white noise)."""
    sf = ell / math.sqrt(2.0)
    r = int(math.ceil(4.0 * sf))
    x = torch.arange(-r, r + 1, dtype=torch.float64)
    w = torch.exp(-0.5 * (x / sf) ** 2)
    return w / torch.sqrt((w * w).sum())


def grf(frames, height, width, channels, ell, gen, device) -> torch.Tensor:
    """[frames*height*width, channels] fp32, each channel an independent unit
    variance Gaussian random field with correlation exp(-r^2/(2 ell^2))."""
    taps = gaussian_taps(ell).to(device=device, dtype=torch.float32)
    r = (taps.numel() - 1) // 2
    z = torch.randn(channels, frames + 2 * r, height + 2 * r, width + 2 * r,
                    generator=gen, device=device, dtype=torch.float32)
    for axis, size in ((1, frames), (2, height), (3, width)):
        acc = torch.zeros_like(z.narrow(axis, 0, size))
        for t in range(taps.numel()):
            acc += taps[t] * z.narrow(axis, t, size)
        z = acc
    return z.permute(1, 2, 3, 0).reshape(frames * height * width, channels).contiguous()


def rope_dims(d: int) -> tuple:
    return (d // 4, 3 * d // 8, 3 * d // 8)


def rope3d(x: torch.Tensor, frames, height, width, base=10000.0) -> torch.Tensor:
    """3D rotary embedding of x [N, d] (raster token order): columns split into
    t/h/w slices of widths d/4, 3d/8, 3d/8; inside slice s, the pair
    (2p, 2p+1) rotates by pos_s * base^(-2p/d_s)."""
    N, d = x.shape
    dev = x.device
    n = torch.arange(N, device=dev, dtype=torch.int64)
    pos = (n // (height * width), (n // width) % height, n % width)
    out = x.clone()
    off = 0
    for s, ds in enumerate(rope_dims(d)):
        p = torch.arange(ds // 2, device=dev, dtype=torch.float64)
        theta = base ** (-2.0 * p / ds)
        ang = pos[s].to(torch.float64)[:, None] * theta[None, :]
        cos = torch.cos(ang).to(torch.float32)
        sin = torch.sin(ang).to(torch.float32)
        a = x[:, off:off + ds:2]
        b = x[:, off + 1:off + ds:2]
        out[:, off:off + ds:2] = a * cos - b * sin
        out[:, off + 1:off + ds:2] = a * sin + b * cos
        off += ds
    return out


def make_head(w: Workload, head: int, device="cpu"):
    """fp32 (q, k, v) [N, d] of one head."""
    N, d = w.n, w.d
    if w.tokens == "grf":
        z = grf(w.frames, w.height, w.width, d, 2.0, _gen(w.seed, _STREAM_FIELD, head, device), device)
        eq = torch.randn(N, d, generator=_gen(w.seed, _STREAM_EQ, head, device), device=device)
        ek = torch.randn(N, d, generator=_gen(w.seed, _STREAM_EK, head, device), device=device)
        q = rope3d(z + 0.1 * eq, w.frames, w.height, w.width)
        k = rope3d(z + 0.1 * ek, w.frames, w.height, w.width)
    elif w.tokens == "gmm":
        mu = torch.randn(512, d, generator=_gen(w.seed, _STREAM_MU, head, device), device=device)
        comp = torch.randint(0, 512, (N,), generator=_gen(w.seed, _STREAM_C, head, device), device=device)
        eq = torch.randn(N, d, generator=_gen(w.seed, _STREAM_EQ, head, device), device=device)
        ek = torch.randn(N, d, generator=_gen(w.seed, _STREAM_EK, head, device), device=device)
        q = mu[comp] + 0.3 * eq
        k = mu[comp] + 0.3 * ek
    else:
        raise ValueError(w.tokens)
    v = torch.randn(N, d, generator=_gen(w.seed, _STREAM_V, head, device), device=device)
    return q, k, v


def torch_dtype(w: Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def make_inputs(w: Workload, device="cpu", heads=None):
    """(q, k, v) [H, N, d] in the workload's dtype on `device`; `heads` selects
    a subset of head indices (default all)."""
    hs = range(w.heads) if heads is None else heads
    dt = torch_dtype(w)
    qs, ks, vs = [], [], []
    for h in hs:
        q, k, v = make_head(w, h, device)
        qs.append(q.to(dt))
        ks.append(k.to(dt))
        vs.append(v.to(dt))
    return torch.stack(qs), torch.stack(ks), torch.stack(vs)
