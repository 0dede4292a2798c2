"""Pins of the synthetic input generators (CPU): the textbook RoPE
properties, the random field's variance and correlation law, the mixture's
statistics and seed reproducibility."""

import math

import numpy as np
import torch

from clustered_block_sparse_amd import workloads as wl


def test_rope_preserves_norm():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(4 * 5 * 6, 64, generator=g)
    y = wl.rope3d(x, 4, 5, 6)
    torch.testing.assert_close(y.norm(dim=1), x.norm(dim=1), rtol=1e-5, atol=1e-5)


def test_rope_relative_position():
    """<RoPE(a, p), RoPE(b, p')> depends only on p - p' (per t/h/w axis)."""
    F, H, W, d = 6, 5, 7, 64
    g = torch.Generator().manual_seed(2)
    a = torch.randn(d, generator=g, dtype=torch.float64)
    b = torch.randn(d, generator=g, dtype=torch.float64)
    X = torch.zeros(F * H * W, d, dtype=torch.float64)
    Y = torch.zeros(F * H * W, d, dtype=torch.float64)
    X[:] = a
    Y[:] = b
    RX = wl.rope3d(X.float(), F, H, W).double()
    RY = wl.rope3d(Y.float(), F, H, W).double()

    def tok(t, h, w):
        return (t * H + h) * W + w

    ref = float(RX[tok(2, 1, 3)] @ RY[tok(1, 3, 0)])
    same = float(RX[tok(4, 2, 6)] @ RY[tok(3, 4, 3)])  # same offsets (1, -2, 3)
    other = float(RX[tok(4, 2, 6)] @ RY[tok(3, 4, 4)])
    assert abs(ref - same) < 1e-4
    assert abs(ref - other) > 1e-3
    # zero offset: rotation cancels
    assert abs(float(RX[tok(3, 3, 3)] @ RY[tok(3, 3, 3)]) - float(a @ b)) < 1e-4


def test_rope_dims_split():
    assert wl.rope_dims(64) == (16, 24, 24)
    assert wl.rope_dims(128) == (32, 48, 48)


def test_grf_unit_variance_and_correlation():
    g = torch.Generator().manual_seed(3)
    F, H, W, C = 16, 16, 16, 64
    z = wl.grf(F, H, W, C, 2.0, g, "cpu").reshape(F, H, W, C).double()
    assert abs(float(z.var()) - 1.0) < 0.05
    for r in (1, 2, 3):
        corr = float((z[:, :, :-r] * z[:, :, r:]).mean() / z.var())
        assert abs(corr - math.exp(-r * r / 8.0)) < 0.05, (r, corr)
        corr_t = float((z[:-r] * z[r:]).mean() / z.var())
        assert abs(corr_t - math.exp(-r * r / 8.0)) < 0.05, (r, corr_t)


def test_gaussian_taps():
    t = wl.gaussian_taps(2.0)
    assert t.numel() == 13  # radius ceil(4 * sqrt(2)) = 6
    assert abs(float((t * t).sum()) - 1.0) < 1e-12


def test_gmm_statistics():
    w = wl.TABULAR
    q, k, v = wl.make_head(w, 0, "cpu")
    # q - k = 0.3 (e_q - e_k): variance 2 * 0.09
    assert abs(float((q - k).var()) - 0.18) < 0.01
    assert abs(float(v.var()) - 1.0) < 0.01
    # a token's query lies near one of 512 means: nearest-mean distance^2 ~ 0.09 d
    mu = torch.randn(512, w.d, generator=wl._gen(w.seed, wl._STREAM_MU, 0, "cpu"))
    dist = torch.cdist(q[:2000], mu).min(dim=1).values ** 2
    assert abs(float(dist.mean()) / w.d - 0.09) < 0.01


def test_seed_reproducible_and_heads_differ():
    w = wl.TINY
    a = wl.make_inputs(w)
    b = wl.make_inputs(w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    w2 = w.with_heads(2)
    q2, _, _ = wl.make_inputs(w2)
    assert not torch.equal(q2[0], q2[1])
    assert torch.equal(q2[0], a[0][0])


def test_presets_shapes():
    assert wl.WAN.n == 75600 and wl.WAN.key_clusters() == 591
    assert wl.HUNYUAN.n == 118800 and wl.HUNYUAN.query_clusters() == 929
    assert wl.TABULAR.key_clusters() == 1024
    f = wl.WAN.forced_density(0.1)
    assert f.floor == 59 and f.top_p == 0.0 and not f.online_topk
    assert wl.MID.forced_density(0.1).floor == 13
    assert wl.HUNYUAN.forced_density(0.1).floor == 11880
    q, k, v = wl.make_inputs(wl.TINY)
    assert q.shape == (1, 256, 64) and q.dtype == torch.float32
