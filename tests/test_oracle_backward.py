"""Pins of the oracle's block-sparse attention backward (CPU only):
central finite differences of the (separately pinned) forward, and, with every
cluster selected, the gradients of dense softmax attention from torch's
autograd in float64 (an independent library routine)."""

import math

import numpy as np
import torch

import oracle


def random_problem(rng, N=24, d=6, Cq=4, Ck=5):
    q, k, v = (rng.normal(size=(N, d)) for _ in range(3))
    ql = rng.integers(0, Cq, size=N)
    kl = rng.integers(0, Ck, size=N)
    qp, qo = oracle.permute(ql, Cq)
    kp, ko = oracle.permute(kl, Ck)
    mask = rng.random((Cq, Ck)) < 0.5
    mask[:, int(rng.integers(0, Ck))] = True
    return q, k, v, qp, qo, kp, ko, mask


def test_backward_matches_finite_differences(rng):
    for trial in range(3):
        q, k, v, qp, qo, kp, ko, mask = random_problem(rng)
        scale = 1 / math.sqrt(q.shape[1])
        G = rng.normal(size=q.shape)  # loss = sum(O * G), so dO = G

        def loss(q_, k_, v_):
            return float((oracle.attention(q_, k_, v_, qp, qo, kp, ko, mask, scale) * G).sum())

        dq, dk, dv = oracle.attention_backward(q, k, v, qp, qo, kp, ko, mask, scale, G)
        eps = 1e-6
        for x, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            for _ in range(12):
                n, c = int(rng.integers(0, x.shape[0])), int(rng.integers(0, x.shape[1]))
                args = [q.copy(), k.copy(), v.copy()]
                args[which][n, c] += eps
                up = loss(*args)
                args[which][n, c] -= 2 * eps
                dn = loss(*args)
                assert abs((up - dn) / (2 * eps) - g[n, c]) <= 1e-6 * (1 + abs(g[n, c]))


def test_backward_all_selected_is_dense_autograd(rng):
    q, k, v, qp, qo, kp, ko, mask = random_problem(rng, N=30, d=8)
    mask[:] = True
    scale = 1 / math.sqrt(8)
    G = rng.normal(size=q.shape)
    dq, dk, dv = oracle.attention_backward(q, k, v, qp, qo, kp, ko, mask, scale, G)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.softmax((tq @ tk.T) * scale, dim=-1) @ tv
    out.backward(torch.tensor(G))
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_unselected_keys_get_no_gradient(rng):
    q, k, v, qp, qo, kp, ko, mask = random_problem(rng)
    mask[:, 2] = False
    dq, dk, dv = oracle.attention_backward(q, k, v, qp, qo, kp, ko, mask, 0.4, rng.normal(size=q.shape))
    keys = kp[ko[2]:ko[3]]
    assert np.all(dk[keys] == 0) and np.all(dv[keys] == 0)
