"""Pins of the oracle's predictor fitting (loss, gradient, Adam, the fit
loop) against things other than itself: the mathematics of GELU, central
finite differences, closed forms of the loss and of Adam, a fixed point,
and torch's own autograd + Adam on the CPU in float64.

A plausible mistake in the oracle (a dropped chain-rule term, a wrong sign
or transpose in a weight gradient, a missing bias correction, rows gathered
from the wrong sequence) fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O


def test_gelu_grad_closed_forms_and_finite_differences():
    assert O.gelu_grad(np.array([0.0]))[0] == 0.5
    # GELU(x) - GELU(-x) = x, so GELU'(x) + GELU'(-x) = 1
    x = np.linspace(-7, 7, 301)
    assert np.max(np.abs(O.gelu_grad(x) + O.gelu_grad(-x) - 1.0)) < 1e-15
    assert abs(O.gelu_grad(np.array([40.0]))[0] - 1.0) < 1e-15
    assert abs(O.gelu_grad(np.array([-40.0]))[0]) < 1e-15
    h = 1e-5
    fd = (O.gelu(x + h) - O.gelu(x - h)) / (2 * h)
    assert np.max(np.abs(fd - O.gelu_grad(x))) < 1e-9


def _params(rng, d, scale=0.5):
    return (rng.standard_normal((d, d)) * scale, rng.standard_normal(d) * 0.1,
            rng.standard_normal((d, d)) * scale, rng.standard_normal(d) * 0.1)


def test_loss_gradient_matches_central_differences():
    rng = np.random.default_rng(5)
    n, d = 7, 4
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    w = list(_params(rng, d))
    L, *grads = O.predictor_loss_grad(K, V, *w)
    h = 1e-6
    for i in range(4):
        it = np.nditer(w[i], flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            wp = [x.copy() for x in w]
            wm = [x.copy() for x in w]
            wp[i][idx] += h
            wm[i][idx] -= h
            fd = (O.predictor_loss_grad(K, V, *wp)[0] - O.predictor_loss_grad(K, V, *wm)[0]) / (2 * h)
            assert abs(fd - grads[i][idx]) < 1e-8 * max(1.0, abs(fd)), (i, idx, fd, grads[i][idx])


def test_loss_closed_forms_with_zero_first_layer_and_no_rows():
    rng = np.random.default_rng(6)
    n, d = 9, 8
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    _, _, W2, b2 = _params(rng, d)
    Z = np.zeros((d, d))
    z = np.zeros(d)
    # W1 = 0, b1 = 0: the hidden layer is GELU(0) = 0, so f = b2 for every row
    L, dW1, db1, dW2, db2 = O.predictor_loss_grad(K, V, Z, z, W2, b2)
    assert L == pytest.approx(np.mean((b2[None, :] - V) ** 2), rel=1e-14)
    assert np.allclose(db2, 2.0 * (b2 - V.mean(axis=0)) / d, rtol=1e-13, atol=1e-15)
    assert np.all(dW2 == 0.0)
    # GELU'(0) = 1/2: dZ = (dF W2) / 2 on every row, dW1 = dZ^T K
    dF = 2.0 * (b2[None, :] - V) / (n * d)
    assert np.allclose(dW1, 0.5 * (dF @ W2).T @ K, rtol=1e-12, atol=1e-15)
    assert np.allclose(db1, 0.5 * (dF @ W2).sum(axis=0), rtol=1e-12, atol=1e-15)
    out = O.predictor_loss_grad(np.zeros((0, d)), np.zeros((0, d)), W2, b2, W2, b2)
    assert out[0] == 0.0 and all(np.all(g == 0) for g in out[1:])


def test_adam_constant_gradient_moves_lr_per_step():
    # with a constant gradient the bias-corrected moments equal g and g^2
    # exactly, so every step moves each weight by lr * |g| / (|g| + eps)
    g = np.array([3.0, -0.25, 1e-3, 0.0, -7.5])
    w = np.zeros_like(g)
    m = np.zeros_like(g)
    s = np.zeros_like(g)
    lr, eps = 0.01, 1e-12
    for t in range(1, 13):
        w, m, s = O.adam_update(w, g, m, s, t, lr, 0.9, 0.999, eps)
        expect = -t * lr * g / (np.abs(g) + eps)
        assert np.allclose(w, expect, rtol=1e-12, atol=1e-15), t


def test_adam_without_moments_is_sign_descent():
    # beta1 = beta2 = 0: m^ = g, s^ = g^2 at every step (textbook special case)
    rng = np.random.default_rng(7)
    w = rng.standard_normal(50)
    m = np.zeros(50)
    s = np.zeros(50)
    w0 = w.copy()
    for t in range(1, 6):
        g = rng.standard_normal(50)
        w, m, s = O.adam_update(w, g, m, s, t, 0.1, 0.0, 0.0, 0.0)
        w0 = w0 - 0.1 * np.sign(g)
        assert np.allclose(w, w0, rtol=0, atol=1e-14)


def _fit_inputs(rng, B=2, G=2, H=2, d=8, N=12, r=16, n_body=(12, 9), P=None, teacher=None):
    D = G * H * d
    basis = np.linalg.qr(rng.standard_normal((D, r)))[0].T[None].repeat(B, 0)   # [B, r, D]
    coef = rng.standard_normal((B, N, r))
    P = B if P is None else P
    W1 = rng.standard_normal((P, G, H, d, d)) / math.sqrt(d)
    b1 = rng.standard_normal((P, G, H, d)) * 0.1
    W2 = rng.standard_normal((P, G, H, d, d)) / math.sqrt(d)
    b2 = rng.standard_normal((P, G, H, d)) * 0.1
    v = rng.standard_normal((B, G, N, H, d))
    if teacher is not None:
        for b in range(B):
            kh = (coef[b] @ basis[b]).reshape(N, G, H, d)
            for l in range(G):
                for h in range(H):
                    p = 0 if P == 1 else b
                    v[b, l, :, h] = O.predictor(kh[:, l, h], W1[p, l, h], b1[p, l, h],
                                                W2[p, l, h], b2[p, l, h]) + teacher * v[b, l, :, h]
    return dict(coef_stored=coef, coef_kind="f64", n_body=np.array(n_body), basis=basis, v=v,
                W1=W1, b1=b1, W2=W2, b2=b2)


def test_fit_matches_torch_autograd_and_adam():
    # library routine: torch autograd through nn.functional.gelu (exact erf)
    # and torch.optim.Adam, float64 on the CPU, one predictor per head
    rng = np.random.default_rng(8)
    x = _fit_inputs(rng)
    steps, lr, b1_, b2_, eps = 15, 3e-3, 0.85, 0.995, 1e-7
    res = O.fit_predictor(**x, steps=steps, lr=lr, beta1=b1_, beta2=b2_, eps=eps)
    B, G, N, H, d = x["v"].shape
    for b in range(B):
        n = int(x["n_body"][b])
        kh = torch.from_numpy(x["coef_stored"][b, :n] @ x["basis"][b]).reshape(n, G, H, d)
        for l in range(G):
            for h in range(H):
                K = kh[:, l, h]
                V = torch.from_numpy(x["v"][b, l, :n, h])
                ps = [torch.tensor(x[k][b, l, h], requires_grad=True) for k in ("W1", "b1", "W2", "b2")]
                opt = torch.optim.Adam(ps, lr=lr, betas=(b1_, b2_), eps=eps)
                for t in range(steps):
                    opt.zero_grad()
                    f = torch.nn.functional.gelu(K @ ps[0].T + ps[1]) @ ps[2].T + ps[3]
                    loss = torch.mean((f - V) ** 2)
                    loss.backward()
                    assert res.losses[t, b, l, h] == pytest.approx(loss.item(), rel=1e-12)
                    if t == 0:
                        for k, p_ in enumerate(ps):
                            assert np.allclose(res.grad0[k][b, l, h], p_.grad.numpy(), rtol=1e-10, atol=1e-14)
                    opt.step()
                for got, p_ in zip((res.W1, res.b1, res.W2, res.b2), ps):
                    assert np.allclose(got[b, l, h], p_.detach().numpy(), rtol=1e-9, atol=1e-12)


def test_fit_teacher_is_a_fixed_point_and_empty_heads_do_not_move():
    rng = np.random.default_rng(9)
    x = _fit_inputs(rng, n_body=(12, 0), teacher=0.0)     # values exactly f(k^) at the initial weights
    res = O.fit_predictor(**x, steps=6, lr=0.05)
    assert np.max(res.losses) < 1e-28
    for got, k in zip((res.W1, res.b1, res.W2, res.b2), ("W1", "b1", "W2", "b2")):
        assert np.max(np.abs(got - x[k])) < 1e-7 * 0.05
    # the second sequence has no rows: its predictor keeps its weights exactly
    for got, k in zip((res.W1, res.b1, res.W2, res.b2), ("W1", "b1", "W2", "b2")):
        assert np.array_equal(got[1], x[k][1])


def test_fit_reduces_the_loss_and_shared_predictor_pools_the_rows():
    rng = np.random.default_rng(10)
    x = _fit_inputs(rng, P=1, n_body=(12, 7), teacher=0.05)
    # start away from the teacher
    for k in ("W1", "W2"):
        x[k] = x[k] + rng.standard_normal(x[k].shape) * 0.3
    res = O.fit_predictor(**x, steps=40, lr=1e-2)
    L = res.losses[:, 0]
    assert np.all(L[-1] < 0.5 * L[0])
    # the shared predictor sees the rows of both sequences: the same fit on
    # one sequence holding all those rows (same basis) gives the same weights
    B, G, N, H, d = x["v"].shape
    n0, n1 = 12, 7
    coef1 = np.concatenate([x["coef_stored"][0, :n0], x["coef_stored"][1, :n1]])[None]
    v1 = np.concatenate([x["v"][0, :, :n0], x["v"][1, :, :n1]], axis=1)[None]
    y = dict(x, coef_stored=coef1, v=v1, n_body=np.array([n0 + n1]), basis=x["basis"][:1])
    res1 = O.fit_predictor(**y, steps=40, lr=1e-2)
    for a, b in zip((res.W1, res.b1, res.W2, res.b2), (res1.W1, res1.b1, res1.W2, res1.b2)):
        assert np.allclose(a, b, rtol=1e-12, atol=1e-14)
    # rounding at the end only: the stored weights are the rounding of the fp64 ones
    res_bf = O.fit_predictor(**x, steps=40, lr=1e-2, weight_kind="bf16")
    assert np.array_equal(res_bf.stored[0], O.f64_to_bf16_bits(res.W1))
