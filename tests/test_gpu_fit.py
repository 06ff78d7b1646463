"""GPU parity of lowram_fit_predictor (test-time fitting of the value
predictors) against the oracle's fit_predictor on the oracle's stored cache.

The stored coefficients are the oracle's own prefill of the seeded workload
(CPU), uploaded in storage form, so no input of the oracle comes from the
library.  Checked per case:
  * the gradient at the initial weights, every element, against a
    first-order bound of the library's arithmetic (see grad_bound);
  * the loss of every step;
  * the fitted weights after several Adam steps: elementwise when eps is
    large against the gradient's error (the update is then Lipschitz in the
    gradient), and with the default eps within Adam's step bound for every
    element and 1e-2 lr per step for almost all (a weight whose gradient is
    below the arithmetic's resolution may take the opposite sign step);
  * a predictor with no rows keeps its weights bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_05_amd import device as dev
from decode_attention_05_amd import lowram as L
from decode_attention_05_amd import synth

from gpu_helpers import EPS_BOUND, fit_rows as _rows, flat_params as _flat, grad_bound, kind, np_in, oracle_inputs

pytestmark = pytest.mark.gpu

@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.library()


C = synth.CONFIGS
CASES = {
    # name: (shape, seed, n_body or None, predictor_shared, init)
    "bf16-d128-own-scratch": (synth.scaled(C[2], batch=2, context=350, tail=20, rank=64, latent_rank=32,
                                           n_kv_heads=2, n_q_heads=8, group_layers=2), 41, [330, 201], 0, "scratch"),
    "int4-shared-teacher": (synth.scaled(C[4], batch=2, context=400, tail=16, rank=96, latent_rank=48,
                                         n_kv_heads=2, n_q_heads=4, group_layers=2, keep_frac=None, sinks=0),
                            42, [384, 129], 1, "teacher"),
    "f32-d64-shared-scratch": (C[1], 43, None, 1, "scratch"),
    "bf16-d64-own-empty": (synth.scaled(C[2], batch=3, context=150, tail=10, rank=32, latent_rank=16, head_dim=64,
                                        n_kv_heads=1, n_q_heads=2, group_layers=3), 44, [140, 0, 65], 0, "scratch"),
}


def _upload_coef(stored, k, device="cuda"):
    if k == "int4":
        packed, scales = stored
        return torch.from_numpy(np.ascontiguousarray(packed)).to(device), \
            torch.from_numpy(np.ascontiguousarray(scales).view(np.int16)).view(torch.float16).to(device)
    if k == "bf16":
        return torch.from_numpy(np.ascontiguousarray(stored).view(np.int16)).view(torch.bfloat16).to(device), None
    return torch.from_numpy(np.ascontiguousarray(stored, dtype=np.float32)).to(device), None


def _setup(name):
    s, seed, nb, shared, init = CASES[name]
    print(f"[fit {name}] B={s.batch} G={s.group_layers} Hkv={s.n_kv_heads} d={s.head_dim} N={s.n_rows} "
          f"r={s.rank} shared={shared}", flush=True)
    w = synth.make_workload(s, seed, n_body=nb)
    t = dev.upload(w)
    o = oracle_inputs(t)
    ck = kind(s, "coef")
    ora = O.prefill(o["k_post"], o["v"], o["pos"], o["n_body"], o["basis"], o["w1"], o["b1"], o["w2"], o["b2"],
                    0, s.theta, ck, kind(s, "resid"))
    coef, scale = _upload_coef(ora.coef, ck)
    Bp = 1 if shared else s.batch
    G, H, d = s.group_layers, s.n_kv_heads, s.head_dim
    if init == "teacher":
        base = [w.w1, w.b1, w.w2, w.b2]            # the workload's predictor: the teacher plus noise
        base = [np.repeat(x, Bp, axis=0) for x in base]
    else:                                          # from scratch: W ~ N(0, 1/d), b = 0
        rng = np.random.default_rng(seed + 100)
        base = [rng.standard_normal((Bp, G, H, d, d)) / math.sqrt(d), np.zeros((Bp, G, H, d)),
                rng.standard_normal((Bp, G, H, d, d)) / math.sqrt(d), np.zeros((Bp, G, H, d))]
    dt = dev.tdtype(s)
    w0 = [torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda", dt) for x in base]
    w0_np = [np_in(x) for x in w0]                 # exact values of the stored initial weights
    return s, t, o, ora, dict(coef=coef, coef_scale=scale), shared, w0, w0_np


def _run_gpu(s, t, c, shared, w0, steps, lr, beta1=0.9, beta2=0.999, eps=1e-8):
    tw = dict(t, w1=w0[0].clone(), b1=w0[1].clone(), w2=w0[2].clone(), b2=w0[3].clone())
    loss, grad = dev.fit(s, tw, c, steps=steps, lr=lr, beta1=beta1, beta2=beta2, eps=eps,
                         predictor_shared=shared)
    torch.cuda.synchronize()
    ws = [np_in(tw[k]) for k in ("w1", "b1", "w2", "b2")]
    return ws, (loss.cpu().numpy().astype(np.float64) if loss is not None else None), \
        grad.cpu().numpy().astype(np.float64)


def _run_oracle(s, o, ora, w0_np, steps, lr, beta1=0.9, beta2=0.999, eps=1e-8):
    return O.fit_predictor(ora.coef, kind(s, "coef"), o["n_body"], o["basis"], o["v"], *w0_np,
                           steps=steps, lr=lr, beta1=beta1, beta2=beta2, eps=eps)


@pytest.mark.parametrize("name", list(CASES))
def test_fit_gradient_and_first_step(name):
    s, t, o, ora, c, shared, w0, w0_np = _setup(name)
    lr = 1e-3
    ws, loss, grad = _run_gpu(s, t, c, shared, w0, 1, lr)
    ref = _run_oracle(s, o, ora, w0_np, 1, lr)
    Bp, G, H = (1 if shared else s.batch), s.group_layers, s.n_kv_heads
    for p in range(Bp):
        for l in range(G):
            for h in range(H):
                K, Km, V = _rows(s, o, ora, p, l, h, shared)
                bounds, loss_m = grad_bound(K, Km, V, *(x[p, l, h] for x in w0_np))
                g_ref = _flat(ref.grad0, p, l, h)
                bnd = EPS_BOUND * np.concatenate([bounds[0].ravel(), bounds[1], bounds[2].ravel(), bounds[3]])
                err = np.abs(grad[p, l, h] - g_ref)
                worst = np.max(err / np.maximum(bnd, 1e-300))
                assert np.all(err <= bnd + 1e-30), f"{name} p{p} l{l} h{h}: gradient error {worst:.3g} x bound"
                # the bound above is a worst case (magnitudes add up without cancelling); rounding errors
                # of the pairs are unbiased, so a whole tensor's error stays near 2^-16 of its norm
                # per product along the chain: allow 2^-12 (a dropped pair term gives ~2^-9)
                d2 = s.head_dim * s.head_dim
                cuts = [0, d2, d2 + s.head_dim, 2 * d2 + s.head_dim, 2 * d2 + 2 * s.head_dim]
                for k in range(4):
                    e_k = np.linalg.norm(err[cuts[k]:cuts[k + 1]])
                    g_k = np.linalg.norm(g_ref[cuts[k]:cuts[k + 1]])
                    assert e_k <= EPS_BOUND * g_k + 1e-30, f"{name} p{p} l{l} h{h} tensor {k}: {e_k / g_k:.3g}"
                assert abs(loss[0, p, l, h] - ref.losses[0, p, l, h]) <= EPS_BOUND * loss_m + 1e-30, \
                    f"{name}: loss {loss[0, p, l, h]} vs {ref.losses[0, p, l, h]}"
                if K.shape[0] == 0:
                    # no rows: zero gradient, zero loss, weights kept bit for bit
                    assert np.all(grad[p, l, h] == 0) and loss[0, p, l, h] == 0
                    for a, b in zip(ws, w0_np):
                        assert np.array_equal(a[p, l, h], b[p, l, h])


@pytest.mark.parametrize("name", list(CASES))
def test_fit_trajectory_large_eps(name):
    # eps at the scale of the largest gradient: each update is lr g / (sqrt(s^) + eps) with a
    # derivative in g of at most ~2 lr / eps, so a gradient error e moves a weight by <= 2 lr e / eps
    s, t, o, ora, c, shared, w0, w0_np = _setup(name)
    steps, lr = 6, 2e-3
    g0 = _run_oracle(s, o, ora, w0_np, 1, lr).grad0
    eps = max(float(max(np.abs(x).max() for x in g0)), 1e-12)
    ws, loss, _ = _run_gpu(s, t, c, shared, w0, steps, lr, eps=eps)
    ref = _run_oracle(s, o, ora, w0_np, steps, lr, eps=eps)
    Bp, G, H = (1 if shared else s.batch), s.group_layers, s.n_kv_heads
    unit = 2.0 ** -8 if s.dtype == "bf16" else 2.0 ** -23       # one unit in the last place, relative
    for p in range(Bp):
        for l in range(G):
            for h in range(H):
                K, Km, V = _rows(s, o, ora, p, l, h, shared)
                bounds, loss_m = grad_bound(K, Km, V, *(x[p, l, h] for x in w0_np))
                bnd = EPS_BOUND * np.concatenate([bounds[0].ravel(), bounds[1], bounds[2].ravel(), bounds[3]])
                got = _flat(ws, p, l, h)
                want = _flat([ref.W1, ref.b1, ref.W2, ref.b2], p, l, h)
                # weights move by <= steps * lr, so the bound at the initial weights holds along the way
                # to first order; the stored weight adds one unit of its rounding
                tol = steps * 2.0 * lr * bnd / eps + 4 * steps * 2.0 ** -24 * np.abs(want) + unit * np.abs(want)
                err = np.abs(got - want)
                assert np.all(err <= tol + 1e-30), f"{name} p{p} l{l} h{h}: {np.max(err / (tol + 1e-30)):.3g} x tol"
                if s.dtype == "f32":
                    # against the distance travelled: the fp32 weights follow the oracle's path closely
                    moved = np.linalg.norm(want - _flat(w0_np, p, l, h))
                    assert np.linalg.norm(err) <= EPS_BOUND * moved + 1e-30
                else:
                    # the fp32 weights sit far below one bf16 unit from the oracle's, so the stored
                    # weights equal its rounding except next to a rounding boundary
                    same = O.f64_to_bf16_bits(got) == O.f64_to_bf16_bits(want)
                    assert same.mean() >= 0.99, f"{name} p{p} l{l} h{h}: {same.mean():.4f} equal in bf16"
                assert np.all(np.abs(loss[:, p, l, h] - ref.losses[:, p, l, h]) <= 2 * EPS_BOUND * loss_m + 1e-30)


@pytest.mark.parametrize("name", list(CASES))
def test_fit_trajectory_default_eps(name):
    s, t, o, ora, c, shared, w0, w0_np = _setup(name)
    steps, lr = 8, 1e-3
    ws, loss, _ = _run_gpu(s, t, c, shared, w0, steps, lr)
    ref = _run_oracle(s, o, ora, w0_np, steps, lr)
    # Adam's step is at most ~1.2 lr per weight for the default betas over the first 10 steps, so two
    # runs differ by at most 2.4 lr per step; almost every weight follows the oracle closely
    for k, (a, b) in enumerate(zip(ws, (ref.W1, ref.b1, ref.W2, ref.b2))):
        unit = (2.0 ** -8 if s.dtype == "bf16" else 2.0 ** -23) * np.abs(b)
        err = np.abs(a - b)
        assert np.all(err <= 2.4 * lr * steps + unit), f"{name} tensor {k}: max err {err.max():.3g}"
        close = err <= 1e-2 * lr * steps + unit
        assert close.mean() >= 0.995, f"{name} tensor {k}: {close.mean():.4f} within 1e-2 lr per step"
    # the loss trajectory: a weight that steps the other way has a gradient below the arithmetic's
    # resolution, so it changes the loss by a second-order amount; the evaluation itself carries the
    # first-order bound of the gradient test
    Bp, G, H = (1 if shared else s.batch), s.group_layers, s.n_kv_heads
    for p in range(Bp):
        for l in range(G):
            for h in range(H):
                K, Km, V = _rows(s, o, ora, p, l, h, shared)
                _, loss_m = grad_bound(K, Km, V, *(x[p, l, h] for x in w0_np))
                err = np.abs(loss[:, p, l, h] - ref.losses[:, p, l, h])
                assert np.all(err <= 1e-4 * ref.losses[:, p, l, h] + 2 * EPS_BOUND * loss_m + 1e-30), \
                    f"{name} p{p} l{l} h{h}: loss err {err.max():.3g}"
    if name.endswith("teacher"):
        assert np.all(loss[-1] <= loss[0])
