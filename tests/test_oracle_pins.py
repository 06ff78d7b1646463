"""Pins of the CPU oracle against things other than itself.

The LowRAM pages print no worked example, so every pin here comes from a
definition, a textbook value, a reduction to a library routine, a closed
form of the mathematics, or brute force on tiny inputs.  Each test says
which part of the oracle a plausible mistake in it would break.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "textbook_values.json")))


# --------------------------------------------------------------------------- formats

def test_bf16_rne_golden():
    g = GOLD["bf16_rne"]
    bits = O.f64_to_bf16_bits(np.array(g["value"]))
    assert [int(b) for b in bits] == [int(h, 16) for h in g["bits"]]


def test_bf16_matches_torch_on_fp32_inputs():
    # library routine: torch's float32 -> bfloat16 cast is round-to-nearest-even
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [0.0, -0.0, 1.0, -1.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = O.f64_to_bf16_bits(x.astype(np.float64))
    assert np.array_equal(got, ref)
    # and widening is exact
    assert np.array_equal(O.bf16_bits_to_f64(ref),
                          torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_f16_golden():
    g = GOLD["f16_rne"]
    got = O.f64_to_f16(np.array(g["value"])).view(np.uint16)
    assert [int(b) for b in got] == [int(h, 16) for h in g["bits"]]


def test_int4_hand_and_bounds():
    g = GOLD["int4_hand"]
    x = np.zeros(32)
    x[:len(g["x_head"])] = g["x_head"]
    codes, scales = O.int4_quantize_g32(x)
    assert float(scales[0]) == g["scale"]
    assert list(codes[:len(g["codes_head"])]) == g["codes_head"]
    packed = O.int4_pack(np.array(g["pack_codes"], dtype=np.int8))
    assert [int(b) for b in packed] == [int(h, 16) for h in g["pack_bytes"]]
    # round trip, error bound |x - xhat| <= s/2, exact on multiples of s
    rng = np.random.default_rng(1)
    y = rng.standard_normal((50, 128)) * rng.uniform(0.01, 100, (50, 1))
    c, s = O.int4_quantize_g32(y)
    assert np.array_equal(O.int4_unpack(O.int4_pack(c)), c)
    yh = O.int4_dequantize_g32(c, s)
    sg = np.repeat(s.astype(np.float64), 32, axis=-1)
    # inside the clamp range the error is at most s/2; max|x|/7 is rounded to
    # fp16, so the largest element may sit just outside 7 s and be clamped
    inside = np.abs(y) <= 7 * sg
    assert np.all(np.abs(y - yh)[inside] <= sg[inside] / 2 * (1 + 1e-12))
    assert np.all(np.abs(y - yh)[~inside] <= np.abs(y)[~inside] - 7 * sg[~inside] + 1e-12)
    assert np.all(np.abs(c) <= 7)
    # all-zero group -> scale 0 and codes 0
    cz, sz = O.int4_quantize_g32(np.zeros(64))
    assert np.all(cz == 0) and np.all(sz == 0)


def test_int4_exact_on_multiples():
    s = np.float16(0.25)
    k = np.arange(-7, 8)
    x = np.resize(k, 32).astype(np.float64) * float(s)
    x[0] = 7 * float(s)                     # make max|x| = 7 s exactly
    c, sc = O.int4_quantize_g32(x)
    assert float(sc[0]) == float(s)
    assert np.array_equal(O.int4_dequantize_g32(c, sc), x)


# --------------------------------------------------------------------------- RoPE

def test_rope_golden_cases():
    for case in GOLD["rope_rotate_half"]["cases"]:
        y = O.rope_rotate(np.array([case["x"]]), np.array([case["pos"]]), case["theta"])[0]
        assert np.allclose(y, case["y"], atol=1e-15), case


def test_rope_matches_complex_multiplication_and_closed_forms():
    rng = np.random.default_rng(2)
    d, T, theta = 16, 9, 500000.0
    x = rng.standard_normal((T, d))
    pos = rng.integers(0, 200000, T)
    y = O.rope_rotate(x, pos, theta)
    # textbook equivalence: pair (x_i, x_{i+d/2}) as a complex number times e^{i pos w_i}
    w = theta ** (-np.arange(d // 2) * 2.0 / d)
    z = (x[:, :d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos[:, None] * w[None, :])
    assert np.allclose(y, np.concatenate([z.real, z.imag], 1), atol=1e-12)
    # R(-t) R(t) = I, norm preserved
    assert np.allclose(O.rope_rotate(y, pos, theta, inverse=True), x, atol=1e-12)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1))
    # (R(a) q) . (R(b) k) depends only on a - b
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    dots = [O.rope_rotate(q[None], np.array([a + 7]), theta)[0] @
            O.rope_rotate(k[None], np.array([a]), theta)[0] for a in (0, 5, 1234, 99999)]
    assert np.allclose(dots, dots[0], atol=1e-12)


# --------------------------------------------------------------------------- GELU, predictor

def test_gelu_textbook():
    g = GOLD["normal_cdf"]
    x = np.array(g["x"])
    assert np.allclose(O.gelu(x), x * np.array(g["phi"]), rtol=0, atol=1e-15)
    xs = np.linspace(-8, 8, 101)
    assert np.allclose(O.gelu(xs) - O.gelu(-xs), xs, atol=1e-14)   # GELU(x) - GELU(-x) = x
    assert O.gelu(np.array([30.0]))[0] == 30.0


def test_predictor_hand_example_fixes_weight_orientation():
    g = GOLD["predictor_hand"]
    f = O.predictor(np.array([g["k"]]), g["W1"], g["b1"], g["W2"], g["b2"])[0]
    assert np.allclose(f, g["f"], atol=1e-12)


def test_predictor_constant_when_weights_zero():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((5, 8))
    c = rng.standard_normal(8)
    f = O.predictor(k, np.zeros((8, 8)), rng.standard_normal(8), np.zeros((8, 8)), c)
    assert np.allclose(f, c[None].repeat(5, 0), atol=0)


# --------------------------------------------------------------------------- selection

def test_selection_hand():
    g = GOLD["selection_hand"]
    e = np.array([np.nan if v == "nan" else v for v in g["err"]], dtype=np.float64)
    assert list(O.select_worst(e, g["m"])) == g["rows"]


def test_selection_special_cases_and_rank_definition():
    rng = np.random.default_rng(4)
    for trial in range(30):
        n = int(rng.integers(1, 40))
        e = rng.integers(0, 5, n).astype(np.float64)        # many ties
        if trial % 3 == 0:
            e[rng.integers(0, n)] = np.nan
        for m in range(0, n + 1):
            S = O.select_worst(e, m)
            # independent definition: t is selected iff fewer than m rows beat it
            def beats(u, t):
                eu, et = e[u], e[t]
                if np.isnan(eu) != np.isnan(et):
                    return np.isnan(eu)
                if np.isnan(eu):
                    return u < t
                return eu > et or (eu == et and u < t)
            ref = [t for t in range(n) if sum(beats(u, t) for u in range(n) if u != t) < m]
            assert list(S) == ref
        assert len(O.select_worst(e, 0)) == 0
        assert list(O.select_worst(e, n)) == list(range(n))
    # permuting distinct scores permutes the selected rows
    e = rng.standard_normal(50)
    perm = rng.permutation(50)
    S = O.select_worst(e, 12)
    Sp = O.select_worst(e[perm], 12)
    assert sorted(perm[Sp]) == list(S)


# --------------------------------------------------------------------------- whole-path invariants

def _tiny(rng, B=2, G=2, H=2, grp=2, d=8, N=20, Te=3, theta=10000.0):
    D = G * H * d
    kpost = rng.standard_normal((B, G, N, H, d))
    v = rng.standard_normal((B, G, N, H, d))
    tk = rng.standard_normal((B, G, Te, H, d))
    tv = rng.standard_normal((B, G, Te, H, d))
    q = rng.standard_normal((B, H * grp, d))
    W1 = rng.standard_normal((1, G, H, d, d)) / math.sqrt(d)
    W2 = rng.standard_normal((1, G, H, d, d)) / math.sqrt(d)
    b1 = rng.standard_normal((1, G, H, d)) * 0.1
    b2 = rng.standard_normal((1, G, H, d)) * 0.1
    return dict(B=B, G=G, H=H, grp=grp, d=d, N=N, Te=Te, D=D, theta=theta, kpost=kpost, v=v,
                tk=tk, tv=tv, q=q, W1=W1, W2=W2, b1=b1, b2=b2)


def _run(t, basis, m, coef_kind="f64", resid_kind="f64", pos=None, subset=None,
         n_body=None, tail_len=None, layer=0, W=None, return_probs=False):
    B, N, Te = t["B"], t["N"], t["Te"]
    n_body = np.full(B, N) if n_body is None else n_body
    tail_len = np.full(B, Te) if tail_len is None else tail_len
    W1, b1, W2, b2 = W if W is not None else (t["W1"], t["b1"], t["W2"], t["b2"])
    c = O.prefill(t["kpost"], t["v"], pos, n_body, basis, W1, b1, W2, b2, m, t["theta"],
                  coef_kind, resid_kind)
    res = O.decode(layer, t["q"], c.coef, coef_kind, pos, n_body, basis, W1, b1, W2, b2,
                   c.resid_idx, c.resid_val, resid_kind, t["tk"], t["tv"], tail_len, t["theta"],
                   subset=subset, return_probs=return_probs)
    return c, res


def _exact(t, layer, subset=None, tail_len=None):
    """Uncompressed attention over body (post-RoPE keys as given) + tail."""
    B, H, grp = t["B"], t["H"], t["grp"]
    out = np.zeros(t["q"].shape)
    lse = np.zeros(t["q"].shape[:2])
    for b in range(B):
        A = np.arange(t["N"]) if subset is None else np.asarray(subset[b], dtype=int)
        tl = t["Te"] if tail_len is None else tail_len[b]
        for qh in range(H * grp):
            h = qh // grp
            K = np.concatenate([t["kpost"][b, layer, A, h], t["tk"][b, layer, :tl, h]])
            V = np.concatenate([t["v"][b, layer, A, h], t["tv"][b, layer, :tl, h]])
            out[b, qh], lse[b, qh], _ = O.attention_exact(t["q"][b, qh], K, V)
    return out, lse


def test_full_rank_all_residuals_is_exact_attention():
    """Invariant: a full-rank basis with residuals for every row reproduces
    exact uncompressed attention (any orthonormal basis, any predictor)."""
    rng = np.random.default_rng(5)
    t = _tiny(rng)
    Q, _ = np.linalg.qr(rng.standard_normal((t["D"], t["D"])))
    basis = np.stack([Q.T] * t["B"])
    for layer in range(t["G"]):
        _, (out, lse) = _run(t, basis, m=t["N"], layer=layer)
        ref, ref_lse = _exact(t, layer)
        assert np.allclose(out, ref, atol=1e-11, rtol=0)
        assert np.allclose(lse, ref_lse, atol=1e-11, rtol=0)


def test_identity_basis_zero_predictor_matches_torch_sdpa():
    """Reduction to a library routine: torch SDPA (CPU, fp64, GQA by
    repeating each KV head over its contiguous query heads)."""
    rng = np.random.default_rng(6)
    t = _tiny(rng, grp=3)
    z = (np.zeros_like(t["W1"]), np.zeros_like(t["b1"]), np.zeros_like(t["W2"]), np.zeros_like(t["b2"]))
    basis = np.stack([np.eye(t["D"])] * t["B"])
    for layer in range(t["G"]):
        _, (out, lse) = _run(t, basis, m=t["N"], layer=layer, W=z)
        K = np.concatenate([t["kpost"][:, layer], t["tk"][:, layer]], axis=1)   # [B, n, H, d]
        V = np.concatenate([t["v"][:, layer], t["tv"][:, layer]], axis=1)
        Kt = torch.from_numpy(K).permute(0, 2, 1, 3).repeat_interleave(t["grp"], dim=1)
        Vt = torch.from_numpy(V).permute(0, 2, 1, 3).repeat_interleave(t["grp"], dim=1)
        qt = torch.from_numpy(t["q"])[:, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt.contiguous(), Vt.contiguous())[:, :, 0]
        assert np.allclose(out, ref.numpy(), atol=1e-12)


def test_softmax_weights_sum_to_one_and_constant_values():
    rng = np.random.default_rng(7)
    t = _tiny(rng)
    Q, _ = np.linalg.qr(rng.standard_normal((t["D"], 12)))
    basis = np.stack([Q.T] * t["B"])
    _, (out, lse, probs) = _run(t, basis, m=5, coef_kind="bf16", resid_kind="bf16", return_probs=True)
    for p in probs.values():
        assert abs(p.sum() - 1.0) <= 1e-12
    # W2 = 0, b2 = 1, no residuals, tail values 1 -> every output is 1
    W = (t["W1"], t["b1"], np.zeros_like(t["W2"]), np.ones_like(t["b2"]))
    t1 = dict(t)
    t1["tv"] = np.ones_like(t["tv"])
    _, (out1, _) = _run(t1, basis, m=0, W=W)
    assert np.allclose(out1, 1.0, atol=1e-14)


def test_eckart_young_projection_and_inverse_rope():
    """Closed form: with the SVD basis of the pre-RoPE keys, the rebuild error
    ||X - X B^T B||_F^2 equals the sum of the discarded sigma_i^2.  The keys
    are rotated here by complex multiplication, so a wrong sign or pairing in
    the oracle's inverse rotation breaks the identity."""
    rng = np.random.default_rng(8)
    G, H, d, N, theta, r = 2, 2, 8, 40, 10000.0, 9
    D = G * H * d
    X = rng.standard_normal((N, 6)) @ rng.standard_normal((6, D)) + 0.3 * rng.standard_normal((N, D))
    pos = np.sort(rng.choice(5000, N, replace=False))
    w = theta ** (-np.arange(d // 2) * 2.0 / d)
    Xg = X.reshape(N, G, H, d)
    z = (Xg[..., :d // 2] + 1j * Xg[..., d // 2:]) * np.exp(1j * pos[:, None, None, None] * w)
    kpost = np.concatenate([z.real, z.imag], -1).transpose(1, 0, 2, 3)[None]      # [1, G, N, H, d]
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    basis = Vt[:r][None]
    zeros = np.zeros((1, G, H, d, d)), np.zeros((1, G, H, d))
    c = O.prefill(kpost, np.zeros_like(kpost), pos[None], np.array([N]), basis,
                  zeros[0], zeros[1], zeros[0], zeros[1], 0, theta, "f64", "f64")
    err = np.sum((X - c.khat_pre[0]) ** 2)
    assert abs(err - np.sum(S[r:] ** 2)) <= 1e-9 * np.sum(S ** 2)
    assert np.allclose(c.coef[0], X @ Vt[:r].T, atol=1e-10)


def test_predictor_exact_gives_zero_error_at_full_rank():
    rng = np.random.default_rng(9)
    t = _tiny(rng, B=1)
    B, G, N, H, d = t["kpost"].shape
    pos = np.arange(N)
    # values generated by the predictor itself from the pre-RoPE keys (no noise)
    kpre = O.rope_rotate(t["kpost"][0].transpose(0, 2, 1, 3), pos, t["theta"], inverse=True)
    v = np.zeros_like(t["v"])
    for l in range(G):
        for h in range(H):
            v[0, l, :, h] = O.predictor(kpre[l, h], t["W1"][0, l, h], t["b1"][0, l, h],
                                        t["W2"][0, l, h], t["b2"][0, l, h])
    t["v"] = v
    basis = np.eye(t["D"])[None]
    c, _ = _run(t, basis, m=3)
    assert np.max(c.err) < 1e-24
    # and a constant predictor scores the squared distance to that constant
    W = (np.zeros_like(t["W1"]), np.zeros_like(t["b1"]), np.zeros_like(t["W2"]), np.full_like(t["b2"], 0.25))
    c2, _ = _run(t, basis, m=3, W=W)
    assert np.allclose(c2.err[0], ((v[0] - 0.25) ** 2).sum(-1).transpose(0, 2, 1), atol=1e-12)


def test_subset_special_cases_and_split_merge():
    rng = np.random.default_rng(10)
    t = _tiny(rng, N=30)
    Q, _ = np.linalg.qr(rng.standard_normal((t["D"], 10)))
    basis = np.stack([Q.T] * t["B"])
    _, (full, full_lse) = _run(t, basis, m=7, coef_kind="bf16", resid_kind="bf16")
    allrows = [np.arange(t["N"])] * t["B"]
    _, (sub, sub_lse) = _run(t, basis, m=7, coef_kind="bf16", resid_kind="bf16", subset=allrows)
    assert np.array_equal(full, sub) and np.array_equal(full_lse, sub_lse)
    # empty subset -> attention over the tail only
    empty = [np.zeros(0, dtype=int)] * t["B"]
    _, (tail_only, tl_lse) = _run(t, basis, m=7, subset=empty)
    for b in range(t["B"]):
        for qh in range(t["H"] * t["grp"]):
            h = qh // t["grp"]
            o, l, _ = O.attention_exact(t["q"][b, qh], t["tk"][b, 0, :, h], t["tv"][b, 0, :, h])
            assert np.allclose(tail_only[b, qh], o, atol=1e-13) and abs(tl_lse[b, qh] - l) < 1e-13
    # empty attended set: o = 0, lse = -inf
    _, (o0, l0) = _run(t, basis, m=7, subset=empty, tail_len=np.zeros(t["B"], dtype=int))
    assert np.all(o0 == 0) and np.all(np.isneginf(l0))
    # split-K: any partition of the rows, merged by log-sum-exp, equals one pass
    perm = rng.permutation(t["N"])
    parts_rows = [np.sort(perm[:11]), np.sort(perm[11:12]), np.sort(perm[12:])]
    parts = []
    for rows in parts_rows:
        _, (o, l) = _run(t, basis, m=7, coef_kind="bf16", resid_kind="bf16",
                         subset=[rows] * t["B"], tail_len=np.zeros(t["B"], dtype=int))
        parts.append((o, l))
    _, (tailpart, tail_l) = _run(t, basis, m=7, coef_kind="bf16", resid_kind="bf16", subset=empty)
    parts.append((tailpart, tail_l))
    for b in range(t["B"]):
        for qh in range(t["H"] * t["grp"]):
            o, l = O.merge_partials([(p[0][b, qh], p[1][b, qh]) for p in parts])
            assert np.allclose(o, full[b, qh], atol=1e-12) and abs(l - full_lse[b, qh]) < 1e-12


def test_eviction_keep_all_equals_no_eviction_and_gqa_special_cases():
    rng = np.random.default_rng(11)
    t = _tiny(rng, grp=1)
    Q, _ = np.linalg.qr(rng.standard_normal((t["D"], 16)))
    basis = np.stack([Q.T] * t["B"])
    _, (x, lx) = _run(t, basis, m=4, coef_kind="bf16", resid_kind="bf16")
    pos = np.stack([np.arange(t["N"])] * t["B"])
    _, (y, ly) = _run(t, basis, m=4, coef_kind="bf16", resid_kind="bf16", pos=pos)
    assert np.array_equal(x, y) and np.array_equal(lx, ly)
    # MHA (one query head per KV head): each output uses its own head only
    ref, _ = _exact(t, 0)
    Qf, _ = np.linalg.qr(rng.standard_normal((t["D"], t["D"])))
    _, (mha, _) = _run(t, np.stack([Qf.T] * t["B"]), m=t["N"])
    assert np.allclose(mha, ref, atol=1e-11)
    # identical queries within a GQA group give identical outputs
    t2 = _tiny(rng, grp=4)
    t2["q"][:, 1:4] = t2["q"][:, 0:1]
    t2["q"][:, 5:8] = t2["q"][:, 4:5]
    _, (g, _) = _run(t2, basis, m=4, coef_kind="bf16", resid_kind="bf16")
    assert np.array_equal(g[:, 0], g[:, 3]) and np.array_equal(g[:, 4], g[:, 7])


def test_ragged_body_padding_rules():
    rng = np.random.default_rng(12)
    t = _tiny(rng, N=16)
    Q, _ = np.linalg.qr(rng.standard_normal((t["D"], 8)))
    basis = np.stack([Q.T] * t["B"])
    n_body = np.array([16, 5])
    c, (out, _) = _run(t, basis, m=7, coef_kind="f32", resid_kind="f32", n_body=n_body)
    assert np.all(c.coef[1, 5:] == 0)
    assert list(c.resid_idx[1, 0, 0, 5:]) == [O.INT32_MAX] * 2
    assert np.all(O.dequant_store(c.resid_val, "f32")[1, :, :, 5:] == 0)
    assert np.all(c.err[1, :, :, 5:] == 0)
    # the short sequence attends to its 5 body rows only
    t5 = dict(t)
    _, (o5, _) = _run(t5, basis, m=7, coef_kind="f32", resid_kind="f32", n_body=n_body,
                      subset=[np.arange(16), np.arange(5)])
    assert np.array_equal(out, o5)


def test_int4_storage_roundtrip_in_decode():
    """Storage rounding is the only difference between int4 and f64 modes:
    decoding the int4 cache equals decoding an f64 cache holding the
    dequantised values."""
    rng = np.random.default_rng(13)
    t = _tiny(rng, d=32)                      # d and r multiples of 32 (int4 groups)
    Q, _ = np.linalg.qr(rng.standard_normal((t["D"], 32)))
    basis = np.stack([Q.T] * t["B"])
    c, (out, lse) = _run(t, basis, m=6, coef_kind="int4", resid_kind="int4")
    C = O.dequant_store(c.coef, "int4")
    R = O.dequant_store(c.resid_val, "int4")
    out2, lse2 = O.decode(0, t["q"], C, "f64", None, np.full(t["B"], t["N"]), basis, t["W1"], t["b1"],
                          t["W2"], t["b2"], c.resid_idx, R, "f64", t["tk"], t["tv"],
                          np.full(t["B"], t["Te"]), t["theta"])
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# --------------------------------------------------------------------------- appending rows (tail lifecycle)

def _prefill_part(t, basis, n0, m, coef_kind="f64", resid_kind="f64", pos=None):
    """Prefill of the first n0 body rows into a cache with room for all N."""
    B = t["B"]
    return O.prefill(t["kpost"], t["v"], pos, np.full(B, n0), basis, t["W1"], t["b1"], t["W2"], t["b2"],
                     m, t["theta"], coef_kind, resid_kind)


def _with_slots(c, m_total):
    """The cache with its residual arrays padded to m_total slots (INT32_MAX
    indices, zero residuals), as a caller allocates room for later rows."""
    idx = c.resid_idx
    pad = m_total - idx.shape[-1]
    idx = np.concatenate([idx, np.full(idx.shape[:-1] + (pad,), O.INT32_MAX, dtype=idx.dtype)], axis=-1)

    def padv(a):
        return np.concatenate([a, np.zeros(a.shape[:3] + (pad,) + a.shape[4:], dtype=a.dtype)], axis=3)
    val = (padv(c.resid_val[0]), padv(c.resid_val[1])) if c.resid_kind == "int4" else padv(c.resid_val)
    return O.OracleCache(coef=c.coef, coef_kind=c.coef_kind, resid_idx=idx, resid_val=val,
                         resid_kind=c.resid_kind)


def _append_rest(t, c, basis, n0, m_new, pos=None):
    B, N = t["B"], t["N"]
    pos_new = None if pos is None else pos[:, n0:]
    return O.append_body(c, np.full(B, n0), pos, t["kpost"][:, :, n0:], t["v"][:, :, n0:], pos_new, basis,
                         t["W1"], t["b1"], t["W2"], t["b2"], m_new, t["theta"])


@pytest.mark.parametrize("with_pos", [False, True])
def test_append_full_rank_all_residuals_is_exact_attention(with_pos):
    """Invariant: prefill of part of the body, then the rest appended, with a
    full-rank basis and a residual for every row, decodes to exact attention
    over all body rows and the tail.  A wrong position for an appended row
    (its inverse rotation), a misplaced coefficient row or residual slot, or
    a wrong body length breaks it."""
    rng = np.random.default_rng(41)
    t = _tiny(rng, N=23)
    B, N = t["B"], t["N"]
    Q, _ = np.linalg.qr(rng.standard_normal((t["D"], t["D"])))
    basis = np.stack([Q.T] * B)
    pos = np.cumsum(rng.integers(1, 4, size=(B, N)), axis=1) if with_pos else None
    n0 = 15
    c = _prefill_part(t, basis, n0, m=N, pos=pos)
    c2, nb2, pos2, err_new = _append_rest(t, c, basis, n0, m_new=N - n0, pos=pos)
    assert np.array_equal(nb2, np.full(B, N)) and err_new.shape == (B, t["G"], t["H"], N - n0)
    if with_pos:
        assert np.array_equal(pos2, pos)
    for layer in range(t["G"]):
        out, lse = O.decode(layer, t["q"], c2.coef, "f64", pos2, nb2, basis, t["W1"], t["b1"], t["W2"],
                            t["b2"], c2.resid_idx, c2.resid_val, "f64", t["tk"], t["tv"], np.full(B, t["Te"]),
                            t["theta"])
        ref, ref_lse = _exact(t, layer)
        assert np.allclose(out, ref, atol=1e-11, rtol=0)
        assert np.allclose(lse, ref_lse, atol=1e-11, rtol=0)


def test_append_rows_match_whole_prefill_and_select_among_new_rows():
    """The appended rows get exactly the coefficients and scores a prefill of
    the whole body gives them (the steps are per row); their residual set is
    the brute-force top-m_new of the new rows by (score desc, row asc),
    following the untouched entries of the first part."""
    rng = np.random.default_rng(42)
    t = _tiny(rng, N=30)
    B, G, H, N = t["B"], t["G"], t["H"], t["N"]
    Q, _ = np.linalg.qr(rng.standard_normal((t["D"], 10)))
    basis = np.stack([Q.T] * B)
    n0, m0, m_new = 18, 4, 3
    c = _with_slots(_prefill_part(t, basis, n0, m=m0, coef_kind="bf16", resid_kind="bf16"), m0 + m_new)
    c2, nb2, _, err_new = _append_rest(t, c, basis, n0, m_new)
    whole = O.prefill(t["kpost"], t["v"], None, np.full(B, N), basis, t["W1"], t["b1"], t["W2"], t["b2"],
                      m0 + m_new, t["theta"], "bf16", "bf16")
    assert np.array_equal(O.dequant_store(c2.coef, "bf16"), O.dequant_store(whole.coef, "bf16"))
    assert np.allclose(err_new, whole.err[..., n0:], rtol=1e-12, atol=0)
    for b in range(B):
        for l in range(G):
            for h in range(H):
                got = c2.resid_idx[b, l, h]
                assert np.array_equal(got[:m0], c.resid_idx[b, l, h, :m0])           # first part untouched
                e = err_new[b, l, h]
                top = sorted(range(N - n0), key=lambda i: (-e[i], i))[:m_new]
                assert list(got[m0:]) == sorted(n0 + i for i in top)
                assert np.all(np.diff(got) > 0)
                # the appended residuals are the whole-body prefill's residuals of those rows
                R2 = O.dequant_store(c2.resid_val, "bf16")[b, l, h]
                f_rows = {int(x): k for k, x in enumerate(whole.resid_idx[b, l, h])}
                for k in range(m0, m0 + m_new):
                    if int(got[k]) in f_rows:
                        assert np.array_equal(R2[k], O.dequant_store(whole.resid_val, "bf16")[b, l, h, f_rows[int(got[k])]])


def test_append_zero_rows_is_identity():
    rng = np.random.default_rng(43)
    t = _tiny(rng, N=12)
    Q, _ = np.linalg.qr(rng.standard_normal((t["D"], 6)))
    basis = np.stack([Q.T] * t["B"])
    c = _prefill_part(t, basis, 12, m=3, coef_kind="bf16", resid_kind="bf16")
    z = lambda a: a[:, :, :0]
    c2, nb2, _, err = O.append_body(c, np.full(t["B"], 12), None, z(t["kpost"]), z(t["v"]), None, basis,
                                    t["W1"], t["b1"], t["W2"], t["b2"], 0, t["theta"])
    assert np.array_equal(nb2, np.full(t["B"], 12)) and err.shape[-1] == 0
    assert np.array_equal(c2.coef, c.coef)
    assert np.array_equal(c2.resid_idx, c.resid_idx) and np.array_equal(c2.resid_val, c.resid_val)
