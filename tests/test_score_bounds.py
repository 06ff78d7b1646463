"""CPU checks of the prefill score bounds and of the selection checker
(tests/score_bounds.py) that the GPU parity tests use.

* An emulation of the library's scoring arithmetic in numpy fp32 (the
  rebuild summed in fp32 from the exactly stored coefficients, the rebuilt
  key and the hidden activations split into bf16 pairs, the exact-erf GELU
  rounded to fp32) stays within the bounds on every row, also with stored
  coefficients moved to the other admissible rounding where the projection
  noise allows it.
* Planted mistakes fail the checker: scores 1 % off on ordinary rows; a
  selection in which one chosen row is swapped for a row far below the
  threshold; a list that is not the top-m of the scores it came with.
* The bounds are tight enough to decide almost every row: the fraction of
  rows inside the bound of the threshold is small.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as O
import score_bounds as SB
from decode_attention_05_amd import synth


def _bf16(x):
    return O.bf16_bits_to_f64(O.f64_to_bf16_bits(np.asarray(x, np.float64)))


def _bf16_f32(x):
    return _bf16(x).astype(np.float32)


def _case(cfg: int, **kw):
    s = synth.scaled(synth.CONFIGS[cfg], **kw)
    w = synth.make_workload(s, seed=41 + cfg)
    cvt = _bf16 if s.dtype == "bf16" else (lambda x: np.asarray(x, np.float64))
    o = {k: cvt(getattr(w, k)) for k in ("k_post", "v", "basis", "w1", "b1", "w2", "b2")}
    o["pos"], o["n_body"] = w.pos, w.n_body
    ck = "int4" if s.coef_store == "int4" else ("f32" if s.dtype == "f32" else "bf16")
    oc = O.prefill(o["k_post"], o["v"], o["pos"], o["n_body"], o["basis"], o["w1"], o["b1"], o["w2"], o["b2"],
                   s.n_resid, s.theta, ck, ck)
    noise = 2.0 ** -20 * SB.projection_magnitude(o["k_post"], o["pos"], o["n_body"], o["basis"], s.theta)
    op = SB.SPLIT if s.dtype == "bf16" else SB.U32
    bound = SB.score_bounds(oc.coef, ck, oc.coef_exact, oc.khat_pre, o["basis"], o["w1"], o["b1"], o["w2"],
                            o["b2"], o["v"], o["n_body"], noise, op=op)
    return s, o, oc, ck, noise, bound


_CACHE = {}


def case(name):
    if name not in _CACHE:
        if name == "bf16":
            _CACHE[name] = _case(2, batch=2, context=768, tail=128)
        elif name == "int4":
            _CACHE[name] = _case(4, batch=1, context=4096, tail=256)
        else:
            _CACHE[name] = _case(1)
    return _CACHE[name]


def emulate_scores(C, Bs, W1, b1, W2, b2, v):
    """The library's pair-split scoring arithmetic in numpy fp32: C [n, r]
    stored coefficients (exact in fp32), Bs [r, d] the bf16 basis columns."""
    f32 = np.float32
    k = C.astype(f32) @ Bs.astype(f32)
    kh = _bf16_f32(k)
    kl = _bf16_f32(k - kh)
    W1f, W2f = W1.astype(f32), W2.astype(f32)
    z = (b1.astype(f32) + kh @ W1f.T) + kl @ W1f.T
    from scipy.special import erf
    h = (f32(0.5) * z * (f32(1.0) + erf(z.astype(np.float64) * np.sqrt(0.5)).astype(f32))).astype(f32)
    hh = _bf16_f32(h)
    hl = _bf16_f32(h - hh)
    f = (b2.astype(f32) + hh @ W2f.T) + hl @ W2f.T
    dlt = v.astype(f32) - f
    return np.sum(dlt * dlt, axis=-1, dtype=f32).astype(np.float64)


def _emulated_all(s, o, oc, ck, C):
    B, G, N, H, d = o["v"].shape
    e = np.zeros((B, G, H, N))
    for b in range(B):
        n = int(o["n_body"][b])
        for l in range(G):
            for h in range(H):
                c0 = (l * H + h) * d
                e[b, l, h, :n] = emulate_scores(C[b, :n], o["basis"][b][:, c0:c0 + d], o["w1"][0, l, h],
                                                o["b1"][0, l, h], o["w2"][0, l, h], o["b2"][0, l, h],
                                                o["v"][b, l, :n, h])
    return e


@pytest.mark.parametrize("name", ["bf16", "int4"])
def test_emulated_arithmetic_within_bounds(name):
    s, o, oc, ck, noise, bound = case(name)
    C = O.dequant_store(oc.coef, ck)
    e = _emulated_all(s, o, oc, ck, C)
    nb = o["n_body"]
    for b in range(s.batch):
        n = int(nb[b])
        SB.assert_scores_within(e[b, :, :, :n], oc.err[b, :, :, :n], bound[b, :, :, :n], f"{name} b={b}")
    # the bound is not vacuous: the emulated error uses a visible part of it
    n = int(nb[0])
    ratio = np.abs(e[0, :, :, :n] - oc.err[0, :, :, :n]) / bound[0, :, :, :n]
    assert ratio.max() > 1e-3


def test_other_admissible_coefficient_roundings_within_bounds():
    """bf16: every coefficient whose exact value lies within the projection
    noise of a rounding boundary moved to the other rounding."""
    s, o, oc, ck, noise, bound = case("bf16")
    units = SB.coef_deviation(oc.coef_exact, oc.coef, ck, noise)["amb"][0]
    C = O.dequant_store(oc.coef, ck)
    assert (units > 0).any()
    # the roundings of the ends of [c - noise, c + noise]: take the one that
    # differs from the oracle's stored value (the farther one)
    lo, hi = _bf16(oc.coef_exact - noise), _bf16(oc.coef_exact + noise)
    C_alt = np.where(np.abs(lo - C) >= np.abs(hi - C), lo, hi)
    assert np.array_equal(np.abs(C_alt - C), units)
    e = _emulated_all(s, o, oc, ck, C_alt)
    for b in range(s.batch):
        n = int(o["n_body"][b])
        SB.assert_scores_within(e[b, :, :, :n], oc.err[b, :, :, :n], bound[b, :, :, :n], f"moved b={b}")


def test_other_admissible_int4_scales_and_codes_within_bounds():
    """int4: per 32-value group one admissible scale (fp16 of max|x| / 7
    for a max|x| within the noise), then per value one admissible code under
    that scale, drawn at random; the rows' scores stay within the bounds."""
    s, o, oc, ck, noise, bound = case("int4")
    c = oc.coef_exact
    rng = np.random.default_rng(3)
    grp = c.shape[:-1] + (-1, 32)
    amax = np.abs(c.reshape(grp)).max(-1)
    nz = noise.reshape(grp).max(-1)
    slack = nz / 7.0 + 2.0 ** -23 * amax / 7.0
    ends = [np.maximum(amax / 7.0 - slack, 0.0), amax / 7.0 + slack]
    pick = rng.integers(0, 2, size=amax.shape)
    sc = np.repeat(np.asarray(O.f64_to_f16(np.where(pick == 0, ends[0], ends[1])), np.float64), 32, axis=-1)
    safe = np.where(sc > 0, sc, 1.0)
    side = np.where(rng.integers(0, 2, size=c.shape) == 0, -1.0, 1.0)
    C_alt = np.where(sc > 0, np.clip(np.rint((c + side * noise) / safe), -7, 7) * sc, 0.0)
    C = O.dequant_store(oc.coef, ck)
    n = int(o["n_body"][0])
    assert np.any(C_alt[0, :n] != C[0, :n])
    e = _emulated_all(s, o, oc, ck, C_alt)
    SB.assert_scores_within(e[0, :, :, :n], oc.err[0, :, :, :n], bound[0, :, :, :n], "int4 moved")


@pytest.mark.parametrize("name", ["bf16", "int4", "f32"])
def test_bounds_decide_almost_every_row(name):
    s, o, oc, ck, noise, bound = case(name)
    stats = SB.SelectionStats()
    for b in range(s.batch):
        n = int(o["n_body"][b])
        for l in range(s.group_layers):
            for h in range(s.n_kv_heads):
                SB.check_selection(oc.resid_idx[b, l, h], oc.err[b, l, h], oc.err[b, l, h], bound[b, l, h], n,
                                   s.n_resid, "self", stats)
    assert stats.mismatched == 0
    print(name, stats.summary())
    if name != "int4":            # int4: see gpu_helpers.MAX_BAND_FRAC
        assert stats.band <= 0.05 * stats.rows, stats.summary()


def test_planted_score_error_fails():
    """Scores 1 % off on the ordinary rows (below the 90th percentile of
    their list) fail the per-row check."""
    s, o, oc, ck, noise, bound = case("bf16")
    n = int(o["n_body"][0])
    e = oc.err[0, 0, 0, :n].copy()
    ordinary = e < np.quantile(e, 0.9)
    bad = np.where(ordinary, e * 1.01, e)
    with pytest.raises(AssertionError):
        SB.assert_scores_within(bad, oc.err[0, 0, 0, :n], bound[0, 0, 0, :n], "planted")
    SB.assert_scores_within(e, oc.err[0, 0, 0, :n], bound[0, 0, 0, :n], "unchanged")


def test_planted_swap_fails():
    """A chosen row swapped for the lowest-scoring row: the list is the top-m
    of scores constructed to produce it, but the oracle's scores of the two
    rows are far apart, which the bounds do not allow."""
    s, o, oc, ck, noise, bound = case("bf16")
    n = int(o["n_body"][0])
    m = s.n_resid
    e_ref = oc.err[0, 0, 0]
    ref = SB.top_m_rows(e_ref[:n], m)
    low = int(np.argmin(e_ref[:n]))
    drop = int(ref[len(ref) // 2])
    e_lib = e_ref.copy()
    e_lib[low], e_lib[drop] = e_ref[drop], e_ref[low]
    lst = np.full(m, O.INT32_MAX, dtype=np.int64)
    lst[:m] = SB.top_m_rows(e_lib[:n], m)
    assert low in lst and drop not in lst
    with pytest.raises(AssertionError, match="bounds allow"):
        SB.check_selection(lst, e_lib, e_ref, bound[0, 0, 0], n, m, "planted swap")
    SB.check_selection(ref, e_ref, e_ref, bound[0, 0, 0], n, m, "unchanged")


def test_list_not_top_m_of_its_scores_fails():
    s, o, oc, ck, noise, bound = case("bf16")
    n = int(o["n_body"][0])
    m = s.n_resid
    e_ref = oc.err[0, 0, 0]
    lst = SB.top_m_rows(e_ref[:n], m).copy()
    outside = np.setdiff1d(np.arange(n), lst)
    lst[0] = outside[0]
    with pytest.raises(AssertionError, match="not the top"):
        SB.check_selection(np.sort(lst), e_ref, e_ref, bound[0, 0, 0], n, m, "planted list")


def test_near_tie_swap_is_allowed():
    """Two rows whose exact scores differ by less than their bounds may be
    chosen either way."""
    s, o, oc, ck, noise, bound = case("bf16")
    n = int(o["n_body"][0])
    m = s.n_resid
    e_ref = oc.err[0, 0, 0, :n]
    order = np.lexsort((np.arange(n), -e_ref))
    x, y = int(order[m - 1]), int(order[m])          # the last chosen row and the first unchosen one
    if e_ref[x] - e_ref[y] > bound[0, 0, 0, x] + bound[0, 0, 0, y]:
        pytest.skip("no near-tie at the threshold of this list")
    e_lib = e_ref.copy()
    e_lib[x], e_lib[y] = e_ref[y], e_ref[x]
    lst = SB.top_m_rows(e_lib, m)
    SB.check_selection(lst, e_lib, e_ref, bound[0, 0, 0, :n], n, m, "near tie")
