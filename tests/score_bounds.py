"""Per-row error bounds of the library's prefill scores, and the check of a
residual selection against the oracle's scores with them.  Test
infrastructure: numpy over the oracle's own quantities.

The score of body row t for (sequence b, layer l, KV head h) is
e = sum_j (v_j - f_j)^2, f = W2 gelu(W1 k^ + b1) + b2, k^ the key rebuilt
from the stored coefficients ("LowRAM Paper: Amortised Values and Low-Rank
Keys for KV Compression", section "Value cache amortisation in plain
language": the per-token reconstruction error that decides which rows keep a
residual).  The oracle evaluates it in fp64; the library in fp32 arithmetic
whose activation operands are bf16 pairs (|x - hi - lo| <= 2^-16 |x|) and
whose GELU is the exact-erf form.  A library score may therefore differ from
the oracle's by

  (1) the rounding of that arithmetic, and
  (2) a stored coefficient of the row that differs by one storage unit: where
      the exact coefficient lies within the projection's fp32 noise of a
      rounding boundary, either stored value is correct (the coefficient rule
      of the prefill parity tests).

(1) To first order the score error is a linear form in the individual
rounding errors: e_lib - e = sum_s a_s eps_s with |eps_s| <= b_s, where a_s is
the derivative of e with respect to the rounded quantity (computed here from
the oracle's values: g = W1^T (gelu'(z) o (W2^T r)), r = v - f, carries the
sensitivity of e to the rebuilt key) and b_s the rounding's magnitude bound.
Rounding errors are taken as independent and mean-zero (the standard
probabilistic model of round-to-nearest); an fp32 sum of n terms contributes
n addition roundings each bounded by u * sum |terms| (u = 2^-24; Higham and
Mary, "A New Approach to Probabilistic Rounding Error Analysis", SIAM J. Sci.
Comput. 41 (2019)).  Hoeffding's inequality then gives

  P(|sum_s a_s eps_s| >= lam * sqrt(sum_s a_s^2 b_s^2)) <= 2 exp(-lam^2 / 2),

2.5e-14 per score at lam = 8, the value used here.  Second-order terms are
bounded by norms (GELU' <= 1.13, |GELU''| <= 0.8).

(2) is bounded in the worst case over the admissible stored values: with
G = de/dc = -2 B g, |de| <= the largest over the decided scenarios of
|sum_k dc_k G_k| plus sum over the open values of |dc_k| |G_k|, plus its
second-order term; which values are open, and how far each may move, come
from the oracle's exact (pre-rounding) coefficients alone.

A selection is integer work decided by these scores, so the library's
residual list must be exactly the top-m of its own exported scores, and may
differ from the oracle's own top-m only in a way the bounds allow: for every
row x the library chose and the oracle did not, and every row y the oracle
chose and the library did not, e(x) + bound(x) >= e(y) - bound(y).
"""
from __future__ import annotations

import numpy as np

import oracle as O

LAM = 8.0                   # Hoeffding factor (2 exp(-32) per score)
U32 = 2.0 ** -24            # fp32 unit roundoff
SPLIT = 2.0 ** -16          # bf16 pair split: |x - hi - lo| <= 2^-16 |x| (bf16 inputs)
GELU_D1 = 1.13              # max |GELU'|
GELU_D2 = 0.8               # max |GELU''|
GELU_EVAL = 8 * U32         # exact-erf GELU in fp32: |err| <= 8u (|gelu(z)| + |z|)


def projection_magnitude(k_post, pos, n_body, basis, theta: float) -> np.ndarray:
    """S[b, t, k] = sum_c |basis[b, k, c]| |x[b, t, c]| over the pre-RoPE key
    row x (the oracle's inverse rotation of k_post): the scale of the
    rounding error of coefficient (t, k) when the projection is summed in
    fp32; the coefficient rule of the prefill tests allows 2^-20 S (zero for
    padding rows)."""
    B, G, N, H, d = k_post.shape
    S = np.zeros((B, N, basis.shape[1]))
    for b in range(B):
        n = int(n_body[b])
        if n == 0:
            continue
        p = np.arange(N) if pos is None else np.asarray(pos[b])
        k_pre = O.rope_rotate(k_post[b, :, :n].transpose(0, 2, 1, 3), p[:n], theta, inverse=True)
        X = k_pre.transpose(2, 0, 1, 3).reshape(n, -1)
        S[b, :n] = np.abs(X) @ np.abs(basis[b]).T
    return S


def coef_deviation(coef_exact: np.ndarray, coef_stored, kind: str, noise: np.ndarray) -> dict:
    """How far the library's stored coefficients may lie from the oracle's.
    The library stores the rounding of its own fp32 projection, which lies
    within `noise` (the projection's fp32 noise bound) of the exact
    coefficient c; every value the storage rounding gives for an input in
    [c - noise, c + noise] is admissible.  The rounding is monotone in its
    input, so the interval's ends give every candidate.

    Returns a dict of [..., r] arrays:
      "det": list over scenarios of deviations that are decided once the
             scenario is (int4: the group scale is fp16(max|x| / 7) of the
             library's own values, whose max|x| lies within the group's
             largest noise of the exact one, divided in fp32: one scenario
             per candidate scale; the codes of a scenario move together);
      "amb": per scenario, the largest deviation of a value whose rounding
             the noise leaves open (independent of the others);
      "rand": fp32 storage only: the deviation (noise plus one fp32 unit) is
             the arithmetic's own rounding noise, independent per value.
    bf16 has one scenario with nothing decided: each value rounds on its own.
    """
    c = np.asarray(coef_exact, dtype=np.float64)
    zero = np.zeros_like(c)
    if kind == "f32":
        return {"det": [zero], "amb": [zero], "rand": noise + U32 * np.abs(c)}
    ref = O.dequant_store(coef_stored, kind)
    if kind == "bf16":
        lo = O.bf16_bits_to_f64(O.f64_to_bf16_bits(c - noise))
        hi = O.bf16_bits_to_f64(O.f64_to_bf16_bits(c + noise))
        return {"det": [zero], "amb": [np.maximum(np.abs(lo - ref), np.abs(hi - ref))], "rand": None}
    assert kind == "int4"
    grp = c.shape[:-1] + (-1, 32)
    amax = np.abs(c.reshape(grp)).max(-1)
    nz = noise.reshape(grp).max(-1)
    slack = nz / 7.0 + 2.0 ** -23 * amax / 7.0
    det, amb = [], []
    for s_end in (np.maximum(amax / 7.0 - slack, 0.0), amax / 7.0 + slack):
        sc = np.repeat(np.asarray(O.f64_to_f16(s_end), dtype=np.float64), 32, axis=-1)
        safe = np.where(sc > 0, sc, 1.0)
        v_lo = np.where(sc > 0, np.clip(np.rint((c - noise) / safe), -7, 7) * sc, 0.0)
        v_hi = np.where(sc > 0, np.clip(np.rint((c + noise) / safe), -7, 7) * sc, 0.0)
        same = v_lo == v_hi
        det.append(np.where(same, v_lo - ref, 0.0))
        amb.append(np.where(same, 0.0, np.maximum(np.abs(v_lo - ref), np.abs(v_hi - ref))))
    return {"det": det, "amb": amb, "rand": None}


def deviation_rows(dev: dict, b: int, n: int) -> dict:
    """The deviations of rows [0, n) of sequence b."""
    return {k: (None if v is None else ([x[b, :n] for x in v] if isinstance(v, list) else v[b, :n]))
            for k, v in dev.items()}


def coef_term(dev: dict, G: np.ndarray) -> np.ndarray:
    """Worst case over the admissible stored coefficients of |sum_k dc_k G_k|
    per row, G = de/dc: the largest over the scenarios of the decided
    deviations' signed sum (per 32-value group for int4: a scenario fixes a
    group's scale, not the others') plus the open values' absolute terms."""
    n, r = G.shape
    worst = np.zeros(n)
    grp = (n, r // 32, 32) if r % 32 == 0 else (n, 1, r)
    best = None
    for det, amb in zip(dev["det"], dev["amb"]):
        t = np.abs(np.sum((det * G).reshape(grp), -1)) + np.sum((amb * np.abs(G)).reshape(grp), -1)
        best = t if best is None else np.maximum(best, t)
    worst += best.sum(-1)
    return worst


def deviation_abs(dev: dict) -> np.ndarray:
    """The largest absolute deviation of each value over the scenarios."""
    return np.max([np.abs(d) + a for d, a in zip(dev["det"], dev["amb"])], axis=0)


def head_bounds(k: np.ndarray, C: np.ndarray, Bs: np.ndarray, W1, b1, W2, b2, v: np.ndarray,
                dev: dict | None = None, op: float = SPLIT, lam: float = LAM):
    """Score and score-error bound of n rows of one (sequence, layer, head).

    k [n, d]: the oracle's rebuilt pre-RoPE keys of the head (from its stored
    coefficients); C [n, r]: those stored coefficients (dequantised);
    Bs [r, d]: the head's basis columns; v [n, d]; dev: the rows'
    coefficient deviations (coef_deviation; None: the library's stored
    coefficients are the oracle's); op: the relative rounding of the activation
    operands (SPLIT for bf16 inputs, whose products take bf16 pairs; U32
    for fp32 inputs, whose arithmetic is fp32 throughout).  The stored coefficients
    (bf16, or int4 code * scale as an exact bf16 pair) times the bf16 basis
    are exact products; the rebuild's error is its fp32 sum.  Returns
    (e, bound)."""
    W1, W2 = np.asarray(W1, np.float64), np.asarray(W2, np.float64)
    n, d = k.shape
    r = Bs.shape[0]
    z = k @ W1.T + b1
    hd = O.gelu(z)
    gp = O.gelu_grad(z)
    f = hd @ W2.T + b2
    rr = v - f
    e = np.sum(rr * rr, -1)
    w2r = rr @ W2                        # de/dh = -2 W2^T r
    gz = w2r * gp                        # de/dz = -2 gelu'(z) o W2^T r
    g = gz @ W1                          # de/dk = -2 W1^T (...)
    ak, aC, aB = np.abs(k), np.abs(C), np.abs(Bs)
    Mk = aC @ aB                         # sum_k |c_k B_ki|: scale of the rebuild's fp32 sum (r terms)
    Mz = ak @ np.abs(W1).T               # scale of z's sums (2 d terms: both halves of the pair)
    Mf = np.abs(hd) @ np.abs(W2).T       # scale of f's sums (2 d terms)
    # (1) variance-style sum of (a_s b_s)^2 over the independent roundings
    V = np.sum((2 * g * op * ak) ** 2, -1) + r * np.sum((2 * g * U32 * Mk) ** 2, -1)
    dk2 = (op * ak) ** 2 + r * (U32 * Mk) ** 2
    V += 2 * d * np.sum((2 * gz * U32 * Mz) ** 2, -1)
    dh = GELU_EVAL * (np.abs(hd) + np.abs(z)) + op * np.abs(hd)
    V += np.sum((2 * w2r * dh) ** 2, -1)
    V += 2 * d * np.sum((2 * rr * U32 * Mf) ** 2, -1)
    V += np.sum((2 * rr * U32 * np.abs(rr)) ** 2, -1) + np.sum((U32 * rr * rr) ** 2, -1) + d * (U32 * e) ** 2
    rand = None if dev is None else dev["rand"]
    if rand is not None and rand.any():
        V += np.sum((2 * (g @ Bs.T) * rand) ** 2, -1)
        dk2 += (rand * rand) @ (Bs * Bs)
    bound = lam * np.sqrt(V)
    # second order of (1): |de - linear| <= |df|^2 + 2 |r| |W2| |gelu''|/2 |dz|^2
    nW1, nW2 = np.linalg.norm(W1, 2), np.linalg.norm(W2, 2)
    ndk = lam * np.sqrt(np.sum(dk2, -1))
    ndz = nW1 * ndk + lam * np.sqrt(2 * d * np.sum((U32 * Mz) ** 2, -1))
    ndf = nW2 * (GELU_D1 * ndz + np.linalg.norm(dh, axis=-1)) + lam * np.sqrt(2 * d * np.sum((U32 * Mf) ** 2, -1))
    nr = np.linalg.norm(rr, axis=-1)
    bound += ndf ** 2 + nr * nW2 * GELU_D2 * ndz ** 2
    # (2) stored coefficients that may differ from the oracle's
    if dev is not None:
        units = deviation_abs(dev)
        amb = units.any(-1)
        if amb.any():
            G = np.zeros((n, r))
            G[amb] = -2 * (g[amb] @ Bs.T)                          # de/dc = -2 B (W1^T ...)
            bound += coef_term(dev, G)
            dkc = units @ np.linalg.norm(Bs, axis=-1)             # |dk| <= sum_k |dc_k| |B_k|
            dzc = nW1 * dkc
            bound += (nW2 * GELU_D1 * dzc) ** 2 + nr * nW2 * GELU_D2 * dzc ** 2
    return e, bound


def _pred(arr, b, l, h):
    """Predictor tensor of (b, l, h); a batch dimension of 1 is shared."""
    arr = np.asarray(arr, dtype=np.float64)
    return arr[0 if arr.shape[0] == 1 else b, l, h]


def score_bounds(coef_stored, coef_kind: str, coef_exact, khat, basis, W1, b1, W2, b2, v, n_body,
                 noise: np.ndarray, op: float = SPLIT, lam: float = LAM) -> np.ndarray:
    """bound[b, l, h, t] on |e_library - e_oracle| for every body row (0 for
    padding rows).  coef_stored / coef_exact / khat: the oracle's stored and
    exact coefficients and its rebuilt keys ([B, N, r], [B, N, r],
    [B, N, D]); noise [B, N, r]: the projection's fp32 noise bound of each
    coefficient; v [B, G, N, Hkv, d]; op as in head_bounds."""
    B, G, N, H, d = v.shape
    Cq = O.dequant_store(coef_stored, coef_kind)
    dev = coef_deviation(coef_exact, coef_stored, coef_kind, noise)
    out = np.zeros((B, G, H, N))
    for b in range(B):
        n = int(n_body[b])
        if n == 0:
            continue
        for l in range(G):
            for h in range(H):
                c0 = (l * H + h) * d
                _, bd = head_bounds(khat[b, :n, c0:c0 + d], Cq[b, :n], basis[b][:, c0:c0 + d],
                                    _pred(W1, b, l, h), _pred(b1, b, l, h), _pred(W2, b, l, h), _pred(b2, b, l, h),
                                    v[b, l, :n, h], deviation_rows(dev, b, n), op, lam)
                out[b, l, h, :n] = bd
    return out


def assert_scores_within(e_lib: np.ndarray, e_ref: np.ndarray, bound: np.ndarray, what: str):
    """Every score within its row's bound."""
    err = np.abs(np.asarray(e_lib, np.float64) - e_ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(bound, 1e-300), 0)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} scores outside their bound; worst at {i}: "
                             f"library {e_lib[i]:.9g} oracle {e_ref[i]:.9g} bound {bound[i]:.3g}")


def top_m_rows(e: np.ndarray, m: int) -> np.ndarray:
    """The m rows with the largest finite scores e (ties to the lower row),
    ascending: the selection rule applied to scores the test holds."""
    assert np.all(np.isfinite(e))
    order = np.lexsort((np.arange(len(e)), -e))
    return np.sort(order[:m])


class SelectionStats:
    """Counts over the checked lists: rows, rows chosen differently from the
    oracle's own selection, and rows whose membership in the top-m the score
    bounds leave open (the only rows where a difference is allowed)."""

    def __init__(self):
        self.lists = self.rows = self.mismatched = self.band = 0

    def add(self, n, mism, band):
        self.lists += 1
        self.rows += n
        self.mismatched += mism
        self.band += band

    def summary(self) -> str:
        return (f"{self.lists} lists, {self.rows} rows: {self.mismatched} rows chosen differently from the "
                f"oracle's selection; {self.band} rows ({100.0 * self.band / max(self.rows, 1):.3f} %) whose "
                f"membership the score bounds leave open")


def check_selection(idx_list, e_lib: np.ndarray, e_ref: np.ndarray, bound: np.ndarray, n: int, m: int, what: str,
                    stats: SelectionStats | None = None):
    """One residual list (m slots, ascending, INT32_MAX padding) of the
    library: exactly the top-min(m, n) of its own exported scores e_lib,
    and against the oracle's exact scores e_ref: every difference from the
    oracle's own top-m is one the score bounds allow."""
    k = min(m, n)
    got = np.asarray(idx_list, dtype=np.int64)
    assert np.all(got[k:] == O.INT32_MAX), f"{what}: padding slots"
    chosen = got[:k]
    assert np.array_equal(chosen, top_m_rows(np.asarray(e_lib[:n], np.float64), k)), \
        f"{what}: not the top {k} of the exported scores"
    if k == 0 or k == n:
        if stats is not None:
            stats.add(n, 0, 0)
        return
    e, bd = e_ref[:n], bound[:n]
    ref = top_m_rows(e, k)
    lib_only = np.setdiff1d(chosen, ref)
    ref_only = np.setdiff1d(ref, chosen)
    if len(lib_only):
        lo = np.min(e[lib_only] + bd[lib_only])
        hi = np.max(e[ref_only] - bd[ref_only])
        assert lo >= hi, (f"{what}: the library chose rows {lib_only[:8]} over {ref_only[:8]}; their exact scores "
                          f"differ by more than the bounds allow ({lo:.9g} < {hi:.9g})")
    # rows whose membership the bounds leave open: a chosen row is settled
    # when its lowest admissible score exceeds every unchosen row's highest
    # one, and an unchosen row when its highest is below every chosen row's
    # lowest
    inside = np.zeros(n, dtype=bool)
    inside[ref] = True
    lo_in = np.min(e[inside] - bd[inside])
    hi_out = np.max(e[~inside] + bd[~inside])
    band = int(np.sum(inside & (e - bd <= hi_out)) + np.sum(~inside & (e + bd >= lo_in)))
    if stats is not None:
        stats.add(n, len(lib_only), band)
