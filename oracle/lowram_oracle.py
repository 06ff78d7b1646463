"""Plain, slow fp64 CPU oracle of the LowRAM prefill and decode path.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

Sources (cited by short name below):
  [ABS]  arXiv listing of "LowRAM: Low-Rank Keys and Amortised Values for
         Composable KV Cache Compression at Test-Time" (arXiv:2611.07025),
         Abstract.
  [WIKI] "LowRAM: predict values from keys, store only the misses"
         (cere-bro wiki note): TL;DR, data-flow flowchart, Key points.
  [EXPL] "LowRAM Paper: Amortised Values and Low-Rank Keys for KV
         Compression" (wpnews copy of an explainx.ai post): sections
         "Value cache amortisation in plain language", "Asymmetric key
         compression with xKV", "Step-by-step mental model for one decoding
         session", "Benchmarks and composability".

Arithmetic is float64 throughout.  The only rounding steps are the storage
roundings that are part of the method (stored coefficients, stored residuals
and int4 scales); every other quantity is exact up to fp64 rounding.

Where the pages leave a step open the oracle takes one plain reading; each
such reading is named R<n> in the docstring that applies it.

Pinning: every public function here is pinned by a CPU test against closed
forms, textbook values, library routines or brute force (tests/test_oracle_*).
No function is "parity unpinned".

Array conventions (all row-major, numpy):
  q          [B, Hq, d]               post-RoPE query of the new token
  k_post, v  [B, G, N, Hkv, d]        prompt-body keys (post-RoPE) and values
  pos        [B, N] int or None       original token position of body row t
  n_body     [B] int                  valid body rows per sequence
  basis      [B, r, D], D = G*Hkv*d   column (l*Hkv + h)*d + j
  W1, W2     [B or 1, G, Hkv, d, d]   [out, in]: hidden = W1 @ k + b1
  b1, b2     [B or 1, G, Hkv, d]
  coef       [B, N, r]                stored coefficients
  resid_idx  [B, G, Hkv, m] ascending, padded with INT32_MAX past n_body
  resid_val  [B, G, Hkv, m, d]
  tail_k/v   [B, G, Te, Hkv, d] post-RoPE exact rows, tail_len [B]
  subset     list of B sorted int arrays (body rows) or None
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "INT32_MAX", "bf16_bits_to_f64", "f64_to_bf16_bits", "f64_to_f32",
    "f64_to_f16", "Storage", "round_store", "dequant_store",
    "int4_quantize_g32", "int4_dequantize_g32", "int4_pack", "int4_unpack",
    "rope_inv_freq", "rope_rotate", "gelu", "predictor",
    "select_worst", "prefill", "append_body", "decode", "attention_exact",
    "merge_partials", "OracleCache", "gelu_grad", "predictor_loss_grad",
    "adam_update", "fit_predictor", "FitResult", "pre_rope_keys", "key_basis",
    "orth_columns", "key_basis_iteration", "subset_policy",
]

INT32_MAX = 2**31 - 1


# ---------------------------------------------------------------------------
# number formats (storage rounding; R14, R18)
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to bfloat16 with round-to-nearest-even, directly from
    the fp64 value (no intermediate fp32 rounding).  NaN maps to 0x7FC0.

    bfloat16 keeps 8 significant bits and the fp32 exponent range (smallest
    subnormal 2**-133).  With a = m * 2**e (frexp), the leading bit has
    weight 2**(e-1); the value is rounded to a multiple of
    q = 2**max(e-1-7, -133) with np.rint (ties to even).  Results of 2**128
    or more become infinity.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)
    lead = e.astype(np.int64) - 1
    qexp = np.where(lead < -126, -133, lead - 7)
    with np.errstate(over="ignore", invalid="ignore"):
        n = np.rint(np.ldexp(a, -qexp))
        r = np.ldexp(n, qexp)
        r32 = np.where(r >= 2.0**128, np.inf, r).astype(np.float32)
    bits = (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = np.where(a == 0, np.uint16(0), bits)
    bits = np.where(np.signbit(x), bits | np.uint16(0x8000), bits)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 to float32 (numpy's cast rounds to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f64_to_f16(x: np.ndarray) -> np.ndarray:
    """Round float64 to IEEE binary16, round-to-nearest-even (numpy cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


# ---------------------------------------------------------------------------
# int4 with one fp16 scale per 32 consecutive elements (R13, R14)
# [ABS] composition with quantisation; [EXPL] "Benchmarks and
# composability" (4-bit KV stacked on LowRAM)
# ---------------------------------------------------------------------------

def int4_quantize_g32(x: np.ndarray):
    """Symmetric int4 quantisation in groups of 32 along the last axis.

    Reading R14: s = fp16(max|x| / 7) rounded to nearest even and saturated
    to the largest finite fp16; code = clamp(rint(x / s), -7, 7) using the
    fp16-rounded s; a group whose s rounds to 0 gets codes 0.
    Returns (codes int8 [..., n], scales float16 [..., n // 32]).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % 32:
        raise ValueError("int4 groups need a multiple of 32 elements")
    g = x.reshape(x.shape[:-1] + (n // 32, 32))
    amax = np.abs(g).max(axis=-1)
    s16 = np.minimum(f64_to_f16(amax / 7.0).astype(np.float64), 65504.0)
    s16 = s16.astype(np.float16)
    s = s16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.where(s > 0, np.rint(g / np.where(s > 0, s, 1.0)), 0.0)
    c = np.clip(c, -7, 7).astype(np.int8)
    return c.reshape(x.shape), s16


def int4_dequantize_g32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """x_hat = code * s, exact in float64."""
    codes = np.asarray(codes).astype(np.float64)
    n = codes.shape[-1]
    s = np.asarray(scales).astype(np.float64)
    g = codes.reshape(codes.shape[:-1] + (n // 32, 32)) * s[..., None]
    return g.reshape(codes.shape)


def int4_pack(codes: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, element 2i in the low nibble of byte i."""
    c = np.asarray(codes).astype(np.int16) & 0xF
    lo = c[..., 0::2]
    hi = c[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def int4_unpack(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


@dataclass
class Storage:
    """How one stored tensor is held: 'f64' (no rounding; oracle-only test
    mode), 'f32', 'bf16', or 'int4' (int4 codes + fp16 scale per 32)."""
    kind: str


def round_store(x: np.ndarray, kind: str):
    """Apply the storage rounding of the method (R18).  Returns the stored
    representation: f64/f32 array, bf16 bit patterns, or (packed, scales)."""
    if kind == "f64":
        return np.asarray(x, dtype=np.float64).copy()
    if kind == "f32":
        return f64_to_f32(x)
    if kind == "bf16":
        return f64_to_bf16_bits(x)
    if kind == "int4":
        codes, scales = int4_quantize_g32(x)
        return int4_pack(codes), scales
    raise ValueError(kind)


def dequant_store(stored, kind: str) -> np.ndarray:
    """Exact float64 value of a stored tensor."""
    if kind in ("f64", "f32"):
        return np.asarray(stored, dtype=np.float64)
    if kind == "bf16":
        return bf16_bits_to_f64(stored)
    if kind == "int4":
        packed, scales = stored
        return int4_dequantize_g32(int4_unpack(packed), scales)
    raise ValueError(kind)


# ---------------------------------------------------------------------------
# rotary position embedding (R9)
# [EXPL] "Asymmetric key compression with xKV": RoPE is inverted before the
# keys are compressed and reapplied during attention.
# ---------------------------------------------------------------------------

def rope_inv_freq(d: int, theta: float) -> np.ndarray:
    """omega_i = theta ** (-2 i / d), i = 0 .. d/2-1, in float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return theta ** (-2.0 * i / d)


def rope_rotate(x: np.ndarray, pos: np.ndarray, theta: float,
                inverse: bool = False) -> np.ndarray:
    """Rotate-half RoPE (R9): for i < d/2 the pair (x_i, x_{i+d/2}) turns by
    angle pos * omega_i; inverse=True turns by -pos * omega_i.

    x: [..., T, d] (or any shape whose second-to-last axis matches pos after
    broadcasting); pos: [T] (integer positions).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(d, theta)[None, :]
    if inverse:
        ang = -ang
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    # broadcast [T, half] against [..., T, half]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ---------------------------------------------------------------------------
# value predictor (R1, R15, R16)
# [EXPL] "Value cache amortisation in plain language": a small per-head MLP
# maps each token's key to its value.
# ---------------------------------------------------------------------------

def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def predictor(k: np.ndarray, W1, b1, W2, b2) -> np.ndarray:
    """f(k) = W2 GELU(W1 k + b1) + b2 for rows k [..., d]; W are [out, in]."""
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    hidden = gelu(k @ W1.T + np.asarray(b1, dtype=np.float64))
    return hidden @ W2.T + np.asarray(b2, dtype=np.float64)


# ---------------------------------------------------------------------------
# worst-token selection (R4, R5, R6)
# [ABS] residuals are kept only for the tokens the predictor reconstructs
# worst; [WIKI] data-flow flowchart (the residual store holds the worst
# tokens alone).
# ---------------------------------------------------------------------------

def _desc_key(e: float):
    """Sort key for 'larger error first' with NaN above +inf (R6)."""
    if math.isnan(e):
        return (0, 0.0)
    return (1, -e)


def select_worst(err: np.ndarray, m: int) -> np.ndarray:
    """The m rows with the largest error, ties broken by the lower row index,
    returned in ascending row order (brute force: a full sort)."""
    err = np.asarray(err, dtype=np.float64)
    n = err.shape[0]
    if not 0 <= m:
        raise ValueError("m must be >= 0")
    order = sorted(range(n), key=lambda t: (_desc_key(float(err[t])), t))
    return np.array(sorted(order[:m]), dtype=np.int64)


# ---------------------------------------------------------------------------
# prefill (P1..P6)
# [EXPL] "Step-by-step mental model ..." item 1 and "Value cache amortisation
# in plain language": invert RoPE, compress keys on a shared low-rank basis
# across the layer group, predict values from the keys, score the error per
# token and keep residuals for the worst predictions.
# ---------------------------------------------------------------------------

def _w(arr, b, l, h):
    """Predictor tensor of (sequence b, layer l, head h); batch dim 1 means
    shared by every sequence (R15)."""
    arr = np.asarray(arr)
    bb = 0 if arr.shape[0] == 1 else b
    return arr[bb, l, h]


@dataclass
class OracleCache:
    """Stored compressed cache of one layer group, in storage form."""
    coef: object            # stored coefficients (see round_store)
    coef_kind: str
    resid_idx: np.ndarray   # [B, G, Hkv, m] int64
    resid_val: object       # stored residuals [B, G, Hkv, m, d]
    resid_kind: str
    err: np.ndarray = field(default=None)     # [B, G, Hkv, N] fp64 scores
    khat_pre: np.ndarray = field(default=None)  # [B, N, D] rebuilt pre-RoPE keys
    coef_exact: np.ndarray = field(default=None)  # [B, N, r] coefficients before storage rounding


def prefill(k_post, v, pos, n_body, basis, W1, b1, W2, b2, m: int,
            theta: float, coef_kind: str, resid_kind: str,
            err_override=None) -> OracleCache:
    """Compress one layer group (c2 steps 1-7).

    k_post, v: [B, G, N, Hkv, d] float; basis [B, r, D].  Rows t >= n_body[b]
    are padding: their coefficients are stored as 0, their error is 0 and
    they are never selected; when m > n_body[b] the trailing index slots
    hold INT32_MAX with zero residuals.

    err_override: optional [B, G, Hkv, N] scores used for the selection in
    place of the oracle's own (used to check a selection bit-exactly on
    another implementation's exported scores).
    """
    k_post = np.asarray(k_post, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    basis = np.asarray(basis, dtype=np.float64)
    B, G, N, H, d = k_post.shape
    r, D = basis.shape[1], basis.shape[2]
    assert D == G * H * d
    coef = np.zeros((B, N, r))
    khat_all = np.zeros((B, N, D))
    err = np.zeros((B, G, H, N))
    idx = np.full((B, G, H, m), INT32_MAX, dtype=np.int64)
    res = np.zeros((B, G, H, m, d))
    for b in range(B):
        n = int(n_body[b])
        p = np.arange(N) if pos is None else np.asarray(pos[b])
        # P1: undo the rotation of every key (R9); rows on the second-to-last axis
        k_pre = rope_rotate(k_post[b, :, :n].transpose(0, 2, 1, 3), p[:n], theta,
                            inverse=True)                       # [G, H, n, d]
        # P2: concatenate (layer, head, dim) -> one D-vector per token and
        # project on the basis rows (R7, R8)
        X = k_pre.transpose(2, 0, 1, 3).reshape(n, D)
        coef[b, :n] = X @ basis[b].T
    # storage rounding of the coefficients (part of the method, R18)
    coef_st = round_store(coef, coef_kind)
    coef_q = dequant_store(coef_st, coef_kind)
    for b in range(B):
        n = int(n_body[b])
        # P3: rebuild from the stored coefficients; decode sees only these
        khat = coef_q[b, :n] @ basis[b]                   # [n, D]
        khat_all[b, :n] = khat
        kh = khat.reshape(n, G, H, d)
        for l in range(G):
            for h in range(H):
                # P4: predict and score (R1, R3)
                f = predictor(kh[:, l, h], _w(W1, b, l, h), _w(b1, b, l, h),
                              _w(W2, b, l, h), _w(b2, b, l, h))
                e = np.sum((v[b, l, :n, h] - f) ** 2, axis=-1)
                err[b, l, h, :n] = e
                # P5: exact worst-m selection (R4-R6)
                e_sel = e if err_override is None else np.asarray(err_override)[b, l, h, :n]
                S = select_worst(e_sel, min(m, n))
                idx[b, l, h, :len(S)] = S
                # P6: residual = value - prediction at the selected rows (R2)
                res[b, l, h, :len(S)] = v[b, l, S, h] - f[S]
    res_st = round_store(res, resid_kind)
    return OracleCache(coef=coef_st, coef_kind=coef_kind, resid_idx=idx,
                       resid_val=res_st, resid_kind=resid_kind, err=err,
                       khat_pre=khat_all, coef_exact=coef)


# ---------------------------------------------------------------------------
# appending exact rows to the compressed body (tail lifecycle)
# [EXPL] "Asymmetric key compression with xKV", last paragraph: newly decoded
# tokens keep exact K/V.  Folding some of them into the compressed body is
# read here as the prefill steps applied to those rows with the sequence's
# existing basis and predictor (R23); rows and residuals already stored stay
# as they are, since their exact values are no longer held.
# ---------------------------------------------------------------------------

def _rows_copy(dst, src, kind, put):
    """Apply put(dst_array, src_array) to every array of a storage form."""
    if kind == "int4":
        put(dst[0], src[0])
        put(dst[1], src[1])
    else:
        put(dst, src)


def _storage_copy(x, kind):
    if kind == "int4":
        return (np.array(x[0], copy=True), np.array(x[1], copy=True))
    return np.array(x, copy=True)


def append_body(cache: OracleCache, n_body, pos, k_post_new, v_new, pos_new, basis,
                W1, b1, W2, b2, m_new: int, theta: float, err_override=None):
    """Fold n_new exact rows per sequence into a stored cache (R23).

    cache: stored coefficients [B, N, r] (N = rows allocated, at least
    n_body[b] + n_new), resid_idx [B, G, Hkv, m] ascending with INT32_MAX
    padding, resid_val.  pos: the cache's positions [B, N] or None (then
    body row t sits at position t, and the new rows at n_body[b] + t).
    k_post_new, v_new [B, G, n_new, Hkv, d]; pos_new [B, n_new] (required
    when pos is not None).

    1. the prefill steps 1-7 on the new rows alone, with the given basis and
       predictor, m_new residual rows chosen among them (err_override: the
       scores to select on, as in prefill);
    2. their coefficients become body rows n_body[b] .. n_body[b] + n_new - 1
       (and their positions are stored there when the cache has positions);
    3. per (b, l, h) the chosen rows, shifted by n_body[b], follow the
       entries already stored (those < n_body[b]), so each list stays
       ascending; their residuals go to the same slots;
    4. n_body grows by n_new.

    Returns (cache, n_body, pos, err of the new rows [B, G, Hkv, n_new]).
    """
    k_post_new = np.asarray(k_post_new, dtype=np.float64)
    B, G, n_new, H, d = k_post_new.shape
    nb = np.asarray(n_body, dtype=np.int64)
    if pos is None:
        p_new = nb[:, None] + np.arange(n_new)[None, :]
    else:
        assert pos_new is not None, "a cache with positions needs the new rows' positions"
        p_new = np.asarray(pos_new, dtype=np.int64)
    mini = prefill(k_post_new, v_new, p_new, np.full(B, n_new), basis, W1, b1, W2, b2, m_new,
                   theta, cache.coef_kind, cache.resid_kind, err_override=err_override)
    coef = _storage_copy(cache.coef, cache.coef_kind)
    idx = np.array(cache.resid_idx, dtype=np.int64, copy=True)
    val = _storage_copy(cache.resid_val, cache.resid_kind)
    m = idx.shape[-1]
    N = (coef[0] if cache.coef_kind == "int4" else coef).shape[1]
    pos_out = None if pos is None else np.array(pos, copy=True)
    for b in range(B):
        n0 = int(nb[b])
        assert n0 + n_new <= N, "no room for the new rows"

        def put_rows(dst, src, b=b, n0=n0):
            dst[b, n0:n0 + n_new] = src[b]
        _rows_copy(coef, mini.coef, cache.coef_kind, put_rows)
        if pos_out is not None:
            pos_out[b, n0:n0 + n_new] = p_new[b]
        for l in range(G):
            for h in range(H):
                count = int(np.sum(idx[b, l, h] < n0))
                new = mini.resid_idx[b, l, h]
                k = int(np.sum(new < n_new))
                assert count + k <= m, "no room for the new residual rows"
                idx[b, l, h, count:count + k] = new[:k] + n0

                def put_res(dst, src, b=b, l=l, h=h, count=count, k=k):
                    dst[b, l, h, count:count + k] = src[b, l, h, :k]
                _rows_copy(val, mini.resid_val, cache.resid_kind, put_res)
    out = OracleCache(coef=coef, coef_kind=cache.coef_kind, resid_idx=idx, resid_val=val,
                      resid_kind=cache.resid_kind)
    return out, nb + n_new, pos_out, mini.err


# ---------------------------------------------------------------------------
# fitting the value predictor at test time (R24)
# [EXPL] "Value cache amortisation in plain language": during prefill a small
# per-head MLP is fitted so that each token's key maps to its value;
# [EXPL] "Step-by-step mental model ..." item 1 and [ABS]: the predictors are
# fitted at test time, from scratch or from a meta-learned initialisation.
# The pages give no loss, optimiser or step count.  Reading R24: the loss of
# one predictor is the mean squared error of f(k^) against v over its body
# rows and the d value components, with k^ the rebuilt pre-RoPE key (R1);
# it is minimised by full-batch Adam (Kingma and Ba, "Adam: A Method for
# Stochastic Optimization", ICLR 2015, Algorithm 1: bias-corrected first
# and second moment estimates) for a fixed number of steps from given
# initial weights, with the hyperparameters as arguments.
# ---------------------------------------------------------------------------

def gelu_grad(x: np.ndarray) -> np.ndarray:
    """Derivative of the exact GELU x Phi(x): Phi(x) + x phi(x), with phi
    the standard normal density."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + _erf(x / math.sqrt(2.0))) + x * np.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def predictor_loss_grad(K, V, W1, b1, W2, b2):
    """Loss L = sum over rows t and components j of (f(k_t)_j - v_tj)^2,
    divided by n d, and its exact gradient (R24).

    K, V [n, d]; W [out, in].  Returns (L, dW1, db1, dW2, db2); with n == 0
    the loss and every gradient are 0.  Chain rule through
    f = W2 A + b2, A = GELU(Z), Z = W1 k + b1:
      dL/dF = 2 (F - V) / (n d)
      dW2 = dF^T A, db2 = column sums of dF, dA = dF W2,
      dZ = dA * GELU'(Z), dW1 = dZ^T K, db1 = column sums of dZ.
    """
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    b1 = np.asarray(b1, dtype=np.float64)
    b2 = np.asarray(b2, dtype=np.float64)
    n, d = K.shape
    if n == 0:
        return 0.0, np.zeros_like(W1), np.zeros_like(b1), np.zeros_like(W2), np.zeros_like(b2)
    Z = K @ W1.T + b1
    A = gelu(Z)
    F = A @ W2.T + b2
    E = F - V
    L = float(np.sum(E * E)) / (n * d)
    dF = 2.0 * E / (n * d)
    dW2 = dF.T @ A
    db2 = dF.sum(axis=0)
    dZ = (dF @ W2) * gelu_grad(Z)
    dW1 = dZ.T @ K
    db1 = dZ.sum(axis=0)
    return L, dW1, db1, dW2, db2


def adam_update(w, g, m, s, t: int, lr: float, beta1: float, beta2: float, eps: float):
    """One Adam step at step number t >= 1 (Kingma and Ba, Algorithm 1):
    m <- beta1 m + (1 - beta1) g, s <- beta2 s + (1 - beta2) g^2,
    w <- w - lr m^ / (sqrt(s^) + eps) with m^ = m / (1 - beta1^t) and
    s^ = s / (1 - beta2^t).  Returns (w, m, s)."""
    m = beta1 * m + (1.0 - beta1) * g
    s = beta2 * s + (1.0 - beta2) * g * g
    mh = m / (1.0 - beta1 ** t)
    sh = s / (1.0 - beta2 ** t)
    return w - lr * mh / (np.sqrt(sh) + eps), m, s


@dataclass
class FitResult:
    """Fitted predictor (R24): float64 weights [P, G, Hkv, ...], the same
    rounded to the weight storage kind, and the loss of every step."""
    W1: np.ndarray
    b1: np.ndarray
    W2: np.ndarray
    b2: np.ndarray
    stored: tuple           # (W1, b1, W2, b2) in storage form (round_store)
    losses: np.ndarray      # [steps, P, G, Hkv]: loss at the weights step s starts from
    grad0: tuple            # (dW1, db1, dW2, db2) at the initial weights


def fit_predictor(coef_stored, coef_kind: str, n_body, basis, v, W1, b1, W2, b2,
                  steps: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                  eps: float = 1e-8, weight_kind: str = "f64") -> FitResult:
    """Fit every (layer, head) predictor of one layer group to its rows (R24).

    coef_stored: stored coefficients [B, N, r] (see round_store); basis
    [B, r, D]; v [B, G, N, Hkv, d]; W1, W2 [P, G, Hkv, d, d] and b1, b2
    [P, G, Hkv, d] are the initial weights, P = B (one predictor per
    sequence) or P = 1 (one predictor shared by the batch, fitted on the rows
    of every sequence).  Rows t < n_body[b] of sequence b take part, their
    keys rebuilt from the stored coefficients (k^ = c B, the keys decode
    sees).  steps full-batch Adam steps; the weights are rounded to
    weight_kind only at the end.
    """
    coef_q = dequant_store(coef_stored, coef_kind)
    basis = np.asarray(basis, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, G, N, H, d = v.shape
    W1 = np.array(W1, dtype=np.float64)
    b1 = np.array(b1, dtype=np.float64)
    W2 = np.array(W2, dtype=np.float64)
    b2 = np.array(b2, dtype=np.float64)
    P = W1.shape[0]
    assert P in (1, B)
    khat = [coef_q[b, :int(n_body[b])] @ basis[b] for b in range(B)]   # [n_b, D]
    losses = np.zeros((steps, P, G, H))
    g0 = (np.zeros_like(W1), np.zeros_like(b1), np.zeros_like(W2), np.zeros_like(b2))
    for p in range(P):
        seqs = range(B) if P == 1 else [p]
        for l in range(G):
            for h in range(H):
                c0 = (l * H + h) * d
                K = np.concatenate([khat[b][:, c0:c0 + d] for b in seqs], axis=0)
                V = np.concatenate([v[b, l, :int(n_body[b]), h] for b in seqs], axis=0)
                w = [W1[p, l, h], b1[p, l, h], W2[p, l, h], b2[p, l, h]]
                mom = [np.zeros_like(x) for x in w]
                sec = [np.zeros_like(x) for x in w]
                for t in range(1, steps + 1):
                    L, dW1, db1, dW2, db2 = predictor_loss_grad(K, V, *w)
                    losses[t - 1, p, l, h] = L
                    grads = [dW1, db1, dW2, db2]
                    if t == 1:
                        for acc, gr in zip(g0, grads):
                            acc[p, l, h] = gr
                    for i in range(4):
                        w[i], mom[i], sec[i] = adam_update(w[i], grads[i], mom[i], sec[i], t,
                                                           lr, beta1, beta2, eps)
                W1[p, l, h], b1[p, l, h], W2[p, l, h], b2[p, l, h] = w
    stored = tuple(round_store(x, weight_kind) for x in (W1, b1, W2, b2))
    return FitResult(W1=W1, b1=b1, W2=W2, b2=b2, stored=stored, losses=losses, grad0=g0)


# ---------------------------------------------------------------------------
# decode (D0..D9)
# [EXPL] "Step-by-step mental model ..." item 2 and "Asymmetric key
# compression with xKV": keys are rebuilt and re-rotated, values are
# regenerated from the keys plus residuals, new tokens keep exact K/V;
# [ABS] only a selected subset of KV pairs is rebuilt per step.
# ---------------------------------------------------------------------------

def attention_exact(q, K, V):
    """Softmax attention of one query over rows K, V (scale 1/sqrt d, R17).

    q [d], K [n, d], V [n, d].  Returns (o [d], lse, p [n]).  With n == 0:
    o = 0, lse = -inf (R20).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    d = q.shape[-1]
    if K.shape[0] == 0:
        return np.zeros(d), -np.inf, np.zeros(0)
    s = K @ q / math.sqrt(d)
    M = s.max()
    w = np.exp(s - M)
    L = w.sum()
    p = w / L
    return p @ V, M + math.log(L), p


def decode(layer: int, q, coef_stored, coef_kind: str, pos, n_body, basis,
           W1, b1, W2, b2, resid_idx, resid_val_stored, resid_kind: str,
           tail_k, tail_v, tail_len, theta: float, subset=None,
           return_probs: bool = False):
    """Decode attention of layer `layer` of the group (c3).

    Returns out [B, Hq, d] and lse [B, Hq] (and, with return_probs, the list
    of probability vectors per (b, qh) over body rows then tail rows).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    C = dequant_store(coef_stored, coef_kind)            # [B, N, r]
    R = dequant_store(resid_val_stored, resid_kind)      # [B, G, H, m, d]
    basis = np.asarray(basis, dtype=np.float64)
    tail_k = np.asarray(tail_k, dtype=np.float64)
    tail_v = np.asarray(tail_v, dtype=np.float64)
    H = tail_k.shape[3]
    N = C.shape[1]
    grp = Hq // H                 # contiguous GQA grouping: kv(qh) = qh // grp
    out = np.zeros((B, Hq, d))
    lse = np.zeros((B, Hq))
    probs = {}
    for b in range(B):
        n = int(n_body[b])
        p_all = np.arange(N) if pos is None else np.asarray(pos[b])
        # D0: attended body rows (R11)
        if subset is None:
            A = np.arange(n)
        else:
            A = np.asarray(subset[b], dtype=np.int64)
        tl = int(tail_len[b])
        for h in range(H):
            cols = slice((layer * H + h) * d, (layer * H + h + 1) * d)
            # D2: rebuild pre-RoPE keys of the attended rows
            k_pre = C[b, A] @ basis[b][:, cols]                 # [nA, d]
            # D3: rotate to each row's original position
            k = rope_rotate(k_pre, p_all[A], theta) if len(A) else k_pre
            # D5: predicted values
            vhat = predictor(k_pre, _w(W1, b, layer, h), _w(b1, b, layer, h),
                             _w(W2, b, layer, h), _w(b2, b, layer, h)) if len(A) else np.zeros((0, d))
            # D7: add the stored residual of rows in the residual set
            row_of = {int(t): i for i, t in enumerate(A)}
            for s_i, t in enumerate(resid_idx[b, layer, h]):
                if int(t) in row_of:
                    vhat[row_of[int(t)]] += R[b, layer, h, s_i]
            # D8: exact tail rows
            Kt = tail_k[b, layer, :tl, h]
            Vt = tail_v[b, layer, :tl, h]
            Kall = np.concatenate([k, Kt], axis=0)
            Vall = np.concatenate([vhat, Vt], axis=0)
            for qh in range(h * grp, (h + 1) * grp):
                # D4, D6, D9: softmax attention over body then tail
                o, ls, p = attention_exact(q[b, qh], Kall, Vall)
                out[b, qh] = o
                lse[b, qh] = ls
                probs[(b, qh)] = p
    if return_probs:
        return out, lse, probs
    return out, lse


def merge_partials(parts):
    """Combine attention results over disjoint row sets by log-sum-exp.

    parts: list of (o [d], lse).  Returns (o, lse) of the union.
    """
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    if np.all(np.isneginf(lses)):
        return np.zeros_like(np.asarray(parts[0][0], dtype=np.float64)), -np.inf
    M = lses[np.isfinite(lses)].max()
    w = np.where(np.isneginf(lses), 0.0, np.exp(lses - M))
    L = w.sum()
    o = sum(wi * np.asarray(p[0], dtype=np.float64) for wi, p in zip(w, parts)) / L
    return o, M + math.log(L)


# ---------------------------------------------------------------------------
# the shared key basis of a layer group (R25)
# [EXPL] "Asymmetric key compression with xKV": adjacent layers share
# dominant key subspaces, so a group stores one basis plus small factors,
# computed on the keys with RoPE undone; "Step-by-step mental model ...",
# item 1 (prefill compresses the keys with shared low-rank bases).
# ---------------------------------------------------------------------------

def pre_rope_keys(k_post, pos, n_body, theta: float) -> np.ndarray:
    """The matrix the basis summarises: X[b, t] = concatenation over (layer,
    head) of the key of row t with its rotation undone (the prefill's first
    step), column (l*Hkv + h)*d + j; [B, N, D] fp64, rows t >= n_body[b] 0."""
    k_post = np.asarray(k_post, dtype=np.float64)
    B, G, N, H, d = k_post.shape
    X = np.zeros((B, N, G * H * d))
    for b in range(B):
        n = int(n_body[b])
        p = np.arange(N) if pos is None else np.asarray(pos[b])
        k_pre = rope_rotate(k_post[b, :, :n].transpose(0, 2, 1, 3), p[:n], theta,
                            inverse=True)                       # [G, H, n, d]
        X[b, :n] = k_pre.transpose(2, 0, 1, 3).reshape(n, G * H * d)
    return X


def key_basis(k_post, pos, n_body, theta: float, r: int):
    """Definition of the basis (R25): per sequence, the top-r right singular
    vectors of the uncentred pre-RoPE key matrix X[b, :n] as rows, by the
    fp64 SVD.  Rows past the rank min(n, D) are zero; each row's sign is
    left as the SVD returns it (a basis is defined up to the sign of its
    rows).  Returns (basis [B, r, D], singular values [B, r], zero-padded)."""
    X = pre_rope_keys(k_post, pos, n_body, theta)
    B, N, D = X.shape
    basis = np.zeros((B, r, D))
    sv = np.zeros((B, r))
    for b in range(B):
        n = int(n_body[b])
        if n == 0:
            continue
        _, s, Vt = np.linalg.svd(X[b, :n], full_matrices=False)
        k = min(r, len(s))
        basis[b, :k] = Vt[:k]
        sv[b, :k] = s[:k]
    return basis, sv


def orth_columns(M: np.ndarray, drop_tol: float) -> np.ndarray:
    """Orthonormal columns of Gram-Schmidt on the columns of M in order,
    skipping dependent ones: column j's residual against the span of the
    columns kept before it, if its norm is at most drop_tol times the
    largest column norm of M, marks it linearly dependent (numerical rank
    deficiency): its output column is zero and it takes no part in the
    later columns.  With no column skipped this is the Q factor of the thin
    QR factorisation with R's diagonal non-negative (the unique Q of a
    full-rank M), computed here by Householder QR (numpy)."""
    n, k = M.shape
    Q = np.zeros((n, k))
    if k == 0:
        return Q
    lim = drop_tol * np.max(np.linalg.norm(M, axis=0))
    kept = []                       # accepted columns, in order
    rest = list(range(k))           # columns still to decide, in order
    while rest:
        cols = kept + rest
        Qf, Rf = np.linalg.qr(M[:, cols])
        Qf = Qf * np.where(np.diag(Rf) < 0, -1.0, 1.0)[None, :]
        # a column past the row count has no diagonal entry: once the columns
        # before it span R^n its residual is zero (dependent)
        dg = np.zeros(len(cols))
        dg[:min(n, len(cols))] = np.abs(np.diag(Rf))
        bad = [i for i in range(len(kept), len(cols)) if dg[i] <= lim]
        stop = bad[0] if bad else len(cols)
        for i in range(len(kept), stop):      # nested QR: these are final
            Q[:, cols[i]] = Qf[:, i]
        kept = kept + cols[len(kept):stop]
        if not bad:
            break
        # the first dependent column is skipped; so is every later column
        # already dependent on the kept ones (it stays dependent on more)
        Qk = Q[:, kept]
        rest = [c for c in cols[stop + 1:]
                if np.linalg.norm(M[:, c] - Qk @ (Qk.T @ M[:, c])) > lim]
    return Q


def key_basis_iteration(k_post, pos, n_body, theta: float, start,
                        power_iters: int, drop_tol: float = 1e-5) -> np.ndarray:
    """The basis as the library computes it (R25): randomized subspace
    iteration (Halko, Martinsson and Tropp, "Finding structure with
    randomness", SIAM Review 2011, Algorithm 4.4) on X = pre-RoPE keys,
    started from the caller's r x D Gaussian matrix `start` (the random
    numbers are an input), with power_iters + 1 rounds of
        P = orth(X Q^T);   Q = orth(X^T P)^T
    (Q = start before the first round), orth as in orth_columns.  No
    Rayleigh-Ritz step: the rows are an orthonormal basis of the computed
    subspace, not individual singular vectors.  In exact arithmetic the
    result is the Q factor of (X^T X)^(power_iters+1) start^T, rows with a
    dependent column zero.  Returns [B, r, D] fp64."""
    X = pre_rope_keys(k_post, pos, n_body, theta)
    start = np.asarray(start, dtype=np.float64)
    B, N, D = X.shape
    r = start.shape[1]
    out = np.zeros((B, r, D))
    for b in range(B):
        Xb = X[b]
        Q = start[b]                                    # [r, D] rows
        for _ in range(power_iters + 1):
            P = orth_columns(Xb @ Q.T, drop_tol)        # [N, r]
            Q = orth_columns(Xb.T @ P, drop_tol).T      # [r, D]
        out[b] = Q
    return out


# ---------------------------------------------------------------------------
# a structured subset of attended rows (R26)
# [ABS], [WIKI] flowchart: only a selected subset of KV pairs is rebuilt per
# decode step; the pages do not say how it is chosen.
# ---------------------------------------------------------------------------

def subset_policy(n_body, n_sink: int, n_recent: int, stride: int) -> list:
    """Per sequence, the sorted body rows t < n_body[b] with t < n_sink, or
    t >= n_body[b] - n_recent, or (stride > 0 and (t - n_sink) % stride == 0)
    (R26).  Returns a list of int64 arrays."""
    out = []
    for n in np.asarray(n_body).tolist():
        t = np.arange(int(n))
        keep = (t < n_sink) | (t >= n - n_recent)
        if stride > 0:
            keep |= (t - n_sink) % stride == 0
        out.append(t[keep])
    return out
