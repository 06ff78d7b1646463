"""Seeded synthetic workloads for the LowRAM decode path.

This module only draws inputs: it holds the data recipe of a synthetic
"model" that produced a KV cache, and none of the compression or attention
arithmetic of the method.  Both the HIP library's tests and the CPU oracle
consume what it returns; neither is imported here.

The recipe stands in for the pages' workloads (long-context prompts on
7B-class models, which are not available here):

* pre-RoPE keys of a layer group are low rank plus noise,
  X = Z A^T + 0.05 E, with Z ~ N(0,1) [N, R] per sequence, A ~ N(0, 1/R)
  [D, R] per group and E ~ N(0,1);
* the model's keys are X turned by its rotary embedding at each token's
  position (rotate-half pairs (i, i + d/2), angle pos * theta**(-2i/d));
  this module turns them with complex multiplication;
* values are a teacher network of the pre-RoPE keys,
  V = W2 gelu(W1 x) with W ~ N(0, 1/d) and zero biases, plus 0.05 N(0,1)
  noise, except for 5 % of the tokens (chosen once per sequence) whose
  noise is a standard Student-t with 3 degrees of freedom;
* the caller's predictor is the teacher with N(0, 0.01^2) added to all
  four tensors; queries are N(0,1) and already rotated;
* the exact tail follows the same recipe at positions T_c .. T-1;
* the key basis of a (sequence, group) is the top-r right singular vectors
  of the uncentred pre-RoPE key matrix (the caller's input; computed in
  float64 for small matrices, by randomized subspace iteration otherwise).

Streams: numpy.random.default_rng(SeedSequence(seed)) spawns children in
the fixed order keys, teacher, value-noise, predictor, query, tail, subset,
eviction.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
from scipy.special import erf

INT32_MAX = 2**31 - 1


@dataclass
class Shape:
    """Shape of one layer-group workload."""
    name: str
    batch: int
    group_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    rank: int
    context: int
    tail: int
    resid_frac: tuple          # exact rational (num, den)
    theta: float
    dtype: str                 # "f32" or "bf16"
    latent_rank: int = 384
    coef_store: str = "native"  # "native" or "int4"
    resid_store: str = "native"
    subset_frac: tuple | None = None
    keep_frac: tuple | None = None   # eviction: kept fraction of the body
    sinks: int = 0
    n_groups: int = 1          # layer groups in the model stack

    @property
    def body(self) -> int:     # T_c: prompt body length
        return self.context - self.tail

    @property
    def n_rows(self) -> int:   # N: stored body rows
        if self.keep_frac is None:
            return self.body
        a, b = self.keep_frac
        return -(-self.body * a // b)

    @property
    def n_resid(self) -> int:  # m = ceil(rho * N) with exact rationals
        a, b = self.resid_frac
        return -(-self.n_rows * a // b)

    @property
    def D(self) -> int:
        return self.group_layers * self.n_kv_heads * self.head_dim


# The five workloads: a tiny fp32 shape, Llama-3-shaped layer groups at 8k,
# 32k (with a row subset) and 131k (int4 storage and eviction) context, and
# the 7-group, 7:1-GQA peak-throughput model.  Values their source sizes do
# not fix: 4 layers per group for the int4 workload, a 128-row tail for the
# peak workload, RoPE theta 500000 for the Llama-shaped groups.
CONFIGS = {
    1: Shape("tiny-fp32", 1, 2, 4, 2, 64, 32, 256, 16, (1, 4), 10000.0, "f32",
             latent_rank=16),
    2: Shape("llama3-8b-group-8k", 8, 4, 32, 8, 128, 512, 8192, 128, (1, 5),
             500000.0, "bf16"),
    3: Shape("long-32k-subset", 16, 4, 32, 8, 128, 512, 32768, 512, (1, 5),
             500000.0, "bf16", subset_frac=(1, 4)),
    4: Shape("int4-evict-131k", 4, 4, 32, 8, 128, 384, 131072, 256, (3, 20),
             500000.0, "bf16", coef_store="int4", resid_store="int4",
             keep_frac=(3, 10), sinks=64),
    5: Shape("gqa7-peak-32k", 607, 4, 28, 4, 128, 256, 32768, 128, (1, 5),
             500000.0, "bf16", n_groups=7),
}


def scaled(base: Shape, **kw) -> Shape:
    """Copy of a shape with some fields replaced (smaller test sizes)."""
    d = dict(base.__dict__)
    d.update(kw)
    return Shape(**d)


@dataclass
class Workload:
    shape: Shape
    q: np.ndarray                 # [B, Hq, d] float32
    k_post: np.ndarray            # [B, G, N, Hkv, d] float32
    v: np.ndarray                 # [B, G, N, Hkv, d] float32
    pos: np.ndarray | None        # [B, N] int32 or None
    n_body: np.ndarray            # [B] int32
    basis: np.ndarray             # [B, r, D] float32
    w1: np.ndarray                # [1, G, Hkv, d, d] float32
    b1: np.ndarray                # [1, G, Hkv, d]
    w2: np.ndarray
    b2: np.ndarray
    tail_k: np.ndarray            # [B, G, Te, Hkv, d]
    tail_v: np.ndarray
    tail_len: np.ndarray          # [B] int32
    subset: list | None = None    # per-sequence sorted body rows
    m: int = 0
    extra: dict = field(default_factory=dict)


def _model_rotate(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """The synthetic model's rotary embedding, as complex multiplication of
    z_i = x_i + i x_{i+d/2} by exp(i pos theta^(-2i/d)).  x [..., T, d]."""
    d = x.shape[-1]
    half = d // 2
    freq = np.power(theta, -np.arange(half, dtype=np.float64) * 2.0 / d)
    rot = np.exp(1j * np.outer(pos.astype(np.float64), freq))       # [T, half]
    z = x[..., :half].astype(np.float64) + 1j * x[..., half:].astype(np.float64)
    z = z * rot
    return np.concatenate([z.real, z.imag], axis=-1).astype(np.float32)


def _teacher(x: np.ndarray, w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """Teacher value network of the synthetic model: w2 gelu(w1 x)."""
    a = x @ w1.T
    a = 0.5 * a * (1.0 + erf(a * np.float32(1.0 / math.sqrt(2.0))))
    return (a @ w2.T).astype(np.float32)


def harness_basis(X: np.ndarray, r: int, exact: bool | None = None,
                  rng: np.random.Generator | None = None) -> np.ndarray:
    """Top-r right singular vectors of X [N, D] as rows [r, D], each row's
    largest-magnitude entry made positive.  Exact (float64 eigh of X^T X)
    when the matrix is small, else randomized subspace iteration with 64
    extra columns and two power iterations (Halko, Martinsson and Tropp,
    SIAM Review 2011, Alg. 4.4)."""
    N, D = X.shape
    if exact is None:
        exact = D <= 1024
    if exact or r >= min(N, D):
        Xd = X.astype(np.float64)
        w, V = np.linalg.eigh(Xd.T @ Xd)
        order = np.argsort(w)[::-1][:r]
        Bm = V[:, order].T
        if Bm.shape[0] < r:                      # rank-deficient request
            Bm = np.concatenate([Bm, np.zeros((r - Bm.shape[0], D))], 0)
    else:
        rng = rng or np.random.default_rng(0)
        k = min(r + 64, D)
        Xf = X.astype(np.float32)
        Y = Xf.T @ (Xf @ rng.standard_normal((D, k), dtype=np.float32))
        Q, _ = np.linalg.qr(Y.astype(np.float64))
        for _ in range(2):
            Z = Xf.T @ (Xf @ Q.astype(np.float32))
            Q, _ = np.linalg.qr(Z.astype(np.float64))
        # Rayleigh-Ritz on the subspace
        P = Xf.astype(np.float64) @ Q               # [N, k]
        w, U = np.linalg.eigh(P.T @ P)
        order = np.argsort(w)[::-1][:r]
        Bm = (Q @ U[:, order]).T
    sgn = np.sign(Bm[np.arange(Bm.shape[0]), np.argmax(np.abs(Bm), axis=1)])
    sgn[sgn == 0] = 1.0
    return (Bm * sgn[:, None]).astype(np.float64)


def make_workload(shape: Shape, seed: int, *, with_basis: bool = True,
                  basis_exact: bool | None = None,
                  n_body: np.ndarray | None = None,
                  tail_len: np.ndarray | None = None,
                  distinct: int | None = None) -> Workload:
    """Draw one layer group's workload (see the module docstring).

    distinct: draw only this many sequences and repeat them cyclically to
    fill the batch (large timing workloads); queries stay distinct."""
    if distinct is not None and distinct < shape.batch:
        w = make_workload(scaled(shape, batch=distinct), seed, with_basis=with_basis,
                          basis_exact=basis_exact)
        reps = [b % distinct for b in range(shape.batch)]
        for k in ("k_post", "v", "basis", "tail_k", "tail_v", "pos"):
            a = getattr(w, k)
            if a is not None:
                setattr(w, k, a[reps])
        if w.subset is not None:
            w.subset = [w.subset[i] for i in reps]
        rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
        w.q = rng.standard_normal((shape.batch, shape.n_q_heads, shape.head_dim), dtype=np.float32)
        w.n_body = np.full(shape.batch, shape.n_rows, dtype=np.int32) if n_body is None else np.asarray(n_body, np.int32)
        w.tail_len = np.full(shape.batch, shape.tail, dtype=np.int32) if tail_len is None else np.asarray(tail_len, np.int32)
        w.shape = shape
        return w
    s = shape
    B, G, Hq, H, d, r = (s.batch, s.group_layers, s.n_q_heads, s.n_kv_heads,
                         s.head_dim, s.rank)
    N, Te, D, R = s.n_rows, s.tail, s.D, s.latent_rank
    Tc = s.body
    ss = np.random.SeedSequence(seed)
    (g_key, g_teach, g_noise, g_pred, g_q, g_tail, g_sub, g_evict) = [
        np.random.default_rng(c) for c in ss.spawn(8)]

    # eviction: kept rows and their original positions
    if s.keep_frac is not None:
        pos = np.zeros((B, N), dtype=np.int32)
        for b in range(B):
            rest = g_evict.choice(np.arange(s.sinks, Tc), size=N - s.sinks, replace=False)
            pos[b] = np.sort(np.concatenate([np.arange(s.sinks), rest])).astype(np.int32)
    else:
        pos = None

    A = g_key.standard_normal((D, R), dtype=np.float32) * np.float32(1.0 / math.sqrt(R))
    w1 = g_teach.standard_normal((G, H, d, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))
    w2 = g_teach.standard_normal((G, H, d, d), dtype=np.float32) * np.float32(1.0 / math.sqrt(d))

    k_post = np.empty((B, G, N, H, d), dtype=np.float32)
    v = np.empty((B, G, N, H, d), dtype=np.float32)
    tail_k = np.empty((B, G, Te, H, d), dtype=np.float32)
    tail_v = np.empty((B, G, Te, H, d), dtype=np.float32)
    basis = np.empty((B, r, D), dtype=np.float32) if with_basis else None

    def rows(gen, n):
        Z = gen.standard_normal((n, R), dtype=np.float32)
        E = gen.standard_normal((n, D), dtype=np.float32)
        return Z @ A.T + np.float32(0.05) * E               # [n, D]

    def values(gen, X, n):
        heavy = gen.random(n) < 0.05
        Xg = X.reshape(n, G, H, d)
        out = np.empty((n, G, H, d), dtype=np.float32)
        for l in range(G):
            for h in range(H):
                out[:, l, h] = _teacher(Xg[:, l, h], w1[l, h], w2[l, h])
        noise = np.float32(0.05) * gen.standard_normal(out.shape, dtype=np.float32)
        t3 = gen.standard_t(3, size=(int(heavy.sum()), G, H, d)).astype(np.float32)
        noise[heavy] = t3
        return out + noise

    for b in range(B):
        X = rows(g_key, N)
        p = np.arange(N) if pos is None else pos[b]
        kp = _model_rotate(X.reshape(N, G, H, d).transpose(1, 2, 0, 3), p, s.theta)
        k_post[b] = kp.transpose(0, 2, 1, 3)
        v[b] = values(g_noise, X, N).transpose(1, 0, 2, 3)
        if with_basis:
            basis[b] = harness_basis(X, r, exact=basis_exact,
                                     rng=np.random.default_rng(seed * 1000 + b))
        Xt = rows(g_tail, Te)
        tp = np.arange(Tc, Tc + Te)
        kt = _model_rotate(Xt.reshape(Te, G, H, d).transpose(1, 2, 0, 3), tp, s.theta)
        tail_k[b] = kt.transpose(0, 2, 1, 3)
        tail_v[b] = values(g_tail, Xt, Te).transpose(1, 0, 2, 3)

    pw1 = (w1 + np.float32(0.01) * g_pred.standard_normal(w1.shape, dtype=np.float32))[None]
    pb1 = (np.float32(0.01) * g_pred.standard_normal((G, H, d), dtype=np.float32))[None]
    pw2 = (w2 + np.float32(0.01) * g_pred.standard_normal(w2.shape, dtype=np.float32))[None]
    pb2 = (np.float32(0.01) * g_pred.standard_normal((G, H, d), dtype=np.float32))[None]
    q = g_q.standard_normal((B, Hq, d), dtype=np.float32)

    nb = np.full(B, N, dtype=np.int32) if n_body is None else np.asarray(n_body, dtype=np.int32)
    subset = None
    if s.subset_frac is not None:
        # drawn among each sequence's own body rows (all N when lengths are not ragged)
        a, c = s.subset_frac
        subset = [np.sort(g_sub.choice(int(nb[b]), size=-(-int(nb[b]) * a // c), replace=False)).astype(np.int32)
                  for b in range(B)]

    tl = np.full(B, Te, dtype=np.int32) if tail_len is None else np.asarray(tail_len, dtype=np.int32)
    return Workload(shape=s, q=q, k_post=k_post, v=v, pos=pos, n_body=nb,
                    basis=basis, w1=pw1, b1=pb1, w2=pw2, b2=pb2,
                    tail_k=tail_k, tail_v=tail_v, tail_len=tl, subset=subset,
                    m=s.n_resid)


def subset_csr(subset: list) -> tuple[np.ndarray, np.ndarray]:
    """Per-sequence row lists -> CSR (off [B+1] int32, idx [nnz] int32)."""
    off = np.zeros(len(subset) + 1, dtype=np.int32)
    off[1:] = np.cumsum([len(x) for x in subset])
    idx = (np.concatenate(subset).astype(np.int32) if off[-1] else
           np.zeros(0, dtype=np.int32))
    return off, idx
