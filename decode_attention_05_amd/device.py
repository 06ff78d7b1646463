"""Device plumbing for the LowRAM library: move a seeded workload into HBM
in the storage dtype, allocate the compressed cache and outputs, and call
the library.  Allocation and copies use torch; all method arithmetic runs in
liblowram.so."""
from __future__ import annotations

import math

import numpy as np
import torch

from . import lowram as L
from .synth import Shape, Workload, subset_csr


def tdtype(s: Shape):
    return torch.float32 if s.dtype == "f32" else torch.bfloat16


def abi_shape(s: Shape, *, algo: int = L.ALGO_AUTO, predictor_shared: int = 1,
              n_body_max: int | None = None, n_resid: int | None = None) -> L.lowram_shape:
    return L.make_shape(
        batch=s.batch, group_layers=s.group_layers, n_q_heads=s.n_q_heads,
        n_kv_heads=s.n_kv_heads, head_dim=s.head_dim, rank=s.rank,
        n_body_max=s.n_rows if n_body_max is None else n_body_max,
        n_resid=s.n_resid if n_resid is None else n_resid, tail_max=s.tail,
        rope_theta=s.theta, dtype=L.F32 if s.dtype == "f32" else L.BF16,
        coef_store=L.STORE_INT4 if s.coef_store == "int4" else L.STORE_NATIVE,
        resid_store=L.STORE_INT4 if s.resid_store == "int4" else L.STORE_NATIVE,
        predictor_shared=predictor_shared, algo=algo)


def upload(w: Workload, device="cuda") -> dict:
    """Inputs of prefill and decode as device tensors in the storage dtype."""
    s = w.shape
    dt = tdtype(s)

    def f(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dt)

    def i(x):
        return torch.from_numpy(np.ascontiguousarray(x).astype(np.int32)).to(device)

    t = dict(q=f(w.q), k_post=f(w.k_post), v=f(w.v), basis=None if w.basis is None else f(w.basis),
             w1=f(w.w1), b1=f(w.b1),
             w2=f(w.w2), b2=f(w.b2), tail_k=f(w.tail_k), tail_v=f(w.tail_v),
             n_body=i(w.n_body), tail_len=i(w.tail_len),
             pos=None if w.pos is None else i(w.pos))
    if w.subset is not None:
        off, idx = subset_csr(w.subset)
        t["subset_off"], t["subset_idx"] = i(off), i(idx)
    return t


def alloc_cache(s: Shape, m: int | None = None, device="cuda") -> dict:
    """Empty compressed-cache arrays of one layer group."""
    B, G, H, d, r, N = s.batch, s.group_layers, s.n_kv_heads, s.head_dim, s.rank, s.n_rows
    m = s.n_resid if m is None else m
    dt = tdtype(s)
    c = {}
    if s.coef_store == "int4":
        c["coef"] = torch.empty((B, N, r // 2), dtype=torch.uint8, device=device)
        c["coef_scale"] = torch.empty((B, N, r // 32), dtype=torch.float16, device=device)
    else:
        c["coef"] = torch.empty((B, N, r), dtype=dt, device=device)
    c["resid_idx"] = torch.empty((B, G, H, m), dtype=torch.int32, device=device)
    if s.resid_store == "int4":
        c["resid_val"] = torch.empty((B, G, H, m, d // 2), dtype=torch.uint8, device=device)
        c["resid_scale"] = torch.empty((B, G, H, m, d // 32), dtype=torch.float16, device=device)
    else:
        c["resid_val"] = torch.empty((B, G, H, m, d), dtype=dt, device=device)
    c["err"] = torch.empty((B, G, H, N), dtype=torch.float32, device=device)
    return c


def workspace(nbytes: int, device="cuda"):
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def prefill(s: Shape, t: dict, c: dict, *, m: int | None = None, predictor_shared: int = 1,
            ws=None, algo: int = L.ALGO_AUTO) -> None:
    sh = abi_shape(s, predictor_shared=predictor_shared, n_resid=m, algo=algo)
    if ws is None:
        ws = workspace(L.lowram_workspace_size(sh, 0))
    L.lowram_compress_prefill(sh, t["k_post"], t["v"], t.get("pos"), t["n_body"], t["basis"],
                              t["w1"], t["b1"], t["w2"], t["b2"], c["coef"], c.get("coef_scale"),
                              c["resid_idx"], c["resid_val"], c.get("resid_scale"), c.get("err"), ws)


def fit(s: Shape, t: dict, c: dict, *, steps: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
        eps: float = 1e-8, predictor_shared: int = 1, ws=None, loss: bool = True, grad: bool = True):
    """Fit t's predictor weights in place on the stored cache c (lowram_fit_predictor).
    Returns (loss [steps, Bp, G, Hkv] or None, gradient at the initial weights or None)."""
    sh = abi_shape(s, predictor_shared=predictor_shared)
    if ws is None:
        ws = workspace(L.lowram_fit_workspace_size(sh))
    Bp = 1 if predictor_shared else s.batch
    G, H, d = s.group_layers, s.n_kv_heads, s.head_dim
    dev = t["v"].device
    loss_out = torch.empty((steps, Bp, G, H), dtype=torch.float32, device=dev) if loss and steps > 0 else None
    grad_out = torch.empty((Bp, G, H, 2 * d * d + 2 * d), dtype=torch.float32, device=dev) if grad else None
    L.lowram_fit_predictor(sh, c["coef"], c.get("coef_scale"), t["n_body"], t["basis"], t["v"],
                           L.make_fit_params(steps, lr, beta1, beta2, eps), t["w1"], t["b1"], t["w2"],
                           t["b2"], loss_out, grad_out, ws)
    return loss_out, grad_out


def compute_basis(s: Shape, t: dict, start: torch.Tensor, power_iters: int, *, ws=None,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """The group's key basis [B, r, D] (dtype of s) computed by the library
    from the keys in t, starting from `start` [B, r, D] fp32."""
    sh = abi_shape(s)
    if ws is None:
        ws = workspace(L.lowram_basis_workspace_size(sh), device=t["k_post"].device)
    if out is None:
        out = torch.empty((s.batch, s.rank, s.D), dtype=tdtype(s), device=t["k_post"].device)
    L.lowram_compute_basis(sh, t["k_post"], t.get("pos"), t["n_body"], start, power_iters, out, ws)
    return out


def algorithmic_basis_flops(s: Shape, n_rows: int, power_iters: int) -> int:
    """Algorithmic flops of one basis call over n_rows body rows in total:
    per round the two products X Q^T and X^T P (4 n D r), the Gram matrices
    (symmetric, len r^2 each) and the triangular applications (len r^2
    each) of both orthonormalisations, plus the last one on Q, and per
    orthonormalisation a Cholesky and a triangular inverse (r^3 / 3 each)
    per sequence."""
    r, D, B = s.rank, s.D, s.batch
    rounds = power_iters + 1
    per_round = 4 * n_rows * D * r + 2 * (n_rows + B * D) * r * r
    last = 2 * B * D * r * r
    factor = (2 * rounds + 1) * B * 2 * r ** 3 // 3
    return rounds * per_round + last + factor


def cache_of(t: dict, c: dict) -> dict:
    """The lowram_cache fields from the input and compressed-cache tensors."""
    return dict(coef=c["coef"], coef_scale=c.get("coef_scale"), pos=t.get("pos"),
                n_body=t["n_body"], basis=t["basis"], w1=t["w1"], b1=t["b1"], w2=t["w2"],
                b2=t["b2"], resid_idx=c["resid_idx"], resid_val=c["resid_val"],
                resid_scale=c.get("resid_scale"), tail_k=t["tail_k"], tail_v=t["tail_v"],
                tail_len=t["tail_len"])


class Decoder:
    """One layer group's decode calls with a persistent workspace and outputs."""

    def __init__(self, s: Shape, t: dict, c: dict, *, algo=L.ALGO_AUTO, use_subset=False,
                 predictor_shared: int = 1, m: int | None = None):
        self.s = s
        self.sh = abi_shape(s, algo=algo, predictor_shared=predictor_shared, n_resid=m)
        self.cache = L.make_cache(cache_of(t, c))
        self._keep = (t, c)
        self.q = t["q"]
        self.sub = (t.get("subset_off"), t.get("subset_idx")) if use_subset else (None, None)
        self.ws = workspace(L.lowram_workspace_size(self.sh, 1))
        self.out = torch.empty((s.batch, s.n_q_heads, s.head_dim), dtype=tdtype(s), device=self.q.device)
        self.lse = torch.empty((s.batch, s.n_q_heads), dtype=torch.float32, device=self.q.device)

    def __call__(self, layer: int, q=None, stream=None):
        L.lowram_decode_attn(self.sh, layer, self.q if q is None else q, self.cache, self.sub[0],
                             self.sub[1], self.out, self.lse, self.ws, stream)
        return self.out, self.lse

    def timed(self, layer: int, before_event, after_event, stream=None):
        """The same call, recording two events (raw hipEvent_t) around its body-row kernel."""
        L.lowram_decode_attn_timed(self.sh, layer, self.q, self.cache, self.sub[0], self.sub[1], self.out,
                                   self.lse, self.ws, before_event, after_event, stream)
        return self.out, self.lse


def to_numpy_store(x: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in the oracle's storage form (bf16 as uint16 bits)."""
    x = x.detach().cpu()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def algorithmic_decode_bytes(s: Shape, n_attended: int, with_subset: bool) -> int:
    """Bytes one decode call must move at minimum (one layer, whole batch)."""
    B, H, d, r, m = s.batch, s.n_kv_heads, s.head_dim, s.rank, s.n_resid
    coef_row = r // 2 + (r // 32) * 2 if s.coef_store == "int4" else r * (4 if s.dtype == "f32" else 2)
    el = 4 if s.dtype == "f32" else 2
    res_row = d // 2 + (d // 32) * 2 if s.resid_store == "int4" else d * el
    frac = n_attended / max(s.n_rows, 1)
    b = B * n_attended * coef_row
    if s.keep_frac is not None:
        b += B * n_attended * 4                           # positions
    if with_subset:
        b += B * n_attended * 4                           # subset indices
    b += B * r * H * d * el                               # the layer's basis slice
    b += H * (2 * d * d + 2 * d) * el                     # predictor (shared)
    b += B * H * math.ceil(m * frac) * (res_row + 4)      # attended residual rows + indices
    b += B * H * s.tail * d * el * 2                      # tail K and V
    b += B * s.n_q_heads * d * el * 2                     # q and out
    return b


def algorithmic_body_kernel_flops(s: Shape, n_attended: int) -> int:
    """Flops of the body-row kernel alone, per launch (one layer, whole
    batch): per attended body row 2*r*H*d (key rebuild) + 2*H*d*d (predictor
    hidden layer) + 4*Hq*d (scores and hidden accumulation); per attended
    residual row 2*grp*d per KV head (its weighted sum); per tail row 4*Hq*d
    (scores and weighted values: the launch's last workgroups take the tail)."""
    B, H, Hq, d, r = s.batch, s.n_kv_heads, s.n_q_heads, s.head_dim, s.rank
    frac = n_attended / max(s.n_rows, 1)
    f = n_attended * (2 * r * H * d + 2 * H * d * d + 4 * Hq * d)
    f += math.ceil(s.n_resid * frac) * 2 * Hq * d
    f += s.tail * 4 * Hq * d
    return B * f


def algorithmic_body_kernel_bytes(s: Shape, n_attended: int, with_subset: bool) -> int:
    """Bytes the body-row kernel must read at minimum, per launch: attended
    coefficient rows (+ scales, positions, subset indices), the layer's basis
    slice, W1 and b1, the queries, the attended residual rows with their
    indices, and the tail's keys and values."""
    B, H, d, r, m = s.batch, s.n_kv_heads, s.head_dim, s.rank, s.n_resid
    el = 4 if s.dtype == "f32" else 2
    coef_row = r // 2 + (r // 32) * 2 if s.coef_store == "int4" else r * el
    res_row = d // 2 + (d // 32) * 2 if s.resid_store == "int4" else d * el
    frac = n_attended / max(s.n_rows, 1)
    b = B * n_attended * coef_row
    if s.keep_frac is not None:
        b += B * n_attended * 4
    if with_subset:
        b += B * n_attended * 4
    b += B * r * H * d * el + H * (d * d + d) * el + B * s.n_q_heads * d * el
    b += B * H * math.ceil(m * frac) * (res_row + 4)
    b += B * H * s.tail * d * el * 2
    return b


def algorithmic_prefill_flops(s: Shape) -> int:
    """Flops of one prefill call (whole batch, every body row): projection on
    the basis 2*N*D*r, rebuild from the stored coefficients 2*N*r*D, and both
    predictor layers 4*G*H*d*d per row.  Work an implementation adds (split
    operands, recomputing the selected rows) is not counted."""
    B, G, H, d, r, N = s.batch, s.group_layers, s.n_kv_heads, s.head_dim, s.rank, s.n_rows
    D = G * H * d
    return B * N * (4 * D * r + 4 * G * H * d * d)


def algorithmic_prefill_bytes(s: Shape) -> int:
    """Bytes one prefill call must move at minimum: keys and values in, the
    basis and predictor in, coefficients, scores and residuals out."""
    B, G, H, d, r, N, m = s.batch, s.group_layers, s.n_kv_heads, s.head_dim, s.rank, s.n_rows, s.n_resid
    el = 4 if s.dtype == "f32" else 2
    coef_row = r // 2 + (r // 32) * 2 if s.coef_store == "int4" else r * el
    res_row = d // 2 + (d // 32) * 2 if s.resid_store == "int4" else d * el
    b = 2 * B * G * N * H * d * el                        # keys and values
    b += B * r * G * H * d * el                           # basis
    b += G * H * (2 * d * d + 2 * d) * el                 # predictor (shared)
    if s.keep_frac is not None:
        b += B * N * 4                                    # positions
    b += B * N * coef_row                                 # coefficients
    b += B * G * H * N * 4                                # scores
    b += B * G * H * m * (res_row + 4)                    # residual rows and indices
    return b


def algorithmic_append_flops(s: Shape, n_new: int) -> int:
    """Flops of one lowram_append_body call: the prefill work of n_new rows
    per sequence (projection, rebuild, both predictor layers)."""
    B, G, H, d, r = s.batch, s.group_layers, s.n_kv_heads, s.head_dim, s.rank
    D = G * H * d
    return B * n_new * (4 * D * r + 4 * G * H * d * d)


def algorithmic_append_bytes(s: Shape, n_new: int, m_new: int) -> int:
    """Bytes one lowram_append_body call must move at minimum: the new key
    and value rows, the basis and predictor, the new coefficient rows, their
    scores and residual rows out."""
    B, G, H, d, r = s.batch, s.group_layers, s.n_kv_heads, s.head_dim, s.rank
    el = 4 if s.dtype == "f32" else 2
    coef_row = r // 2 + (r // 32) * 2 if s.coef_store == "int4" else r * el
    res_row = d // 2 + (d // 32) * 2 if s.resid_store == "int4" else d * el
    b = 2 * B * G * n_new * H * d * el + B * r * G * H * d * el + G * H * (2 * d * d + 2 * d) * el
    b += B * n_new * coef_row + B * G * H * n_new * 4 + B * G * H * m_new * (res_row + 4)
    return b


def algorithmic_fit_step_flops(s: Shape, n_rows: int) -> int:
    """Flops of one gradient pass of the fit over n_rows body rows in total
    (all sequences): per row and (layer, head) the two forward products, the
    backward product through W2 and the two weight gradients, 2 d^2 each.
    The bf16-pair splitting (three MFMAs per product) is not counted."""
    G, H, d = s.group_layers, s.n_kv_heads, s.head_dim
    return n_rows * G * H * 5 * 2 * d * d


def algorithmic_fit_step_bytes(s: Shape, n_rows: int, n_predictors: int) -> int:
    """Bytes one gradient pass must move at minimum: the rebuilt keys and the
    values of every row once (fp32 each, the precision the pass computes in)
    and the weights of every predictor."""
    G, H, d = s.group_layers, s.n_kv_heads, s.head_dim
    return n_rows * G * H * d * 8 + n_predictors * G * H * (2 * d * d + 2 * d) * 4


def algorithmic_decode_flops(s: Shape, n_attended: int) -> int:
    B, H, Hq, d, r = s.batch, s.n_kv_heads, s.n_q_heads, s.head_dim, s.rank
    A = n_attended
    f = 2 * A * r * H * d            # key rebuild
    f += 2 * A * H * d * d           # predictor hidden layer
    f += 4 * A * Hq * d              # scores and hidden accumulation
    f += 4 * s.tail * Hq * d         # tail
    f += 2 * Hq * d * d              # hoisted output layer
    return B * f
