"""Helpers shared by the GPU parity tests: run the library on a seeded
workload and compare with the oracle on identical stored data."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from decode_attention_05_amd import device as dev
from decode_attention_05_amd import lowram as L
from decode_attention_05_amd import synth


def kind(s: synth.Shape, which: str) -> str:
    store = s.coef_store if which == "coef" else s.resid_store
    if store == "int4":
        return "int4"
    return "f32" if s.dtype == "f32" else "bf16"


def np_in(x: torch.Tensor) -> np.ndarray:
    """A device input tensor as float64 (exact widening of its stored values)."""
    a = dev.to_numpy_store(x)
    return O.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def stored(c: dict, which: str, k: str):
    """A compressed-cache array in the oracle's storage form."""
    if which == "coef":
        v, sc = c["coef"], c.get("coef_scale")
    else:
        v, sc = c["resid_val"], c.get("resid_scale")
    if k == "int4":
        return (v.cpu().numpy(), sc.cpu().numpy())
    return dev.to_numpy_store(v)


def oracle_inputs(t: dict) -> dict:
    o = {k: np_in(t[k]) for k in ("q", "k_post", "v", "basis", "w1", "b1", "w2", "b2", "tail_k", "tail_v")}
    o["n_body"] = t["n_body"].cpu().numpy()
    o["tail_len"] = t["tail_len"].cpu().numpy()
    o["pos"] = None if t.get("pos") is None else t["pos"].cpu().numpy()
    if t.get("subset_off") is not None:
        off = t["subset_off"].cpu().numpy()
        idx = t["subset_idx"].cpu().numpy()
        o["subset"] = [idx[off[b]:off[b + 1]] for b in range(len(off) - 1)]
    return o


def oracle_decode(s: synth.Shape, o: dict, c: dict, layer: int, subset=None):
    return O.decode(layer, o["q"], stored(c, "coef", kind(s, "coef")), kind(s, "coef"), o["pos"],
                    o["n_body"], o["basis"], o["w1"], o["b1"], o["w2"], o["b2"],
                    c["resid_idx"].cpu().numpy().astype(np.int64),
                    stored(c, "resid", kind(s, "resid")), kind(s, "resid"), o["tail_k"], o["tail_v"],
                    o["tail_len"], s.theta, subset=subset)


def assert_decode_close(s: synth.Shape, out: torch.Tensor, lse: torch.Tensor, ref, ref_lse, what=""):
    got = out.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), fin), what
    if s.dtype == "f32":
        # per (b, qh) row: ||o_gpu - o_ref||_inf <= 1e-5 ||o_ref||_inf
        err = np.abs(got - ref).max(-1)
        bound = 1e-5 * np.maximum(np.abs(ref).max(-1), 1e-30)
        assert np.all(err <= bound), f"{what}: worst rel err {np.max(err / bound) * 1e-5:.3g}"
        assert np.all(np.abs(gl - ref_lse)[fin] <= 1e-5 * np.maximum(1.0, np.abs(ref_lse[fin]))), what
    else:
        err = np.abs(got - ref)
        assert err.max() <= 2e-2, f"{what}: max abs err {err.max():.4g}"
        assert np.all(np.abs(gl - ref_lse)[fin] <= 2e-2), f"{what}: lse err {np.abs(gl - ref_lse)[fin].max():.4g}"
    assert np.all(got[~fin] == 0), what


def assert_prefill_matches(s: synth.Shape, c: dict, o: dict):
    """The library's prefill outputs against the oracle's on the same inputs:
    scores within 1e-5 (fp32) / 2e-2 (bf16) of each row maximum, the
    selection bit-exact on the library's own scores, coefficients and
    residuals within one storage unit (equal for almost all)."""
    e_gpu = c["err"].cpu().numpy().astype(np.float64)
    # the oracle, selecting on the library's own scores
    oc = O.prefill(o["k_post"], o["v"], o["pos"], o["n_body"], o["basis"], o["w1"], o["b1"],
                   o["w2"], o["b2"], s.n_resid, s.theta, kind(s, "coef"), kind(s, "resid"),
                   err_override=e_gpu)
    tol = 1e-5 if s.dtype == "f32" else 2e-2
    nb = o["n_body"]
    for b in range(s.batch):
        n = int(nb[b])
        if n == 0:
            continue
        ref = oc.err[b, :, :, :n]
        scale = np.maximum(ref.max(-1, keepdims=True), 1e-30)
        assert np.all(np.abs(e_gpu[b, :, :, :n] - ref) <= tol * scale), f"scores b={b}"
        assert np.all(e_gpu[b, :, :, n:] == 0)
    # selection: bit-exact on the library's scores
    idx_gpu = c["resid_idx"].cpu().numpy().astype(np.int64)
    assert np.array_equal(idx_gpu, oc.resid_idx), "selected rows differ"
    # stored coefficients
    assert_coef_close(s, o, stored(c, "coef", kind(s, "coef")), oc.coef)
    # stored residuals, on the same selected rows
    rk = kind(s, "resid")
    if s.n_resid:
        if rk == "int4":
            pg, sg = stored(c, "resid", rk)
            po, so = oc.resid_val
            cg, co = O.int4_unpack(pg).astype(int), O.int4_unpack(po).astype(int)
            assert np.abs(cg - co).max() <= 1
            assert np.mean(cg == co) > 0.97
        else:
            g = O.dequant_store(stored(c, "resid", rk), rk)
            r = O.dequant_store(oc.resid_val, rk)
            rel = 2.0 ** -7 if rk == "bf16" else 1e-5
            assert np.all(np.abs(g - r) <= rel * np.abs(r) + (5e-3 if rk == "bf16" else 1e-5)), "residuals"


def assert_decode_matches(s: synth.Shape, t: dict, c: dict, o: dict, algo: int, predictor_shared: int = 1,
                          m: int | None = None, what: str = ""):
    """Decode of every layer (and with the subset, when the workload has one)
    against the oracle's decode of the same stored cache."""
    use_subset = o.get("subset") is not None
    for sub in ([False, True] if use_subset else [False]):
        dcd = dev.Decoder(s, t, c, algo=algo, use_subset=sub, predictor_shared=predictor_shared, m=m)
        for layer in range(s.group_layers):
            out, lse = dcd(layer)
            torch.cuda.synchronize()
            ref, ref_lse = oracle_decode(s, o, c, layer, subset=o.get("subset") if sub else None)
            assert_decode_close(s, out, lse, ref, ref_lse, f"{what} layer {layer} subset={sub} algo={algo}")


def _pad_slots(c: dict, m_total: int) -> dict:
    """Residual arrays widened to m_total slots (INT32_MAX, zero residuals)."""
    out = dict(c)
    idx = c["resid_idx"]
    pad = m_total - idx.shape[-1]
    out["resid_idx"] = torch.cat([idx, torch.full(idx.shape[:-1] + (pad,), O.INT32_MAX, dtype=idx.dtype,
                                                  device=idx.device)], -1).contiguous()
    for k in ("resid_val", "resid_scale"):
        if c.get(k) is not None:
            x = c[k]
            out[k] = torch.cat([x, torch.zeros(x.shape[:3] + (pad,) + x.shape[4:], dtype=x.dtype,
                                               device=x.device)], 3).contiguous()
    return out


def _rows(x: torch.Tensor, n0: np.ndarray, n_new: int) -> torch.Tensor:
    """Rows n0[b] .. n0[b] + n_new - 1 of every sequence of a [B, G, N, H, d] tensor."""
    return torch.stack([x[b, :, int(n0[b]):int(n0[b]) + n_new] for b in range(x.shape[0])]).contiguous()

def assert_append_matches(s: synth.Shape, t: dict, n_new: int, unused, algo: int, name: str = ""):
    """Prefill of the first n0[b] = N - n_new - unused[b] rows of every
    sequence, then lowram_append_body of the next n_new rows, against the
    oracle's append_body on the same stored cache; then decode of the folded
    cache against the oracle's decode of it."""
    B, G, H, N = s.batch, s.group_layers, s.n_kv_heads, s.n_rows
    n0 = np.array([N - n_new - unused[b] for b in range(B)], dtype=np.int64)
    a, den = s.resid_frac
    m_new = -(-n_new * a // den)
    m0 = -(-int(n0.max()) * a // den)
    # prefill of the first n0[b] rows, m0 residual entries each, then room for m_new more
    t0 = dict(t)
    t0["n_body"] = torch.from_numpy(n0.astype(np.int32)).cuda()
    c0 = dev.alloc_cache(s, m=m0)
    dev.prefill(s, t0, c0, m=m0, algo=algo)
    c = _pad_slots(c0, m0 + m_new)
    torch.cuda.synchronize()
    ck, rk = kind(s, "coef"), kind(s, "resid")
    before = dict(coef=stored(c, "coef", ck), idx=c["resid_idx"].cpu().numpy().astype(np.int64),
                  res=stored(c, "resid", rk))
    # the rows to fold
    k_new, v_new = _rows(t["k_post"], n0, n_new), _rows(t["v"], n0, n_new)
    pos_new = None
    pos_dev = None
    if t.get("pos") is not None:
        pos_new = torch.stack([t["pos"][b, int(n0[b]):int(n0[b]) + n_new] for b in range(B)]).contiguous()
        pos_dev = t["pos"].clone()
        for b in range(B):
            pos_dev[b, int(n0[b]):] = -1                 # rows past the body: written by the call
    n_body = t0["n_body"].clone()
    err_new = torch.empty((B, G, H, n_new), dtype=torch.float32, device="cuda")
    sh = dev.abi_shape(s, n_resid=m0 + m_new, algo=algo)
    ws = dev.workspace(L.lowram_append_workspace_size(sh, n_new, m_new))
    L.lowram_append_body(sh, n_new, m_new, k_new, v_new, pos_new, t["basis"], t["w1"], t["b1"], t["w2"], t["b2"],
                         n_body, pos_dev, c["coef"], c.get("coef_scale"), c["resid_idx"], c["resid_val"],
                         c.get("resid_scale"), err_new, ws)
    torch.cuda.synchronize()

    assert np.array_equal(n_body.cpu().numpy(), n0 + n_new)
    if pos_dev is not None:
        for b in range(B):
            assert np.array_equal(pos_dev[b, :int(n0[b]) + n_new].cpu().numpy(),
                                  t["pos"][b, :int(n0[b]) + n_new].cpu().numpy())
    # the oracle's append on the same stored cache, selecting on the library's scores
    o = oracle_inputs(t)
    e_gpu = err_new.cpu().numpy().astype(np.float64)
    pre = O.OracleCache(coef=before["coef"], coef_kind=ck, resid_idx=before["idx"], resid_val=before["res"],
                        resid_kind=rk)
    oc, nb_ref, _, err_ref = O.append_body(
        pre, n0, o["pos"], np_in(k_new), np_in(v_new), None if pos_new is None else pos_new.cpu().numpy(),
        o["basis"], o["w1"], o["b1"], o["w2"], o["b2"], m_new, s.theta, err_override=e_gpu)
    assert np.array_equal(nb_ref, n0 + n_new)
    tol = 1e-5 if s.dtype == "f32" else 2e-2
    scale = np.maximum(err_ref.max(-1, keepdims=True), 1e-30)
    assert np.all(np.abs(e_gpu - err_ref) <= tol * scale), "scores of the new rows"
    # residual lists: old entries kept, new entries the oracle's choice on the library's scores
    assert np.array_equal(c["resid_idx"].cpu().numpy().astype(np.int64), oc.resid_idx), "residual lists"
    # coefficients: every row (the rows before n0 come from the prefill, the
    # others from the append; both are projections of the workload's rows)
    assert_coef_close(s, oracle_inputs(dict(t, n_body=torch.from_numpy((n0 + n_new).astype(np.int32)).cuda())),
                      stored(c, "coef", ck), oc.coef)
    # rows stored before the call: untouched (every array of the storage form)
    after = stored(c, "coef", ck)
    pairs = zip(after, before["coef"]) if ck == "int4" else [(after, before["coef"])]
    for x_after, x_before in pairs:
        for b in range(B):
            assert np.array_equal(x_after[b, :int(n0[b])], x_before[b, :int(n0[b])])
    # residual values
    if rk == "int4":
        pg, _ = stored(c, "resid", rk)
        po, _ = oc.resid_val
        cg, co = O.int4_unpack(pg).astype(int), O.int4_unpack(po).astype(int)
        assert np.abs(cg - co).max() <= 1 and np.mean(cg == co) > 0.97
    else:
        g = O.dequant_store(stored(c, "resid", rk), rk)
        r = O.dequant_store(oc.resid_val, rk)
        rel = 2.0 ** -7 if rk == "bf16" else 1e-5
        assert np.all(np.abs(g - r) <= rel * np.abs(r) + (5e-3 if rk == "bf16" else 1e-5)), "residuals"

    # decode over the folded cache
    tf = dict(t)
    tf["n_body"] = n_body
    if pos_dev is not None:
        tf["pos"] = pos_dev
    of = oracle_inputs(tf)
    dcd = dev.Decoder(s, tf, c, algo=algo, m=m0 + m_new)
    for layer in range(G):
        out, lse = dcd(layer)
        torch.cuda.synchronize()
        ref, ref_lse = oracle_decode(s, of, c, layer)
        assert_decode_close(s, out, lse, ref, ref_lse, f"{name} layer {layer}")


def projection_magnitude(s: synth.Shape, o: dict) -> np.ndarray:
    """S[b, t, k] = sum_c |basis[b, k, c]| |x[b, t, c]| over the pre-RoPE key
    row x: the scale of the rounding error of coefficient (t, k) when the
    projection is summed in fp32 (zero for padding rows)."""
    k_post = o["k_post"]
    B, G, N, H, d = k_post.shape
    S = np.zeros((B, N, s.rank))
    for b in range(B):
        n = int(o["n_body"][b])
        if n == 0:
            continue
        p = np.arange(N) if o["pos"] is None else np.asarray(o["pos"][b])
        k_pre = O.rope_rotate(k_post[b, :, :n].transpose(0, 2, 1, 3), p[:n], s.theta, inverse=True)
        X = k_pre.transpose(2, 0, 1, 3).reshape(n, -1)
        S[b, :n] = np.abs(X) @ np.abs(o["basis"][b]).T
    return S


def assert_coef_close(s: synth.Shape, o: dict, got, ref, what: str = "coefficients"):
    """Stored coefficients against the oracle's: every value within one
    storage unit of the oracle's plus the fp32 accumulation noise of the
    projection (2^-20 S, S from projection_magnitude: sixteen fp32 units of
    the magnitude sum); equal for almost all values far enough above that
    noise for their rounding to be determined.  Where the exact coefficient
    is zero (rows of the basis outside the span of the keys) both sides hold
    rounding noise of their own precision, which only the first rule bounds.
    fp32 storage keeps the fp32 tolerance (1e-5 of the row's largest value)
    and no equality rule: its rounding is that of the arithmetic itself."""
    ck = kind(s, "coef")
    noise = 2.0 ** -20 * projection_magnitude(s, o)
    if ck == "int4":
        pg, sg = got
        po, so = ref
        cg, co = O.int4_unpack(pg).astype(int), O.int4_unpack(po).astype(int)
        g = O.int4_dequantize_g32(cg, sg)
        r = O.int4_dequantize_g32(co, so)
        step = np.repeat(np.maximum(sg.astype(np.float64), so.astype(np.float64)), 32, axis=-1)
        viol = np.abs(g - r) - (step + noise)
        determined = np.repeat(np.abs(r).reshape(r.shape[:-1] + (-1, 32)).max(-1), 32, axis=-1) >= 2 ** 10 * np.repeat(
            noise.reshape(noise.shape[:-1] + (-1, 32)).max(-1), 32, axis=-1)
        same = cg == co
    else:
        g = O.dequant_store(got, ck)
        r = O.dequant_store(ref, ck)
        if ck == "bf16":
            unit = np.where(r != 0, 2.0 ** (np.floor(np.log2(np.abs(np.where(r != 0, r, 1.0)))) - 7), 0.0)
        else:
            unit = 1e-5 * np.abs(r).max(-1, keepdims=True)
        viol = np.abs(g - r) - (unit + noise)
        determined = np.abs(r) >= 2 ** 10 * noise
        same = g == r
    if np.any(viol > 0):
        i = np.unravel_index(np.argmax(viol), viol.shape)
        raise AssertionError(f"{what}: at {tuple(int(x) for x in i)} library {g[i]:.6g} oracle {r[i]:.6g} "
                             f"noise bound {noise[i]:.3g}")
    # equality applies to storage coarser than the fp32 arithmetic (bf16, int4)
    if ck != "f32" and determined.any():
        frac = same[determined].mean()
        assert frac > (0.99 if ck == "int4" else 0.98), f"{what}: {frac:.4f} of the determined values equal"
