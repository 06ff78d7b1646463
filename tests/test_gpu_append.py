"""GPU parity of lowram_append_body (folding exact rows into the compressed
body) against the oracle's append_body on identical stored data.

Each case prefills the first n0[b] rows of a seeded workload (ragged over
the batch) into a cache with room for more residual entries, then appends
the next n_new rows of every sequence.  Checked:
  * rows and residual entries stored before the call are unchanged, n_body
    and the positions grow as documented;
  * the new rows' coefficients within one storage unit of the oracle's
    (equal for almost all), their scores within 1e-5 (fp32) / 2e-2 (bf16)
    of the row maximum;
  * the appended residual entries equal, bit for bit, the oracle's
    selection on the library's own scores, and the residuals match;
  * decode over the folded cache matches the oracle's decode of it.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_05_amd import device as dev
from decode_attention_05_amd import lowram as L
from decode_attention_05_amd import synth

from gpu_helpers import assert_decode_close, kind, np_in, oracle_decode, oracle_inputs, stored

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.library()


C = synth.CONFIGS
CASES = {
    # name: (shape, seed, n_new, rows left unused at the end per sequence, algo)
    "bf16-mfma": (synth.scaled(C[2], batch=2, context=1100, tail=37, rank=128, latent_rank=64), 31, 96,
                  [0, 40], L.ALGO_AUTO),
    "int4-evict-positions": (synth.scaled(C[4], batch=2, context=4096, tail=50, rank=128, latent_rank=64), 32,
                             64, [10, 0], L.ALGO_AUTO),
    "bf16-plain": (synth.scaled(C[2], batch=2, context=700, tail=20, rank=64, latent_rank=32), 33, 50,
                   [0, 7], L.ALGO_PLAIN),
    "fp32-tiny": (C[1], 34, 30, [0], L.ALGO_AUTO),
}


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


@pytest.mark.parametrize("name", list(CASES))
def test_append_parity_and_decode(name):
    s, seed, n_new, unused, algo = CASES[name]
    B, G, H, N = s.batch, s.group_layers, s.n_kv_heads, s.n_rows
    print(f"[append {name}] B={B} N={N} n_new={n_new} r={s.rank}", flush=True)
    w = synth.make_workload(s, seed)
    t = dev.upload(w)
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
    # coefficients: every row
    if ck == "int4":
        pg, sg = stored(c, "coef", ck)
        po, so = oc.coef
        cg, co = O.int4_unpack(pg).astype(int), O.int4_unpack(po).astype(int)
        assert np.abs(cg - co).max() <= 1 and np.mean(cg == co) > 0.99
        assert np.all(np.abs(sg.astype(np.float64) - so.astype(np.float64)) <= 2.0 ** -10 * np.abs(so.astype(np.float64)) + 1e-12)
    else:
        g = O.dequant_store(stored(c, "coef", ck), ck)
        r = O.dequant_store(oc.coef, ck)
        rowmax = np.abs(r).max(-1, keepdims=True)
        if ck == "bf16":
            assert np.all(np.abs(g - r) <= np.abs(r) * 2.0 ** -7 + 1e-6 * rowmax)
            assert np.mean(g == r) > 0.98
        else:
            assert np.all(np.abs(g - r) <= 1e-5 * rowmax)
        for b in range(B):                                   # rows stored before: untouched
            assert np.array_equal(g[b, :int(n0[b])], O.dequant_store(before["coef"], ck)[b, :int(n0[b])])
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
