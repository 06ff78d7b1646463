"""Full-size parity: every workload at its benchmark size, decoded in the same
launch configuration that bench.py times (the default kernel choice), with
the oracle recomputing sampled sequences one at a time.

For each workload: the library compresses the whole batch; the oracle runs
its own prefill of each sampled sequence.  The library's prefill of the first
sample is checked against it (scores and coefficients within tolerance, each
residual list the exact top-m of the library's scores and a valid top-m of
the oracle's, residuals against their definition).  The sampled sequences'
slices of the cache are then replaced by the oracle's stored cache, the
whole batch is decoded as bench.py launches it, and the samples are checked
against the oracle's decode of its cache, every layer.
Large batches repeat a few distinct recipe sequences (queries stay distinct)
so host-side generation stays within seconds.
"""
import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_05_amd import device as dev
from decode_attention_05_amd import lowram as L
from decode_attention_05_amd import synth

import score_bounds as SB
from gpu_helpers import (assert_band_small, assert_decode_close, assert_residuals_close, coef_rows_equal,
                         new_rows_score_bounds, score_bounds_of,
                         kind, np_in, oracle_residuals, upload_cache)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

C = synth.CONFIGS
FULL = {
    "cfg2-llama8b-8k": (C[2], 8, [0, 7]),
    "cfg3-32k-subset": (C[3], 2, [0, 15]),
    "cfg4-int4-evict-131k": (C[4], 2, [1]),
    "cfg5-gqa7-32k-slice": (synth.scaled(C[5], batch=2), 2, [0, 1]),
}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.library()


def _slice_inputs(t: dict, b: int) -> dict:
    o = {k: np_in(t[k][b:b + 1]) for k in ("q", "k_post", "v", "basis", "tail_k", "tail_v")}
    for k in ("w1", "b1", "w2", "b2"):
        o[k] = np_in(t[k])
    o["n_body"] = t["n_body"][b:b + 1].cpu().numpy()
    o["tail_len"] = t["tail_len"][b:b + 1].cpu().numpy()
    o["pos"] = None if t.get("pos") is None else t["pos"][b:b + 1].cpu().numpy()
    if t.get("subset_off") is not None:
        off = t["subset_off"].cpu().numpy()
        o["subset"] = [t["subset_idx"][off[b]:off[b + 1]].cpu().numpy()]
    return o


def _slice_store(c: dict, which: str, k: str, b: int):
    v = c["coef"] if which == "coef" else c["resid_val"]
    sc = c.get("coef_scale") if which == "coef" else c.get("resid_scale")
    if k == "int4":
        return (v[b:b + 1].cpu().numpy(), sc[b:b + 1].cpu().numpy())
    return dev.to_numpy_store(v[b:b + 1])


def _put_sequence(c: dict, oc: O.OracleCache, b: int):
    """Overwrite sequence b of the library's cache with the oracle's stored cache of it."""
    up = upload_cache(None, oc)
    for k in ("coef", "coef_scale", "resid_idx", "resid_val", "resid_scale"):
        if c.get(k) is not None:
            c[k][b:b + 1].copy_(up[k])


@pytest.mark.parametrize("name", list(FULL))
def test_fullsize_prefill_and_decode(name):
    s, distinct, samples = FULL[name]
    print(f"[fullsize {name}] B={s.batch} N={s.n_rows} m={s.n_resid} r={s.rank}", flush=True)
    w = synth.make_workload(s, seed=500 + len(name), distinct=distinct)
    t = dev.upload(w)
    c = dev.alloc_cache(s)
    dev.prefill(s, t, c)
    torch.cuda.synchronize()
    ck, rk = kind(s, "coef"), kind(s, "resid")

    # the oracle's own prefill of each sampled sequence
    ocs = {}
    for b in samples:
        o = _slice_inputs(t, b)
        ocs[b] = O.prefill(o["k_post"], o["v"], o["pos"], o["n_body"], o["basis"], o["w1"], o["b1"], o["w2"],
                           o["b2"], s.n_resid, s.theta, ck, rk)

    # the library's prefill of the first sampled sequence against the oracle's
    b = samples[0]
    o, oc = _slice_inputs(t, b), ocs[b]
    n = int(o["n_body"][0])
    e_gpu = c["err"][b:b + 1].cpu().numpy().astype(np.float64)
    ref = oc.err[0]
    bound = score_bounds_of(s, o, oc)[0]
    SB.assert_scores_within(e_gpu[0, :, :, :n], ref[:, :, :n], bound[:, :, :n], f"{name} scores")
    stats = SB.SelectionStats()
    idx_gpu = c["resid_idx"][b:b + 1].cpu().numpy().astype(np.int64)
    res_gpu = _slice_store(c, "resid", rk, b)
    same = coef_rows_equal(_slice_store(c, "coef", ck, b), oc.coef, ck)
    checked = chosen = 0
    for l in range(s.group_layers):
        for h in range(s.n_kv_heads):
            SB.check_selection(idx_gpu[0, l, h], e_gpu[0, l, h], ref[l, h], bound[l, h], n, s.n_resid,
                               f"{name} b={b} l={l} h={h}", stats)
            k = min(s.n_resid, n)
            sel = np.nonzero(same[0, idx_gpu[0, l, h, :k]])[0]
            chosen += k
            checked += len(sel)
            if len(sel):
                rows = idx_gpu[0, l, h, sel]
                want = oracle_residuals(s, o, oc.khat_pre[0], 0, l, h, rows)
                got = tuple(x[0, l, h, sel] for x in res_gpu) if rk == "int4" else res_gpu[0, l, h, sel]
                assert_residuals_close(s, got, rk, want, f"{name} residuals l={l} h={h}")
    print(f"[fullsize {name}] residuals checked on {checked} of {chosen} chosen rows", flush=True)
    assert_band_small(stats, f"fullsize {name} b={b}", ck)
    assert checked >= max(1, chosen // 20)
    if ck == "int4":
        cg = O.int4_unpack(_slice_store(c, "coef", ck, b)[0]).astype(int)
        co = O.int4_unpack(oc.coef[0]).astype(int)
        assert np.abs(cg - co).max() <= 1 and np.mean(cg == co) > 0.99
    else:
        g = O.dequant_store(_slice_store(c, "coef", ck, b), ck)
        r = O.dequant_store(oc.coef, ck)
        assert np.all(np.abs(g - r) <= np.abs(r) * 2.0 ** -7 + 1e-6 * np.abs(r).max(-1, keepdims=True))
        assert np.mean(g == r) > 0.98

    # decode of the whole batch, as bench.py launches it, with the sampled
    # sequences holding the oracle's stored cache, against the oracle's decode
    for bs in samples:
        _put_sequence(c, ocs[bs], bs)
    for sub in ([False, True] if w.subset is not None else [False]):
        dcd = dev.Decoder(s, t, c, use_subset=sub)
        for layer in range(s.group_layers):
            out, lse = dcd(layer)
            torch.cuda.synchronize()
            for bs in samples:
                ob, ocb = _slice_inputs(t, bs), ocs[bs]
                ref_o, ref_l = O.decode(layer, ob["q"], ocb.coef, ck, ob["pos"], ob["n_body"], ob["basis"],
                                        ob["w1"], ob["b1"], ob["w2"], ob["b2"], ocb.resid_idx, ocb.resid_val, rk,
                                        ob["tail_k"], ob["tail_v"], ob["tail_len"], s.theta,
                                        subset=ob.get("subset") if sub else None)
                assert_decode_close(s, out[bs:bs + 1], lse[bs:bs + 1], ref_o, ref_l,
                                    f"{name} b={bs} layer={layer} subset={sub}")
    del t, c
    torch.cuda.empty_cache()


def test_fullsize_fit_gradient():
    """The predictor fit as bench.py times it (8k Llama-shaped group, one
    predictor per sequence and head: 256 predictors x 8064 rows), one Adam
    step, with sequence 0 holding the oracle's own stored coefficients: the
    gradient and loss of its 32 predictors against the oracle's, under the
    bounds of the small-size fit tests (first-order bound per element, 2^-12
    of each tensor's norm)."""
    from gpu_helpers import EPS_BOUND, flat_params, grad_bound
    s = C[2]
    B, G, H, d = s.batch, s.group_layers, s.n_kv_heads, s.head_dim
    print(f"[fullsize fit] B={B} N={s.n_rows} predictors={B * G * H}", flush=True)
    w = synth.make_workload(s, seed=700, distinct=2)
    t = dev.upload(w)
    c = dev.alloc_cache(s)
    dev.prefill(s, t, c)
    torch.cuda.synchronize()
    ck = kind(s, "coef")
    o = _slice_inputs(t, 0)
    oc = O.prefill(o["k_post"], o["v"], o["pos"], o["n_body"], o["basis"], o["w1"], o["b1"], o["w2"], o["b2"],
                   0, s.theta, ck, kind(s, "resid"))
    c["coef"][0:1].copy_(upload_cache(None, oc)["coef"])
    w0 = {k: t[k].expand(B, *t[k].shape[1:]).contiguous() for k in ("w1", "b1", "w2", "b2")}
    w0_np = [np_in(w0[k][0:1]) for k in ("w1", "b1", "w2", "b2")]
    tw = dict(t, **{k: v.clone() for k, v in w0.items()})
    loss, grad = dev.fit(s, tw, c, steps=1, lr=1e-3, predictor_shared=0)
    torch.cuda.synchronize()
    loss = loss.cpu().numpy().astype(np.float64)
    grad = grad.cpu().numpy().astype(np.float64)
    ref = O.fit_predictor(oc.coef, ck, o["n_body"], o["basis"], o["v"], *w0_np, steps=1, lr=1e-3)
    cq = O.dequant_store(oc.coef, ck)[0]
    n = int(o["n_body"][0])
    cuts = [0, d * d, d * d + d, 2 * d * d + d, 2 * d * d + 2 * d]
    for l in range(G):
        for h in range(H):
            c0 = (l * H + h) * d
            K = cq[:n] @ o["basis"][0][:, c0:c0 + d]
            Km = np.abs(cq[:n]) @ np.abs(o["basis"][0][:, c0:c0 + d])
            V = o["v"][0, l, :n, h]
            bounds, loss_m = grad_bound(K, Km, V, *(x[0, l, h] for x in w0_np))
            bnd = EPS_BOUND * np.concatenate([bounds[0].ravel(), bounds[1], bounds[2].ravel(), bounds[3]])
            g_ref = flat_params(ref.grad0, 0, l, h)
            err = np.abs(grad[0, l, h] - g_ref)
            assert np.all(err <= bnd + 1e-30), f"l={l} h={h}: gradient beyond its bound"
            for k in range(4):
                assert np.linalg.norm(err[cuts[k]:cuts[k + 1]]) <= \
                    EPS_BOUND * np.linalg.norm(g_ref[cuts[k]:cuts[k + 1]]) + 1e-30, f"l={l} h={h} tensor {k}"
            assert abs(loss[0, 0, l, h] - ref.losses[0, 0, l, h]) <= EPS_BOUND * loss_m + 1e-30
    del t, c
    torch.cuda.empty_cache()


def test_fullsize_fold():
    """lowram_append_body as bench.py times it: the last 128 rows of every
    sequence of the 8k workload folded into a body prefilled up to them, with
    sequence 0 holding the oracle's own stored cache of its first rows.
    Sequence 0 against the oracle's append_body of that cache: scores of the
    new rows, the stored entries kept, the new entries the top-m of the
    library's scores and a valid top-m of the oracle's, the new coefficient
    rows, and the new residuals against their definition."""
    from gpu_helpers import _pad_oracle_slots, assert_coef_close, coef_rows_equal, oracle_residuals, stored
    s = C[2]
    B, G, H, N = s.batch, s.group_layers, s.n_kv_heads, s.n_rows
    n_new = min(s.tail, N // 2)
    n0 = N - n_new
    a, den = s.resid_frac
    m_new, m0 = -(-n_new * a // den), -(-n0 * a // den)
    print(f"[fullsize fold] B={B} n0={n0} n_new={n_new} m0={m0} m_new={m_new}", flush=True)
    w = synth.make_workload(s, seed=701, distinct=2)
    t = dev.upload(w)
    t0 = dict(t)
    t0["n_body"] = torch.full((B,), n0, dtype=torch.int32, device="cuda")
    c0 = dev.alloc_cache(s, m=m0)
    dev.prefill(s, t0, c0, m=m0)
    c = dev.alloc_cache(s, m=m0 + m_new)
    c["coef"] = c0["coef"]
    c["resid_idx"].fill_(O.INT32_MAX)
    c["resid_idx"][..., :m0] = c0["resid_idx"]
    c["resid_val"].zero_()
    c["resid_val"][:, :, :, :m0] = c0["resid_val"]
    ck, rk = kind(s, "coef"), kind(s, "resid")
    o0 = _slice_inputs(t0, 0)
    pre = _pad_oracle_slots(O.prefill(o0["k_post"], o0["v"], o0["pos"], o0["n_body"], o0["basis"], o0["w1"],
                                      o0["b1"], o0["w2"], o0["b2"], m0, s.theta, ck, rk), m0 + m_new)
    up = upload_cache(None, pre)
    for k in ("coef", "resid_idx", "resid_val"):
        c[k][0:1].copy_(up[k])
    torch.cuda.synchronize()
    k_new = t["k_post"][:, :, n0:].contiguous()
    v_new = t["v"][:, :, n0:].contiguous()
    n_body = t0["n_body"].clone()
    err_new = torch.empty((B, G, H, n_new), dtype=torch.float32, device="cuda")
    sh = dev.abi_shape(s, n_resid=m0 + m_new)
    ws = dev.workspace(L.lowram_append_workspace_size(sh, n_new, m_new))
    L.lowram_append_body(sh, n_new, m_new, k_new, v_new, None, t["basis"], t["w1"], t["b1"], t["w2"], t["b2"],
                         n_body, None, c["coef"], None, c["resid_idx"], c["resid_val"], None, err_new, ws)
    torch.cuda.synchronize()
    assert torch.all(n_body == N)
    o = _slice_inputs(t, 0)
    oc, nb_ref, _, err_ref = O.append_body(pre, o0["n_body"], None, np_in(k_new[0:1]), np_in(v_new[0:1]), None,
                                           o["basis"], o["w1"], o["b1"], o["w2"], o["b2"], m_new, s.theta)
    e_gpu = err_new[0:1].cpu().numpy().astype(np.float64)
    bound = new_rows_score_bounds(s, o, np_in(k_new[0:1]), np_in(v_new[0:1]),
                                  n0 + np.arange(n_new)[None, :], m_new, err_ref)
    SB.assert_scores_within(e_gpu, err_ref, bound, "fold scores")
    stats = SB.SelectionStats()
    idx = c["resid_idx"][0].cpu().numpy().astype(np.int64)
    res = dev.to_numpy_store(c["resid_val"][0:1])
    got_coef = dev.to_numpy_store(c["coef"][0:1])
    same = coef_rows_equal(got_coef, oc.coef, ck)
    khat = O.dequant_store(oc.coef, ck)[0] @ o["basis"][0]
    checked = 0
    for l in range(G):
        for h in range(H):
            lst, old = idx[l, h], pre.resid_idx[0, l, h]
            k_old = int(np.sum(old < n0))
            assert np.array_equal(lst[:k_old], old[:k_old]), f"l={l} h={h}: stored entries changed"
            assert np.array_equal(res[0, l, h, :k_old], pre.resid_val[0, l, h, :k_old])
            new = lst[k_old:k_old + m_new]
            SB.check_selection(np.where(new == O.INT32_MAX, O.INT32_MAX, new - n0), e_gpu[0, l, h],
                               err_ref[0, l, h], bound[0, l, h], n_new, m_new, f"fold l={l} h={h}", stats)
            k = int(np.sum(new != O.INT32_MAX))
            sel = np.nonzero(same[0, new[:k]])[0]
            checked += len(sel)
            if len(sel):
                want = oracle_residuals(s, o, khat, 0, l, h, new[sel])
                assert_residuals_close(s, res[0, l, h, k_old + sel], rk, want, f"fold residuals l={l} h={h}")
    assert checked > 0
    assert_band_small(stats, "fullsize fold", ck)
    assert np.array_equal(got_coef[0, :n0], pre.coef[0, :n0])
    assert_coef_close(s, o, got_coef, oc.coef, "folded coefficients")
    del t, c, c0
    torch.cuda.empty_cache()


BASIS_FULL = {
    # workload: (shape, sequences checked)
    "cfg2-llama8b-8k": (C[2], (0, 7)),
    "cfg4-int4-evict-131k": (C[4], (1,)),
}


@pytest.mark.parametrize("name", list(BASIS_FULL))
def test_fullsize_basis(name):
    """The key basis as bench.py computes it (two power rounds; the 8k
    Llama-shaped group: 8 sequences of 8064 rows, D = 4096, r = 512; the
    131k workload: 4 sequences of 39,245 kept rows at their original
    positions, r = 384): sampled sequences against the oracle's subspace
    iteration from the same start, under the small-size bounds."""
    from test_gpu_basis import assert_basis_matches
    s, seqs = BASIS_FULL[name]
    print(f"[fullsize basis {name}] B={s.batch} N={s.n_rows} D={s.D} r={s.rank}", flush=True)
    w = synth.make_workload(s, seed=701, with_basis=False, distinct=2)
    t = dev.upload(w)
    start = np.random.default_rng(702).standard_normal((s.batch, s.rank, s.D)).astype(np.float32)
    out = dev.compute_basis(s, t, torch.from_numpy(start).cuda(), 2)
    torch.cuda.synchronize()
    got = np_in(out)
    pos = None if t.get("pos") is None else t["pos"].cpu().numpy()
    for b in seqs:
        k_post = np_in(t["k_post"][b:b + 1])
        print(f"[fullsize basis] oracle sequence {b}", flush=True)
        assert_basis_matches(s, got[b:b + 1], k_post, None if pos is None else pos[b:b + 1],
                             t["n_body"][b:b + 1].cpu().numpy(), start[b:b + 1].astype(np.float64), 2,
                             check_optimum=False)
    del t, out
    torch.cuda.empty_cache()
