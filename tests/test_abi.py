"""The C ABI without a GPU: the library loads, exports every declared
symbol, and the host-side checks return the documented status codes before
anything is launched."""
import ctypes

import numpy as np
import pytest

from decode_attention_05_amd import lowram as L
from decode_attention_05_amd import synth
from decode_attention_05_amd.device import abi_shape


def test_library_exports_every_header_symbol():
    lib = L.library()
    names = L.header_functions()
    assert {"lowram_compress_prefill", "lowram_decode_attn", "lowram_workspace_size",
            "lowram_status_string", "lowram_last_error", "lowram_dense_decode_attn",
            "lowram_dense_workspace_size", "lowram_decode_attn_timed", "lowram_check_decode_indices",
            "lowram_append_body",
            "lowram_append_workspace_size", "lowram_fit_predictor", "lowram_fit_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout():
    assert ctypes.sizeof(L.lowram_fit_params) == 40
    assert L.lowram_fit_params.lr.offset == 8
    assert ctypes.sizeof(L.lowram_shape) == 72
    assert L.lowram_shape.rope_theta.offset == 40
    assert ctypes.sizeof(L.lowram_cache) == 15 * 8


def _shape(**kw):
    base = dict(batch=2, group_layers=2, n_q_heads=8, n_kv_heads=2, head_dim=128, rank=64,
                n_body_max=100, n_resid=20, tail_max=8, rope_theta=10000.0, dtype=L.BF16)
    base.update(kw)
    return L.make_shape(**base)


def test_timed_decode_needs_both_events():
    sh = _shape()
    lib = L.library()
    for before, after in ((None, None), (0x1000, None), (None, 0x1000)):
        st = lib.lowram_decode_attn_timed(ctypes.byref(sh), 0, None, None, None, None, None, None, None, 0, None,
                                          before, after)
        assert st == L.E_ARG and "both" in L.lowram_last_error()


def _valid_indices(sh):
    """Host index arrays of a well-formed decode call of shape sh."""
    B, G, H, N, m, Te = sh.batch, sh.group_layers, sh.n_kv_heads, sh.n_body_max, sh.n_resid, sh.tail_max
    rng = np.random.default_rng(0)
    nb = np.array([N, N // 2], dtype=np.int32)[:B]
    tl = np.array([Te, 0], dtype=np.int32)[:B]
    pos = np.tile(np.arange(N, dtype=np.int32) * 3, (B, 1))
    ridx = np.full((B, G, H, m), 2**31 - 1, dtype=np.int32)
    for b in range(B):
        for l in range(G):
            for h in range(H):
                k = min(m, int(nb[b]))
                ridx[b, l, h, :k] = np.sort(rng.choice(int(nb[b]), k, replace=False))
    rows = [np.sort(rng.choice(int(nb[b]), 7, replace=False)).astype(np.int32) for b in range(B)]
    off = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    idx = np.concatenate(rows).astype(np.int32)
    return dict(n_body=nb, tail_len=tl, pos=pos, resid_idx=ridx, subset_off=off, subset_idx=idx)


def _check(sh, a):
    return L.lowram_check_decode_indices(sh, a["n_body"], a["tail_len"], a["pos"], a["resid_idx"],
                                         a["subset_off"], a["subset_idx"])


def test_index_checker_accepts_valid_indices():
    sh = _shape()
    a = _valid_indices(sh)
    _check(sh, a)
    _check(sh, dict(a, pos=None, tail_len=None, subset_off=None, subset_idx=None))


def _broken(name):
    sh = _shape()
    a = {k: v.copy() for k, v in _valid_indices(sh).items()}
    if name == "n_body above n_body_max":
        a["n_body"][0] = sh.n_body_max + 1
    elif name == "negative tail_len":
        a["tail_len"][1] = -1
    elif name == "tail_len above tail_max":
        a["tail_len"][0] = sh.tail_max + 1
    elif name == "negative position":
        a["pos"][1, 3] = -5
    elif name == "residual list not ascending":
        a["resid_idx"][0, 1, 0, [2, 3]] = a["resid_idx"][0, 1, 0, [3, 2]]
    elif name == "residual list repeats a row":
        a["resid_idx"][1, 0, 1, 4] = a["resid_idx"][1, 0, 1, 3]
    elif name == "residual row past n_body":
        a["resid_idx"][1, 1, 1, :] = 2**31 - 1
        a["resid_idx"][1, 1, 1, 0] = int(a["n_body"][1])
    elif name == "row after padding":
        a["resid_idx"][1, 0, 0, -1] = 0
    elif name == "subset not ascending":
        a["subset_idx"][[1, 2]] = a["subset_idx"][[2, 1]]
    elif name == "subset entry past n_body":
        a["subset_idx"][-1] = int(a["n_body"][1])
    elif name == "subset offsets decrease":
        a["subset_off"][1] = a["subset_off"][2] + 1
    return sh, a


@pytest.mark.parametrize("name", ["n_body above n_body_max", "negative tail_len", "tail_len above tail_max",
                                  "negative position", "residual list not ascending", "residual list repeats a row",
                                  "residual row past n_body", "row after padding", "subset not ascending",
                                  "subset entry past n_body", "subset offsets decrease"])
def test_index_checker_rejects(name):
    sh, a = _broken(name)
    with pytest.raises(L.LowramError) as ei:
        _check(sh, a)
    assert ei.value.status == L.E_ARG


def test_status_strings():
    assert L.status_string(0) == "LOWRAM_OK"
    assert L.status_string(-3) == "LOWRAM_E_WORKSPACE"


@pytest.mark.parametrize("kw,code", [
    (dict(n_q_heads=7), L.E_ARG),
    (dict(head_dim=96), L.E_UNSUPPORTED),
    (dict(rank=48), L.E_ARG),
    (dict(rank=8192), L.E_ARG),
    (dict(n_resid=101), L.E_ARG),
    (dict(batch=0), L.E_ARG),
    (dict(rope_theta=-1.0), L.E_ARG),
    (dict(dtype=L.F32, coef_store=L.STORE_INT4), L.E_UNSUPPORTED),
    (dict(n_q_heads=18, n_kv_heads=2), L.E_UNSUPPORTED),
    (dict(dtype=7), L.E_ARG),
    (dict(algo=9), L.E_ARG),
])
def test_shape_checks(kw, code):
    sh = _shape(**kw)
    n = ctypes.c_size_t()
    assert L.library().lowram_workspace_size(ctypes.byref(sh), 1, ctypes.byref(n)) == code
    assert L.lowram_last_error() != ""


def test_struct_size_checked():
    sh = _shape()
    sh.struct_size = 64
    n = ctypes.c_size_t()
    assert L.library().lowram_workspace_size(ctypes.byref(sh), 0, ctypes.byref(n)) == L.E_ARG


def test_workspace_sizes():
    sh = _shape()
    # prefill, plain kernels: fp32 scores [B, G, Hkv, N] (rounded up to 256 bytes)
    scores = -(-2 * 2 * 2 * 100 * 4 // 256) * 256
    assert L.lowram_workspace_size(_shape(algo=L.ALGO_PLAIN), 0) == scores
    # MFMA kernels, at most 256 rows per sequence: each workgroup runs the whole
    # contraction, so the scores are all
    assert L.lowram_workspace_size(sh, 0) == scores
    # more rows: the scores, then fp32 partial coefficients [splits, B, N, r]: two sequences
    # of three 128-row tiles give 6 workgroups, so the contraction over the 4 (layer, head)
    # blocks splits 4 ways
    sh3 = _shape(n_body_max=300)
    scores3 = -(-2 * 2 * 2 * 300 * 4 // 256) * 256
    assert L.lowram_workspace_size(sh3, 0) == scores3 + 4 * 2 * 300 * 64 * 4
    # decode, plain kernel: one (M, L, acc1, pad, acc_h[d], acc_v[d]) record per (b, qh, split)
    shp = _shape(algo=L.ALGO_PLAIN)
    ws = L.lowram_workspace_size(shp, 1)
    assert ws == 2 * 8 * ((100 + 63) // 64 + 1) * (4 + 2 * 128) * 4
    # MFMA kernel: the records plus its per-call staging, larger than the records alone
    assert L.lowram_workspace_size(_shape(), 1) > 2 * 8 * 2 * (4 + 2 * 128) * 4
    assert L.lowram_dense_workspace_size(2, 8, 2, 128, 1000) == 2 * 8 * 2 * (4 + 256) * 4


def test_decode_checks_before_launch():
    lib = L.library()
    sh = _shape()
    fake = ctypes.c_void_p(0x1000)          # never dereferenced: the checks fail first
    cache = L.lowram_cache(*([0x1000] * 15))
    args = lambda layer, q, c, off, idx, out, ws, wsb: lib.lowram_decode_attn(
        ctypes.byref(sh), layer, q, c, off, idx, out, None, ws, wsb, None)
    assert args(2, fake, ctypes.byref(cache), None, None, fake, fake, 1 << 30) == L.E_ARG   # layer
    assert args(-1, fake, ctypes.byref(cache), None, None, fake, fake, 1 << 30) == L.E_ARG
    assert args(0, None, ctypes.byref(cache), None, None, fake, fake, 1 << 30) == L.E_ARG   # q
    assert args(0, fake, None, None, None, fake, fake, 1 << 30) == L.E_ARG                   # cache
    assert args(0, fake, ctypes.byref(cache), fake, None, fake, fake, 1 << 30) == L.E_ARG   # subset idx
    assert args(0, fake, ctypes.byref(cache), None, None, fake, fake, 16) == L.E_WORKSPACE
    assert args(0, fake, ctypes.byref(cache), None, None, fake, None, 1 << 30) == L.E_WORKSPACE
    bad = L.lowram_cache(*([0x1000] * 15))
    bad.basis = None
    assert args(0, fake, ctypes.byref(bad), None, None, fake, fake, 1 << 30) == L.E_ARG
    # MFMA forced on an fp32 shape
    sh32 = _shape(dtype=L.F32, algo=L.ALGO_MFMA)
    assert lib.lowram_decode_attn(ctypes.byref(sh32), 0, fake, ctypes.byref(cache), None, None, fake,
                                  None, fake, 1 << 30, None) == L.E_UNSUPPORTED


def test_prefill_checks_before_launch():
    lib = L.library()
    sh = _shape()
    f = ctypes.c_void_p(0x1000)
    call = lambda sh, resid_idx, err, ws, wsb: lib.lowram_compress_prefill(
        ctypes.byref(sh), f, f, None, f, f, f, f, f, f, f, None, resid_idx, f, None, err, ws, wsb, None)
    assert call(sh, None, f, None, 0) == L.E_ARG                      # residual outputs needed
    assert call(sh, f, None, None, 0) == L.E_WORKSPACE                # no err_out and no workspace
    assert call(sh, f, None, f, 10) == L.E_WORKSPACE
    sh4 = _shape(coef_store=L.STORE_INT4)
    assert call(sh4, f, f, None, 0) == L.E_ARG                        # int4 needs coef_scale_out
    # the MFMA prefill forced on shapes it does not cover
    for kw in (dict(dtype=L.F32), dict(head_dim=64), dict(rank=96), dict(rank=640, group_layers=4)):
        assert call(_shape(algo=L.ALGO_MFMA, **kw), f, f, None, 0) == L.E_UNSUPPORTED, kw


def test_dense_checks():
    lib = L.library()
    f = ctypes.c_void_p(0x1000)
    assert lib.lowram_dense_decode_attn(2, 7, 2, 128, 64, f, f, f, f, f, None, f, 1 << 30, None) == L.E_ARG
    assert lib.lowram_dense_decode_attn(2, 8, 2, 80, 64, f, f, f, f, f, None, f, 1 << 30, None) == L.E_UNSUPPORTED
    assert lib.lowram_dense_decode_attn(2, 8, 2, 128, 64, f, f, f, f, f, None, f, 8, None) == L.E_WORKSPACE


def test_bench_shapes_pass_host_checks():
    for k, s in synth.CONFIGS.items():
        n = ctypes.c_size_t()
        sh = abi_shape(s)
        assert L.library().lowram_workspace_size(ctypes.byref(sh), 1, ctypes.byref(n)) == L.OK, (k, L.lowram_last_error())


def test_append_checks_before_launch():
    lib = L.library()
    sh = _shape()                                   # N = 100, m = 20
    f = ctypes.c_void_p(0x1000)
    call = lambda sh, n_new, m_new, pos=None, pos_new=None, resid=f, ws=f, wsb=1 << 30: lib.lowram_append_body(
        ctypes.byref(sh), n_new, m_new, f, f, pos_new, f, f, f, f, f, f, pos, f, None, resid, resid, None, None,
        ws, wsb, None)
    assert call(sh, -1, 0) == L.E_ARG                                 # counts
    assert call(sh, 101, 0) == L.E_ARG
    assert call(sh, 10, 11) == L.E_ARG                                # m_new > n_new
    assert call(_shape(n_resid=4), 10, 5) == L.E_ARG                  # m_new > n_resid
    assert call(sh, 10, 3, resid=None) == L.E_ARG                     # residual arrays needed
    assert call(sh, 10, 3, pos=f) == L.E_ARG                          # cached positions need pos_new
    assert call(sh, 10, 3, ws=None, wsb=0) == L.E_WORKSPACE
    need = L.lowram_append_workspace_size(sh, 10, 3)
    assert call(sh, 10, 3, wsb=need - 1) == L.E_WORKSPACE
    assert need >= 2 * 10 * 64 * 2 + 2 * 4 * 3 * 128 * 2              # new coefficient and residual rows
    assert call(_shape(algo=L.ALGO_MFMA, head_dim=64), 10, 3) == L.E_UNSUPPORTED
    with pytest.raises(L.LowramError):
        L.lowram_append_workspace_size(sh, 10, 11)


def test_fit_checks_before_launch():
    lib = L.library()
    sh = _shape()                                   # B 2, G 2, Hkv 2, d 128, N 100
    f = ctypes.c_void_p(0x1000)
    need = L.lowram_fit_workspace_size(sh)

    def call(sh=sh, params=None, coef=f, scale=None, w=f, ws=f, wsb=need, **pk):
        prm = params if params is not None else L.make_fit_params(**{**dict(steps=3, lr=1e-3), **pk})
        return lib.lowram_fit_predictor(ctypes.byref(sh), coef, scale, f, f, f, ctypes.byref(prm), w, f, f, f,
                                        None, None, ws, wsb, None)
    assert call(steps=-1) == L.E_ARG
    assert call(lr=0.0) == L.E_ARG
    assert call(lr=float("inf")) == L.E_ARG
    assert call(beta1=1.0) == L.E_ARG
    assert call(beta2=-0.1) == L.E_ARG
    assert call(eps=0.0) == L.E_ARG
    bad = L.make_fit_params(3, 1e-3)
    bad.struct_size = 8
    assert call(params=bad) == L.E_ARG
    assert lib.lowram_fit_predictor(ctypes.byref(sh), f, None, f, f, f, None, f, f, f, f, None, None, f, need,
                                    None) == L.E_ARG                # params NULL
    assert call(w=None) == L.E_ARG                                    # predictor arrays are in/out
    assert call(coef=None) == L.E_ARG
    assert call(sh=_shape(coef_store=L.STORE_INT4)) == L.E_ARG        # int4 needs the scales
    assert call(ws=None, wsb=0) == L.E_WORKSPACE
    assert call(wsb=need - 1) == L.E_WORKSPACE
    assert call(sh=_shape(head_dim=96)) == L.E_UNSUPPORTED
    # steps = 0 launches nothing and succeeds
    assert call(steps=0) == L.OK
    # the workspace holds the rebuilt keys and both transposed copies (12 bytes per row, head and dim),
    # three fp32 copies of the parameters and the bf16 pairs of W1, W2, W2^T of each predictor
    rows = 2 * 2 * 2 * 128                          # B G Hkv x 100 rows rounded up to 128
    preds = 2 * 2                                   # shared over the batch: G Hkv predictors
    assert need >= rows * 128 * 12 + preds * (2 * 128 * 128 + 2 * 128) * 12 + preds * 6 * 128 * 128 * 2
    own = L.lowram_fit_workspace_size(_shape(predictor_shared=0))
    assert own - need >= preds * ((2 * 128 * 128 + 2 * 128) * 12 + 6 * 128 * 128 * 2)


def test_basis_checks_before_launch():
    lib = L.library()
    sh = _shape()                                   # B 2, G 2, Hkv 2, d 128, N 100
    f = ctypes.c_void_p(0x1000)
    need = L.lowram_basis_workspace_size(sh)

    def call(sh=sh, k=f, nb=f, start=f, q=2, out=f, ws=f, wsb=need):
        return lib.lowram_compute_basis(ctypes.byref(sh), k, None, nb, start, q, out, ws, wsb, None)
    assert call(q=-1) == L.E_ARG
    assert call(q=65) == L.E_ARG
    assert call(start=None) == L.E_ARG
    assert call(out=None) == L.E_ARG
    assert call(nb=None) == L.E_ARG
    assert call(k=None) == L.E_ARG
    assert call(start=ctypes.c_void_p(0x1004)) == L.E_ARG           # start must be 16-byte aligned
    assert call(ws=ctypes.c_void_p(0x1008)) == L.E_ARG              # so must the workspace
    assert call(ws=None, wsb=0) == L.E_WORKSPACE
    assert call(wsb=need - 1) == L.E_WORKSPACE
    big = _shape(rank=544, n_kv_heads=4)
    assert call(sh=big, wsb=1 << 40) == L.E_UNSUPPORTED
    with pytest.raises(L.LowramError):
        L.lowram_basis_workspace_size(big)
    # the workspace holds the pre-RoPE keys (100 rows rounded up to 128) and the iterates
    r, D = sh.rank, 2 * 2 * 128
    assert need >= 2 * 128 * D * 4 + 2 * (2 * 128 * r * 4) + 2 * (2 * r * D * 4) + 2 * r * r * (8 + 8 + 4)


def test_subset_checks_before_launch():
    lib = L.library()
    f = ctypes.c_void_p(0x1000)
    pol = L.make_subset_policy(4, 16, 3)
    # count(100) = 4 sinks + 16 recent + ceil((84 - 4) / 3) = 27 strided
    assert L.lowram_subset_capacity(2, 100, pol) == 2 * (4 + 16 + 27)
    assert L.lowram_subset_capacity(1, 0, pol) == 0

    def call(batch=2, nb=f, nmax=100, pol=pol, off=f, idx=f, cap=94):
        return lib.lowram_select_subset(batch, nb, nmax, ctypes.byref(pol), off, idx, cap, None)
    assert call(batch=0) == L.E_ARG
    assert call(nmax=-1) == L.E_ARG
    assert call(pol=L.make_subset_policy(-1, 0, 0)) == L.E_ARG
    assert call(pol=L.make_subset_policy(0, 0, -2)) == L.E_ARG
    bad = L.make_subset_policy(1, 1, 1)
    bad.struct_size = 4
    assert call(pol=bad) == L.E_ARG
    assert call(nb=None) == L.E_ARG
    assert call(off=None) == L.E_ARG
    assert call(cap=93) == L.E_ARG                                  # below the bound
