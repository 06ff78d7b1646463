"""Python binding of liblowram.so: argument marshalling only.

Every function here has the name of the C entry point it calls and passes
torch tensors as raw device pointers plus the current HIP stream.  All work
runs in the library's HIP kernels; torch only owns device memory and
streams.  A missing library raises at load time — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblowram.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
HEADERS = [os.path.join(INCLUDE, f) for f in ("lowram.h", "lowram_basis.h", "lowram_subset.h", "lowram_timing.h")]

F32, BF16 = 0, 1
STORE_NATIVE, STORE_INT4 = 0, 1
ALGO_AUTO, ALGO_PLAIN, ALGO_MFMA = 0, 1, 2
OK, E_ARG, E_UNSUPPORTED, E_WORKSPACE, E_HIP = 0, -1, -2, -3, -4


class lowram_shape(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("batch", ctypes.c_int32), ("group_layers", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("n_body_max", ctypes.c_int32), ("n_resid", ctypes.c_int32),
        ("tail_max", ctypes.c_int32), ("rope_theta", ctypes.c_double),
        ("dtype", ctypes.c_int32), ("coef_store", ctypes.c_int32),
        ("resid_store", ctypes.c_int32), ("predictor_shared", ctypes.c_int32),
        ("algo", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class lowram_cache(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "coef", "coef_scale", "pos", "n_body", "basis", "w1", "b1", "w2", "b2",
        "resid_idx", "resid_val", "resid_scale", "tail_k", "tail_v", "tail_len")]


class lowram_fit_params(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("steps", ctypes.c_int32), ("lr", ctypes.c_double),
                ("beta1", ctypes.c_double), ("beta2", ctypes.c_double), ("eps", ctypes.c_double)]


def make_fit_params(steps: int, lr: float, beta1: float = 0.9, beta2: float = 0.999,
                    eps: float = 1e-8) -> lowram_fit_params:
    return lowram_fit_params(ctypes.sizeof(lowram_fit_params), steps, lr, beta1, beta2, eps)


class lowram_subset_policy(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("n_sink", ctypes.c_int32), ("n_recent", ctypes.c_int32),
                ("stride", ctypes.c_int32)]


def make_subset_policy(n_sink: int, n_recent: int, stride: int) -> lowram_subset_policy:
    return lowram_subset_policy(ctypes.sizeof(lowram_subset_policy), n_sink, n_recent, stride)


class LowramError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


_lib = None


def library():
    """Load liblowram.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lib.lowram_workspace_size.argtypes = [ctypes.POINTER(lowram_shape), i32, ctypes.POINTER(sz)]
        lib.lowram_compress_prefill.argtypes = [ctypes.POINTER(lowram_shape)] + [vp] * 16 + [sz, vp]
        lib.lowram_decode_attn.argtypes = [ctypes.POINTER(lowram_shape), i32, vp,
                                           ctypes.POINTER(lowram_cache), vp, vp, vp, vp, vp, sz, vp]
        lib.lowram_dense_workspace_size.argtypes = [i32] * 5 + [ctypes.POINTER(sz)]
        lib.lowram_dense_decode_attn.argtypes = [i32] * 5 + [vp] * 7 + [sz, vp]
        lib.lowram_decode_attn_timed.argtypes = [ctypes.POINTER(lowram_shape), i32, vp,
                                                 ctypes.POINTER(lowram_cache), vp, vp, vp, vp, vp, sz, vp, vp, vp]
        lib.lowram_check_decode_indices.argtypes = [ctypes.POINTER(lowram_shape)] + [vp] * 6
        lib.lowram_decode_attn_noalloc.argtypes = [ctypes.POINTER(lowram_shape), i32, vp,
                                                   ctypes.POINTER(lowram_cache), vp, vp, vp, vp, vp]
        lib.lowram_append_workspace_size.argtypes = [ctypes.POINTER(lowram_shape), i32, i32, ctypes.POINTER(sz)]
        lib.lowram_append_body.argtypes = [ctypes.POINTER(lowram_shape), i32, i32] + [vp] * 17 + [sz, vp]
        lib.lowram_fit_workspace_size.argtypes = [ctypes.POINTER(lowram_shape), ctypes.POINTER(sz)]
        lib.lowram_fit_predictor.argtypes = ([ctypes.POINTER(lowram_shape)] + [vp] * 5 +
                                             [ctypes.POINTER(lowram_fit_params)] + [vp] * 7 + [sz, vp])
        lib.lowram_basis_workspace_size.argtypes = [ctypes.POINTER(lowram_shape), ctypes.POINTER(sz)]
        lib.lowram_compute_basis.argtypes = [ctypes.POINTER(lowram_shape)] + [vp] * 4 + [i32] + [vp] * 2 + [sz, vp]
        lib.lowram_subset_capacity.argtypes = [i32, i32, ctypes.POINTER(lowram_subset_policy),
                                               ctypes.POINTER(ctypes.c_int64)]
        lib.lowram_select_subset.argtypes = [i32, vp, i32, ctypes.POINTER(lowram_subset_policy), vp, vp,
                                             ctypes.c_int64, vp]
        for f in ("lowram_workspace_size", "lowram_compress_prefill", "lowram_decode_attn",
                  "lowram_dense_workspace_size", "lowram_dense_decode_attn", "lowram_decode_attn_timed",
                  "lowram_check_decode_indices", "lowram_decode_attn_noalloc",
                  "lowram_append_workspace_size", "lowram_append_body", "lowram_fit_workspace_size",
                  "lowram_fit_predictor", "lowram_basis_workspace_size", "lowram_compute_basis",
                  "lowram_subset_capacity", "lowram_select_subset"):
            getattr(lib, f).restype = i32
        lib.lowram_status_string.argtypes = [i32]
        lib.lowram_status_string.restype = ctypes.c_char_p
        lib.lowram_last_error.argtypes = []
        lib.lowram_last_error.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in the public headers."""
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(lowram_\w+)\s*\(", text, re.M)))


def status_string(st: int) -> str:
    return library().lowram_status_string(st).decode()


def lowram_last_error() -> str:
    return library().lowram_last_error().decode()


def _check(st: int):
    if st != OK:
        raise LowramError(st, lowram_last_error())


def _p(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to liblowram must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_shape(*, batch, group_layers, n_q_heads, n_kv_heads, head_dim, rank, n_body_max,
               n_resid, tail_max, rope_theta, dtype, coef_store=STORE_NATIVE,
               resid_store=STORE_NATIVE, predictor_shared=1, algo=ALGO_AUTO) -> lowram_shape:
    return lowram_shape(ctypes.sizeof(lowram_shape), batch, group_layers, n_q_heads, n_kv_heads,
                        head_dim, rank, n_body_max, n_resid, tail_max, float(rope_theta), dtype,
                        coef_store, resid_store, predictor_shared, algo, 0)


def lowram_workspace_size(shape: lowram_shape, op: int) -> int:
    n = ctypes.c_size_t(0)
    _check(library().lowram_workspace_size(ctypes.byref(shape), op, ctypes.byref(n)))
    return n.value


def lowram_compress_prefill(shape, k_post, v, pos, n_body, basis, w1, b1, w2, b2, coef_out,
                            coef_scale_out, resid_idx_out, resid_val_out, resid_scale_out,
                            err_out, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().lowram_compress_prefill(
        ctypes.byref(shape), _p(k_post), _p(v), _p(pos), _p(n_body), _p(basis), _p(w1), _p(b1),
        _p(w2), _p(b2), _p(coef_out), _p(coef_scale_out), _p(resid_idx_out), _p(resid_val_out),
        _p(resid_scale_out), _p(err_out), _p(workspace), ws_bytes, _stream(stream)))


def lowram_append_workspace_size(shape: lowram_shape, n_new: int, m_new: int) -> int:
    n = ctypes.c_size_t(0)
    _check(library().lowram_append_workspace_size(ctypes.byref(shape), n_new, m_new, ctypes.byref(n)))
    return n.value


def lowram_append_body(shape, n_new, m_new, k_post_new, v_new, pos_new, basis, w1, b1, w2, b2, n_body, pos,
                       coef, coef_scale, resid_idx, resid_val, resid_scale, err_out, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().lowram_append_body(
        ctypes.byref(shape), n_new, m_new, _p(k_post_new), _p(v_new), _p(pos_new), _p(basis), _p(w1), _p(b1),
        _p(w2), _p(b2), _p(n_body), _p(pos), _p(coef), _p(coef_scale), _p(resid_idx), _p(resid_val),
        _p(resid_scale), _p(err_out), _p(workspace), ws_bytes, _stream(stream)))


def lowram_fit_workspace_size(shape: lowram_shape) -> int:
    n = ctypes.c_size_t(0)
    _check(library().lowram_fit_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def lowram_fit_predictor(shape, coef, coef_scale, n_body, basis, v, params, w1, b1, w2, b2, loss_out,
                         grad_out, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().lowram_fit_predictor(
        ctypes.byref(shape), _p(coef), _p(coef_scale), _p(n_body), _p(basis), _p(v), ctypes.byref(params),
        _p(w1), _p(b1), _p(w2), _p(b2), _p(loss_out), _p(grad_out), _p(workspace), ws_bytes,
        _stream(stream)))


def lowram_basis_workspace_size(shape: lowram_shape) -> int:
    n = ctypes.c_size_t(0)
    _check(library().lowram_basis_workspace_size(ctypes.byref(shape), ctypes.byref(n)))
    return n.value


def lowram_compute_basis(shape, k_post, pos, n_body, start, power_iters, basis_out, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().lowram_compute_basis(
        ctypes.byref(shape), _p(k_post), _p(pos), _p(n_body), _p(start), power_iters, _p(basis_out),
        _p(workspace), ws_bytes, _stream(stream)))


def lowram_subset_capacity(batch: int, n_body_max: int, policy: lowram_subset_policy) -> int:
    n = ctypes.c_int64(0)
    _check(library().lowram_subset_capacity(batch, n_body_max, ctypes.byref(policy), ctypes.byref(n)))
    return n.value


def lowram_select_subset(batch, n_body, n_body_max, policy, subset_off, subset_idx, stream=None):
    cap = subset_idx.numel() if subset_idx is not None else 0
    _check(library().lowram_select_subset(batch, _p(n_body), n_body_max, ctypes.byref(policy), _p(subset_off),
                                          _p(subset_idx), cap, _stream(stream)))


def make_cache(t: dict) -> lowram_cache:
    """lowram_cache from a dict of tensors (missing keys -> NULL)."""
    return lowram_cache(*[(t[k].data_ptr() if t.get(k) is not None else None)
                          for k, _ in lowram_cache._fields_])


def lowram_decode_attn(shape, layer, q, cache, subset_off, subset_idx, out, lse_out, workspace,
                       stream=None):
    c = cache if isinstance(cache, lowram_cache) else make_cache(cache)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().lowram_decode_attn(
        ctypes.byref(shape), layer, _p(q), ctypes.byref(c), _p(subset_off), _p(subset_idx),
        _p(out), _p(lse_out), _p(workspace), ws_bytes, _stream(stream)))


def lowram_dense_workspace_size(batch, n_q_heads, n_kv_heads, head_dim, max_ctx) -> int:
    n = ctypes.c_size_t(0)
    _check(library().lowram_dense_workspace_size(batch, n_q_heads, n_kv_heads, head_dim, max_ctx,
                                                 ctypes.byref(n)))
    return n.value


def lowram_dense_decode_attn(batch, n_q_heads, n_kv_heads, head_dim, max_ctx, q, k, v, ctx_len,
                             out, lse_out, workspace, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().lowram_dense_decode_attn(
        batch, n_q_heads, n_kv_heads, head_dim, max_ctx, _p(q), _p(k), _p(v), _p(ctx_len),
        _p(out), _p(lse_out), _p(workspace), ws_bytes, _stream(stream)))


def lowram_decode_attn_timed(shape, layer, q, cache, subset_off, subset_idx, out, lse_out, workspace,
                             before_event, after_event, stream=None):
    """lowram_decode_attn that records two caller events (raw hipEvent_t
    handles, e.g. torch.cuda.Event.cuda_event after a first record()) around
    its body-row kernel."""
    c = cache if isinstance(cache, lowram_cache) else make_cache(cache)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(library().lowram_decode_attn_timed(
        ctypes.byref(shape), layer, _p(q), ctypes.byref(c), _p(subset_off), _p(subset_idx),
        _p(out), _p(lse_out), _p(workspace), ws_bytes, _stream(stream),
        ctypes.c_void_p(before_event), ctypes.c_void_p(after_event)))


def lowram_decode_attn_noalloc(shape, layer, q, cache, subset_off, subset_idx, out, lse_out, stream=None):
    """lowram_decode_attn with the library's own device scratch (no workspace)."""
    c = cache if isinstance(cache, lowram_cache) else make_cache(cache)
    _check(library().lowram_decode_attn_noalloc(
        ctypes.byref(shape), layer, _p(q), ctypes.byref(c), _p(subset_off), _p(subset_idx),
        _p(out), _p(lse_out), _stream(stream)))


def lowram_check_decode_indices(shape, n_body, tail_len, pos, resid_idx, subset_off, subset_idx):
    """The decode call's index preconditions on host arrays (numpy int32,
    contiguous, or None)."""
    def hp(a):
        return None if a is None else ctypes.c_void_p(a.ctypes.data)
    _check(library().lowram_check_decode_indices(ctypes.byref(shape), hp(n_body), hp(tail_len), hp(pos),
                                                 hp(resid_idx), hp(subset_off), hp(subset_idx)))
