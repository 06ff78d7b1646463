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
