#!/usr/bin/env python3
"""Decode throughput of the LowRAM path on one MI355X.

Default workload: the 32k-context layer group (B = 16, G = 4, Hq/Hkv =
32/8, d = 128, r = 512, exact tail of 512 rows).  A step is one decode step
of every sequence in the batch through the layer group: G calls of
lowram_decode_attn (one per layer), each attending every body row of the
compressed cache of its layer.  Inputs are resident in HBM before the timed
region; the compressed cache is replicated and the copies rotate from call
to call so that no call is served from the 256 MB Infinity Cache.  Every
timed call records events around itself and around its body-row kernel;
medians over all timed calls give the call and kernel durations.

Prints one JSON line: the metric and its value (tokens/s with every row
attended), the roofline of the body-row kernel, the same measurements over
the workload's 25 % row subset ("subset"), the uncompressed comparator, the
prefill, fold, predictor-fit and key-basis measurements, the peak-throughput
comparison at a fixed HBM budget ("peak": the 28-layer, 7:1-GQA model) and
the oracle's CPU baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 << 20


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# the sources the body-row kernel is compiled from: stored HBM-traffic
# figures apply only while these are unchanged
BODY_KERNEL_SOURCES = ("decode_mfma.hip", "mfma_common.h", "dense_body.h", "lowram_internal.h")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "decode_attention_05_amd", "csrc")
    for f in BODY_KERNEL_SOURCES:
        h.update(open(os.path.join(d, f), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "lowram.h"), "rb").read())
    return h.hexdigest()[:16]


def prefill_roof(s, prefill_ms, peak_flops):
    """Roofline of one prefill call (every kernel of it) on its algorithmic work."""
    from decode_attention_05_amd import device as dev
    fl, by = dev.algorithmic_prefill_flops(s), dev.algorithmic_prefill_bytes(s)
    sec = prefill_ms / 1e3
    bound = "mfma" if fl / (peak_flops * 1e12) >= by / (HBM_PEAK_GBS * 1e9) else "hbm"
    roof = max(fl / (peak_flops * 1e12), by / (HBM_PEAK_GBS * 1e9))
    return {"ms": round(prefill_ms, 3), "bound": bound, "algorithmic_flops": fl, "algorithmic_bytes": by,
            "achieved_tflops": round(fl / sec / 1e12, 2), "achieved_gbs": round(by / sec / 1e9, 1),
            "frac": round(roof / sec, 4)}


def fold_measure(s, t, peak_flops, reps=5):
    """Time lowram_append_body folding one exact tail's worth of rows (the
    last `tail` body rows of every sequence) into a body prefilled up to
    them; the cache state is restored between calls, outside the events.
    `us` is the call from an idle GPU (its kernels wait for the host to
    enqueue them); `us_device` is the same call queued behind ~1 ms of other
    GPU work, as a decode loop issues it, so that the host has enqueued every
    kernel before the first starts: the fold's own device time."""
    import torch
    from decode_attention_05_amd import device as dev
    from decode_attention_05_amd import lowram as L
    B, N = s.batch, s.n_rows
    n_new = min(s.tail, N // 2)
    n0 = N - n_new
    a, den = s.resid_frac
    m_new, m0 = -(-n_new * a // den), -(-n0 * a // den)
    t0 = dict(t)
    t0["n_body"] = torch.full((B,), n0, dtype=torch.int32, device="cuda")
    c = dev.alloc_cache(s, m=m0 + m_new)
    c0 = dev.alloc_cache(s, m=m0)
    dev.prefill(s, t0, c0, m=m0)
    c["coef"] = c0["coef"]
    if c0.get("coef_scale") is not None:
        c["coef_scale"] = c0["coef_scale"]
    c["resid_idx"].fill_(2**31 - 1)
    c["resid_idx"][..., :m0] = c0["resid_idx"]
    c["resid_val"].zero_()
    c["resid_val"][:, :, :, :m0] = c0["resid_val"]
    if c.get("resid_scale") is not None:
        c["resid_scale"].zero_()
        c["resid_scale"][:, :, :, :m0] = c0["resid_scale"]
    k_new = t["k_post"][:, :, n0:].contiguous()
    v_new = t["v"][:, :, n0:].contiguous()
    pos_new = None if t.get("pos") is None else t["pos"][:, n0:].contiguous()
    pos = None if t.get("pos") is None else t["pos"].clone()
    idx0 = c["resid_idx"].clone()
    n_body = t0["n_body"].clone()
    sh = dev.abi_shape(s, n_resid=m0 + m_new)
    ws = dev.workspace(L.lowram_append_workspace_size(sh, n_new, m_new))
    times, queued = [], []
    for i in range(2 * (reps + 1)):
        n_body.copy_(t0["n_body"])
        c["resid_idx"].copy_(idx0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        behind = i % 2 == 1
        if behind:
            torch.cuda._sleep(2_000_000)                  # a bounded spin of ~1 ms ahead of the call
        e0.record()
        L.lowram_append_body(sh, n_new, m_new, k_new, v_new, pos_new, t["basis"], t["w1"], t["b1"], t["w2"],
                             t["b2"], n_body, pos, c["coef"], c.get("coef_scale"), c["resid_idx"], c["resid_val"],
                             c.get("resid_scale"), None, ws)
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            (queued if behind else times).append(e0.elapsed_time(e1))
    assert int(n_body[0]) == N
    ms = sum(times) / len(times)
    ms_dev = sum(queued) / len(queued)
    fl = dev.algorithmic_append_flops(s, n_new)
    by = dev.algorithmic_append_bytes(s, n_new, m_new)
    roof = max(fl / (peak_flops * 1e12), by / (HBM_PEAK_GBS * 1e9))
    return {"rows_per_sequence": n_new, "residual_rows_per_list": m_new, "us": round(ms * 1e3, 1),
            "us_device": round(ms_dev * 1e3, 1), "rows_per_s": round(B * n_new / (ms / 1e3), 1),
            "algorithmic_flops": fl, "algorithmic_bytes": by,
            "bound": "mfma" if fl / (peak_flops * 1e12) >= by / (HBM_PEAK_GBS * 1e9) else "hbm",
            "frac": round(roof / (ms / 1e3), 4)}


def fit_measure(s, t, c, steps_lo=2, steps_hi=12):
    """Time lowram_fit_predictor fitting one predictor per sequence, layer and
    KV head on the compressed cache c: two calls with steps_lo and steps_hi
    Adam steps separate the per-step time (one gradient pass over every body
    row plus the Adam update) from the one-time preparation (rebuilt keys and
    transposed copies).  Weights are restored between calls, outside the
    events.  The products run on bf16 matrix cores for every dtype, so the
    bf16 MFMA peak is the roof."""
    import torch
    from decode_attention_05_amd import device as dev
    from decode_attention_05_amd import lowram as L
    peak_flops = BF16_MFMA_PEAK_TFLOPS
    B, G, H, d, N = s.batch, s.group_layers, s.n_kv_heads, s.head_dim, s.n_rows
    sh = dev.abi_shape(s, predictor_shared=0)
    ws = dev.workspace(L.lowram_fit_workspace_size(sh))
    w0 = {k: t[k].expand(B, *t[k].shape[1:]).contiguous() for k in ("w1", "b1", "w2", "b2")}
    tw = dict(t, **{k: v.clone() for k, v in w0.items()})

    def run(steps):
        for k in w0:
            tw[k].copy_(w0[k])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        L.lowram_fit_predictor(sh, c["coef"], c.get("coef_scale"), t["n_body"], t["basis"], t["v"],
                               L.make_fit_params(steps, 1e-3), tw["w1"], tw["b1"], tw["w2"], tw["b2"],
                               None, None, ws)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    run(steps_lo)                                   # warm-up
    lo = min(run(steps_lo) for _ in range(2))
    hi = min(run(steps_hi) for _ in range(2))
    step_ms = (hi - lo) / (steps_hi - steps_lo)
    prep_ms = lo - steps_lo * step_ms
    fl = dev.algorithmic_fit_step_flops(s, B * N)
    by = dev.algorithmic_fit_step_bytes(s, B * N, B)
    sec = step_ms / 1e3
    return {"predictors": B * G * H, "rows_per_predictor": N, "step_ms": round(step_ms, 4),
            "prep_ms": round(prep_ms, 3), "algorithmic_flops_per_step": fl, "algorithmic_bytes_per_step": by,
            "achieved_tflops": round(fl / sec / 1e12, 2),
            "bound": "mfma" if fl / (peak_flops * 1e12) >= by / (HBM_PEAK_GBS * 1e9) else "hbm",
            "frac": round(max(fl / (peak_flops * 1e12), by / (HBM_PEAK_GBS * 1e9)) / sec, 4),
            "arithmetic": "bf16 pairs, three MFMAs per product (not counted in the flops)"}


def basis_measure(s, t, power_iters=2, reps=3):
    """Time lowram_compute_basis on the workload's keys (every sequence, the
    given power rounds) with HIP events on the stream it runs on.  Its
    dominant products run on the fp32 matrix cores (the Gram matrices and
    factors in fp64), so the fp32 MFMA peak is the roof of the whole call."""
    import torch
    from decode_attention_05_amd import device as dev
    from decode_attention_05_amd import lowram as L
    sh = dev.abi_shape(s)
    ws = dev.workspace(L.lowram_basis_workspace_size(sh))
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    start = torch.randn((s.batch, s.rank, s.D), generator=g, device="cuda", dtype=torch.float32)
    out = torch.empty((s.batch, s.rank, s.D), dtype=t["k_post"].dtype, device="cuda")

    def run():
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dev.compute_basis(s, t, start, power_iters, ws=ws, out=out)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    run()                                           # warm-up
    ms = min(run() for _ in range(reps))
    n_rows = int(t["n_body"].sum().item())
    fl = dev.algorithmic_basis_flops(s, n_rows, power_iters)
    sec = ms / 1e3
    return {"ms": round(ms, 3), "power_iters": power_iters, "algorithmic_flops": fl,
            "achieved_tflops": round(fl / sec / 1e12, 2), "peak_tflops": FP32_PEAK_TFLOPS,
            "frac": round(fl / (FP32_PEAK_TFLOPS * 1e12) / sec, 4),
            "arithmetic": "fp32 matrix-core products; Gram matrices, Cholesky and inverse in fp64",
            "residual_energy_vs_optimum": basis_quality(s, t, out, seq=0)}


def basis_quality(s, t, basis, seq=0):
    """Residual energy of the keys outside the span of the library's basis,
    over the optimum (the keys' top-r singular subspace), for one sequence:
    X = its body keys with RoPE undone (fp64), G = X^T X; the optimum leaves
    tr G minus the r largest eigenvalues of G, the basis tr G minus
    tr(Q^T G Q), Q an orthonormal basis of its rows' span."""
    import torch
    n = int(t["n_body"][seq].item())
    G_, H, d = s.group_layers, s.n_kv_heads, s.head_dim
    k = t["k_post"][seq, :, :n].to(torch.float64)                  # [G, n, H, d]
    pos = (t["pos"][seq, :n] if t.get("pos") is not None else torch.arange(n, device=k.device)).to(torch.float64)
    half = d // 2
    inv = torch.pow(torch.tensor(s.theta, dtype=torch.float64, device=k.device),
                    -2.0 * torch.arange(half, dtype=torch.float64, device=k.device) / d)
    ang = pos[:, None] * inv[None, :]                                # [n, half]
    cs, sn = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]
    lo, hi = k[..., :half], k[..., half:]
    x = torch.cat([lo * cs + hi * sn, hi * cs - lo * sn], dim=-1)    # the rotation undone
    X = x.permute(1, 0, 2, 3).reshape(n, G_ * H * d)                # columns (l * H + h) * d + j
    gram = X.T @ X
    total = float(torch.trace(gram))
    top = float(torch.linalg.eigvalsh(gram).flip(0)[:s.rank].sum())
    qb, _ = torch.linalg.qr(basis[seq].to(torch.float64).T)
    captured = float(torch.trace(qb.T @ gram @ qb))
    opt = total - top
    del k, x, X, gram
    return {"sequence": seq, "rows": n, "ratio": round((total - captured) / opt, 4) if opt > 0 else None,
            "basis_residual_frac": (total - captured) / total, "optimum_residual_frac": opt / total,
            "how": "fp64 Gram matrix of the RoPE-undone keys, its eigenvalues, and the span of the basis rows"}


def subset_policy_measure(s, t, c, algo, n_sink=64, n_recent=1024, stride=4, steps=10):
    """lowram_select_subset (sinks, a stride through the middle, a recent
    window) on the workload's body lengths, event-timed, and decode steps of
    the group over that subset (every layer, tokens/s as the main metric)."""
    import torch
    from decode_attention_05_amd import device as dev
    from decode_attention_05_amd import lowram as L
    pol = L.make_subset_policy(n_sink, n_recent, stride)
    B, N = s.batch, s.n_rows
    cap = L.lowram_subset_capacity(B, N, pol)
    off = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    idx = torch.empty(max(cap, 1), dtype=torch.int32, device="cuda")

    def sel():
        L.lowram_select_subset(B, t["n_body"], N, pol, off, idx)
    sel()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        sel()
    e1.record()
    torch.cuda.synchronize()
    sel_us = e0.elapsed_time(e1) * 1e3 / 20
    entries = int(off[-1].item())
    dec = dev.Decoder(s, dict(t, subset_off=off, subset_idx=idx), c, algo=algo, use_subset=True)
    for layer in range(s.group_layers):
        dec(layer)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        for layer in range(s.group_layers):
            dec(layer)
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / steps
    return {"policy": {"n_sink": n_sink, "n_recent": n_recent, "stride": stride}, "select_us": round(sel_us, 2),
            "attended_rows": entries, "attended_frac": round(entries / max(B * N, 1), 4),
            "decode_tokens_per_s": round(B / (step_ms / 1e3), 1), "decode_ms_per_step": round(step_ms, 4)}


def time_decode(decs, layers, group_layers, steps, warmup):
    """Decode steps of `layers` calls each (layer li % group_layers of the
    group), the decoders `decs` taken in turn call by call.  W untimed
    warm-up steps, then exactly K steps between two device
    synchronisations: the wall time per step, and per call the event-timed
    duration of the whole call and of its body-row kernel (the events of
    every timed call are created and first recorded before the timed
    region, on the stream the library runs on)."""
    import torch
    stream = torch.cuda.current_stream()
    n = steps * layers
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(n)]
    for e in evs:
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    calls = 0

    def step(timed):
        nonlocal calls
        for li in range(layers):
            d = decs[calls % len(decs)]
            if timed is not None:
                a, b, ka, kb = evs[timed[0]]
                a.record(stream)
                d.timed(li % group_layers, ka.cuda_event, kb.cuda_event)
                b.record(stream)
                timed[0] += 1
            else:
                d(li % group_layers)
            calls += 1

    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    cursor = [0]
    t_start = time.perf_counter()
    for _ in range(steps):
        step(cursor)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    call_ms = [a.elapsed_time(b) for a, b, _, _ in evs]
    kern_ms = [ka.elapsed_time(kb) for _, _, ka, kb in evs]
    return (t_end - t_start) * 1e3 / steps, call_ms, kern_ms


def stored_profile(workload: str, subset: bool):
    """HBM traffic and achieved clock of the body-row kernel from the
    committed rocprofv3 summary of this workload, when it was taken on the
    current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"decode_counters_{workload}{'_subset' if subset else ''}.json")
    if not os.path.exists(path):
        return None
    tf = json.load(open(path))
    if tf.get("kernel_source_hash") != kernel_source_hash():
        return None
    return tf


def decode_roofline(s, n_att, use_subset, kern_ms_list, call_ms_list, workload):
    """Roofline of the body-row kernel (the call's dominant kernel) from its
    median event-timed duration, and the whole call beside it."""
    import numpy as np
    from decode_attention_05_amd import device as dev
    is_f32 = s.dtype == "f32"
    peak_flops = FP32_PEAK_TFLOPS if is_f32 else BF16_MFMA_PEAK_TFLOPS
    kern = float(np.median(kern_ms_list))
    call = float(np.median(call_ms_list))
    kbytes = dev.algorithmic_body_kernel_bytes(s, n_att, use_subset)
    kflops = dev.algorithmic_body_kernel_flops(s, n_att)
    bound = "mfma" if kflops / (peak_flops * 1e12) >= kbytes / (HBM_PEAK_GBS * 1e9) else "hbm"
    prof = stored_profile(workload, use_subset)
    traffic = None if prof is None else prof.get("body_kernel_bytes_per_launch")
    k_tflops = kflops / (kern / 1e3) / 1e12
    k_gbs = kbytes / (kern / 1e3) / 1e9
    if bound == "mfma":
        roof = {"bound": "mfma", "achieved": round(k_tflops, 2), "peak": peak_flops, "unit": "TFLOP/s",
                "frac": round(k_tflops / peak_flops, 4), "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(k_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(k_gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    roof.update({"kernel": "body-row kernel (key rebuild, RoPE, scores, predictor hidden layer)",
                 "kernel_us_median": round(kern * 1e3, 2), "kernel_us_mean": round(float(np.mean(kern_ms_list)) * 1e3, 2),
                 "timed_launches": len(kern_ms_list), "algorithmic_flops": kflops, "algorithmic_bytes": kbytes,
                 "achieved_gbs_on_algorithmic_bytes": round(k_gbs, 1)})
    if prof is not None:
        roof["clock_mhz"] = prof.get("clock_mhz")
        roof["counters"] = prof.get("summary")
    bytes_call = dev.algorithmic_decode_bytes(s, n_att, use_subset)
    flops_call = dev.algorithmic_decode_flops(s, n_att)
    call_info = {
        "decode_call_us_median": round(call * 1e3, 2),
        "call_roofline_frac": round(max(bytes_call / (HBM_PEAK_GBS * 1e9), flops_call / (peak_flops * 1e12))
                                    / (call / 1e3), 4),
        "hbm": {"algorithmic_bytes_per_call": bytes_call, "achieved_gbs": round(bytes_call / (call / 1e3) / 1e9, 1),
                "pct_of_peak": round(100 * bytes_call / (call / 1e3) / 1e9 / HBM_PEAK_GBS, 2)},
        "mfma": {"algorithmic_flops_per_call": flops_call,
                 "achieved_tflops": round(flops_call / (call / 1e3) / 1e12, 2),
                 "pct_of_peak": round(100 * flops_call / (call / 1e3) / 1e12 / peak_flops, 2)},
    }
    return roof, call_info


def comparator_measure(s, t, reps_per_layer=8):
    """The uncompressed bf16 decode over the same shape (rotated copies of
    exact K/V, each call reading HBM), event-timed."""
    import torch
    from decode_attention_05_amd import device as dev
    from decode_attention_05_amd import lowram as L
    B, T, H, d = s.batch, s.context, s.n_kv_heads, s.head_dim
    kv_bytes = B * T * H * d * 2 * 2
    nk = max(2, math.ceil(4 * MALL_BYTES / kv_bytes))
    g = torch.Generator(device="cuda").manual_seed(7)
    kvs = [(torch.randn((B, T, H, d), device="cuda", dtype=torch.bfloat16, generator=g),
            torch.randn((B, T, H, d), device="cuda", dtype=torch.bfloat16, generator=g)) for _ in range(nk)]
    ctx = torch.full((B,), T, dtype=torch.int32, device="cuda")
    out = torch.empty((B, s.n_q_heads, d), dtype=torch.bfloat16, device="cuda")
    ws = dev.workspace(L.lowram_dense_workspace_size(B, s.n_q_heads, H, d, T))
    qd = t["q"].to(torch.bfloat16)
    for i in range(2 * nk):
        k_, v_ = kvs[i % nk]
        L.lowram_dense_decode_attn(B, s.n_q_heads, H, d, T, qd, k_, v_, ctx, out, None, ws)
    torch.cuda.synchronize()
    reps = reps_per_layer * s.group_layers
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        k_, v_ = kvs[i % nk]
        L.lowram_dense_decode_attn(B, s.n_q_heads, H, d, T, qd, k_, v_, ctx, out, None, ws)
    b.record()
    torch.cuda.synchronize()
    dcall = a.elapsed_time(b) / reps
    dgbs = (kv_bytes + 2 * B * s.n_q_heads * d * 2) / (dcall / 1e3) / 1e9
    log(f"comparator call {dcall * 1e3:.1f} us, {dgbs:.0f} GB/s")
    del kvs
    torch.cuda.empty_cache()
    return {"kind": "uncompressed bf16 decode attention (lowram_dense_decode_attn)",
            "tokens_per_s": round(B / (dcall * s.group_layers / 1e3), 1),
            "call_us": round(dcall * 1e3, 2), "hbm_gbs": round(dgbs, 1),
            "hbm_pct_of_peak": round(100 * dgbs / HBM_PEAK_GBS, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3,
                    help="workload 1-4 (default 3: 32k context, every body row attended, with the 25 %% "
                         "subset reported beside it); 5 = peak throughput at the batch a fixed HBM budget holds")
    ap.add_argument("--algo", default="auto", choices=["auto", "plain", "mfma"])
    ap.add_argument("--subset", action="store_true",
                    help="make the workload's row subset the headline (it is always reported in 'subset')")
    ap.add_argument("--fit-only", action="store_true",
                    help="prefill the workload, then time only the predictor fit and print its JSON object")
    ap.add_argument("--basis-only", action="store_true",
                    help="time only the key-basis computation on the workload and print its JSON object")
    ap.add_argument("--fold-only", action="store_true",
                    help="prefill the workload, then time only the fold of one tail's worth of rows and print "
                         "its JSON object")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode measurements (for profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-comparator", action="store_true")
    ap.add_argument("--no-peak", action="store_true", help="leave out the peak-throughput object")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library runs each GPU's share on that GPU alone "
              "(sequences are independent, so more GPUs would each hold their own sequences and run "
              "this same path). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from decode_attention_05_amd import device as dev
    from decode_attention_05_amd import lowram as L
    from decode_attention_05_amd import synth

    L.library()
    torch.cuda.set_device(0)
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": n,
                          "bytes_written_per_copy": n, "copies": 3}), flush=True)
        return
    if args.config == 5:
        print(json.dumps(peak_bench(args, standalone=True)), flush=True)
        return
    s = synth.CONFIGS[args.config]
    algo = {"auto": L.ALGO_AUTO, "plain": L.ALGO_PLAIN, "mfma": L.ALGO_MFMA}[args.algo]
    log(f"workload {s.name}: B={s.batch} G={s.group_layers} Hq={s.n_q_heads} Hkv={s.n_kv_heads} "
        f"d={s.head_dim} r={s.rank} T={s.context} N={s.n_rows} m={s.n_resid} Te={s.tail}")
    t0 = time.time()
    # large batches repeat two distinct recipe sequences (queries stay distinct)
    distinct = 2 if args.config in (3, 4) else None
    w = synth.make_workload(s, seed=1000 + args.config, distinct=distinct)
    log(f"host generation {time.time() - t0:.1f}s")
    t = dev.upload(w)
    c = dev.alloc_cache(s)
    has_subset = w.subset is not None
    headline_subset = args.subset and has_subset
    n_sub = len(w.subset[0]) if has_subset else 0
    # prefill: one untimed call, then the mean of a few timed calls (the same
    # inputs give the same outputs, so repeating it leaves the cache as is)
    prefill_ws = dev.workspace(L.lowram_workspace_size(dev.abi_shape(s), 0))
    dev.prefill(s, t, c, ws=prefill_ws)
    torch.cuda.synchronize()
    n_pre = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n_pre):
        dev.prefill(s, t, c, ws=prefill_ws)
    e1.record()
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1) / n_pre
    del prefill_ws
    log(f"prefill {prefill_ms:.3f} ms")
    if args.fit_only:
        print(json.dumps({"workload": s.name, "fit": fit_measure(s, t, c)}), flush=True)
        return
    if args.basis_only:
        print(json.dumps({"workload": s.name, "basis": basis_measure(s, t)}), flush=True)
        return
    if args.fold_only:
        peak = BF16_MFMA_PEAK_TFLOPS if s.dtype != "f32" else FP32_PEAK_TFLOPS
        print(json.dumps({"workload": s.name, "fold": fold_measure(s, t, peak)}), flush=True)
        return
    host_sample = dict(w=w)
    del w

    # replicate the compressed cache so consecutive calls never share data in the MALL
    cache_keys = ["coef", "coef_scale", "resid_idx", "resid_val", "resid_scale"]
    input_keys = ["basis", "tail_k", "tail_v", "pos", "subset_idx"]
    per_copy = sum(x.numel() * x.element_size() for k, x in c.items() if k in cache_keys and x is not None)
    per_copy += sum(t[k].numel() * t[k].element_size() for k in input_keys if t.get(k) is not None)
    n_copies = max(2, math.ceil(4 * MALL_BYTES / per_copy))
    copies = [(t, c)]
    for _ in range(n_copies - 1):
        tc = dict(t)
        for k in input_keys:
            if t.get(k) is not None:
                tc[k] = t[k].clone()
        cc = {k: (v.clone() if (k in cache_keys and v is not None) else v) for k, v in c.items()}
        copies.append((tc, cc))
    log(f"{n_copies} cache copies of {per_copy / 2**20:.0f} MiB")

    runs = {}
    for sub in ([False, True] if has_subset else [False]):
        decs = [dev.Decoder(s, tc, cc, algo=algo, use_subset=sub) for tc, cc in copies]
        ms_step, call_ms, kern_ms = time_decode(decs, s.group_layers, s.group_layers, args.steps, args.warmup)
        n_att = n_sub if sub else s.n_rows
        roof, call_info = decode_roofline(s, n_att, sub, kern_ms, call_ms, s.name)
        runs[sub] = dict(ms_step=ms_step, n_att=n_att, roof=roof, call=call_info)
        log(f"{'subset' if sub else 'all rows'}: step {ms_step:.3f} ms; call median {call_info['decode_call_us_median']} us; "
            f"body-row kernel median {roof['kernel_us_median']} us (frac {roof['frac']})")
        del decs
    head = runs[headline_subset]
    value = s.batch / (head["ms_step"] / 1e3)

    # stored bytes vs the uncompressed bf16 K+V of every layer of the group
    stored = per_copy + sum(t[k].numel() * t[k].element_size() for k in ("w1", "b1", "w2", "b2"))
    if t.get("subset_idx") is not None:
        stored -= t["subset_idx"].numel() * t["subset_idx"].element_size()
    dense_bytes = s.batch * s.group_layers * s.context * s.n_kv_heads * s.head_dim * 2 * 2
    result = {
        "metric": "decode tokens/s over LowRAM-compressed KV; HBM GB/s as % of peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(head["ms_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32" if s.dtype == "f32" else "bf16",
        "data": "synthetic (seeded recipe of decode_attention_05_amd/synth.py)",
        "config": {"workload": s.name, "batch": s.batch, "group_layers": s.group_layers,
                   "n_q_heads": s.n_q_heads, "n_kv_heads": s.n_kv_heads, "head_dim": s.head_dim,
                   "rank": s.rank, "context": s.context, "tail": s.tail, "n_body": s.n_rows,
                   "n_resid": s.n_resid, "attended_rows": head["n_att"], "subset": bool(headline_subset),
                   "coef_store": s.coef_store, "resid_store": s.resid_store,
                   "algo": args.algo, "cache_copies": n_copies},
        "roofline": head["roof"],
    }
    result.update(head["call"])
    if has_subset:
        other = runs[not headline_subset]
        result["subset" if not headline_subset else "all_rows"] = {
            "attended_rows": other["n_att"], "tokens_per_s": round(s.batch / (other["ms_step"] / 1e3), 1),
            "ms_per_step": round(other["ms_step"], 4), "roofline": other["roof"], **other["call"]}
    result["compression_ratio"] = round(dense_bytes / stored, 3)
    if not args.no_comparator:
        result["comparator"] = comparator_measure(s, t)
        result["comparator"]["lowram_over_comparator"] = round(value / result["comparator"]["tokens_per_s"], 3)
    if not args.decode_only:
        result["prefill_ms"] = round(prefill_ms, 3)
        result["prefill"] = prefill_roof(s, prefill_ms, BF16_MFMA_PEAK_TFLOPS if s.dtype != "f32" else FP32_PEAK_TFLOPS)
        result["fold"] = fold_measure(s, t, BF16_MFMA_PEAK_TFLOPS if s.dtype != "f32" else FP32_PEAK_TFLOPS)
        result["fit"] = fit_measure(s, t, c)
        result["basis"] = basis_measure(s, t)
        result["subset_policy"] = subset_policy_measure(s, t, c, algo)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(s, copies[0][0], host_sample["w"], args.cpu_seconds, headline_subset)
    del copies, c, t, host_sample
    torch.cuda.empty_cache()
    if not args.no_peak and not args.decode_only:
        result["peak"] = peak_bench(args, standalone=False)
    print(json.dumps(result), flush=True)


def peak_bench(args, standalone: bool):
    """Peak decode throughput at the batch a fixed HBM budget holds.

    The budget is what the 7-group, 28-layer model's compressed caches of
    the workload's batch (607 sequences) occupy; the uncompressed bf16
    comparator gets the batch that the same budget holds for exact K/V of
    all 28 layers.  A step is one decode step of the whole batch through all
    28 layers.  Caches are filled on the device with seeded random content
    (timing does not depend on the values); one group's buffers (and one
    layer's K/V for the comparator) serve every group (layer) of the step:
    each call streams gigabytes, far beyond the 256 MB Infinity Cache, so
    the reuse changes no traffic.  Returns the JSON object (a whole result
    line when standalone).
    """
    import numpy as np
    import torch

    from decode_attention_05_amd import device as dev
    from decode_attention_05_amd import lowram as L
    from decode_attention_05_amd import synth

    s = synth.CONFIGS[5]
    B, G, H, Hq, d, r = s.batch, s.group_layers, s.n_kv_heads, s.n_q_heads, s.head_dim, s.rank
    N, m, Te, T, ng = s.n_rows, s.n_resid, s.tail, s.context, s.n_groups
    layers = G * ng
    per_seq = ng * (N * r * 2 + G * H * m * (d * 2 + 4) + r * G * H * d * 2 + 2 * G * Te * H * d * 2 + 8)
    budget = B * per_seq
    dense_per_seq = layers * T * H * d * 2 * 2
    Bd = budget // dense_per_seq
    log(f"peak: {layers} layers; LowRAM {per_seq / 1e6:.1f} MB per sequence -> B={B} "
        f"({budget / 1e9:.1f} GB); exact K/V {dense_per_seq / 1e9:.2f} GB per sequence -> B={Bd}")
    gen = torch.Generator(device="cuda").manual_seed(5005)
    bf = torch.bfloat16
    t0 = time.time()

    def rnd(shape, scale):
        x = torch.empty(shape, dtype=bf, device="cuda")
        x.normal_(0.0, scale, generator=gen)
        return x

    coef = rnd((B, N, r), 1.0)
    basis = rnd((B, r, G * H * d), 1.0 / math.sqrt(r))
    w1, w2 = rnd((1, G, H, d, d), 1.0 / math.sqrt(d)), rnd((1, G, H, d, d), 1.0 / math.sqrt(d))
    b1, b2 = torch.zeros((1, G, H, d), dtype=bf, device="cuda"), torch.zeros((1, G, H, d), dtype=bf, device="cuda")
    ridx = torch.empty((B * G * H, m), dtype=torch.int32, device="cuda")
    for i0 in range(0, B * G * H, 512):             # m distinct sorted rows per (b, layer, head)
        i1 = min(B * G * H, i0 + 512)
        keys = torch.rand((i1 - i0, N), generator=gen, device="cuda")
        ridx[i0:i1] = keys.topk(m, dim=1).indices.sort(dim=1).values.to(torch.int32)
        del keys
    rval = rnd((B, G, H, m, d), 0.05)
    t = dict(q=rnd((B, Hq, d), 1.0), basis=basis, w1=w1, b1=b1, w2=w2, b2=b2,
             tail_k=rnd((B, G, Te, H, d), 1.0), tail_v=rnd((B, G, Te, H, d), 1.0),
             n_body=torch.full((B,), N, dtype=torch.int32, device="cuda"),
             tail_len=torch.full((B,), Te, dtype=torch.int32, device="cuda"), pos=None)
    c = dict(coef=coef, resid_idx=ridx.view(B, G, H, m), resid_val=rval)
    dcd = dev.Decoder(s, t, c)
    torch.cuda.synchronize()
    log(f"peak: filled {torch.cuda.memory_allocated() / 1e9:.1f} GB in {time.time() - t0:.1f}s")
    steps = max(1, min(args.steps, 3))
    step_ms, call_ms, kern_ms = time_decode([dcd], layers, G, steps, 1)
    step_s = step_ms / 1e3
    value = B / step_s
    out_ok = bool(torch.isfinite(dcd.out.float()).all().item())
    roof, call_info = decode_roofline(s, N, False, kern_ms, call_ms, s.name)
    log(f"peak: LowRAM step {step_ms:.1f} ms ({step_ms / layers * 1e3:.0f} us per layer call), "
        f"body kernel {roof['kernel_us_median']} us, {value:.1f} tokens/s")
    del dcd, c, coef, basis, rval, ridx, t
    torch.cuda.empty_cache()

    # the comparator at the batch the same budget holds
    k = rnd((Bd, T, H, d), 1.0)
    v = rnd((Bd, T, H, d), 1.0)
    qd = rnd((Bd, Hq, d), 1.0)
    ctx = torch.full((Bd,), T, dtype=torch.int32, device="cuda")
    outd = torch.empty((Bd, Hq, d), dtype=bf, device="cuda")
    wsd = dev.workspace(L.lowram_dense_workspace_size(Bd, Hq, H, d, T))
    for _ in range(2):
        L.lowram_dense_decode_attn(Bd, Hq, H, d, T, qd, k, v, ctx, outd, None, wsd)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(steps * layers):
        L.lowram_dense_decode_attn(Bd, Hq, H, d, T, qd, k, v, ctx, outd, None, wsd)
    torch.cuda.synchronize()
    dstep_s = (time.perf_counter() - t_start) / steps
    dvalue = Bd / dstep_s
    dgbs = Bd * T * H * d * 4 / (dstep_s / layers) / 1e9
    log(f"peak: comparator step {dstep_s * 1e3:.1f} ms, {dvalue:.1f} tokens/s, {dgbs:.0f} GB/s")
    del k, v, qd, outd, wsd
    torch.cuda.empty_cache()
    peak = {"workload": s.name, "batch": B, "layers": layers, "tokens_per_s": round(value, 1),
            "ms_per_step": round(step_ms, 3), "steps": steps, "roofline": roof, **call_info,
            "hbm_budget_bytes": budget, "lowram_bytes_per_sequence": per_seq,
            "exact_kv_bytes_per_sequence": dense_per_seq, "comparator_batch": int(Bd),
            "comparator_tokens_per_s": round(dvalue, 1), "comparator_hbm_gbs": round(dgbs, 1),
            "lowram_over_comparator": round(value / dvalue, 3), "outputs_finite": out_ok,
            "data": "seeded random device fill (timing does not depend on values)"}
    if not standalone:
        return peak
    return {
        "metric": "decode tokens/s over LowRAM-compressed KV; HBM GB/s as % of peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": 1,
        "ms_per_step": round(step_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": peak["data"],
        "config": {"workload": s.name, "batch": B, "layers": layers, "group_layers": G,
                   "n_q_heads": Hq, "n_kv_heads": H, "head_dim": d, "rank": r, "context": T,
                   "tail": Te, "n_body": N, "n_resid": m},
        "roofline": roof, "peak": peak}


def cpu_baseline(s, t, w, budget_s, use_subset):
    """The oracle as it stands on whole sequences of the same workload: per
    sequence its own prefill (not timed), then its decode through all G
    layers (timed), until about budget_s seconds of decode work; tokens/s is
    scaled like the GPU figure (sequences decoded through all G layers per
    second of decode)."""
    import numpy as np

    import oracle as O
    from decode_attention_05_amd import device as dev
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    ck = "int4" if s.coef_store == "int4" else ("f32" if s.dtype == "f32" else "bf16")
    rk = "int4" if s.resid_store == "int4" else ("f32" if s.dtype == "f32" else "bf16")

    def f64(x):
        a = dev.to_numpy_store(x)
        return O.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)

    w1, b1, w2, b2 = f64(t["w1"]), f64(t["b1"]), f64(t["w2"]), f64(t["b2"])
    nb = t["n_body"].cpu().numpy()
    tl = t["tail_len"].cpu().numpy()
    pos = t["pos"].cpu().numpy() if t.get("pos") is not None else None
    done, el = 0, 0.0
    while done < s.batch and el < budget_s:
        b = done
        sl = slice(b, b + 1)
        q, basis = f64(t["q"][sl]), f64(t["basis"][sl])
        ps = None if pos is None else pos[sl]
        oc = O.prefill(f64(t["k_post"][sl]), f64(t["v"][sl]), ps, nb[sl], basis, w1, b1, w2, b2, s.n_resid,
                       s.theta, ck, rk)
        tk, tv = f64(t["tail_k"][sl]), f64(t["tail_v"][sl])
        sub = [w.subset[b]] if use_subset else None
        t0 = time.perf_counter()
        for layer in range(s.group_layers):
            O.decode(layer, q, oc.coef, ck, ps, nb[sl], basis, w1, b1, w2, b2, oc.resid_idx, oc.resid_val, rk,
                     tk, tv, tl[sl], s.theta, subset=sub)
        el += time.perf_counter() - t0
        done += 1
    return {"value": round(done / el, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {s.batch} sequences decoded through all {s.group_layers} layers on the "
                      f"oracle's own prefill of each ({el:.1f} s of decode, numpy fp64)"}


if __name__ == "__main__":
    main()
