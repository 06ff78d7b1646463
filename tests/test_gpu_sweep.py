"""Seeded sweep of random shapes through the whole library against the oracle.

Each case draws a shape from the supported space: batch 1-3 with ragged body
and tail lengths, 1-4 layers per group, 1-8 KV heads and 1-8 query heads per
KV head, head_dim 64 or 128, any rank that is a multiple of 32 up to
min(D, 512), native or int4 storage, eviction positions, a subset, from no
residual rows to all of them.  The library picks its kernels as a caller's
call would (MFMA where the shape allows, plain otherwise); decode also runs
with the plain kernels forced.  Checked with the parity rules of the fixed
cases: prefill scores, selection (the exact top-m of the library's scores and
a valid top-m of the oracle's), stored coefficients and residuals; decode of
every layer (and the subset) on the oracle's stored cache; an append of a few
rows and decode of the folded cache; one step of the predictor fit
(gradient and loss); the key basis of the same keys (one power round)
against the oracle's subspace iteration from the same start.
"""
import numpy as np
import pytest
import torch

from decode_attention_05_amd import device as dev
from decode_attention_05_amd import lowram as L
from decode_attention_05_amd import synth

from gpu_helpers import (assert_append_matches, assert_decode_matches, assert_fit_gradient_matches,
                         assert_prefill_matches, oracle_inputs)
from test_gpu_basis import assert_basis_matches

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.library()


def _draw(seed: int):
    rng = np.random.default_rng(1000 + seed)
    d = 128 if rng.random() < 0.7 else 64
    f32 = rng.random() < 0.15
    H = int(rng.choice([1, 2, 4, 8]))
    grp = int(rng.choice([1, 2, 3, 4, 7, 8]))
    G = int(rng.integers(1, 5))
    D = G * H * d
    r = int(rng.choice([x for x in (32, 64, 96, 128, 192, 256, 384, 512) if x <= D]))
    body = int(rng.integers(8, 600))
    tail = int(rng.integers(1, 70))
    resid = [(1, 5), (3, 20), (1, 1), (0, 1)][int(rng.choice(4, p=[0.4, 0.3, 0.15, 0.15]))]
    int4_c = (not f32) and rng.random() < 0.3
    int4_r = (not f32) and rng.random() < 0.3
    keep = (3, 10) if rng.random() < 0.25 else None
    sub = (1, 4) if rng.random() < 0.3 else None
    B = int(rng.integers(1, 4))
    s = synth.Shape(f"sweep{seed}", B, G, H * grp, H, d, r, body + tail, tail, resid,
                    float(rng.choice([10000.0, 500000.0])), "f32" if f32 else "bf16",
                    latent_rank=int(min(32, r)), coef_store="int4" if int4_c else "native",
                    resid_store="int4" if int4_r else "native", subset_frac=sub, keep_frac=keep,
                    sinks=4 if keep else 0)
    N = s.n_rows
    n_body = [N] + [int(rng.integers(0, N + 1)) for _ in range(B - 1)]
    tail_len = [int(rng.integers(0, tail + 1)) for _ in range(B)]
    return s, n_body, tail_len


SEEDS = list(range(32))


@pytest.mark.parametrize("seed", SEEDS)
def test_sweep(seed):
    s, n_body, tail_len = _draw(seed)
    print(f"[sweep {seed}] B={s.batch} G={s.group_layers} Hq/H={s.n_q_heads}/{s.n_kv_heads} d={s.head_dim} "
          f"r={s.rank} N={s.n_rows} m={s.n_resid} Te={s.tail} {s.dtype} coef={s.coef_store} "
          f"resid={s.resid_store} keep={s.keep_frac} subset={s.subset_frac} n_body={n_body}", flush=True)
    w = synth.make_workload(s, seed, n_body=n_body, tail_len=tail_len)
    t = dev.upload(w)
    c = dev.alloc_cache(s)
    dev.prefill(s, t, c)
    torch.cuda.synchronize()
    o = oracle_inputs(t)
    oc, _ = assert_prefill_matches(s, c, o)
    for algo in (L.ALGO_AUTO, L.ALGO_PLAIN):
        assert_decode_matches(s, t, oc, o, algo, what=f"sweep {seed}")
    # one step of the predictor fit on the oracle's stored coefficients
    assert_fit_gradient_matches(s, t, oc, o, shared=1, what=f"sweep {seed}")
    # the key basis of the same keys (ragged and empty sequences are rank deficient)
    start = np.random.default_rng(5000 + seed).standard_normal((s.batch, s.rank, s.D)).astype(np.float32)
    basis = dev.compute_basis(s, t, torch.from_numpy(start).cuda(), 1)
    torch.cuda.synchronize()
    from gpu_helpers import np_in
    assert_basis_matches(s, np_in(basis), o["k_post"], o["pos"], o["n_body"], start.astype(np.float64), 1)
    # an append of a few rows into the full-length sequences
    N = s.n_rows
    n_new = min(24, N // 2)
    if n_new >= 1 and s.n_resid > 0:
        unused = [0] * s.batch
        ta = dict(t)
        ta["n_body"] = torch.full((s.batch,), N, dtype=torch.int32, device="cuda")
        assert_append_matches(s, ta, n_new, unused, L.ALGO_AUTO, f"sweep {seed}")
