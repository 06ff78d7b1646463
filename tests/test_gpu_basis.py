"""GPU parity of lowram_compute_basis (the key basis by randomized subspace
iteration) against the oracle.

Each case draws a seeded workload and a seeded Gaussian start, runs the
library, and checks, per sequence:
  * element by element against the oracle's key_basis_iteration (the same
    steps in fp64 from the same start and the uploaded keys): within
    5e-5 + 4 * 64 * 2^-24 * sens_j for row j, sens_j the largest change of
    the oracle's row j per unit relative perturbation of the keys (measured
    by rerunning the oracle on keys perturbed by 1e-6); 64 * 2^-24 is the
    relative error of an fp32 sum of 4096 products, the factor 4 the fp32
    products of two power rounds (P = X Q^T and Y^T = P~^T X each; the
    Gram matrices and their factorisation are fp64), and the floor 5e-5
    (0.3 % of a typical entry D^-1/2) covers the one-sample estimate of
    sens_j.  Rows at a
    near-degenerate step of the Gram-Schmidt order (where the latent signal
    ends and noise begins) move by up to ~1e-4 under fp32 rounding, the
    others by ~1e-6.  For bf16 output: one bf16 unit (at most 2^-7
    relative, where the two sides round across a boundary) plus that;
  * rows past the numerical rank are exactly zero where the oracle's are;
  * the other rows are orthonormal (fp32: 1e-5; bf16: 2e-2);
  * the captured energy ||X B^T||^2 equals the oracle iteration's to 1e-5
    of ||X||^2 (fp32 output), and no basis captures more than the SVD's
    top-r (the oracle's definition, Eckart-Young; 1e-5 relative slack for
    fp32 output, 1e-2 for bf16, whose rounding perturbs orthonormality);
  * with two or more power rounds, the residual energy of the span of the
    library's rows (||X||^2 minus the energy captured by their orthonormal
    completion, so bf16 rounding of the rows' lengths does not count) is at
    most 1.10 times the SVD's, the bound the CPU pin puts on the oracle's
    iteration: a basis that captured much less than xKV's top-r subspace
    would fail it even where the iteration itself agreed.  With fewer rounds
    the iteration is the plain randomized range finder (measured 1.03-1.15
    times the optimum on the recipe); those cases check parity only.
Tolerances: the iteration's fp32 rounding, measured against the fp64 steps
on the workload recipe, stays near 1e-6 absolute (entries ~ D^-1/2).
"""
import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_05_amd import device as dev
from decode_attention_05_amd import lowram as L
from decode_attention_05_amd import synth

from gpu_helpers import np_in

pytestmark = pytest.mark.gpu

# relative perturbation used to measure each row's sensitivity, and the
# relative error of an fp32 sum of up to 4096 products (~sqrt(K) u, K = D)
DELTA = 1e-6
FP32_SUM_REL = 64 * 2.0 ** -24

C = synth.CONFIGS


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.library()


CASES = {
    # name: (shape, seed, power_iters, n_body or None)
    "f32-tiny": (C[1], 61, 2, None),
    "bf16-ragged-evicted-positions": (synth.scaled(C[4], batch=2, context=1500, tail=20, rank=64, latent_rank=48,
                                                   group_layers=2, n_kv_heads=2, n_q_heads=8), 62, 1,
                                      lambda N: [N, N - 157]),
    "f32-rank-deficient": (synth.scaled(C[1], batch=3, context=300, tail=16, rank=64, latent_rank=24), 63, 2,
                           lambda N: [N, 40, 0]),
    "bf16-d128-r256-one-sequence": (synth.scaled(C[2], batch=1, context=1200, tail=16, rank=256, latent_rank=160),
                                    64, 2, None),
    "f32-r96-no-power-round": (synth.scaled(C[1], batch=2, context=700, tail=20, rank=96, latent_rank=40,
                                            group_layers=3), 65, 0, lambda N: [N - 13, N]),
    # the largest supported shape: D = 8 * 8 * 128 = 8192 columns, rank 512
    "bf16-max-D-8192-r512": (synth.scaled(C[2], batch=1, context=700, tail=16, rank=512, latent_rank=300,
                                          group_layers=8), 66, 3, None),
}


def run_case(s, seed, q, nb):
    n_body = None if nb is None else np.array(nb(s.n_rows), dtype=np.int32)
    w = synth.make_workload(s, seed, with_basis=False, n_body=n_body)
    t = dev.upload(w)
    start = np.random.default_rng(seed + 1000).standard_normal((s.batch, s.rank, s.D)).astype(np.float32)
    start_t = torch.from_numpy(start).cuda()
    out = dev.compute_basis(s, t, start_t, q)
    torch.cuda.synchronize()
    k_post = np_in(t["k_post"])
    pos = None if t.get("pos") is None else t["pos"].cpu().numpy()
    nbody = t["n_body"].cpu().numpy()
    return np_in(out), k_post, pos, nbody, start.astype(np.float64)


def assert_basis_matches(s, got, k_post, pos, nbody, start, q, check_optimum=True):
    """got [B', r, D] against the oracle on the matching inputs (B' sequences);
    check_optimum also compares with the SVD (slow at full size; without it
    the optimum for the residual-energy bound comes from the eigenvalues of
    X^T X)."""
    sub = list(range(got.shape[0]))
    ref = O.key_basis_iteration(k_post, pos, nbody, s.theta, start, q)
    # each row's sensitivity to the rounding of the arithmetic: the oracle
    # rerun on keys perturbed by DELTA relative (rows at a near-degenerate
    # step of the Gram-Schmidt order move the most)
    pert = 1.0 + DELTA * np.random.default_rng(99).standard_normal(k_post.shape)
    ref2 = O.key_basis_iteration(k_post * pert, pos, nbody, s.theta, start, q)
    sens = np.max(np.abs(ref2 - ref), axis=-1, keepdims=True) / DELTA          # [B', r, 1]
    row_tol = 5e-5 + 4.0 * FP32_SUM_REL * sens
    X = O.pre_rope_keys(k_post, pos, nbody, s.theta)
    sv = O.key_basis(k_post, pos, nbody, s.theta, s.rank)[1] if check_optimum else None
    for i, b in enumerate(sub):
        g, rf = got[b], ref[i]
        if s.dtype == "f32":
            err = np.abs(g - rf)
            assert np.all(err <= row_tol[i]), (b, err.max(), float(row_tol[i].min()))
        else:
            rb = O.bf16_bits_to_f64(O.f64_to_bf16_bits(rf))
            err = np.abs(g - rb)
            assert np.all(err <= 2.0 ** -7 * np.abs(rb) + row_tol[i]), (b, err.max())
        zero = np.all(rf == 0, axis=1)
        assert np.all(g[zero] == 0), b
        keep = ~zero
        gram = g[keep] @ g[keep].T
        tol = 1e-5 if s.dtype == "f32" else 2e-2
        if keep.any():
            assert np.max(np.abs(gram - np.eye(int(keep.sum())))) <= tol, b
        total = np.sum(X[i] ** 2)
        e_got = np.sum((X[i] @ g.T) ** 2)
        e_ref = np.sum((X[i] @ rf.T) ** 2)
        if s.dtype == "f32":
            assert abs(e_got - e_ref) <= 1e-5 * total + 1e-30, (b, e_got, e_ref, total)
        if check_optimum:        # rounding the rows to bf16 perturbs their orthonormality by ~2^-8
            assert e_got <= np.sum(sv[i] ** 2) * (1 + (1e-5 if s.dtype == "f32" else 1e-2)) + 1e-30, b
        if q >= 2 and keep.any() and total > 0:
            top = (np.sum(sv[i] ** 2) if check_optimum else
                   np.sum(np.sort(np.linalg.eigvalsh(X[i].T @ X[i]))[::-1][:s.rank]))
            qb, _ = np.linalg.qr(g[keep].T)                          # orthonormal basis of the rows' span
            resid = total - np.sum((X[i] @ qb) ** 2)
            resid_opt = total - top
            print(f"  b={b}: residual energy {resid / total:.3e} of the total, "
                  f"{resid / max(resid_opt, 1e-300):.4f} x the SVD's", flush=True)
            # slack: the rows' own rounding moves their span by ~2^-20 (fp32) or
            # 2^-9 (bf16) per row, adding up to that squared times the total
            slack = (1e-9 if s.dtype == "f32" else 2.0 ** -16) * total
            assert resid <= 1.10 * resid_opt + slack, (b, resid, resid_opt)


@pytest.mark.parametrize("name", list(CASES))
def test_basis_parity(name):
    s, seed, q, nb = CASES[name]
    print(f"[basis {name}] B={s.batch} N={s.n_rows} D={s.D} r={s.rank} q={q}", flush=True)
    got, k_post, pos, nbody, start = run_case(s, seed, q, nb)
    assert_basis_matches(s, got, k_post, pos, nbody, start, q)



def test_basis_without_body_rows_is_zero():
    # n_body_max = 0: no key rows at all, so every row of the basis is zero
    s = synth.scaled(C[1], batch=2, rank=32)
    sh = dev.abi_shape(s, n_body_max=0, n_resid=0)
    ws = dev.workspace(L.lowram_basis_workspace_size(sh))
    start = torch.randn((2, s.rank, s.D), device="cuda")
    out = torch.full((2, s.rank, s.D), 7.0, device="cuda")
    nb = torch.zeros(2, dtype=torch.int32, device="cuda")
    L.lowram_compute_basis(sh, None, None, nb, start, 2, out, ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
