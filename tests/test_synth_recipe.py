"""The seeded input recipe: sizes of the five workloads, and agreement of the
synthetic model's rotation with the oracle's inverse rotation (the recovered
pre-RoPE keys must be low rank)."""
import numpy as np

import oracle as O
from decode_attention_05_amd import synth


def test_config_sizes():
    got = {k: (c.n_rows, c.n_resid) for k, c in synth.CONFIGS.items()}
    assert got == {1: (240, 60), 2: (8064, 1613), 3: (32256, 6452), 4: (39245, 5887), 5: (32640, 6528)}


def test_recipe_keys_are_low_rank_before_rope_and_seeded():
    s = synth.CONFIGS[1]
    w = synth.make_workload(s, seed=1)
    w2 = synth.make_workload(s, seed=1)
    assert np.array_equal(w.k_post, w2.k_post) and np.array_equal(w.q, w2.q)
    kp = w.k_post[0].transpose(0, 2, 1, 3)                       # [G, H, N, d]
    pre = O.rope_rotate(kp, np.arange(s.n_rows), s.theta, inverse=True)
    X = pre.transpose(2, 0, 1, 3).reshape(s.n_rows, s.D)
    sv = np.linalg.svd(X, compute_uv=False)
    # rank-16 signal with N(0,1) entries, then noise of std 0.05
    assert sv[15] > 20 * sv[16]
    # without the inverse rotation the keys are not low rank
    sv_post = np.linalg.svd(w.k_post[0].transpose(1, 0, 2, 3).reshape(s.n_rows, s.D), compute_uv=False)
    assert sv_post[16] > 0.2 * sv_post[15]
    # the basis rows are orthonormal and span the signal
    Bm = w.basis[0].astype(np.float64)
    assert np.allclose(Bm @ Bm.T, np.eye(s.rank), atol=1e-5)
    resid = X - (X @ Bm.T) @ Bm
    assert np.linalg.norm(resid) < 0.06 * np.sqrt(X.size)


def test_eviction_and_subset_recipes():
    s = synth.scaled(synth.CONFIGS[4], batch=2, context=2048, tail=64, rank=64, latent_rank=32)
    w = synth.make_workload(s, seed=3, with_basis=False)
    assert w.pos.shape == (2, s.n_rows)
    for b in range(2):
        assert np.all(np.diff(w.pos[b]) > 0) and np.array_equal(w.pos[b, :64], np.arange(64))
        assert w.pos[b, -1] < s.body
    s3 = synth.scaled(synth.CONFIGS[3], batch=2, context=1024, tail=32, rank=64, latent_rank=32)
    w3 = synth.make_workload(s3, seed=4, with_basis=False)
    off, idx = synth.subset_csr(w3.subset)
    assert off[-1] == 2 * (-(-s3.n_rows // 4))
    for b in range(2):
        rows = idx[off[b]:off[b + 1]]
        assert np.all(np.diff(rows) > 0) and rows[-1] < s3.n_rows
