"""GPU parity of lowram_select_subset (the structured subset, R26) against
the oracle's subset_policy: the CSR offsets and indices bit-exact for ragged
batches and edge policies, then decode over the policy's subset (the
oracle's own lists, uploaded) against the oracle's decode with that subset."""
import numpy as np
import pytest
import torch

import oracle as O
from decode_attention_05_amd import device as dev
from decode_attention_05_amd import lowram as L
from decode_attention_05_amd import synth
from decode_attention_05_amd.synth import subset_csr

from gpu_helpers import assert_decode_matches, oracle_inputs, oracle_prefill

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.library()


def select(n_body, N, policy):
    B = len(n_body)
    cap = L.lowram_subset_capacity(B, N, policy)
    nb = torch.tensor(n_body, dtype=torch.int32, device="cuda")
    off = torch.full((B + 1,), -1, dtype=torch.int32, device="cuda")
    idx = torch.full((max(cap, 1),), -1, dtype=torch.int32, device="cuda")
    L.lowram_select_subset(B, nb, N, policy, off, idx if cap > 0 else None)
    torch.cuda.synchronize()
    return off.cpu().numpy(), idx.cpu().numpy(), cap


POLICIES = [(4, 64, 3), (0, 0, 1), (64, 1024, 4), (16, 0, 0), (0, 10, 0), (1000, 5, 2), (2, 2, 1000)]


@pytest.mark.parametrize("policy", POLICIES)
def test_subset_csr_bit_exact(policy):
    rng = np.random.default_rng(sum(policy))
    N = 5000
    n_body = [N, 0, 1, 7] + rng.integers(0, N + 1, size=12).tolist()
    if policy == POLICIES[0]:                      # lengths outside [0, N] are clamped
        n_body += [-5, N + 100]
    pol = L.make_subset_policy(*policy)
    off, idx, cap = select(n_body, N, pol)
    ref_off, ref_idx = subset_csr(O.subset_policy(np.clip(n_body, 0, N), *policy))
    assert np.array_equal(off, ref_off)
    assert np.array_equal(idx[:off[-1]], ref_idx)
    assert off[-1] <= cap and np.all(idx[off[-1]:] == -1)          # nothing written past the end


def test_subset_csr_large_batch():
    # 700 sequences: every workgroup sums the closed-form counts before it
    rng = np.random.default_rng(77)
    N = 40000
    n_body = rng.integers(0, N + 1, size=700).tolist()
    policy = (64, 1024, 4)
    off, idx, cap = select(n_body, N, L.make_subset_policy(*policy))
    ref_off, ref_idx = subset_csr(O.subset_policy(n_body, *policy))
    assert np.array_equal(off, ref_off) and np.array_equal(idx[:off[-1]], ref_idx)


def test_decode_over_the_policy_subset():
    s = synth.scaled(synth.CONFIGS[2], batch=3, context=1500, tail=40, rank=128, latent_rank=64)
    n_body = np.array([s.n_rows, s.n_rows - 211, 300], dtype=np.int32)
    w = synth.make_workload(s, 71, n_body=n_body)
    t = dev.upload(w)
    policy = (16, 128, 5)
    off, idx, _ = select(n_body.tolist(), s.n_rows, L.make_subset_policy(*policy))
    ref_off, ref_idx = subset_csr(O.subset_policy(n_body, *policy))
    assert np.array_equal(off, ref_off) and np.array_equal(idx[:off[-1]], ref_idx)
    t["subset_off"] = torch.from_numpy(ref_off).cuda()
    t["subset_idx"] = torch.from_numpy(ref_idx.astype(np.int32)).cuda()
    o = oracle_inputs(t)
    oc = oracle_prefill(s, o)
    assert_decode_matches(s, t, oc, o, L.ALGO_AUTO, what="policy subset")
