"""GPU parity of lowram_append_body (folding exact rows into the compressed
body) against the oracle's append_body of the same stored cache.

Each case takes the oracle's prefill of the first n0[b] rows of a seeded
workload (ragged over the batch), with room for more residual entries,
uploads it, and appends the next n_new rows of every sequence.  Checked:
  * rows and residual entries stored before the call are unchanged, n_body
    and the positions grow as documented;
  * the new rows' coefficients within one storage unit of the oracle's
    (equal for almost all), their scores within 1e-5 (fp32) / 2e-2 (bf16)
    of the row maximum;
  * the appended residual entries are the top-m_new of the library's
    exported scores of the new rows and a valid top-m_new of the oracle's;
    their residuals against the definition v - f(k^) at those rows;
  * decode over the oracle's folded cache matches the oracle's decode of it.
"""
import pytest
import torch

from decode_attention_05_amd import device as dev
from decode_attention_05_amd import lowram as L
from decode_attention_05_amd import synth

from gpu_helpers import assert_append_matches

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
    # more than 256 new rows: the selection runs as its own launch before the merge
    "bf16-mfma-600-rows": (synth.scaled(C[2], batch=2, context=1100, tail=37, rank=128, latent_rank=64), 35, 600,
                           [0, 40], L.ALGO_AUTO),
    "int4-evict-positions": (synth.scaled(C[4], batch=2, context=4096, tail=50, rank=128, latent_rank=64), 32,
                             64, [10, 0], L.ALGO_AUTO),
    "bf16-plain": (synth.scaled(C[2], batch=2, context=700, tail=20, rank=64, latent_rank=32), 33, 50,
                   [0, 7], L.ALGO_PLAIN),
    "fp32-tiny": (C[1], 34, 30, [0], L.ALGO_AUTO),
}


@pytest.mark.parametrize("name", list(CASES))
def test_append_parity_and_decode(name):
    s, seed, n_new, unused, algo = CASES[name]
    print(f"[append {name}] B={s.batch} N={s.n_rows} n_new={n_new} r={s.rank}", flush=True)
    t = dev.upload(synth.make_workload(s, seed))
    assert_append_matches(s, t, n_new, unused, algo, name)
