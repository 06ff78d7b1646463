"""The allocation-free decode entry (lowram_decode_attn_noalloc) against
lowram_decode_attn with a workspace: bit-identical outputs on two calls in a
row, the second on a smaller input, through the C ABI."""
import numpy as np
import pytest
import torch

from decode_attention_05_amd import device as dev
from decode_attention_05_amd import lowram as L
from decode_attention_05_amd import synth

pytestmark = pytest.mark.gpu

C = synth.CONFIGS
CALLS = [
    # larger first, then a smaller input (batch, rows, rank and heads all smaller)
    ("cfg2-scaled", synth.scaled(C[2], batch=4, context=3000, tail=100, rank=512, latent_rank=64), 31, 2, False),
    ("cfg3-small-subset", synth.scaled(C[3], batch=2, context=900, tail=40, rank=128, latent_rank=64), 32, 1, True),
]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.library()


def test_noalloc_matches_the_workspace_entry_on_two_calls():
    for name, s, seed, layer, sub in CALLS:
        print(f"[noalloc {name}] B={s.batch} N={s.n_rows} r={s.rank} subset={sub}", flush=True)
        w = synth.make_workload(s, seed)
        t = dev.upload(w)
        c = dev.alloc_cache(s)
        dev.prefill(s, t, c)
        dcd = dev.Decoder(s, t, c, use_subset=sub)
        assert L.lowram_workspace_size(dcd.sh, 1) <= 64 << 20
        ref_out, ref_lse = [x.clone() for x in dcd(layer)]
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        L.lowram_decode_attn_noalloc(dcd.sh, layer, t["q"], dcd.cache, dcd.sub[0], dcd.sub[1], out, lse)
        torch.cuda.synchronize()
        assert torch.isfinite(ref_out.float()).all()
        assert torch.equal(out, ref_out), f"{name}: max diff {(out.float() - ref_out.float()).abs().max().item()}"
        assert torch.equal(lse, ref_lse), name


def test_noalloc_rejects_calls_beyond_its_scratch():
    """A shape whose decode workspace exceeds the 64 MiB scratch returns
    LOWRAM_E_WORKSPACE before any launch (the arrays are never read)."""
    s = synth.CONFIGS[5]
    sh = dev.abi_shape(s)
    assert L.lowram_workspace_size(sh, 1) > 64 << 20
    dummy = torch.zeros(16, dtype=torch.int32, device="cuda")
    cache = {k: dummy for k, _ in L.lowram_cache._fields_ if k not in ("coef_scale", "resid_scale", "pos")}
    with pytest.raises(L.LowramError) as ei:
        L.lowram_decode_attn_noalloc(sh, 0, dummy, cache, None, None, dummy, None)
    assert ei.value.status == L.E_WORKSPACE and "allocation-free" in str(ei.value)
