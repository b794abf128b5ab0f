"""GPU parity of the naive path (mla_naive_run: per-head K and V
materialised from the latent cache, then causal softmax attention) against
the fp64 oracle, which is that same definition written out; through the C ABI.

Cases: prefill (every prompt token a query, Sq = L) at sizes that span
several 128-token expansion tiles, 256-query attention tiles and 64-key tiles
with ragged tails; chunked prefill (Sq < L); rows that see nothing (L < Sq);
decode-shaped batches, also against the absorbed decode on the GPU; and the
prompt length 4096 on sampled heads. Bar: the decode's parity tolerance
(max|err| <= 1e-2 max|ref|, sum|err| / sum|ref| <= 2e-3).
"""

import numpy as np
import pytest

from mla_latent_kv_amd import synth
from tests.parity import assert_parity, oracle, run_gpu, say

pytestmark = pytest.mark.gpu


def run_naive(batch, dec=None):
    import torch
    from mla_latent_kv_amd import binding, device
    d = device.upload(batch)
    own = dec is None
    dec = dec or binding.MLADecoder(0, max_q_tokens=2)
    w_uk, w_uv = dec.pack(d["w_uk"]), dec.pack(d["w_uv"])
    o = dec.naive(d["q_nope"], d["q_pe"], w_uk, w_uv, d["kv_cache"], d["block_table"], d["seq_lens"],
                  d["max_seq_len"])
    torch.cuda.synchronize()
    got = o.cpu().numpy().astype(np.float64)
    if own:
        dec.close()
    return got


@pytest.mark.parametrize("spec", [
    synth.Spec("prefill_l300", 1, 300, (300,)),
    synth.Spec("prefill_l64", 1, 64, (64,)),
    synth.Spec("prefill_l1", 1, 1, (1,)),
    synth.Spec("prefill_b2_l257", 2, 257, (257, 257)),
], ids=lambda s: s.name)
def test_prefill_every_head(spec):
    batch = synth.make_batch(spec, seed=len(spec.name) + spec.q_tokens)
    say(f"case naive {spec.name}")
    assert_parity(run_naive(batch), oracle(batch), spec.name)


@pytest.mark.parametrize("spec", [
    synth.Spec("chunked_prefill", 2, 100, (200, 129)),
    synth.Spec("rows_see_nothing", 2, 70, (50, 300)),
    synth.Spec("decode_sq2_ragged", 3, 2, (2, 129, 1000)),
    synth.Spec("empty_and_single", 3, 2, (0, 1, 65), max_seq_len=128),
], ids=lambda s: s.name)
def test_partial_prefill_and_short_sequences(spec):
    batch = synth.make_batch(spec, seed=7 + spec.q_tokens)
    say(f"case naive {spec.name}")
    ref = oracle(batch)
    got = run_naive(batch)
    if spec.name == "rows_see_nothing":
        # sequence 0 (L = 50 < Sq = 70): rows 0..19 see no position -> zeros
        assert np.all(got[0, :20] == 0.0)
    if spec.name == "empty_and_single":
        # L = 0: no row sees anything; L = 1: row 0 sees nothing
        assert np.all(got[0] == 0.0) and np.all(got[1, 0] == 0.0)
    assert_parity(got, ref, spec.name)


def test_naive_equals_absorbed_decode():
    """The two orders of the same sums on the GPU (decode shape, Sq = 1)."""
    spec = synth.Spec("naive_vs_absorb", 3, 1, (700, 64, 2500))
    batch = synth.make_batch(spec, seed=11)
    say("case naive vs absorb")
    naive = run_naive(batch)
    absorb = run_gpu(batch)
    assert_parity(naive, oracle(batch), "naive vs oracle")
    assert_parity(naive, absorb, "naive vs absorbed decode")


def test_prefill_4096_sampled_heads():
    """Prompt length 4096 (the prefill workload), every row of two heads."""
    spec = synth.Spec("prefill_l4096", 1, 4096, ("fixed", 4096))
    batch = synth.make_batch(spec, seed=4096)
    say("case naive prefill L=4096")
    got = run_naive(batch)
    heads = (5, 77)
    ref = oracle(batch, sample=[(0, h) for h in heads])
    assert np.isfinite(got).all()
    assert_parity(got[:, :, list(heads)], ref[:, :, list(heads)], "prefill 4096, heads 5 and 77")
