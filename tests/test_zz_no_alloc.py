"""The allocation-free decode entry point (mla_decode_run_noalloc) against
the workspace entry point (mla_decode_run), through the C ABI.

Two calls in a row, the second with a smaller input (fewer sequences, shorter
histories, the other q_tokens), each compared with mla_decode_run on the same
inputs and with the oracle under the parity tolerance; the benchmark's uniform
shape, where both entry points choose the same one-round plan, must agree
bit for bit; a batch above the split target is refused before any launch.
"""

import numpy as np
import pytest

from mla_latent_kv_amd import synth
from tests.parity import assert_parity, metrics, oracle, say

pytestmark = pytest.mark.gpu


def _both(batch, split_target=0):
    import torch
    from mla_latent_kv_amd import binding, device
    d = device.upload(batch)
    dec = binding.MLADecoder(0, max_q_tokens=2, split_target=split_target)
    args = (d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"], d["block_table"], d["seq_lens"],
            d["max_seq_len"])
    B, Sq = batch["q_nope"].shape[:2]
    out_na = torch.full((B, Sq, 128, 128), float("nan"), dtype=torch.float32, device="cuda")
    binding.mla_decode_run_noalloc(dec.ctx, *args, out=out_na)
    torch.cuda.synchronize()
    got = out_na.cpu().numpy().astype(np.float64)
    ref = dec(*args).cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    dec.close()
    return got, ref


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    first = synth.make_batch(synth.Spec("na_first", 6, 1, (100, 1000, 3000, 333, 64, 2049)), seed=61)
    second = synth.make_batch(synth.Spec("na_second", 3, 2, (97, 700, 1025)), seed=62)
    for name, batch in (("first", first), ("second, smaller", second)):
        say(f"case noalloc {name}: lens={batch['seq_lens'].tolist()}")
        got, ref = _both(batch)
        assert np.isfinite(got).all()
        mt = metrics(got, ref)
        say(f"noalloc vs mla_decode_run ({name}): {mt}")
        assert mt["max_rel"] <= 1e-2 and mt["mean_rel"] <= 2e-3, mt
        assert_parity(got, oracle(batch), f"noalloc {name}")


def test_noalloc_uniform_workload_is_bitwise_the_workspace_result():
    batch = synth.make_batch(synth.CONFIGS[1], seed=1)
    say("case noalloc uniform B=32 x 4096")
    got, ref = _both(batch)
    assert np.array_equal(got, ref)


def test_noalloc_refuses_a_batch_above_the_split_target():
    import torch
    from mla_latent_kv_amd import binding, device
    batch = synth.make_batch(synth.Spec("na_big", 8, 1, (64,) * 8), seed=63)
    d = device.upload(batch)
    dec = binding.MLADecoder(0, max_q_tokens=2, split_target=7)
    out = torch.zeros((8, 1, 128, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        binding.mla_decode_run_noalloc(dec.ctx, d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"],
                                       d["block_table"], d["seq_lens"], d["max_seq_len"], out=out)
    torch.cuda.synchronize()
    assert bool((out == 0).all())
    dec.close()
