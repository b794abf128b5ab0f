"""The fp16 range rules on the GPU, through the C ABI.

* q_abs past fp16's 65504 (but inside 2^20 - 2^9 after the 2^-4 scaling):
  queries scaled by 2^16 with the softmax scale divided by 2^16 (the same
  attention) stay finite, match the oracle, and raise no range flag.
* q_abs past 2^20 - 2^9: the range flag is set and the binding's check raises.
* c_KV past 65504: the output equals the oracle's with those values clamped
  to +-65504 (the saturation rule the C header states).
"""

import numpy as np
import pytest

from mla_latent_kv_amd import synth
from tests.parity import assert_parity, say

pytestmark = pytest.mark.gpu


def _run(batch, scale=0.0, check_range=False):
    import torch
    from mla_latent_kv_amd import binding, device
    d = device.upload(batch)
    dec = binding.MLADecoder(0, max_q_tokens=2, softmax_scale=scale)
    ws = torch.empty(dec.workspace_size(batch["seq_lens"].shape[0], batch["q_nope"].shape[1],
                                        d["max_seq_len"]), dtype=torch.uint8, device="cuda")
    o = dec(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"], d["block_table"],
            d["seq_lens"], d["max_seq_len"], workspace=ws, check_range=check_range)
    torch.cuda.synchronize()
    flags = binding.mla_decode_range_flags(dec.ctx, ws)
    out = o.cpu().numpy().astype(np.float64)
    dec.close()
    return out, flags


def _oracle(batch, scale):
    from oracle import mla_oracle as orc
    return orc.decode_batch(batch["q_nope"], batch["q_pe"], batch["w_uk"], batch["w_uv"], batch["cache"],
                            batch["block_table"], batch["seq_lens"], 64, scale=scale, path="absorb")


def test_large_q_abs_inside_the_scaled_range():
    from oracle import mla_oracle as orc
    big = 2.0 ** 16
    spec = synth.Spec("q_big", 2, 2, (700, 1500), q_scale=big)
    batch = synth.make_batch(spec, seed=51)
    q_abs = orc.absorb_query(orc.bf16_bits_to_f64(batch["q_nope"]).reshape(-1, 128, 128),
                             orc.bf16_bits_to_f64(batch["w_uk"]))
    qmax = float(np.abs(q_abs).max())
    say(f"case q_big: max |q_abs| = {qmax:.4g}")
    assert 65504.0 < qmax < 1048064.0
    scale = orc.default_scale() / big
    got, flags = _run(batch, scale, check_range=True)
    assert flags == 0
    assert_parity(got, _oracle(batch, scale), "q_abs past 65504")


def test_q_abs_past_the_scaled_range_is_flagged():
    from mla_latent_kv_amd import binding
    spec = synth.Spec("q_huge", 1, 1, (300,), q_scale=2.0 ** 24)
    batch = synth.make_batch(spec, seed=52)
    say("case q_huge: the range flag must be set")
    with pytest.raises(FloatingPointError):
        _run(batch, 1e-9, check_range=True)
    _, flags = _run(batch, 1e-9)
    assert flags == binding.MLA_RANGE_QABS


def test_range_flags_rewritten_by_either_absorb_tile():
    """Batches below 128 query rows run the narrow absorb tile, from 128 rows on
    the wide one (half as many workgroups, each writing two flags): every call
    rewrites every flag, so a flagged call followed by a clean one on the same
    workspace reads clean, in either order."""
    import torch
    from mla_latent_kv_amd import binding, device
    cases = {
        "narrow_huge": synth.Spec("narrow_huge", 1, 1, (300,), q_scale=2.0 ** 24),
        "wide_clean": synth.Spec("wide_clean", 128, 1, ("uniform", 1, 150)),
        "wide_huge": synth.Spec("wide_huge", 128, 1, ("uniform", 1, 150), q_scale=2.0 ** 24),
        "narrow_clean": synth.Spec("narrow_clean", 2, 1, (300, 64)),
    }
    dec = binding.MLADecoder(0, max_q_tokens=2, softmax_scale=1e-9)
    batches = {k: synth.make_batch(v, seed=54 + i) for i, (k, v) in enumerate(cases.items())}
    ws_bytes = max(dec.workspace_size(b["seq_lens"].shape[0], b["q_nope"].shape[1],
                                      int(b["seq_lens"].max())) for b in batches.values())
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    expect = {"narrow_huge": binding.MLA_RANGE_QABS, "wide_clean": 0,
              "wide_huge": binding.MLA_RANGE_QABS, "narrow_clean": 0}
    for name in ("narrow_huge", "wide_clean", "wide_huge", "narrow_clean"):
        say(f"case {name}")
        d = device.upload(batches[name])
        dec(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"], d["block_table"],
            d["seq_lens"], d["max_seq_len"], workspace=ws)
        torch.cuda.synchronize()
        assert binding.mla_decode_range_flags(dec.ctx, ws) == expect[name], name
    dec.close()


def test_c_kv_past_fp16_range_saturates():
    spec = synth.Spec("c_big", 2, 1, (200, 333))
    batch = synth.make_batch(spec, seed=53)
    rng = np.random.default_rng(7)
    cache = batch["cache"]
    # 40 latent values of used rows set to +-2^17 (exact in bf16)
    for _ in range(40):
        b = int(rng.integers(0, 2))
        j = int(rng.integers(0, int(batch["seq_lens"][b])))
        blk, slot, col = batch["block_table"][b, j // 64], j % 64, int(rng.integers(0, 512))
        cache[blk, slot, col] = (0x8000 if rng.integers(0, 2) else 0) | 0x4800
    say("case c_big")
    got, flags = _run(batch)
    assert flags == 0
    assert_parity(got, _oracle_clamped(batch), "c_KV saturation")


def _oracle_clamped(batch):
    """The oracle over the cache with every value past 65504 replaced by
    +-65504 (in fp64, where the clamp is exact)."""
    import unittest.mock as um
    from oracle import mla_oracle as orc
    real = orc.bf16_bits_to_f64
    with um.patch.object(orc, "bf16_bits_to_f64", side_effect=lambda b: np.clip(real(b), -65504.0, 65504.0)):
        return orc.decode_batch(batch["q_nope"], batch["q_pe"], batch["w_uk"], batch["w_uv"], batch["cache"],
                                batch["block_table"], batch["seq_lens"], 64, path="absorb")
