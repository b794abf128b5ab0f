"""GPU parity of the output projection y = W_O x against the fp64 oracle,
through the C ABI.

Bar (from the arithmetic): x enters the bf16 matrix cores as hi + lo, within
2^-17 of x, and the products accumulate in fp32 over 16384 terms, so every
output must satisfy |y - y_exact| <= 4e-5 * sum_k |w_nk x_k| (about three
times the two error terms together).
"""

import numpy as np
import pytest

from mla_latent_kv_amd import synth
from tests.parity import assert_parity, oracle, run_gpu, say

pytestmark = pytest.mark.gpu

ALLOW = 4e-5


def _w_o_tensor(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run(x, w_bits):
    import torch
    from mla_latent_kv_amd import binding
    dec = binding.MLADecoder(0, max_q_tokens=2)
    y = dec.output_project(torch.from_numpy(np.ascontiguousarray(x)).cuda(), dec.pack(_w_o_tensor(w_bits)))
    torch.cuda.synchronize()
    dec.close()
    return y.cpu().numpy().astype(np.float64)


def _check(x, w_bits, got, what):
    from oracle import mla_oracle as orc
    w = orc.bf16_bits_to_f64(w_bits)
    ref = orc.output_project(x.astype(np.float64), w)
    mag = np.abs(x.astype(np.float64)) @ np.abs(w).T
    err = np.abs(got - ref)
    ratio = float((err / (ALLOW * mag)).max())
    rel = float(err.sum() / np.abs(ref).sum())
    say(f"oproj {what}: {got.size} values, worst err / allowance {ratio:.3f}, mean rel {rel:.2e}")
    assert np.isfinite(got).all()
    assert ratio <= 1.0, f"{what}: error {ratio:.2f} x the allowance"


@pytest.mark.parametrize("rows", [1, 5, 32, 33, 256])
def test_output_project_against_oracle(rows):
    inp = synth.make_oproj_inputs(rows, seed=60 + rows)
    say(f"case oproj rows={rows}")
    _check(inp["x"], inp["w_o"], _run(inp["x"], inp["w_o"]), f"rows {rows}")


def test_decode_then_output_project():
    """The decode's fp32 output projected on the GPU against the oracle's
    decode projected in fp64 (the decode tolerance applies)."""
    spec = synth.Spec("oproj_after_decode", 3, 2, (300, 1200, 2048))
    batch = synth.make_batch(spec, seed=67)
    w_bits = synth.make_oproj_inputs(1, seed=71)["w_o"]
    o = run_gpu(batch)                                   # [B, Sq, 128, 128] fp32 values
    x = o.reshape(-1, 128 * 128).astype(np.float32)
    got = _run(x, w_bits)
    _check(x, w_bits, got, "on the decode output")
    from oracle import mla_oracle as orc
    ref = orc.output_project(oracle(batch).reshape(-1, 128 * 128), orc.bf16_bits_to_f64(w_bits))
    assert_parity(got, ref, "decode + output projection vs oracle")
