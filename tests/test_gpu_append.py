"""GPU parity of the cache-append producer against the fp64 oracle, through
the C ABI.

Bar: the producer accumulates W h in fp32 and rounds each finished value to
bf16 once. Every written value must lie within one bf16 step of the oracle's
exact value plus the fp32 accumulation allowance 64 * 2^-24 * sum_k |h_k
w_nk| (for a RoPE pair, the allowance of both inputs), and at least 99 % must
equal the exact value rounded to nearest (only values whose exact result lies
within the accumulation error of a rounding midpoint may land on the other
neighbour). Every other cache byte must be left as it was.
"""

import numpy as np
import pytest

from mla_latent_kv_amd import synth
from tests.parity import assert_parity, oracle, run_gpu, say

pytestmark = pytest.mark.gpu

def _bf16_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _exact_to_bf16_bits(x):
    """Round fp64 values to bf16 (nearest, ties to even) through an exact split."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    # fp64 -> fp32 may round; correct the fp32 rounding direction for the bf16 step
    u = f.view(np.uint32).astype(np.uint64)
    lo = (u >> 16) << 16
    down = lo.astype(np.uint32).view(np.float32).astype(np.float64)
    up = (lo + (1 << 16)).astype(np.uint32).view(np.float32).astype(np.float64)
    mag = np.abs(x)
    d_down, d_up = mag - np.abs(down), np.abs(up) - mag
    pick_up = (d_up < d_down) | ((d_up == d_down) & (((lo >> 16) & 1) == 1))
    return np.where(pick_up, (lo >> 16) + 1, lo >> 16).astype(np.uint16)


def _run_append(batch, inp, rope_base=0.0):
    import torch
    from mla_latent_kv_amd import binding, device
    d = device.upload(batch)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    dec = binding.MLADecoder(0, max_q_tokens=2)
    w_kv = dec.pack(bf16(np.concatenate([inp["w_dkv"], inp["w_kr"]])))   # stacked [W_DKV; W_KR]
    dec.append(bf16(inp["hidden"]), w_kv, d["kv_cache"], d["block_table"], d["seq_lens"],
               rope_base=rope_base)
    torch.cuda.synchronize()
    cache = d["kv_cache"].view(torch.int16).cpu().numpy().view(np.uint16)
    dec.close()
    return cache


def _slots(batch, q_tokens):
    """(b, i, block, slot) of every new token."""
    out = []
    for b, L in enumerate(batch["seq_lens"]):
        for i in range(q_tokens):
            pos = int(L) - q_tokens + i
            out.append((b, i, int(batch["block_table"][b, pos // 64]), pos % 64))
    return out


def _check_append(batch, inp, q_tokens, got_cache, rope_base=10000.0, what="", skip=()):
    """Rows of sequences in `skip` must not have been written at all."""
    from oracle import mla_oracle as orc
    exact = orc.append_batch(inp["hidden"], inp["w_dkv"], inp["w_kr"], batch["seq_lens"],
                             q_tokens, base=rope_base)
    # accumulation allowance per value: 64 u sum_k |h_k w_nk|, u = 2^-24
    h_abs = np.abs(orc.bf16_bits_to_f64(inp["hidden"]))
    mag = np.concatenate([h_abs @ np.abs(orc.bf16_bits_to_f64(inp["w_dkv"])).T,
                          h_abs @ np.abs(orc.bf16_bits_to_f64(inp["w_kr"])).T], axis=-1)
    d = orc.D_LATENT
    pair = mag[..., d::2] + mag[..., d + 1::2]          # a rotation mixes both inputs
    mag[..., d::2], mag[..., d + 1::2] = pair, pair
    allow = 64 * 2.0 ** -24 * mag
    before = batch["cache"]
    mask = np.ones(before.shape[:2], dtype=bool)
    n_exact = n_total = 0
    worst = 0.0
    for b, i, blk, slot in _slots(batch, q_tokens):
        if b in skip:
            continue
        g = got_cache[blk, slot]
        e = exact[b, i]
        gv = _bf16_f64(g)
        rne = _exact_to_bf16_bits(e)
        # one bf16 step: the spacing of bf16 values in e's binade [2^k, 2^(k+1))
        k = np.floor(np.log2(np.maximum(np.abs(e), 2.0 ** -126))).astype(int)
        step = np.ldexp(1.0, k - 7)
        err = np.abs(gv - e)
        bound = step + allow[b, i]
        j = int(np.argmax(err / bound))
        assert np.all(err <= bound), (what, b, i, j, float(e[j]), float(gv[j]), float(bound[j]))
        worst = max(worst, float((err / np.maximum(np.abs(e), 1e-30)).max()))
        n_exact += int((g == rne).sum())
        n_total += g.size
        mask[blk, slot] = False
    frac = n_exact / n_total
    say(f"append {what}: {n_total} values, {frac:.5f} equal to the exact value rounded, "
        f"max rel err {worst:.2e}")
    assert frac >= 0.99, f"{what}: only {frac:.4f} rounded like the exact value"
    # every other row untouched, bit for bit (NaN padding included)
    np.testing.assert_array_equal(got_cache[mask], before[mask])
    return exact


@pytest.mark.parametrize("spec", [
    synth.Spec("app_b5_ragged", 5, 1, (1, 64, 65, 1000, 4096)),
    synth.Spec("app_b3_sq2", 3, 2, (2, 129, 3000)),
], ids=lambda s: s.name)
def test_append_small_batches_every_value(spec):
    batch = synth.make_batch(spec, seed=23)
    inp = synth.make_append_inputs(spec.batch, spec.q_tokens, seed=29)
    say(f"case {spec.name}: lens={batch['seq_lens'].tolist()}")
    got = _run_append(batch, inp)
    _check_append(batch, inp, spec.q_tokens, got, what=spec.name)


@pytest.mark.parametrize("idx", [1, 3, 4])
def test_append_full_size_workloads(idx):
    """The batch shapes of the uniform, long (positions up to 131071) and
    two-token workloads, every written value."""
    spec = synth.CONFIGS[idx]
    batch = synth.make_batch(spec, seed=idx)
    inp = synth.make_append_inputs(spec.batch, spec.q_tokens, seed=100 + idx)
    say(f"case append {spec.name}: B={spec.batch} Sq={spec.q_tokens}")
    got = _run_append(batch, inp)
    _check_append(batch, inp, spec.q_tokens, got, what=spec.name)


def test_append_rope_base_argument():
    spec = synth.Spec("app_base", 2, 1, (300, 5000))
    batch = synth.make_batch(spec, seed=31)
    inp = synth.make_append_inputs(2, 1, seed=37)
    got = _run_append(batch, inp, rope_base=500.0)
    _check_append(batch, inp, 1, got, rope_base=500.0, what="rope base 500")


def test_append_skips_an_invalid_block_id():
    """A block id outside the cache is never written through: that token's
    row is skipped (its proper slot keeps its old bytes), the others are
    written as usual."""
    spec = synth.Spec("app_bad_block", 3, 1, (100, 200, 300))
    batch = synth.make_batch(spec, seed=41)
    inp = synth.make_append_inputs(3, 1, seed=43)
    bad = dict(batch)
    bad["block_table"] = batch["block_table"].copy()
    bad["block_table"][1, (200 - 1) // 64] = 10 ** 6
    got = _run_append(bad, inp)
    _check_append(batch, inp, 1, got, what="invalid block id", skip={1})


def test_append_then_decode_matches_oracle():
    """End to end: the producer writes the new tokens' rows, the decode step
    reads them; the decode is compared with the oracle on the cache the
    producer left."""
    spec = synth.Spec("app_decode", 3, 2, (130, 700, 2049))
    batch = synth.make_batch(spec, seed=47)
    inp = synth.make_append_inputs(3, 2, seed=53)
    got_cache = _run_append(batch, inp)
    _check_append(batch, inp, 2, got_cache, what="before decode")
    after = dict(batch)
    after["cache"] = got_cache
    assert_parity(run_gpu(after), oracle(after), "decode after append")
