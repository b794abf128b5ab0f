"""GPU parity of the query side (h -> q_nope, q_pe) against the fp64 oracle,
and of the whole attention block of a decode step (cache append, query side,
decode, output projection) against the oracle's chain, through the C ABI.

Bar for q: each value is rounded to bf16 once, so it must lie within one
bf16 step of the exact value plus the accumulation allowance
2^-15 * (|W_UQ| (|W_DQ| |h|)) (two fp32 sums and the hi + lo split of c_Q;
a RoPE pair takes the allowance of both inputs), and at least 99 % must
equal the exact value rounded to nearest.
"""

import numpy as np
import pytest

from mla_latent_kv_amd import synth
from tests.parity import assert_parity, say

pytestmark = pytest.mark.gpu


def _bf16_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rne_bits(x):
    from tests.test_gpu_append import _exact_to_bf16_bits
    return _exact_to_bf16_bits(x)


def _t(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run_q(inp, seq_lens):
    import torch
    from mla_latent_kv_amd import binding
    dec = binding.MLADecoder(0, max_q_tokens=2)
    qn, qp = dec.query_project(_t(inp["hidden"]), dec.pack(_t(inp["w_dq"])), dec.pack(_t(inp["w_uq"])),
                               torch.from_numpy(np.ascontiguousarray(seq_lens)).cuda())
    torch.cuda.synchronize()
    dec.close()
    f = lambda a: a.view(torch.int16).cpu().numpy().view(np.uint16)
    return f(qn), f(qp)


def _check_q(inp, seq_lens, q_tokens, got_n, got_p, what):
    from oracle import mla_oracle as orc
    qn, qp = orc.query_batch(inp["hidden"], inp["w_dq"], inp["w_uq"], seq_lens, q_tokens)
    h = np.abs(orc.bf16_bits_to_f64(inp["hidden"])).reshape(-1, orc.D_HIDDEN)
    c_mag = h @ np.abs(orc.bf16_bits_to_f64(inp["w_dq"])).T                   # [n, 1536]
    q_mag = np.einsum("hrq,nq->nhr", np.abs(orc.bf16_bits_to_f64(inp["w_uq"])), c_mag)
    allow = 2.0 ** -15 * q_mag.reshape(*qn.shape[:3], -1)
    a_n = allow[..., :orc.D_NOPE]
    a_p = allow[..., orc.D_NOPE:].copy()
    pair = a_p[..., 0::2] + a_p[..., 1::2]
    a_p[..., 0::2], a_p[..., 1::2] = pair, pair
    frac_all = []
    for got, ex, al, nm in ((got_n, qn, a_n, "q_nope"), (got_p, qp, a_p, "q_pe")):
        gv = _bf16_f64(got)
        k = np.floor(np.log2(np.maximum(np.abs(ex), 2.0 ** -126))).astype(int)
        step = np.ldexp(1.0, k - 7)
        err = np.abs(gv - ex)
        ratio = float((err / (step + al)).max())
        frac = float((got == _rne_bits(ex)).mean())
        frac_all.append(frac)
        say(f"qproj {what} {nm}: {got.size} values, worst err / bound {ratio:.3f}, "
            f"{frac:.5f} rounded like the exact value")
        assert ratio <= 1.0, f"{what} {nm}: {ratio:.2f} x the bound"
        assert frac >= 0.99, f"{what} {nm}: only {frac:.4f} rounded exactly"


@pytest.mark.parametrize("batch,q_tokens,lens", [
    (3, 1, (1, 700, 5000)),
    (2, 2, (2, 131071)),
    (32, 1, None),
    (128, 2, None),
])
def test_query_project_against_oracle(batch, q_tokens, lens):
    if lens is None:
        lens = tuple(int(x) for x in np.random.default_rng(batch).integers(2, 16384, batch))
    seq_lens = np.asarray(lens, dtype=np.int32)
    inp = synth.make_query_inputs(batch, q_tokens, seed=80 + batch)
    say(f"case qproj B={batch} Sq={q_tokens}")
    got_n, got_p = _run_q(inp, seq_lens)
    _check_q(inp, seq_lens, q_tokens, got_n, got_p, f"B{batch} Sq{q_tokens}")


def test_attention_block_end_to_end():
    """h -> cache rows (append) and queries (query side) -> decode -> W_O, all
    on the GPU, against the oracle's chain (its exact intermediates rounded to
    bf16 where the GPU path stores bf16: the cache rows and the queries)."""
    import torch
    from mla_latent_kv_amd import binding, device
    from oracle import mla_oracle as orc
    spec = synth.Spec("block", 3, 2, (130, 900, 2049))
    batch = synth.make_batch(spec, seed=91)
    hid = synth.make_query_inputs(3, 2, seed=93)
    app = synth.make_append_inputs(3, 2, seed=95)
    app["hidden"] = hid["hidden"]                  # one hidden state feeds both
    w_o = synth.make_oproj_inputs(1, seed=97)["w_o"]
    say("case attention block B=3 Sq=2")
    d = device.upload(batch)
    dec = binding.MLADecoder(0, max_q_tokens=2)
    w_kv = dec.pack(_t(np.concatenate([app["w_dkv"], app["w_kr"]])))
    w_dq, w_uq, w_o_p = dec.pack(_t(hid["w_dq"])), dec.pack(_t(hid["w_uq"])), dec.pack(_t(w_o))
    dec.append(_t(app["hidden"]), w_kv, d["kv_cache"], d["block_table"], d["seq_lens"])
    qn, qp = dec.query_project(_t(hid["hidden"]), w_dq, w_uq, d["seq_lens"])
    out = dec(qn, qp, d["w_uk"], d["w_uv"], d["kv_cache"], d["block_table"], d["seq_lens"],
              d["max_seq_len"])
    y = dec.output_project(out, w_o_p)
    torch.cuda.synchronize()
    got = y.cpu().numpy().astype(np.float64)
    dec.close()
    # oracle chain
    rows = orc.append_batch(app["hidden"], app["w_dkv"], app["w_kr"], batch["seq_lens"], 2)
    cache = batch["cache"].copy()
    for b, L in enumerate(batch["seq_lens"]):
        for i in range(2):
            pos = int(L) - 2 + i
            cache[batch["block_table"][b, pos // 64], pos % 64] = _rne_bits(rows[b, i])
    q_n, q_p = orc.query_batch(hid["hidden"], hid["w_dq"], hid["w_uq"], batch["seq_lens"], 2)
    o = orc.decode_batch(_rne_bits(q_n), _rne_bits(q_p), batch["w_uk"], batch["w_uv"], cache,
                         batch["block_table"], batch["seq_lens"], 64)
    ref = orc.output_project(o.reshape(-1, 128 * 128), orc.bf16_bits_to_f64(w_o))
    assert_parity(got, ref, "attention block (append, query side, decode, W_O)")
