"""GPU parity of the decode-step prologue (mla_project_new_tokens: the cache
append and the query side of the same new tokens in one call) against the
fp64 oracle, through the C ABI.

Bars: the cache rows take the cache append's bound (tests/test_gpu_append.py)
and every other cache byte stays as it was; q_nope / q_pe take the query
side's bound (tests/test_gpu_qproj.py) and must agree with what
mla_query_project returns for the same inputs: the two calls split the
compressed query's fp32 sums differently, so a q value may differ by its
rounding; at least 99 % are identical.
"""

import numpy as np
import pytest

from mla_latent_kv_amd import synth
from tests.parity import say
from tests.test_gpu_append import _check_append
from tests.test_gpu_qproj import _check_q

pytestmark = pytest.mark.gpu


def _t(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _u16(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _same_q(a, b, what):
    """bf16 bit patterns a (prologue) and b (mla_query_project): >= 99 %
    identical. Each side is held to the oracle's bound on its own (a here, b
    in tests/test_gpu_qproj.py), which bounds their difference; a value
    within rounding of zero may even take opposite signs in the two orders."""
    frac = float((a == b).mean())
    say(f"prologue {what}: {frac:.5f} of q values identical to mla_query_project's")
    assert frac >= 0.99, (what, frac)


def _run(batch, hid, app, rope_base=0.0):
    import torch
    from mla_latent_kv_amd import binding, device
    d = device.upload(batch)
    dec = binding.MLADecoder(0, max_q_tokens=2)
    w_kv = dec.pack(_t(np.concatenate([app["w_dkv"], app["w_kr"]])))
    w_dq, w_uq = dec.pack(_t(hid["w_dq"])), dec.pack(_t(hid["w_uq"]))
    h = _t(hid["hidden"])
    qn, qp = dec.project_new_tokens(h, w_dq, w_uq, w_kv, d["kv_cache"], d["block_table"], d["seq_lens"],
                                    rope_base=rope_base)
    qn2, qp2 = dec.query_project(h, w_dq, w_uq, d["seq_lens"], rope_base=rope_base)
    torch.cuda.synchronize()
    out = _u16(d["kv_cache"]), _u16(qn), _u16(qp), _u16(qn2), _u16(qp2)
    dec.close()
    return out


@pytest.mark.parametrize("spec", [
    synth.Spec("pro_b5_ragged", 5, 1, (1, 64, 65, 1000, 4096)),
    synth.Spec("pro_b3_sq2", 3, 2, (2, 129, 131071)),
    synth.Spec("pro_b1", 1, 1, (7,)),
], ids=lambda s: s.name)
def test_prologue_small_batches(spec):
    batch = synth.make_batch(spec, seed=41)
    hid = synth.make_query_inputs(spec.batch, spec.q_tokens, seed=43)
    app = synth.make_append_inputs(spec.batch, spec.q_tokens, seed=47)
    app["hidden"] = hid["hidden"]
    say(f"case prologue {spec.name}: lens={batch['seq_lens'].tolist()}")
    cache, qn, qp, qn2, qp2 = _run(batch, hid, app)
    _same_q(qn, qn2, spec.name + " q_nope")
    _same_q(qp, qp2, spec.name + " q_pe")
    _check_q(hid, batch["seq_lens"], spec.q_tokens, qn, qp, spec.name)
    _check_append(batch, app, spec.q_tokens, cache, what=spec.name)


@pytest.mark.parametrize("idx", [1, 4])
def test_prologue_full_size_workloads(idx):
    """The batch shapes of the uniform decode (B = 32) and the two-token
    workload, every written value."""
    spec = synth.CONFIGS[idx]
    batch = synth.make_batch(spec, seed=idx)
    hid = synth.make_query_inputs(spec.batch, spec.q_tokens, seed=200 + idx)
    app = synth.make_append_inputs(spec.batch, spec.q_tokens, seed=300 + idx)
    app["hidden"] = hid["hidden"]
    say(f"case prologue {spec.name}: B={spec.batch} Sq={spec.q_tokens}")
    cache, qn, qp, qn2, qp2 = _run(batch, hid, app)
    _same_q(qn, qn2, spec.name + " q_nope")
    _same_q(qp, qp2, spec.name + " q_pe")
    _check_q(hid, batch["seq_lens"], spec.q_tokens, qn, qp, spec.name)
    _check_append(batch, app, spec.q_tokens, cache, what=spec.name)


def test_prologue_rope_base_argument():
    spec = synth.Spec("pro_base", 2, 2, (5, 3000))
    batch = synth.make_batch(spec, seed=51)
    hid = synth.make_query_inputs(2, 2, seed=53)
    app = synth.make_append_inputs(2, 2, seed=55)
    app["hidden"] = hid["hidden"]
    say("case prologue rope_base 50000")
    cache, qn, qp, qn2, qp2 = _run(batch, hid, app, rope_base=50000.0)
    _same_q(qn, qn2, "base 50000 q_nope")
    _same_q(qp, qp2, "base 50000 q_pe")
    _check_append(batch, app, 2, cache, rope_base=50000.0, what="base 50000")
