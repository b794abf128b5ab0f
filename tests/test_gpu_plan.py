"""The split plan as the GPU writes it (prep kernel, read back from the
workspace after a decode call) equals the host mirror's plan entry for
entry (each position's entries up to the first unused one, which the
attention pass stops at), on the workload shapes (uniform, ragged, two-token), small and empty
sequences, a small split target, and a batch past the searched plan's limit
(the simple plan). The mirror's invariants (coverage, contiguous slots, dense
positions, capacity) are asserted on the same batches.
"""

import numpy as np
import pytest

from mla_latent_kv_amd import synth
from tests import plan_mirror as pm
from tests.parity import say

pytestmark = pytest.mark.gpu


def _align(x, a=256):
    return (x + a - 1) // a * a


def _device_plan(spec, seed, split_target=0):
    import torch
    from mla_latent_kv_amd import binding, device
    batch = synth.make_batch(spec, seed=seed)
    d = device.upload(batch)
    dec = binding.MLADecoder(0, max_q_tokens=2, split_target=split_target)
    B, Sq = spec.batch, spec.q_tokens
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    P = split_target or (n_cu if Sq == 1 else n_cu // 2)
    positions, depth, max_chunks = pm.layout(B, Sq, d["max_seq_len"], P)
    ws = torch.zeros(dec.workspace_size(B, Sq, d["max_seq_len"]), dtype=torch.uint8, device="cuda")
    binding.mla_decode_run(dec.ctx, d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"],
                           d["block_table"], d["seq_lens"], d["max_seq_len"], workspace=ws)
    torch.cuda.synchronize()
    raw = ws.cpu().numpy()
    dec.close()
    n_work = depth * positions
    off = _align(4 * 512)   # the range flags (one int per absorb workgroup) come first
    work = raw[off:off + n_work * 32].view(np.int32).reshape(n_work, 8)
    off = _align(off + n_work * 32)
    seqinfo = raw[off:off + B * 16].view(np.int32).reshape(B, 4)
    off = _align(off + B * 16)
    meta = raw[off:off + 16].view(np.int32)
    max_len = min(batch["block_table"].shape[1] * 64, d["max_seq_len"])
    return batch, work, seqinfo, meta, (P, positions, depth, max_chunks, max_len)


CASES = [
    ("uniform_b32_l4096", synth.CONFIGS[1], 1, 0),
    ("ragged_b64", synth.CONFIGS[2], 2, 0),
    ("mtp_b128_sq2", synth.CONFIGS[4], 4, 0),
    ("small", synth.Spec("plan_small", 3, 1, (1, 130, 5000)), 5, 0),
    ("with_empty", synth.Spec("plan_empty", 4, 1, (0, 64, 65, 0)), 6, 0),
    ("target_7", synth.Spec("plan_t7", 4, 1, (700, 64, 4096, 1)), 7, 7),
    ("simple_b1100", synth.Spec("plan_b1100", 1100, 1, ("uniform", 1, 200)), 8, 0),
    # searched plans with the largest sorts: 1024 sequences only fit in four
    # rounds (1024 keys), 700 sequences pad the sort to 1024
    ("sorted_b1024", synth.Spec("plan_b1024", 1024, 1, ("uniform", 1, 300)), 9, 0),
    ("sorted_b700", synth.Spec("plan_b700", 700, 1, ("uniform", 1, 2000)), 10, 0),
]


@pytest.mark.parametrize("name,spec,seed,target", CASES, ids=[c[0] for c in CASES])
def test_device_plan_equals_mirror(name, spec, seed, target):
    say(f"case plan {name}: B={spec.batch} Sq={spec.q_tokens} target={target}")
    batch, work, seqinfo, meta, (P, positions, depth, max_chunks, max_len) = _device_plan(spec, seed, target)
    lens = batch["seq_lens"]
    table = np.asarray(batch["block_table"])
    pm.check(lens, max_len, P)
    ref = pm.plan(lens, max_len, P, positions, depth, max_chunks)
    say(f"plan {name}: search={ref['search']} C={ref['C']} items={ref['n_items']} "
        f"rounds={-(-ref['n_items'] // P)}")
    assert int(meta[0]) == ref["n_items"] and int(meta[1]) == ref["C"]
    # each position's entries up to its first unused one, which must be marked
    for pos in range(positions):
        j = 0
        while j < depth and j * positions + pos in ref["work"]:
            e = j * positions + pos
            b, t0, t1, sl = ref["work"][e]
            assert tuple(work[e, :5]) == (b, t0, t1, sl, ref["L"][b]), (name, e)
            # the cache blocks of the split's first two 64-token blocks
            blk0 = int(table[b, t0 // 64])
            blk1 = int(table[b, t0 // 64 + 1]) if t1 - t0 > 64 else blk0
            assert (int(work[e, 5]), int(work[e, 6])) == (blk0, blk1), (name, e)
            j += 1
        if j < depth:
            assert work[j * positions + pos, 3] == -1, (name, pos, j)
    for b in range(len(lens)):
        assert tuple(seqinfo[b, :3]) == ref["seqinfo"][b], (name, b)
