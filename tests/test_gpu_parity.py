"""GPU parity: the HIP library against the fp64 oracle, through the C ABI.

Every case compares every output: small batches against the naive oracle,
the four full-size workloads against the oracle's absorb-order routine
(pinned to the naive definition on the CPU).
Tolerance: max|err| <= 1e-2 * max|o_ref| and sum|err| / sum|o_ref| <= 2e-3.
"""

import numpy as np
import pytest

from mla_latent_kv_amd import synth
from tests.parity import assert_parity, metrics, oracle, run_gpu, say

pytestmark = pytest.mark.gpu

SMALL = [
    synth.Spec("b3_ragged", 3, 1, (100, 1000, 2500)),
    synth.Spec("b2_sq2", 2, 2, (97, 1500)),
    synth.Spec("edges_sq1", 6, 1, (1, 31, 32, 33, 64, 65)),
    synth.Spec("edges_sq2", 5, 2, (2, 3, 32, 33, 129)),
    synth.Spec("qx3_b2", 2, 1, (700, 3000), q_scale=3.0),
    # 128 and more query rows: the absorb runs its wide tile (4 heads x 64 columns)
    synth.Spec("rows128_sq1", 128, 1, ("uniform", 1, 200)),
    synth.Spec("rows129_sq1", 129, 1, ("uniform", 1, 100)),   # one row in the last 32-row tile
    synth.Spec("rows160_sq2", 80, 2, ("uniform", 2, 150)),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
def test_small_batches_every_output(spec):
    batch = synth.make_batch(spec, seed=17)
    say(f"case {spec.name}: lens={batch['seq_lens'].tolist()}")
    got = run_gpu(batch)
    ref = oracle(batch)
    assert_parity(got, ref, spec.name)


def test_tiny_unpaged_config_every_output():
    spec = synth.CONFIGS[0]
    batch = synth.make_batch(spec, seed=0)
    say(f"case {spec.name}")
    assert_parity(run_gpu(batch), oracle(batch), spec.name)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_full_size_config_every_output(idx):
    """The four full-size workloads, in the launch configuration the benchmark
    times (default split target), every output against the oracle's absorb-
    order routine. That routine is the naive definition regrouped by the
    identity q^T (U c) = (U^T q)^T c (wq-win.github.io DeepSeek-V3 notes,
    section 2 algebra check); the CPU tier pins the two together to 1e-10."""
    spec = synth.CONFIGS[idx]
    batch = synth.make_batch(spec, seed=idx)
    say(f"case {spec.name}: B={spec.batch} Sq={spec.q_tokens} tokens={int(batch['seq_lens'].sum())}")
    got = run_gpu(batch)
    ref = oracle(batch, path="absorb")
    assert_parity(got, ref, f"{spec.name} every output")


# small batches whose split plan gives each attention workgroup several items
# in a row (the item loop reuses its LDS rings), partial last blocks
MULTI_ROUND = [
    (synth.Spec("rounds_sq1", 8, 1, (100, 1000, 2500, 333, 64, 1500, 777, 2049)), 5),
    (synth.Spec("rounds_sq2", 6, 2, (97, 1500, 2600, 130, 65, 1025)), 4),
]


@pytest.mark.parametrize("spec,split", MULTI_ROUND, ids=lambda x: getattr(x, "name", str(x)))
def test_multi_round_plan_every_output(spec, split):
    from tests import plan_mirror as pm
    batch = synth.make_batch(spec, seed=41)
    lens = batch["seq_lens"].tolist()
    mx = int(batch["max_seq_len"])
    r = pm.check(lens, mx, split)
    rounds = -(-r["n_items"] // split)
    assert rounds >= 2, rounds
    say(f"case {spec.name}: lens={lens} split {split}: {r['n_items']} items, {rounds} rounds")
    got = run_gpu(batch, split_target=split)
    assert_parity(got, oracle(batch), spec.name)


def test_block_permutation_is_bitwise_invariant():
    spec = synth.Spec("perm", 3, 2, (300, 1100, 64))
    batch = synth.make_batch(spec, seed=3)
    rng = np.random.default_rng(1)
    nb = batch["cache"].shape[0]
    perm = rng.permutation(nb)
    inv = np.argsort(perm)
    b2 = dict(batch)
    b2["cache"] = batch["cache"][perm]
    b2["block_table"] = np.where(batch["block_table"] >= 0,
                                 inv[np.maximum(batch["block_table"], 0)], -1).astype(np.int32)
    say("case permutation")
    o1 = run_gpu(batch)
    o2 = run_gpu(b2)
    assert np.array_equal(o1, o2)


def test_repeat_is_bitwise_identical_and_split_count_within_tolerance():
    spec = synth.Spec("repeat", 4, 1, (4096, 1000, 77, 2048))
    batch = synth.make_batch(spec, seed=5)
    say("case repeat / split target")
    o1 = run_gpu(batch)
    o2 = run_gpu(batch)
    assert np.array_equal(o1, o2)
    o3 = run_gpu(batch, split_target=7)
    o4 = run_gpu(batch, split_target=1000)
    ref = oracle(batch, sample=[(0, 3), (1, 50), (2, 127), (3, 0)])
    for o, name in ((o1, "default"), (o3, "split 7"), (o4, "split 1000")):
        assert_parity(o, ref, name)
    # different split plans round differently; they must agree to well within
    # the parity tolerance (the split merge is exact up to rounding)
    mt = metrics(o3, o1)
    assert mt["max_rel"] <= 2e-3 and mt["mean_rel"] <= 5e-4, mt


def test_zero_query_is_uniform_average():
    spec = synth.Spec("zeroq", 2, 1, (513, 64))
    batch = synth.make_batch(spec, seed=8)
    batch["q_nope"][:] = 0
    batch["q_pe"][:] = 0
    say("case zero query")
    got = run_gpu(batch)
    from oracle import mla_oracle as orc
    w_uv = orc.bf16_bits_to_f64(batch["w_uv"])
    for b in range(2):
        rows = orc.gather_sequence(batch["cache"], batch["block_table"][b],
                                   int(batch["seq_lens"][b]), 64)
        want = np.einsum("hvc,c->hv", w_uv, rows[:, :512].mean(axis=0))
        assert_parity(got[b, 0], want, f"zero query b={b}")


def test_second_token_row_matches_shorter_single_token_run():
    spec2 = synth.Spec("sq2", 2, 2, (700, 2049))
    batch2 = synth.make_batch(spec2, seed=9)
    # the same cache viewed as Sq = 1 with one token less, query = row 0
    batch1 = dict(batch2)
    batch1["q_nope"] = np.ascontiguousarray(batch2["q_nope"][:, :1])
    batch1["q_pe"] = np.ascontiguousarray(batch2["q_pe"][:, :1])
    batch1["seq_lens"] = batch2["seq_lens"] - 1
    say("case causal row")
    o2 = run_gpu(batch2)
    o1 = run_gpu(batch1)
    mt = metrics(o2[:, 0], o1[:, 0])
    say(f"row0 vs Sq=1: {mt}")
    assert mt["max_rel"] <= 1e-3 and mt["mean_rel"] <= 2e-4


def test_shared_workspace_after_a_larger_plan():
    """A workspace that held a larger split plan (more work-list entries) must
    not leak any of them into a later call with a smaller plan."""
    import torch
    from mla_latent_kv_amd import binding, device
    spec = synth.Spec("reuse", 4, 1, (4096, 1000, 77, 2048))
    batch = synth.make_batch(spec, seed=11)
    d = device.upload(batch)
    big = binding.MLADecoder(0, max_q_tokens=2, split_target=1000)
    small = binding.MLADecoder(0, max_q_tokens=2, split_target=7)
    n = max(big.workspace_size(4, 1, d["max_seq_len"]), small.workspace_size(4, 1, d["max_seq_len"]))
    args = (d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["kv_cache"], d["block_table"],
            d["seq_lens"], d["max_seq_len"])
    say("case shared workspace: split 1000 then split 7")
    fresh = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bytes everywhere
    want = small(*args, workspace=fresh).cpu().numpy()
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    big(*args, workspace=ws)
    got = small(*args, workspace=ws).cpu().numpy()
    torch.cuda.synchronize()
    assert np.isfinite(want).all()
    assert np.array_equal(got, want)


def test_rows_that_see_nothing_are_zero():
    """L = 0 (both rows see nothing) and L = 1 < Sq = 2 (row 0 sees nothing,
    row 1 sees position 0): those rows are zeros; the rest match the oracle."""
    spec = synth.Spec("short_seqs", 4, 2, (1, 0, 2, 70), max_seq_len=128)
    batch = synth.make_batch(spec, seed=29)
    say(f"case {spec.name}: lens={batch['seq_lens'].tolist()}")
    got = run_gpu(batch)
    assert np.all(got[1] == 0.0) and np.all(got[0, 0] == 0.0)
    assert_parity(got, oracle(batch), spec.name)


@pytest.mark.parametrize("sq", [1, 2])
def test_one_item_longer_than_a_block_table_window(sq):
    """A split target of 1 makes the whole 20,000-token history one work item
    (313 cache blocks): the attention pass reloads its window of 64 block ids
    four times within the item. Every head against the oracle (absorb order,
    itself pinned to the naive definition)."""
    spec = synth.Spec(f"long_item_sq{sq}", 1, sq, (20000 + sq - 1,))
    batch = synth.make_batch(spec, seed=31 + sq)
    say(f"case {spec.name}: one item of {int(batch['seq_lens'][0])} tokens")
    got = run_gpu(batch, split_target=1)
    ref = oracle(batch, path="absorb")
    assert_parity(got, ref, spec.name)


# batches past the searched plan's reach: the simple plan (every sequence cut
# at one chunk length, full chunks first), and the largest searched sort
# (the oracle's per-sequence cost makes every output of a thousand sequences
# a minute of host time: 256 sampled (sequence, head) pairs each, every output
# finite)
LARGE_BATCH = [
    synth.Spec("simple_b1100", 1100, 1, ("uniform", 1, 200)),
    synth.Spec("sorted_b1024", 1024, 1, ("uniform", 1, 300)),
    # 8192 sequences (8192 query rows for the absorb, 256 row tiles of the
    # wide tile) and 4096 two-token sequences
    synth.Spec("simple_b8192", 8192, 1, ("uniform", 1, 64)),
    synth.Spec("simple_b4096_sq2", 4096, 2, ("uniform", 2, 64)),
]


@pytest.mark.parametrize("spec", LARGE_BATCH, ids=lambda s: s.name)
def test_large_batches(spec, n_sample=256):
    from tests import plan_mirror as pm
    import torch
    batch = synth.make_batch(spec, seed=43)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    P = n_cu if spec.q_tokens == 1 else n_cu // 2
    r = pm.check(batch["seq_lens"], int(batch["max_seq_len"]), P)
    say(f"case {spec.name}: B={spec.batch} Sq={spec.q_tokens} tokens={int(batch['seq_lens'].sum())} "
        f"search={r['search']} items={r['n_items']}")
    got = run_gpu(batch)
    assert np.isfinite(got).all()
    rng = np.random.default_rng(44)
    bs = rng.choice(spec.batch, n_sample, replace=False)
    sample = [(int(b), int(rng.integers(0, 128))) for b in bs]
    assert_parity(got, oracle(batch, sample=sample), f"{spec.name} {n_sample} sampled (b, h)")


def _random_case(k):
    """Seeded random batch k: batch size, query tokens, a length mix with
    empty sequences, histories shorter than the query tokens and ragged long
    ones, host bound slack, a split target and the query scale."""
    rng = np.random.default_rng(1000 + k)
    B = int(rng.integers(1, 49))
    sq = int(rng.integers(1, 3))
    kinds = rng.random(B)
    lens = np.where(kinds < 0.15, 0,
                    np.where(kinds < 0.25, rng.integers(1, sq + 1, B), rng.integers(1, 4001, B)))
    if lens.max() == 0:
        lens[0] = 1
    slack = int(rng.choice([0, 1, 63, 200]))
    spec = synth.Spec(f"random{k}", B, sq, tuple(int(x) for x in lens),
                      q_scale=float(rng.choice([1.0, 3.0])), max_seq_len=int(lens.max()) + slack)
    split = int(rng.choice([0, 1, 5, 13, 64, 300]))
    return spec, split


@pytest.mark.parametrize("k", range(10))
def test_random_batches_every_output(k):
    spec, split = _random_case(k)
    batch = synth.make_batch(spec, seed=2000 + k)
    say(f"case {spec.name}: B={spec.batch} Sq={spec.q_tokens} split={split} "
        f"max_seq_len={batch['max_seq_len']} lens={batch['seq_lens'].tolist()}")
    got = run_gpu(batch, split_target=split)
    assert_parity(got, oracle(batch, path="absorb"), f"{spec.name} every output")


def _far_cache_batch():
    """One two-token sequence of 2^20 + 1000 cached tokens whose blocks sit
    at ids 23000 and up of a 40000-block cache (2.95 GB, so block byte
    offsets pass 2^31); every other block is bf16 NaN, so a read of any block
    the table does not name would show in the output."""
    batch = synth.make_batch(synth.Spec("far_1m", 1, 2, ((1 << 20) + 1000,)), seed=77)
    nb = batch["cache"].shape[0]
    far = np.full((40000,) + batch["cache"].shape[1:], synth.BF16_NAN, dtype=batch["cache"].dtype)
    far[23000:23000 + nb] = batch["cache"]
    batch["cache"] = far
    batch["block_table"] = np.where(batch["block_table"] >= 0, batch["block_table"] + 23000, -1).astype(np.int32)
    return batch


def test_cache_past_2gib_and_a_million_token_history():
    batch = _far_cache_batch()
    say(f"case far_1m: L={int(batch['seq_lens'][0])} Sq=2, cache {batch['cache'].nbytes / 1e9:.2f} GB, "
        f"blocks {int(batch['block_table'].min())}..{int(batch['block_table'].max())}")
    got = run_gpu(batch)
    assert np.isfinite(got).all()
    assert_parity(got, oracle(batch, path="absorb"), "far_1m every output")
