"""The seeded input generator: determinism, table structure, poison placement."""

import numpy as np

from mla_latent_kv_amd import synth


def test_same_seed_same_bytes():
    spec = synth.Spec("t", 3, 2, ("uniform", 70, 300))
    a, b = synth.make_batch(spec, 4), synth.make_batch(spec, 4)
    for k in ("q_nope", "q_pe", "w_uk", "w_uv", "cache", "block_table", "seq_lens"):
        assert np.array_equal(a[k], b[k])
    c = synth.make_batch(spec, 5)
    assert not np.array_equal(a["cache"], c["cache"])


def test_block_table_is_permutation_and_poison_only_past_lengths():
    spec = synth.Spec("t", 5, 1, ("uniform", 1, 400))
    d = synth.make_batch(spec, 9)
    lens, table, cache = d["seq_lens"], d["block_table"], d["cache"]
    nblk = (lens + 63) // 64
    used = np.concatenate([table[b, :nblk[b]] for b in range(5)])
    assert sorted(used.tolist()) == list(range(cache.shape[0]))
    for b in range(5):
        assert np.all(table[b, nblk[b]:] == -1)
        rows = cache[table[b, :nblk[b]]].reshape(-1, 576)
        nan = (rows & 0x7FFF) > 0x7F80
        assert not nan[:lens[b]].any()
        assert nan[lens[b]:].all()


def test_unpaged_is_identity_table():
    d = synth.make_batch(synth.CONFIGS[0], 0)
    assert d["block_table"].tolist() == [list(range(8))]
    assert d["seq_lens"].tolist() == [512]


def test_bf16_rounding_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9], dtype=np.float32)
    got = synth.f32_to_bf16_bits(x)
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 tie -> 1+2^-6 (even); 1+2^-9 rounds down
    assert got.tolist() == [0x3F80, 0x3F82, 0x3F80]


def test_config_distributions():
    d = synth.make_batch(synth.Spec("t", 2, 1, ("fixed", 64), q_scale=3.0), 1)
    qn = (d["q_nope"].astype(np.uint32) << 16).view(np.float32)
    wk = (d["w_uk"].astype(np.uint32) << 16).view(np.float32)
    assert abs(qn.std() - 3.0) < 0.1
    assert abs(wk.var() * 512 - 1.0) < 0.01
