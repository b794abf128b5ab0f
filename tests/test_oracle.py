"""Pins of the fp64 oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
printed value, a closed form, a special case that reduces to a library routine
(torch's scaled-dot-product attention in fp64 on the CPU), scalar brute force,
or an invariant of the exact arithmetic.
"""

import math
import os

import numpy as np
import pytest

from oracle import mla_oracle as orc
from mla_latent_kv_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape, std=1.0):
    return rng.standard_normal(shape) * std


def _full_dims_case(rng, n_heads=4, length=300, sq=1, q_std=1.0):
    qn = _rand(rng, sq, n_heads, 128, std=q_std)
    qp = _rand(rng, sq, n_heads, 64, std=q_std)
    wk = _rand(rng, n_heads, 128, 512, std=1 / math.sqrt(512))
    wv = _rand(rng, n_heads, 128, 512, std=1 / math.sqrt(512))
    c = _rand(rng, length, 512)
    kr = _rand(rng, length, 64)
    return qn, qp, wk, wv, c, kr


# --------------------------------------------------------------------------
# Printed counts ("DeepSeek-V3" page, MLA section; golden/cache_counts.txt).

def test_cache_counts_match_printed_values():
    want = {}
    with open(os.path.join(GOLDEN, "cache_counts.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                want[k] = float(v)
    got = orc.cache_counts()
    assert got["mha"] == want["mha"]
    assert got["mla"] == want["mla"]
    assert got["naive"] == want["naive"]
    assert round(100 * got["reduction"], 2) == want["reduction_percent"]
    assert got["reduction"] == 0.982421875


def test_cache_layout_bytes_per_token():
    spec = synth.Spec("t", 2, 1, (100, 70))
    d = synth.make_batch(spec, 0)
    cache = d["cache"]
    assert cache.shape[1:] == (64, 576)
    assert cache.itemsize * cache.shape[2] == 1152   # 576 bf16 per token


# --------------------------------------------------------------------------
# The absorb identity q^T (U c) = (U^T q)^T c ([P1], section 2 algebra check).

@pytest.mark.parametrize("sq", [1, 2])
def test_absorb_order_equals_naive(sq):
    rng = np.random.default_rng(11 + sq)
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=4, length=333, sq=sq)
    scale = orc.default_scale()
    ref = orc.naive_decode(qn, qp, wk, wv, c, kr, scale)
    got = orc.absorb_decode(qn, qp, wk, wv, c, kr, scale)
    assert np.max(np.abs(got - ref)) <= 1e-10 * np.max(np.abs(ref))


def test_absorb_identity_single_dot():
    rng = np.random.default_rng(5)
    u = rng.standard_normal((128, 512))
    q = rng.standard_normal(128)
    cs = rng.standard_normal((50, 512))
    lhs = np.array([q @ (u @ c) for c in cs])
    q_abs = orc.absorb_query(q[None, None, :], u[None])[0, 0]
    rhs = cs @ q_abs
    assert np.max(np.abs(lhs - rhs)) <= 1e-10 * np.max(np.abs(lhs))


# --------------------------------------------------------------------------
# Softmax normalisation.

def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(3)
    for n in (1, 2, 17, 4096):
        s = rng.standard_normal(n) * 7
        p = orc.softmax(s)
        assert abs(p.sum() - 1.0) <= 1e-12
        assert np.all(p >= 0)


def test_softmax_extreme_scores_stay_finite():
    p = orc.softmax(np.array([1000.0, 999.0, -1000.0]))
    assert np.all(np.isfinite(p))
    assert abs(p[0] / p[1] - math.e) < 1e-12


# --------------------------------------------------------------------------
# Scalar brute force on tiny dims.

@pytest.mark.parametrize("length", [1, 2, 3, 7])
@pytest.mark.parametrize("sq", [1, 2])
def test_brute_force_tiny(length, sq):
    if length < sq:
        pytest.skip("a sequence holds at least its new tokens")
    rng = np.random.default_rng(100 * length + sq)
    H, dn, dr, dc, dv = 2, 3, 2, 5, 4
    qn, qp = rng.standard_normal((sq, H, dn)), rng.standard_normal((sq, H, dr))
    wk, wv = rng.standard_normal((H, dn, dc)), rng.standard_normal((H, dv, dc))
    c, kr = rng.standard_normal((length, dc)), rng.standard_normal((length, dr))
    scale = 1 / math.sqrt(dn + dr)
    want = orc.brute_force_decode(qn, qp, wk, wv, c, kr, scale)
    got = orc.naive_decode(qn, qp, wk, wv, c, kr, scale)
    got_abs = orc.absorb_decode(qn, qp, wk, wv, c, kr, scale)
    tol = 1e-12 * max(1.0, np.max(np.abs(want)))
    assert np.max(np.abs(got - want)) <= tol
    assert np.max(np.abs(got_abs - want)) <= tol


# --------------------------------------------------------------------------
# Closed-form special cases.

def test_single_visible_token_returns_its_value():
    rng = np.random.default_rng(7)
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=3, length=1)
    o = orc.naive_decode(qn, qp, wk, wv, c, kr, orc.default_scale())
    want = np.einsum("hvc,c->hv", wv, c[0])
    assert np.max(np.abs(o[0] - want)) <= 1e-12 * np.max(np.abs(want))


def test_zero_query_gives_uniform_average():
    rng = np.random.default_rng(8)
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=3, length=257, sq=2)
    qn[:] = 0
    qp[:] = 0
    o = orc.naive_decode(qn, qp, wk, wv, c, kr, orc.default_scale())
    for i in range(2):
        n = 257 - 2 + i + 1
        want = np.einsum("hvc,c->hv", wv, c[:n].mean(axis=0))
        assert np.max(np.abs(o[i] - want)) <= 1e-12 * np.max(np.abs(want))


def test_constant_cache_ignores_query():
    rng = np.random.default_rng(9)
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=3, length=40)
    c[:] = c[0]
    kr[:] = kr[0]
    o = orc.naive_decode(qn, qp, wk, wv, c, kr, orc.default_scale())
    want = np.einsum("hvc,c->hv", wv, c[0])
    assert np.max(np.abs(o[0] - want)) <= 1e-12 * np.max(np.abs(want))


def test_reduces_to_library_attention_with_selection_weights():
    """With W_UK[h] selecting latent dims [a_h, a_h+128) and W_UV[h] selecting
    [b_h, b_h+128), MLA is plain softmax attention with K = [c[a..] ; k_R] and
    V = c[b..]: compare with torch's scaled_dot_product_attention in fp64."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    H, L, sq = 4, 129, 2
    qn, qp, _, _, c, kr = _full_dims_case(rng, n_heads=H, length=L, sq=sq)
    a = [0, 100, 384, 7]
    b = [128, 0, 250, 384]
    wk = np.zeros((H, 128, 512))
    wv = np.zeros((H, 128, 512))
    for h in range(H):
        wk[h, np.arange(128), a[h] + np.arange(128)] = 1.0
        wv[h, np.arange(128), b[h] + np.arange(128)] = 1.0
    scale = orc.default_scale()
    got = orc.naive_decode(qn, qp, wk, wv, c, kr, scale)
    for h in range(H):
        q = torch.tensor(np.concatenate([qn[:, h], qp[:, h]], axis=1))[None]   # [1, sq, 192]
        k = torch.tensor(np.concatenate([c[:, a[h]:a[h] + 128], kr], axis=1))[None]
        v = torch.tensor(c[:, b[h]:b[h] + 128])[None]
        mask = torch.tensor([[j <= L - sq + i for j in range(L)] for i in range(sq)])
        want = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, attn_mask=mask[None], scale=scale)[0].numpy()
        assert np.max(np.abs(got[:, h] - want)) <= 1e-12 * np.max(np.abs(want))


# --------------------------------------------------------------------------
# Invariants of the exact arithmetic.

def test_split_merge_equals_single_pass():
    rng = np.random.default_rng(31)
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=2, length=1000, q_std=3.0)
    scale = orc.default_scale()
    _, o_lat = orc.absorb_decode(qn, qp, wk, wv, c, kr, scale, return_latent=True)
    q_abs = orc.absorb_query(qn, wk)
    for bounds in ([0, 1000], [0, 64, 500, 1000], [0, 1, 2, 999, 1000],
                   [0, 333, 666, 1000, 1200]):
        for h in range(2):
            parts = [orc.absorb_partial(q_abs[0, h], qp[0, h], c, kr, scale, t0, t1, 1000)
                     for t0, t1 in zip(bounds[:-1], bounds[1:])]
            merged = orc.merge_partials(parts)
            assert np.max(np.abs(merged - o_lat[0, h])) <= 1e-12 * np.max(np.abs(o_lat[0, h]))


def test_causal_rule_second_token_matches_shorter_single():
    """Sq = 2: query 0 sees positions <= L-2, exactly an Sq = 1 decode of L-1."""
    rng = np.random.default_rng(41)
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=3, length=90, sq=2)
    scale = orc.default_scale()
    both = orc.naive_decode(qn, qp, wk, wv, c, kr, scale)
    first = orc.naive_decode(qn[:1], qp[:1], wk, wv, c[:-1], kr[:-1], scale)
    last = orc.naive_decode(qn[1:], qp[1:], wk, wv, c, kr, scale)
    assert np.max(np.abs(both[0] - first[0])) <= 1e-12 * np.max(np.abs(first))
    assert np.max(np.abs(both[1] - last[0])) <= 1e-12 * np.max(np.abs(last))


def test_linear_in_value_weights():
    rng = np.random.default_rng(51)
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=2, length=70)
    wv2 = _rand(rng, 2, 128, 512)
    s = orc.default_scale()
    lhs = orc.naive_decode(qn, qp, wk, wv + wv2, c, kr, s)
    rhs = orc.naive_decode(qn, qp, wk, wv, c, kr, s) + orc.naive_decode(qn, qp, wk, wv2, c, kr, s)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(lhs))


def test_latent_is_convex_combination():
    rng = np.random.default_rng(52)
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=3, length=200, q_std=3.0)
    _, o_lat = orc.absorb_decode(qn, qp, wk, wv, c, kr, orc.default_scale(), return_latent=True)
    lo, hi = c.min(axis=0), c.max(axis=0)
    assert np.all(o_lat >= lo - 1e-12) and np.all(o_lat <= hi + 1e-12)


# --------------------------------------------------------------------------
# Score scale: Var(s) = (1/192)(512 * 128/512 + 64) = 1 for the workloads'
# distributions, and 9 with queries scaled by 3.

@pytest.mark.parametrize("q_std,want", [(1.0, 1.0), (3.0, 3.0)])
def test_score_std_closed_form(q_std, want):
    rng = np.random.default_rng(61)
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=64, length=512, q_std=q_std)
    s = np.concatenate([orc.naive_scores(qn[0, h], qp[0, h], wk[h], c, kr, orc.default_scale())
                        for h in range(64)])
    assert abs(s.std() / want - 1) < 0.03


# --------------------------------------------------------------------------
# Paged layout.

def test_gather_and_block_permutation_invariance():
    spec = synth.Spec("t", 3, 1, (130, 64, 1), paged=True)
    d = synth.make_batch(spec, 5)
    # rebuild the same logical content under a different physical placement
    rng = np.random.default_rng(0)
    nb = d["cache"].shape[0]
    perm = rng.permutation(nb)
    inv = np.argsort(perm)
    cache2 = d["cache"][perm]                 # new block k holds old block perm[k]
    table2 = np.where(d["block_table"] >= 0, inv[np.maximum(d["block_table"], 0)], -1)
    for b in range(3):
        L = int(d["seq_lens"][b])
        r1 = orc.gather_sequence(d["cache"], d["block_table"][b], L, 64)
        r2 = orc.gather_sequence(cache2, table2[b], L, 64)
        assert np.array_equal(r1, r2)
        assert not np.isnan(r1).any()
    o1 = orc.decode_batch(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], d["cache"],
                          d["block_table"], d["seq_lens"], 64, sample=[(0, 1), (2, 5)])
    o2 = orc.decode_batch(d["q_nope"], d["q_pe"], d["w_uk"], d["w_uv"], cache2,
                          table2, d["seq_lens"], 64, sample=[(0, 1), (2, 5)])
    assert np.array_equal(o1, o2, equal_nan=True)
    assert np.isfinite(o1[0, 0, 1]).all() and np.isfinite(o1[2, 0, 5]).all()


PAGED_LENGTHS = (1, 63, 64, 65, 130)


def scatter_paged(rows_by_seq, block_size, seed):
    """Scatter known contiguous rows (uint16 bits, one [L_b, W] array per
    sequence) into a paged cache, token by token: token j of sequence b goes
    to physical block table[b, j // block_size], slot j % block_size. The
    physical blocks are a random permutation (so a table is out of order and
    sequences interleave), unused slots of a last block hold bf16 NaN and
    table entries past a sequence's blocks are -1."""
    rng = np.random.default_rng(seed)
    width = rows_by_seq[0].shape[1]
    nblk = [-(-r.shape[0] // block_size) for r in rows_by_seq]
    total = sum(nblk)
    perm = rng.permutation(total)
    cache = np.full((total, block_size, width), synth.BF16_NAN, dtype=np.uint16)
    table = np.full((len(rows_by_seq), max(nblk)), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(nblk):
        table[b, :n] = perm[k:k + n]
        k += n
    for b, rows in enumerate(rows_by_seq):
        for j in range(rows.shape[0]):
            cache[table[b, j // block_size], j % block_size, :] = rows[j]
    return cache, table


def paged_roundtrip_failures(gather, block_size=64, seed=3):
    """Sequences of PAGED_LENGTHS tokens scattered into one paged cache must
    come back from ``gather`` exactly (same shape, bit-identical values).
    Returns the lengths that fail."""
    rng = np.random.default_rng(seed)
    known = [synth.f32_to_bf16_bits(rng.standard_normal((L, 576)).astype(np.float32))
             for L in PAGED_LENGTHS]
    cache, table = scatter_paged(known, block_size, seed)
    bad = []
    for b, L in enumerate(PAGED_LENGTHS):
        got = gather(cache, table[b], L, block_size)
        want = orc.bf16_bits_to_f64(known[b])
        if got.shape != want.shape or not np.array_equal(got, want):
            bad.append(L)
    return bad


def test_paged_reader_returns_the_scattered_rows_exactly():
    """The paged reader against known contiguous rows scattered token by token
    through an out-of-order block table: lengths 1, 63, 64, 65 and 130 (one
    partial block, one block minus one, exactly one, one plus one, and a
    partial third block), NaN in every unused slot, -1 table tails. The layout
    is 576 values per token in 64-token blocks ("DeepSeek-V3" page, MLA cache
    comparison: 512 + 64 = 576)."""
    assert paged_roundtrip_failures(orc.gather_sequence) == []
    assert paged_roundtrip_failures(orc.gather_sequence, block_size=16, seed=4) == []


@pytest.mark.parametrize("sq", [1, 2])
def test_decode_batch_through_the_paged_cache_equals_brute_force(sq):
    """decode_batch over a paged, permuted, NaN-padded cache equals scalar
    brute force over the same rows kept contiguous (tiny dims: H=2, d_nope=3,
    d_rope=2, d_latent=5, d_v=4; lengths 1, 63, 64, 65 and 130 with 64-token
    blocks), on both of the oracle's paths."""
    rng = np.random.default_rng(70 + sq)
    H, dn, dr, dc, dv = 2, 3, 2, 5, 4
    lens = [max(L, sq) for L in PAGED_LENGTHS]
    bits = lambda *s: synth.f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32))
    rows = [bits(L, dc + dr) for L in lens]
    cache, table = scatter_paged(rows, 64, seed=sq)
    qn, qp = bits(len(lens), sq, H, dn), bits(len(lens), sq, H, dr)
    wk, wv = bits(H, dn, dc), bits(H, dv, dc)
    scale = 1 / math.sqrt(dn + dr)
    for path in ("naive", "absorb"):
        got = orc.decode_batch(qn, qp, wk, wv, cache, table, np.array(lens, dtype=np.int32), 64,
                               scale=scale, path=path)
        for b, L in enumerate(lens):
            r = orc.bf16_bits_to_f64(rows[b])
            want = orc.brute_force_decode(orc.bf16_bits_to_f64(qn[b]), orc.bf16_bits_to_f64(qp[b]),
                                          orc.bf16_bits_to_f64(wk), orc.bf16_bits_to_f64(wv),
                                          r[:, :dc], r[:, dc:], scale)
            assert np.max(np.abs(got[b] - want)) <= 1e-12 * np.max(np.abs(want)), (path, L)


def test_absorb_path_rows_that_see_nothing_are_zero():
    """L < Sq on the absorb-order routine: rows i < Sq - L see no position and
    are zeros, as on the naive path; the other rows equal the naive path."""
    rng = np.random.default_rng(64)
    L, sq = 3, 5
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=2, length=L, sq=sq)
    scale = orc.default_scale()
    got = orc.absorb_decode(qn, qp, wk, wv, c, kr, scale)
    ref = orc.naive_decode(qn, qp, wk, wv, c, kr, scale)
    assert np.all(got[:sq - L] == 0.0) and np.all(ref[:sq - L] == 0.0)
    assert np.max(np.abs(got - ref)) <= 1e-10 * np.max(np.abs(ref))


def test_bf16_decode_is_exact():
    vals = np.array([0.0, 1.0, -2.5, 3.140625, 1e-3, -65504.0], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(vals)
    back = orc.bf16_bits_to_f64(bits)
    assert back[1] == 1.0 and back[2] == -2.5 and back[3] == 3.140625
    assert abs(back[4] - 1e-3) <= 2 ** -9 * 1e-3


# --------------------------------------------------------------------------
# Prefill: every prompt token is a query (Sq = L), attention is causal.

def test_prefill_reduces_to_library_causal_attention():
    """Sq = L with selection weights is plain causal attention: torch's
    scaled_dot_product_attention with its own is_causal rule (query i sees
    keys 0..i when the query and key counts agree), fp64 on the CPU."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(61)
    H, L = 3, 150
    qn, qp, _, _, c, kr = _full_dims_case(rng, n_heads=H, length=L, sq=L)
    a, b = [64, 0, 300], [0, 384, 200]
    wk = np.zeros((H, 128, 512))
    wv = np.zeros((H, 128, 512))
    for h in range(H):
        wk[h, np.arange(128), a[h] + np.arange(128)] = 1.0
        wv[h, np.arange(128), b[h] + np.arange(128)] = 1.0
    scale = orc.default_scale()
    got = orc.naive_decode(qn, qp, wk, wv, c, kr, scale)
    for h in range(H):
        q = torch.tensor(np.concatenate([qn[:, h], qp[:, h]], axis=1))[None]
        k = torch.tensor(np.concatenate([c[:, a[h]:a[h] + 128], kr], axis=1))[None]
        v = torch.tensor(c[:, b[h]:b[h] + 128])[None]
        want = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)[0]
        assert np.max(np.abs(got[:, h] - want.numpy())) <= 1e-12 * float(want.abs().max())


def test_prefill_row_equals_decode_of_its_prefix():
    """Prompt token i of a prefill sees exactly positions 0..i: the same
    result as a one-token decode of the first i + 1 cached tokens."""
    rng = np.random.default_rng(62)
    L = 70
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=2, length=L, sq=L)
    scale = orc.default_scale()
    full = orc.naive_decode(qn, qp, wk, wv, c, kr, scale)
    for i in (0, 1, 31, 63, 64, 69):
        one = orc.naive_decode(qn[i:i + 1], qp[i:i + 1], wk, wv, c[:i + 1], kr[:i + 1], scale)
        assert np.max(np.abs(full[i] - one[0])) <= 1e-12 * np.max(np.abs(one))
    # the first prompt token attends only to itself: its output is its own value
    np.testing.assert_allclose(full[0], np.einsum("hvc,c->hv", wv, c[0]), rtol=1e-12, atol=1e-13)


def test_rows_that_see_nothing_are_zero_and_the_rest_unchanged():
    """L < Sq: rows i < Sq - L see no position and yield zeros (the reading
    the C ABI states); row i >= Sq - L sees positions 0..L-Sq+i, exactly a
    one-token decode of that prefix."""
    rng = np.random.default_rng(63)
    L, sq = 5, 9
    qn, qp, wk, wv, c, kr = _full_dims_case(rng, n_heads=2, length=L, sq=sq)
    scale = orc.default_scale()
    got = orc.naive_decode(qn, qp, wk, wv, c, kr, scale)
    assert np.all(got[:sq - L] == 0.0)
    for i in range(sq - L, sq):
        n = L - sq + i + 1
        one = orc.naive_decode(qn[i:i + 1], qp[i:i + 1], wk, wv, c[:n], kr[:n], scale)
        assert np.max(np.abs(got[i] - one[0])) <= 1e-12 * np.max(np.abs(one))
