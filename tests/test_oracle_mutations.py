"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case patches one plausible error into the oracle and checks that the
independent reference it is pinned to disagrees.
"""

import math

import numpy as np
import pytest

from oracle import mla_oracle as orc


def _case(rng, H=3, L=50, sq=1):
    qn = rng.standard_normal((sq, H, 128))
    qp = rng.standard_normal((sq, H, 64))
    wk = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    wv = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    c = rng.standard_normal((L, 512))
    kr = rng.standard_normal((L, 64))
    return qn, qp, wk, wv, c, kr


def _brute_tiny_mismatch(monkeypatch, patch):
    rng = np.random.default_rng(1)
    H, dn, dr, dc, dv, L = 2, 3, 2, 5, 4, 6
    args = (rng.standard_normal((2, H, dn)), rng.standard_normal((2, H, dr)),
            rng.standard_normal((H, dn, dc)), rng.standard_normal((H, dv, dc)),
            rng.standard_normal((L, dc)), rng.standard_normal((L, dr)))
    want = orc.brute_force_decode(*args, 1 / math.sqrt(dn + dr))
    with monkeypatch.context() as m:
        patch(m)
        got = orc.naive_decode(*args, 1 / math.sqrt(dn + dr))
    return np.max(np.abs(got - want))


def test_dropped_rope_term_is_caught(monkeypatch):
    def patch(m):
        m.setattr(orc, "naive_scores",
                  lambda qn, qp, wk, c, kr, s: s * (qn @ (c @ wk.T).T))
    assert _brute_tiny_mismatch(monkeypatch, patch) > 1e-3


def test_wrong_rope_sign_is_caught(monkeypatch):
    def patch(m):
        m.setattr(orc, "naive_scores",
                  lambda qn, qp, wk, c, kr, s: s * (qn @ (c @ wk.T).T - qp @ kr.T))
    assert _brute_tiny_mismatch(monkeypatch, patch) > 1e-3


def test_off_by_one_visibility_is_caught(monkeypatch):
    def patch(m):
        m.setattr(orc, "visible_len", lambda L, sq, i: L - sq + i)
    assert _brute_tiny_mismatch(monkeypatch, patch) > 1e-3


def test_wrong_scale_is_caught_by_score_std():
    rng = np.random.default_rng(61)
    qn, qp, wk, wv, c, kr = _case(rng, H=64, L=512)
    for bad in (1 / 192, 1 / math.sqrt(128)):
        s = np.concatenate([orc.naive_scores(qn[0, h], qp[0, h], wk[h], c, kr, bad)
                            for h in range(64)])
        assert abs(s.std() - 1) >= 0.03


def test_unshifted_merge_weights_are_caught():
    rng = np.random.default_rng(3)
    qn, qp, wk, wv, c, kr = _case(rng, H=1, L=300)
    qn *= 3
    s = orc.default_scale()
    _, o_lat = orc.absorb_decode(qn, qp, wk, wv, c, kr, s, return_latent=True)
    q_abs = orc.absorb_query(qn, wk)
    parts = [orc.absorb_partial(q_abs[0, 0], qp[0, 0], c, kr, s, t0, t0 + 100, 300)
             for t0 in (0, 100, 200)]
    # a merge that forgets the exp(m_s - M) rescale disagrees with one pass
    bad = sum(o for o, _, _ in parts) / sum(l for _, _, l in parts)
    assert np.max(np.abs(bad - o_lat[0, 0])) > 1e-3
    assert np.max(np.abs(orc.merge_partials(parts) - o_lat[0, 0])) < 1e-12


# ---- cache-append producer: planted mistakes in the rotary embedding must
# move it away from the library rotary embedding it is pinned to

def _rope_gap(monkeypatch, patch):
    pytest.importorskip("transformers")
    from tests.test_oracle_append import _library_rope
    x = np.random.default_rng(8).standard_normal((6, 64))
    pos = np.array([1, 2, 7, 31, 63, 500])
    want = _library_rope(x, pos, 10000.0)
    with monkeypatch.context() as m:
        patch(m)
        got = orc.rope_rotate(x, pos)
    return np.max(np.abs(got - want))


def test_rope_frequency_exponent_mistake_is_caught(monkeypatch):
    def patch(m):
        m.setattr(orc, "rope_inv_freq",
                  lambda d=64, base=10000.0: base ** (-np.arange(d // 2, dtype=np.float64) / d))
    assert _rope_gap(monkeypatch, patch) > 1e-2


def test_rope_clockwise_rotation_is_caught(monkeypatch):
    real = orc.rope_rotate
    def patch(m):
        m.setattr(orc, "rope_rotate", lambda x, pos, base=10000.0: real(x, -np.asarray(pos), base))
    assert _rope_gap(monkeypatch, patch) > 1e-2


def test_rope_half_split_pairing_is_caught(monkeypatch):
    real = orc.rope_rotate
    def half_split(x, pos, base=10000.0):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        inter = np.empty_like(x)
        inter[..., 0::2], inter[..., 1::2] = x[..., : d // 2], x[..., d // 2:]
        y = real(inter, pos, base)
        return np.concatenate([y[..., 0::2], y[..., 1::2]], axis=-1)
    def patch(m):
        m.setattr(orc, "rope_rotate", half_split)
    assert _rope_gap(monkeypatch, patch) > 1e-2


# ---- paged reader: a block count rounded down (drops a partial last block)
# and two full blocks read in swapped order must both fail the round trip of
# known rows through an out-of-order block table, and the paged decode's
# agreement with brute force on the same rows kept contiguous

def _gather_floor(cache_bits, table_row, length, block_size):
    nblk = length // block_size
    blocks = cache_bits[np.asarray(table_row[:nblk], dtype=np.int64)]
    rows = blocks.reshape(nblk * block_size, cache_bits.shape[-1])[:length]
    return orc.bf16_bits_to_f64(rows)


def _gather_swapped(cache_bits, table_row, length, block_size):
    nblk = -(-length // block_size)
    ids = np.asarray(table_row[:nblk], dtype=np.int64).copy()
    if nblk >= 2:
        ids[[0, 1]] = ids[[1, 0]]
    rows = cache_bits[ids].reshape(nblk * block_size, cache_bits.shape[-1])[:length]
    return orc.bf16_bits_to_f64(rows)


@pytest.mark.parametrize("mutant", [_gather_floor, _gather_swapped], ids=["floor", "swap"])
def test_paged_reader_mistakes_are_caught(mutant):
    from tests.test_oracle import paged_roundtrip_failures
    assert paged_roundtrip_failures(mutant) != []


@pytest.mark.parametrize("mutant", [_gather_floor, _gather_swapped], ids=["floor", "swap"])
def test_paged_reader_mistakes_move_the_paged_decode(monkeypatch, mutant):
    from tests import test_oracle as t
    with monkeypatch.context() as m:
        m.setattr(orc, "gather_sequence", mutant)
        with pytest.raises((AssertionError, ValueError, IndexError)):
            t.test_decode_batch_through_the_paged_cache_equals_brute_force(1)
