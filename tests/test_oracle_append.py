"""Pins of the oracle's cache-append producer, query side and output projection
(CPU only).

The pages give c_KV = W_DKV h and a RoPE-rotated, head-shared k_R without the
rotary formula, so the rotation is pinned by the properties that define a
rotary embedding (norm preservation, identity at position 0, composition of
angles, scores that depend only on the relative position) and against an
independent library implementation (transformers' Llama rotary embedding,
whose half-split pairing equals the consecutive-pair one after de-interleaving
the 64 channels). The projection and the row layout are pinned by scalar
brute force on tiny shapes. The output projection W_O concat_h(o_h) is pinned
by scalar brute force (which also fixes the head-major concatenation order),
linearity and unit vectors.
"""

import math

import numpy as np
import pytest

from oracle import mla_oracle as orc


def _rng(seed):
    return np.random.default_rng(seed)


def test_rope_preserves_norm_and_is_identity_at_zero():
    x = _rng(0).standard_normal((7, 64))
    pos = np.array([0, 1, 5, 63, 4096, 131071, 2 ** 20])
    y = orc.rope_rotate(x, pos)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(orc.rope_rotate(x, np.zeros(7, dtype=int)), x)


def test_rope_angles_compose():
    x = _rng(1).standard_normal((5, 64))
    a = np.array([3, 17, 250, 1000, 9])
    b = np.array([4, 1, 6, 2047, 0])
    np.testing.assert_allclose(orc.rope_rotate(orc.rope_rotate(x, a), b), orc.rope_rotate(x, a + b),
                               rtol=1e-10, atol=1e-11)


def test_rope_scores_depend_only_on_relative_position():
    r = _rng(2)
    q, k = r.standard_normal(64), r.standard_normal(64)
    for m, n in [(10, 3), (500, 499), (7, 40), (4096, 0), (123, 123)]:
        lhs = orc.rope_rotate(q, m) @ orc.rope_rotate(k, n)
        rhs = orc.rope_rotate(q, m - n) @ k
        assert abs(lhs - rhs) < 1e-10 * (1 + abs(rhs)), (m, n, lhs, rhs)
    # and the dependence is real: a different offset gives a different score
    assert abs(orc.rope_rotate(q, 5) @ k - orc.rope_rotate(q, 6) @ k) > 1e-3


def _library_rope(x, pos, base):
    """transformers' rotary embedding (default type) applied to the
    de-interleaved vector: channel 2i -> i, 2i+1 -> i + d/2."""
    import torch
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb
    d = x.shape[-1]
    cfg = LlamaConfig(hidden_size=d * 2, num_attention_heads=2, head_dim=d,
                      max_position_embeddings=1 << 20, rope_theta=base)
    emb = LlamaRotaryEmbedding(cfg)
    inv = emb.inv_freq.double()                                   # library frequencies
    freqs = torch.tensor(np.asarray(pos, dtype=np.float64))[:, None] * inv[None, :]
    ang = torch.cat((freqs, freqs), dim=-1)
    cos, sin = ang.cos()[None], ang.sin()[None]                   # [1, n, d]
    y = torch.tensor(np.concatenate([x[..., 0::2], x[..., 1::2]], axis=-1))[None, None]
    yq, _ = apply_rotary_pos_emb(y, y, cos, sin, unsqueeze_dim=1)
    yq = yq[0, 0].numpy()
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = yq[..., : d // 2], yq[..., d // 2:]
    return out


@pytest.mark.parametrize("base", [10000.0, 500.0])
def test_rope_matches_library_rotary_embedding(base):
    pytest.importorskip("transformers")
    x = _rng(3).standard_normal((6, 64))
    small = np.array([0, 1, 2, 7, 31, 63])
    # inv_freq is fp32 in the library: tight at small positions ...
    np.testing.assert_allclose(orc.rope_rotate(x, small, base), _library_rope(x, small, base),
                               rtol=0, atol=5e-6)
    # ... and still within the fp32 frequency rounding at long ones
    big = np.array([100, 1000, 4095, 30000, 65535, 131071])
    np.testing.assert_allclose(orc.rope_rotate(x, big, base), _library_rope(x, big, base),
                               rtol=0, atol=0.05)


def test_append_rows_scalar_brute_force():
    r = _rng(4)
    d_h, d_c, d_r = 5, 3, 4
    h = r.standard_normal((3, d_h))
    w_dkv = r.standard_normal((d_c, d_h))
    w_kr = r.standard_normal((d_r, d_h))
    pos = np.array([0, 2, 9])
    got = orc.append_rows(h, w_dkv, w_kr, pos, base=100.0)
    for t in range(3):
        for n in range(d_c):
            want = sum(w_dkv[n, k] * h[t, k] for k in range(d_h))
            assert abs(got[t, n] - want) < 1e-12
        kr = [sum(w_kr[n, k] * h[t, k] for k in range(d_h)) for n in range(d_r)]
        # the k_R block is the rotation of W_KR h (checked above against the library)
        np.testing.assert_allclose(got[t, d_c:], orc.rope_rotate(np.array(kr), pos[t], 100.0),
                                   rtol=0, atol=1e-12)
        # position 0 leaves W_KR h as is, so the row is plain [W_DKV h | W_KR h]
        if pos[t] == 0:
            np.testing.assert_allclose(got[t, d_c:], kr, rtol=0, atol=1e-12)


def test_append_rows_linear_in_hidden():
    r = _rng(5)
    h1, h2 = r.standard_normal((2, 4, 40))
    w_dkv, w_kr = r.standard_normal((12, 40)), r.standard_normal((8, 40))
    pos = np.array([3, 0, 77, 5000])
    a, b = 0.75, -2.5
    lhs = orc.append_rows(a * h1 + b * h2, w_dkv, w_kr, pos)
    rhs = a * orc.append_rows(h1, w_dkv, w_kr, pos) + b * orc.append_rows(h2, w_dkv, w_kr, pos)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_append_positions_are_the_last_q_tokens():
    pos = orc.append_positions(np.array([1, 5, 64]), 1)
    np.testing.assert_array_equal(pos, [[0], [4], [63]])
    pos = orc.append_positions(np.array([2, 130]), 2)
    np.testing.assert_array_equal(pos, [[0, 1], [128, 129]])


def test_append_batch_unit_hidden_selects_weight_columns():
    """h = e_k gives c_KV = column k of W_DKV and k_R = RoPE(column k of W_KR)."""
    r = _rng(6)
    from mla_latent_kv_amd import synth
    d_h = 48
    w_dkv = synth.f32_to_bf16_bits(r.standard_normal((orc.D_LATENT, d_h)).astype(np.float32))
    w_kr = synth.f32_to_bf16_bits(r.standard_normal((orc.D_ROPE, d_h)).astype(np.float32))
    hid = np.zeros((2, 1, d_h), dtype=np.uint16)
    hid[0, 0, 7] = 0x3F80   # bf16 1.0
    hid[1, 0, 30] = 0x3F80
    rows = orc.append_batch(hid, w_dkv, w_kr, np.array([1, 1000]), 1)
    wd, wk = orc.bf16_bits_to_f64(w_dkv), orc.bf16_bits_to_f64(w_kr)
    np.testing.assert_array_equal(rows[0, 0, :orc.D_LATENT], wd[:, 7])
    np.testing.assert_array_equal(rows[0, 0, orc.D_LATENT:], wk[:, 7])   # position 0
    np.testing.assert_array_equal(rows[1, 0, :orc.D_LATENT], wd[:, 30])
    np.testing.assert_allclose(rows[1, 0, orc.D_LATENT:], orc.rope_rotate(wk[:, 30], 999),
                               rtol=0, atol=1e-13)
    assert not np.allclose(rows[1, 0, orc.D_LATENT:], wk[:, 30])
    assert math.isclose(np.linalg.norm(rows[1, 0, orc.D_LATENT:]), np.linalg.norm(wk[:, 30]),
                        rel_tol=1e-13)


# ---- output projection pins

def test_output_project_scalar_brute_force_and_head_order():
    r = _rng(9)
    n, H, dv, dm = 2, 3, 4, 5
    o = r.standard_normal((n, H, dv))
    w = r.standard_normal((dm, H * dv))
    y = orc.output_project(o, w)
    for t in range(n):
        for m in range(dm):
            want = sum(w[m, h * dv + v] * o[t, h, v] for h in range(H) for v in range(dv))
            assert abs(y[t, m] - want) < 1e-12
    # a head's block of W_O acts only on that head's output
    o2 = np.zeros_like(o)
    o2[:, 1] = o[:, 1]
    np.testing.assert_allclose(orc.output_project(o2, w), o[:, 1] @ w[:, dv:2 * dv].T,
                               rtol=1e-13, atol=1e-13)


def test_output_project_linear_and_unit_columns():
    r = _rng(10)
    o1, o2 = r.standard_normal((2, 3, 8, 16))
    w = r.standard_normal((12, 128))
    np.testing.assert_allclose(orc.output_project(2 * o1 - 3 * o2, w),
                               2 * orc.output_project(o1, w) - 3 * orc.output_project(o2, w),
                               rtol=1e-12, atol=1e-12)
    e = np.zeros((1, 8, 16))
    e[0, 5, 7] = 1.0
    np.testing.assert_array_equal(orc.output_project(e, w)[0], w[:, 5 * 16 + 7])


# ---- query side pins

def test_query_project_scalar_brute_force():
    r = _rng(11)
    n, d_h, d_q, H, dn, dr = 2, 6, 4, 3, 2, 4
    h = r.standard_normal((n, d_h))
    w_dq = r.standard_normal((d_q, d_h))
    w_uq = r.standard_normal((H, dn + dr, d_q))
    pos = np.array([0, 7])
    qn, qp = orc.query_project(h, w_dq, w_uq, pos, base=50.0, d_nope=dn, d_rope=dr)
    for t in range(n):
        c = [sum(w_dq[j, k] * h[t, k] for k in range(d_h)) for j in range(d_q)]
        for hh in range(H):
            full = [sum(w_uq[hh, rr, j] * c[j] for j in range(d_q)) for rr in range(dn + dr)]
            np.testing.assert_allclose(qn[t, hh], full[:dn], rtol=0, atol=1e-12)
            np.testing.assert_allclose(qp[t, hh], orc.rope_rotate(np.array(full[dn:]), pos[t], 50.0),
                                       rtol=0, atol=1e-12)
            if pos[t] == 0:
                np.testing.assert_allclose(qp[t, hh], full[dn:], rtol=0, atol=1e-12)


def test_query_and_key_rotations_give_relative_scores():
    """q_pe . k_R of the same projected vectors depends only on the distance
    between the query's and the key's positions."""
    r = _rng(12)
    qv, kv = r.standard_normal(64), r.standard_normal(64)
    s1 = orc.rope_rotate(qv, 1000) @ orc.rope_rotate(kv, 990)
    s2 = orc.rope_rotate(qv, 40) @ orc.rope_rotate(kv, 30)
    assert abs(s1 - s2) < 1e-10


def test_query_project_linear_in_hidden():
    r = _rng(13)
    h1, h2 = r.standard_normal((2, 3, 20))
    w_dq, w_uq = r.standard_normal((8, 20)), r.standard_normal((2, 6, 8))
    pos = np.array([1, 2, 300])
    a = orc.query_project(h1 - 2 * h2, w_dq, w_uq, pos, d_nope=2, d_rope=4)
    b1 = orc.query_project(h1, w_dq, w_uq, pos, d_nope=2, d_rope=4)
    b2 = orc.query_project(h2, w_dq, w_uq, pos, d_nope=2, d_rope=4)
    for i in range(2):
        np.testing.assert_allclose(a[i], b1[i] - 2 * b2[i], rtol=1e-12, atol=1e-12)
