"""The fp16 range rules of the GPU path, emulated on the host.

The matrix-core products run on fp16 operands: the bf16 latent converted to
fp16, and the absorbed query q_abs rounded to fp16 after an exact scaling by
2^-4 (q_pe gets the same scaling, the softmax scale undoes it). No page states
value ranges; these tests show what the two rules mean:

* c_KV: a bf16 value converts to fp16 exactly when 2^-14 <= |x| <= 65504
  (fp16's normal range holds every 8-bit bf16 significand), with an absolute
  error below 2^-24 under it; above it the conversion saturates.
* q_abs: without the scaling, |q_abs| > 65504 overflows fp16 and the scores
  become inf; with it the bound is 2^20 - 2^9 = 1048064, and a decode whose
  q_abs exceeds 65504 (but not that bound) stays within the parity tolerance.
"""

import math

import numpy as np

from oracle import mla_oracle as orc

Q_SCALE = 2.0 ** -4
Q_ABS_MAX = 65504.0 / Q_SCALE


def _all_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = orc.bf16_bits_to_f64(bits)
    return x[np.isfinite(x)]


def test_bf16_values_in_fp16_normal_range_convert_exactly():
    x = _all_bf16()
    inside = (np.abs(x) >= 2.0 ** -14) & (np.abs(x) <= 65504.0)
    h = x[inside].astype(np.float16).astype(np.float64)
    assert np.array_equal(h, x[inside])
    tiny = np.abs(x) < 2.0 ** -14
    err = np.abs(x[tiny].astype(np.float16).astype(np.float64) - x[tiny])
    assert err.max() <= 2.0 ** -25   # nearest rounding; toward zero stays below 2^-24
    assert Q_ABS_MAX == 2.0 ** 20 - 2.0 ** 9


def _emulated_decode(qn, qp, wk, wv, c, kr, scale, pre_scale):
    """Absorb-order decode of one sequence with q_abs rounded to fp16 after
    multiplying by ``pre_scale`` (everything else exact), fp64."""
    q_abs = orc.absorb_query(qn, wk) * pre_scale
    with np.errstate(over="ignore", invalid="ignore"):
        q16 = q_abs.astype(np.float16).astype(np.float64)
        s = (scale / pre_scale) * (np.einsum("ihc,jc->ihj", q16, c)
                                   + np.einsum("ihr,jr->ihj", qp * pre_scale, kr))
        e = np.exp(s - s.max(axis=2, keepdims=True))
        p = e / e.sum(axis=2, keepdims=True)
    return np.einsum("hvc,ihc->ihv", wv, np.einsum("ihj,jc->ihc", p, c))


def test_scaled_q_abs_keeps_large_queries_finite_and_accurate():
    """q scaled by 2^16 with the softmax scale divided by 2^16: the same
    attention, but q_abs reaches ~1e5. Unscaled fp16 overflows; the 2^-4
    scaling keeps every value finite and the output within the parity bar."""
    rng = np.random.default_rng(90)
    H, L, big = 8, 256, 2.0 ** 16
    qn = rng.standard_normal((1, H, 128)) * big
    qp = rng.standard_normal((1, H, 64)) * big
    wk = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    wv = rng.standard_normal((H, 128, 512)) / math.sqrt(512)
    c = rng.standard_normal((L, 512))
    kr = rng.standard_normal((L, 64))
    scale = orc.default_scale() / big
    q_abs = orc.absorb_query(qn, wk)
    assert 65504.0 < np.abs(q_abs).max() < Q_ABS_MAX
    ref = orc.absorb_decode(qn, qp, wk, wv, c, kr, scale)
    plain = _emulated_decode(qn, qp, wk, wv, c, kr, scale, 1.0)
    assert not np.isfinite(plain).all()
    got = _emulated_decode(qn, qp, wk, wv, c, kr, scale, Q_SCALE)
    err = np.abs(got - ref)
    assert np.isfinite(got).all()
    assert err.max() <= 1e-2 * np.abs(ref).max()
    assert err.sum() <= 2e-3 * np.abs(ref).sum()
