"""Seeded synthetic inputs for MLA decode (shared by the GPU tests, the bench
and the oracle checks).

This module only draws random numbers and lays them out: it holds none of the
attention arithmetic. Floating tensors are drawn as fp32 from NumPy's
``default_rng`` and rounded to bf16 (round-to-nearest-even) so that both sides
consume the very same bf16 bit patterns (uint16 arrays here).

Workload shapes follow DeepSeek-V3's MLA dimensions as printed in the
configuration table of the "DeepSeek-V3" page (ailearn.mscapital.top): 128
heads, 512-d KV latent, 64-d RoPE key, 128-d non-positional query, 128-d value;
and the five decode workloads this library is measured on (tiny unpaged,
uniform 32 x 4K, ragged 64 x U[1K, 32K], long 4 x 128K with queries scaled by 3,
speculative-verify 128 x 2 queries x U[2K, 16K]).
"""

from __future__ import annotations

import dataclasses

import numpy as np

BF16_NAN = 0x7FC0
BLOCK = 64


@dataclasses.dataclass(frozen=True)
class Spec:
    """One synthetic decode batch.

    lengths: either a tuple of explicit per-sequence lengths, or ("uniform", lo, hi)
    for i.i.d. integer lengths in [lo, hi] inclusive, or ("fixed", L).
    """
    name: str
    batch: int
    q_tokens: int
    lengths: tuple
    q_scale: float = 1.0
    paged: bool = True            # False: identity block table (contiguous cache)
    max_seq_len: int = 0          # host-side upper bound; 0 = max drawn length
    n_heads: int = 128
    d_nope: int = 128
    d_rope: int = 64
    d_latent: int = 512
    d_v: int = 128
    block_size: int = BLOCK


# The five measured workloads (seed = index).
CONFIGS = (
    Spec("tiny_b1_l512_unpaged", 1, 1, ("fixed", 512), paged=False),
    Spec("uniform_b32_l4096", 32, 1, ("fixed", 4096)),
    Spec("ragged_b64_l1k_32k", 64, 1, ("uniform", 1024, 32768), max_seq_len=32768),
    Spec("long_b4_l128k_qx3", 4, 1, ("fixed", 131072), q_scale=3.0),
    Spec("mtp_b128_sq2_l2k_16k", 128, 2, ("uniform", 2048, 16384), max_seq_len=16384),
)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); finite inputs only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal_bits(rng: np.random.Generator, shape, std: float = 1.0,
                 chunk: int = 1 << 24) -> np.ndarray:
    """N(0, std^2) drawn in fp32 and rounded to bf16, generated in fixed chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x = rng.standard_normal(e - s, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = f32_to_bf16_bits(x)
    return out.reshape(shape)


def draw_lengths(spec: Spec, rng: np.random.Generator) -> np.ndarray:
    kind = spec.lengths[0]
    if kind == "fixed":
        lens = np.full(spec.batch, int(spec.lengths[1]), dtype=np.int32)
    elif kind == "uniform":
        lo, hi = int(spec.lengths[1]), int(spec.lengths[2])
        lens = rng.integers(lo, hi, size=spec.batch, endpoint=True).astype(np.int32)
    else:
        lens = np.asarray(spec.lengths, dtype=np.int32)
        assert lens.shape == (spec.batch,)
    return lens


def make_tables(spec: Spec, seed: int):
    """The lengths and the block table of make_batch(spec, seed) alone (same
    draws): (seq_lens [B], block_table [B, max_blocks_per_seq] with unused
    tail entries -1, max_seq_len, total blocks). Each sequence owns
    ceil(L_b / block) physical blocks, a random permutation of all blocks
    when the spec is paged, in order otherwise."""
    ss = np.random.SeedSequence(seed).spawn(7)
    r_len, r_perm = np.random.default_rng(ss[0]), np.random.default_rng(ss[1])
    lens = draw_lengths(spec, r_len)
    bs = spec.block_size
    nblk = (lens + bs - 1) // bs
    total_blocks = int(nblk.sum())
    max_seq = int(spec.max_seq_len or lens.max())
    assert max_seq >= int(lens.max())
    max_blocks = (max_seq + bs - 1) // bs
    if spec.paged:
        perm = r_perm.permutation(total_blocks).astype(np.int32)
    else:
        perm = np.arange(total_blocks, dtype=np.int32)
    table = np.full((spec.batch, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(spec.batch):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += int(nblk[b])
    return lens, table, max_seq, total_blocks


def make_batch(spec: Spec, seed: int, poison: bool = True) -> dict:
    """Draw one batch. Returns uint16 bf16-bit arrays and int32 tables:

    q_nope [B, Sq, H, d_nope], q_pe [B, Sq, H, d_rope], w_uk [H, d_nope, d_latent],
    w_uv [H, d_v, d_latent], cache [num_blocks, block, d_latent + d_rope],
    block_table [B, max_blocks_per_seq] (unused tail entries -1),
    seq_lens [B], plus the host-side ``max_seq_len``.

    Cache row j of sequence b is [c_KV (d_latent) | k_R (d_rope)] in physical
    block block_table[b, j // block], slot j % block. The unused slots of each
    sequence's last block hold bf16 NaN when ``poison`` is set.
    """
    ss = np.random.SeedSequence(seed).spawn(7)
    r_qn, r_qp, r_wk, r_wv, r_c = (np.random.default_rng(s) for s in ss[2:])
    lens, table, max_seq, total_blocks = make_tables(spec, seed)
    bs = spec.block_size
    nblk = (lens + bs - 1) // bs

    B, Sq, H = spec.batch, spec.q_tokens, spec.n_heads
    q_nope = _normal_bits(r_qn, (B, Sq, H, spec.d_nope), spec.q_scale)
    q_pe = _normal_bits(r_qp, (B, Sq, H, spec.d_rope), spec.q_scale)
    w_std = float(1.0 / np.sqrt(spec.d_latent))        # variance 1/512
    w_uk = _normal_bits(r_wk, (H, spec.d_nope, spec.d_latent), w_std)
    w_uv = _normal_bits(r_wv, (H, spec.d_v, spec.d_latent), w_std)
    row = spec.d_latent + spec.d_rope
    cache = _normal_bits(r_c, (total_blocks, bs, row))
    if poison:
        for b in range(spec.batch):
            tail = int(lens[b]) % bs
            if tail:
                cache[table[b, nblk[b] - 1], tail:, :] = BF16_NAN
    return {
        "q_nope": q_nope, "q_pe": q_pe, "w_uk": w_uk, "w_uv": w_uv,
        "cache": cache, "block_table": table, "seq_lens": lens,
        "max_seq_len": max_seq, "block_size": bs, "spec": spec,
    }


D_HIDDEN = 7168   # model width (input of the cache-append producer)


def make_append_inputs(batch: int, q_tokens: int, seed: int, d_hidden: int = D_HIDDEN,
                       d_latent: int = 512, d_rope: int = 64) -> dict:
    """Inputs of the cache-append producer as bf16 bits: hidden [B, Sq, d_hidden]
    ~ N(0, 1), w_dkv [d_latent, d_hidden] and w_kr [d_rope, d_hidden] ~ N(0,
    1/d_hidden), so each appended value has unit variance like the synthetic
    cache rows."""
    r_h, r_d, r_k = (np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3))
    w_std = 1.0 / np.sqrt(d_hidden)
    return {
        "hidden": _normal_bits(r_h, (batch, q_tokens, d_hidden)),
        "w_dkv": _normal_bits(r_d, (d_latent, d_hidden), std=w_std),
        "w_kr": _normal_bits(r_k, (d_rope, d_hidden), std=w_std),
    }


def make_oproj_inputs(rows: int, seed: int, d_in: int = 128 * 128, d_model: int = D_HIDDEN) -> dict:
    """Inputs of the output projection: x fp32 [rows, d_in] ~ N(0, 1) (the
    attention outputs it consumes are fp32) and w_o as bf16 bits [d_model,
    d_in] ~ N(0, 1/d_in)."""
    r_x, r_w = (np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(2))
    return {"x": r_x.standard_normal((rows, d_in), dtype=np.float32),
            "w_o": _normal_bits(r_w, (d_model, d_in), std=1.0 / np.sqrt(d_in))}


def make_query_inputs(batch: int, q_tokens: int, seed: int, d_hidden: int = D_HIDDEN,
                      d_q: int = 1536, heads: int = 128, d_qk: int = 192) -> dict:
    """Inputs of the query side as bf16 bits: hidden [B, Sq, d_hidden] ~ N(0, 1),
    w_dq [d_q, d_hidden] ~ N(0, 1/d_hidden), w_uq [heads, d_qk, d_q] ~ N(0, 1/d_q)
    (unit-variance c_Q and queries, like the decode workloads' q)."""
    r_h, r_d, r_u = (np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(3))
    return {
        "hidden": _normal_bits(r_h, (batch, q_tokens, d_hidden)),
        "w_dq": _normal_bits(r_d, (d_q, d_hidden), std=1.0 / np.sqrt(d_hidden)),
        "w_uq": _normal_bits(r_u, (heads, d_qk, d_q), std=1.0 / np.sqrt(d_q)),
    }
