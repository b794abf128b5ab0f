"""Algorithmic work of one absorbed MLA decode call (used for roofline figures).

Bytes: every cached row (c_KV | k_R, 576 bf16) is read once, both per-head
weight tensors W_UK and W_UV once, the queries once, and the fp32 output is
written once. Work buffers (partial softmax states, the absorbed queries) and
padding are excluded: they are the implementation's, not the method's.

Flops: per (query row, visible cached token) and head, a 576-wide score dot
product and a 512-wide accumulation of the latent, 2*(576 + 512); per query row
and head the two weight products, 2*128*512 each.
"""

from __future__ import annotations


def visible(length: int, q_tokens: int, i: int) -> int:
    """Positions query i (of q_tokens new tokens) attends to: j <= L - Sq + i."""
    return length - q_tokens + i + 1


def algorithmic_work(seq_lens, q_tokens, n_heads=128, d_nope=128, d_rope=64,
                     d_latent=512, d_v=128, elem_bytes=2, out_bytes=4) -> dict:
    row = d_latent + d_rope
    lens = [int(x) for x in seq_lens]
    cache = sum(lens) * row * elem_bytes
    weights = n_heads * (d_nope + d_v) * d_latent * elem_bytes
    n_q = len(lens) * q_tokens
    q = n_q * n_heads * (d_nope + d_rope) * elem_bytes
    out = n_q * n_heads * d_v * out_bytes
    vis = sum(visible(l, q_tokens, i) for l in lens for i in range(q_tokens))
    attn_flops = vis * 2 * n_heads * (row + d_latent)
    proj_flops = n_q * 2 * n_heads * (d_nope + d_v) * d_latent
    return {
        "cache_bytes": cache,
        "weight_bytes": weights,
        "total_bytes": cache + weights + q + out,
        "attn_flops": attn_flops,
        "flops": attn_flops + proj_flops,
        "query_tokens": n_q,
    }
