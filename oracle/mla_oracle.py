"""fp64 CPU oracle for Multi-head Latent Attention decode.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import or call this module. The product
path (the HIP library and its Python binding) never imports it, and this
module imports nothing from the product path: it takes plain NumPy arrays.

Sources (the pages are web write-ups of the DeepSeek-V3 technical report):

* [P1] "092 | DeepSeek-V3: model, numeric precision and communication under one
  cost budget" (wq-win.github.io), section 2 "MLA: cache the compressed
  history": each cached token keeps a 512-d joint KV latent c plus a 64-d
  decoupled RoPE key; the algebra check there gives the identity
  q_t^T (U c_s) = (U^T q_t)^T c_s with U in R^{d_h x d_c}, exact in exact
  arithmetic, and states that the RoPE branch is computed separately.
* [P3] "DeepSeek-V3" (ailearn.mscapital.top), the MLA paragraphs under the
  state-flow figures and the configuration table: 128 heads, KV rank 512,
  per-head non-positional q/k width 128, RoPE width 64, V width 128; the
  absorb order (q_nope x W_UK against every cached c_KV, the RoPE part
  multiplied separately and added; sum_j p_j c_KV,j first, then W_UV); the
  naive branch that expands K and V per head; cache element counts
  128x(128+128) = 32,768, 512+64 = 576 (98.24 % fewer), 128x(192+128) = 40,960.
* [P5] DeepSeek-V3 article at m.lsln.cn (news 222502), section 2.1 (decode
  attention softmax(Q_t K_{1:t}^T) V_{1:t}; MHA caches about 2 n_h d_h per
  token), section 2.2 (absorb W_UK into the query side and W_UV into the
  output side), section 2.3 (decoupled RoPE: q^R per head, k^R shared across
  heads).

Readings where the pages are silent or garbled:

* softmax scale: no page gives one; 1/sqrt(d_nope + d_rope) = 1/sqrt(192),
  the width of the per-head query/key each score is a dot product over.
* the decode path takes q_pe and k_R already rotated; only the cache-append
  producer below applies RoPE.
* RoPE (the pages name it, for the decoupled 64-d branch, without a formula):
  the rotary embedding's own definition, consecutive pairs (x_2i, x_2i+1)
  turned counter-clockwise by the angle pos * base^(-2i/64), base 10000, no
  length scaling (the pages name YaRN for 128K contexts but give no
  parameters).
* the appended latent is c_KV = W_DKV h exactly as the pages write it (no
  normalisation of c_KV), and k_R = RoPE(W_KR h) at the new token's position
  L - Sq + i.
* output projection: W_O in R^{7168 x 16384} maps the heads' outputs,
  concatenated head-major (index h * 128 + v), back to the model width.
* query side: the query is compressed to rank 1536 ([P3] configuration
  table): c_Q = W_DQ h (7168 -> 1536), then per head q = W_UQ[h] c_Q
  (1536 -> 192), rows 0..127 the non-positional part q_nope and rows
  128..191 the position part, rotated like k_R at the token's position:
  q_pe = RoPE(q[128:], L - Sq + i). No normalisation of c_Q (the pages give
  none).
* with Sq new tokens per sequence (all already in the cache, counted in L),
  query i sees cached positions j <= L - Sq + i; a row that sees no position
  (L < Sq, i < Sq - L) yields zeros (no page covers it).
* k_R is one 64-d key per token shared by every head ([P5] section 2.3).
* W_UK[h], W_UV[h] are [128, 512]: k = W_UK[h] c, v = W_UV[h] c.

The naive path (``naive_decode``) is the definition the method must equal: it
materialises per head K_h[j] = [W_UK[h] c_j ; k_R,j] and V_h[j] = W_UV[h] c_j
and runs a standard softmax attention. ``absorb_decode`` reorders the same
sums the way the pages describe; the tests hold the two together (the [P1]
identity) and pin both against closed forms, a library attention routine and
scalar brute force.

Parity pins: every function here is pinned by a test in tests/test_oracle.py,
except the behaviour on trained weights and real activation statistics, which
no page prints (parity unpinned for real-model numerics).
"""

from __future__ import annotations

import math

import numpy as np

# ----------------------------------------------------------------------------
# Dimensions of DeepSeek-V3's MLA ([P3] configuration table; [P5] section 5).
N_HEADS = 128
D_NOPE = 128
D_ROPE = 64
D_LATENT = 512
D_V = 128
ROW = D_LATENT + D_ROPE  # 576 cached elements per token ([P3]: 512 + 64)
D_HIDDEN = 7168          # model width ([P5] section 5 configuration skeleton)
ROPE_BASE = 10000.0      # reading: the rotary embedding's own base


def default_scale(d_nope: int = D_NOPE, d_rope: int = D_ROPE) -> float:
    """Softmax scale 1/sqrt(d_nope + d_rope) (reading: no page states it)."""
    return 1.0 / math.sqrt(d_nope + d_rope)


# ----------------------------------------------------------------------------
# Input decoding (no arithmetic of the method).

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp64: a bf16 pattern is the top half of an fp32 pattern."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gather_sequence(cache_bits: np.ndarray, table_row: np.ndarray, length: int,
                    block_size: int) -> np.ndarray:
    """Logical rows 0..length-1 of one sequence from the paged cache, as fp64.

    cache_bits: uint16 [num_blocks, block_size, 576]; table_row: int32 block ids.
    Row j lives in physical block table_row[j // block_size], slot j % block_size.
    """
    nblk = -(-length // block_size)
    blocks = cache_bits[np.asarray(table_row[:nblk], dtype=np.int64)]
    rows = blocks.reshape(nblk * block_size, cache_bits.shape[-1])[:length]
    return bf16_bits_to_f64(rows)


def visible_len(length: int, sq: int, i: int) -> int:
    """Number of cached positions query i (of sq new tokens) may attend to."""
    return length - sq + i + 1


# ----------------------------------------------------------------------------
# Naive path: materialise per-head K and V ([P3] naive branch; [P5] 2.1, 2.3).

def naive_scores(q_nope_h, q_pe_h, w_uk_h, c_kv, k_r, scale):
    """Scores of query rows (one head) against every given cached token.

    K_h[j] = [W_UK[h] c_j ; k_R,j] (192 wide), q_h = [q_nope ; q_pe];
    s_j = scale * q_h . K_h[j]. q_nope_h [..., 128], q_pe_h [..., 64] (one
    query or a block of them); returns [..., L].
    """
    k_nope = c_kv @ w_uk_h.T                                    # [L, 128]: W_UK[h] c_j per row
    k_full = np.concatenate([k_nope, k_r], axis=1)               # [L, 192]
    q_full = np.concatenate([q_nope_h, q_pe_h], axis=-1)         # [..., 192]
    return scale * (q_full @ k_full.T)


def softmax(s: np.ndarray) -> np.ndarray:
    """exp(s - max s) / sum: the standard softmax (the shift is exact in reals)."""
    e = np.exp(s - np.max(s))
    return e / np.sum(e)


def naive_decode(q_nope, q_pe, w_uk, w_uv, c_kv, k_r, scale, heads=None,
                 chunk: int = 8192):
    """Naive MLA decode of one sequence, fp64.

    q_nope [Sq, H, 128], q_pe [Sq, H, 64], w_uk / w_uv [H, 128, 512],
    c_kv [L, 512], k_r [L, 64]. Returns o [Sq, H, 128] (rows of heads not in
    ``heads`` are NaN). Tokens are processed in chunks so that no more than
    ``chunk`` rows of K_h, V_h exist at once.
    """
    sq, n_heads = q_nope.shape[0], q_nope.shape[1]
    length = c_kv.shape[0]
    heads = range(n_heads) if heads is None else heads
    out = np.full((sq, n_heads, w_uv.shape[1]), np.nan)
    for h in heads:
        # scores for all queries of this head; K_h chunk by chunk, each chunk
        # materialised once for every query row
        s = np.empty((sq, length))
        for t0 in range(0, length, chunk):
            t1 = min(length, t0 + chunk)
            s[:, t0:t1] = naive_scores(q_nope[:, h], q_pe[:, h], w_uk[h], c_kv[t0:t1], k_r[t0:t1], scale)
        p = np.zeros_like(s)
        for i in range(sq):
            n = visible_len(length, sq, i)
            if n > 0:               # a row that sees no position keeps p = 0: output 0
                p[i, :n] = softmax(s[i, :n])
        acc = np.zeros((sq, w_uv.shape[1]))
        for t0 in range(0, length, chunk):
            t1 = min(length, t0 + chunk)
            v = c_kv[t0:t1] @ w_uv[h].T              # V_h rows: W_UV[h] c_j
            acc += p[:, t0:t1] @ v
        out[:, h] = acc
    return out


# ----------------------------------------------------------------------------
# Absorb order ([P1] identity; [P3] absorb path; [P5] 2.2). Used only to pin
# the identity and as the algorithmic CPU baseline, never by the GPU path.

def absorb_query(q_nope, w_uk):
    """q_abs[i, h, :] = W_UK[h]^T q_nope[i, h, :]  (128 -> 512)."""
    return np.einsum("hnc,ihn->ihc", w_uk, q_nope, optimize=True)


def absorb_scores(q_abs, q_pe, c_kv, k_r, scale):
    """s[i, h, j] = scale * (q_abs[i,h] . c_j + q_pe[i,h] . k_R,j)."""
    return scale * (np.einsum("ihc,jc->ihj", q_abs, c_kv, optimize=True)
                    + np.einsum("ihr,jr->ihj", q_pe, k_r, optimize=True))


def absorb_decode(q_nope, q_pe, w_uk, w_uv, c_kv, k_r, scale, return_latent=False):
    """Absorb-order MLA decode of one sequence, fp64: q_abs, scores, softmax,
    o_lat = sum_j p_j c_j, then o = W_UV[h] o_lat."""
    sq = q_nope.shape[0]
    length = c_kv.shape[0]
    q_abs = absorb_query(q_nope, w_uk)
    s = absorb_scores(q_abs, q_pe, c_kv, k_r, scale)          # [Sq, H, L]
    p = np.zeros_like(s)
    for i in range(sq):
        n = visible_len(length, sq, i)
        if n <= 0:                  # a row that sees no position keeps p = 0: output 0
            continue
        e = np.exp(s[i, :, :n] - s[i, :, :n].max(axis=1, keepdims=True))
        p[i, :, :n] = e / e.sum(axis=1, keepdims=True)
    o_lat = np.einsum("ihj,jc->ihc", p, c_kv, optimize=True)
    o = np.einsum("hvc,ihc->ihv", w_uv, o_lat, optimize=True)
    return (o, o_lat) if return_latent else o


def absorb_partial(q_abs, q_pe, c_kv, k_r, scale, t0, t1, n_vis):
    """Softmax statistics of one query row over cached tokens [t0, t1) clipped
    to the first n_vis positions: (O = sum e^{s-m} c, m, l = sum e^{s-m}).
    An empty range gives (0, -inf, 0)."""
    t1 = min(t1, n_vis)
    if t1 <= t0:
        return np.zeros(c_kv.shape[1]), -np.inf, 0.0
    s = scale * (c_kv[t0:t1] @ q_abs + k_r[t0:t1] @ q_pe)
    m = float(np.max(s))
    e = np.exp(s - m)
    return e @ c_kv[t0:t1], m, float(np.sum(e))


def merge_partials(parts):
    """Log-sum-exp merge of (O, m, l) partials into the normalised o_lat."""
    m_all = max(m for _, m, _ in parts)
    num = sum(np.exp(m - m_all) * o for o, m, _ in parts if m > -np.inf)
    den = sum(np.exp(m - m_all) * l for _, m, l in parts if m > -np.inf)
    return num / den


# ----------------------------------------------------------------------------
# Scalar brute force for tiny shapes: plain Python loops, no BLAS.

def brute_force_decode(q_nope, q_pe, w_uk, w_uv, c_kv, k_r, scale):
    """Naive decode with nested Python loops (tiny dims only)."""
    sq, n_heads, d_nope = q_nope.shape
    d_rope = q_pe.shape[2]
    d_v, d_c = w_uv.shape[1], w_uv.shape[2]
    length = c_kv.shape[0]
    out = np.zeros((sq, n_heads, d_v))
    for i in range(sq):
        n = visible_len(length, sq, i)
        for h in range(n_heads):
            scores = []
            for j in range(n):
                acc = 0.0
                for a in range(d_nope):
                    k_a = 0.0
                    for c in range(d_c):
                        k_a += float(w_uk[h, a, c]) * float(c_kv[j, c])
                    acc += float(q_nope[i, h, a]) * k_a
                for r in range(d_rope):
                    acc += float(q_pe[i, h, r]) * float(k_r[j, r])
                scores.append(acc * scale)
            top = max(scores)
            weights = [math.exp(x - top) for x in scores]
            total = sum(weights)
            for v in range(d_v):
                val = 0.0
                for j in range(n):
                    vj = 0.0
                    for c in range(d_c):
                        vj += float(w_uv[h, v, c]) * float(c_kv[j, c])
                    val += weights[j] / total * vj
                out[i, h, v] = val
    return out


# ----------------------------------------------------------------------------
# Batch driver over the paged layout.

def decode_batch(q_nope_bits, q_pe_bits, w_uk_bits, w_uv_bits, cache_bits,
                 block_table, seq_lens, block_size, scale=None, sample=None,
                 path="naive"):
    """Oracle output for a paged batch.

    All floating inputs are bf16 bit patterns (uint16): q_nope [B, Sq, H, 128],
    q_pe [B, Sq, H, 64], w_uk / w_uv [H, 128, 512], cache [NB, block, 576].
    ``sample``: optional iterable of (b, h) pairs; only those are computed
    (other entries are NaN). Returns fp64 [B, Sq, H, 128].
    """
    scale = default_scale() if scale is None else scale
    w_uk = bf16_bits_to_f64(w_uk_bits)
    w_uv = bf16_bits_to_f64(w_uv_bits)
    n_b, sq, n_heads = q_nope_bits.shape[:3]
    out = np.full((n_b, sq, n_heads, w_uv.shape[1]), np.nan)
    by_seq = {}
    if sample is None:
        by_seq = {b: None for b in range(n_b)}
    else:
        for b, h in sample:
            by_seq.setdefault(int(b), []).append(int(h))
    d_c = w_uk.shape[2]
    for b, heads in sorted(by_seq.items()):
        rows = gather_sequence(cache_bits, block_table[b], int(seq_lens[b]), block_size)
        c_kv, k_r = rows[:, :d_c], rows[:, d_c:]
        qn = bf16_bits_to_f64(q_nope_bits[b])
        qp = bf16_bits_to_f64(q_pe_bits[b])
        if path == "naive":
            out[b] = naive_decode(qn, qp, w_uk, w_uv, c_kv, k_r, scale, heads=heads)
        else:
            hs = list(range(n_heads)) if heads is None else sorted(set(heads))
            out[b][:, hs] = absorb_decode(qn[:, hs], qp[:, hs], w_uk[hs], w_uv[hs],
                                          c_kv, k_r, scale)
    return out


# ----------------------------------------------------------------------------
# Cache sizes ([P3] cache counts; [P5] 2.1 "about 2 n_h d_h per token").

def cache_counts(n_heads=N_HEADS, d_nope=D_NOPE, d_rope=D_ROPE, d_latent=D_LATENT,
                 d_v=D_V):
    """Per-layer, per-token cache element counts of the three layouts."""
    mha = n_heads * (d_nope + d_v)                # K and V of every head
    mla = d_latent + d_rope                       # c_KV and the shared k_R
    naive = n_heads * (d_nope + d_rope + d_v)     # expanded 192-wide K plus V
    return {"mha": mha, "mla": mla, "naive": naive, "reduction": 1.0 - mla / mha}



# ----------------------------------------------------------------------------
# Cache-append producer ([P5] 2.2: c_t^KV = W^DKV h_t, the short joint latent
# each token caches; [P5] 2.3: the decoupled position branch keeps one small
# key k^R shared by all heads, rotated by RoPE; [P3] MLA paragraphs: per token
# and layer only c_KV in R^512 and the rotated k_R in R^64 are cached).

def rope_inv_freq(d_rope=D_ROPE, base=ROPE_BASE):
    """Angular frequency of pair i: base^(-2i/d_rope), i = 0 .. d_rope/2 - 1."""
    i = np.arange(d_rope // 2, dtype=np.float64)
    return base ** (-2.0 * i / d_rope)


def rope_rotate(x, pos, base=ROPE_BASE):
    """Rotary embedding of x [..., d] at integer positions pos (broadcast over
    the leading axes): pair (x_2i, x_2i+1) turns counter-clockwise by
    pos * theta_i, i.e. (x_2i cos - x_2i+1 sin, x_2i sin + x_2i+1 cos)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def append_rows(hidden, w_dkv, w_kr, positions, base=ROPE_BASE):
    """Cache rows of new tokens, fp64: [c_KV = W_DKV h ; k_R = RoPE(W_KR h, pos)].

    hidden [n, d_hidden], w_dkv [d_latent, d_hidden], w_kr [d_rope, d_hidden],
    positions [n] (each token's index in its sequence). Returns [n, d_latent +
    d_rope] in the cache's row order [c_KV | k_R]."""
    hidden = np.asarray(hidden, dtype=np.float64)
    c = hidden @ np.asarray(w_dkv, dtype=np.float64).T
    k = rope_rotate(hidden @ np.asarray(w_kr, dtype=np.float64).T, positions, base)
    return np.concatenate([c, k], axis=-1)


def append_positions(seq_lens, q_tokens):
    """Position of new token i of sequence b: L_b - Sq + i, as [B, Sq] (the new
    tokens are the last Sq of each sequence, counted in L_b)."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    return lens[:, None] - q_tokens + np.arange(q_tokens)[None, :]


def append_batch(hidden_bits, w_dkv_bits, w_kr_bits, seq_lens, q_tokens, base=ROPE_BASE):
    """Exact (fp64) rows the producer writes for a batch: hidden bf16 bits
    [B, Sq, d_hidden] -> [B, Sq, d_latent + d_rope]."""
    h = bf16_bits_to_f64(hidden_bits)
    n_b, sq, d_h = h.shape
    pos = append_positions(seq_lens, q_tokens)
    rows = append_rows(h.reshape(n_b * sq, d_h), bf16_bits_to_f64(w_dkv_bits),
                       bf16_bits_to_f64(w_kr_bits), pos.reshape(-1), base)
    return rows.reshape(n_b, sq, -1)


# ----------------------------------------------------------------------------
# Output projection (the last step of the attention block, [P3] MLA state
# flow: the attention output goes through an output projection matrix back to
# the model width).

def output_project(o, w_o):
    """y[t, :] = W_O concat_h(o[t, h, :]) for attention outputs o [n, H, d_v]
    (or already flat [n, H * d_v]) and W_O [d_model, H * d_v], fp64."""
    o = np.asarray(o, dtype=np.float64)
    flat = o.reshape(o.shape[0], -1)
    return flat @ np.asarray(w_o, dtype=np.float64).T


# ----------------------------------------------------------------------------
# Query side ([P3] configuration table: Q compression rank 1536, per-head
# non-positional width 128 and RoPE width 64; [P5] 2.3: a small per-head
# position query q^R, rotated like the shared k^R).

D_QRANK = 1536


def query_project(hidden, w_dq, w_uq, positions, base=ROPE_BASE, d_nope=D_NOPE, d_rope=D_ROPE):
    """q_nope [n, H, d_nope] and q_pe [n, H, d_rope] of new tokens, fp64.

    hidden [n, d_hidden], w_dq [d_q, d_hidden], w_uq [H, d_nope + d_rope, d_q],
    positions [n]."""
    hidden = np.asarray(hidden, dtype=np.float64)
    c_q = hidden @ np.asarray(w_dq, dtype=np.float64).T                  # [n, d_q]
    q = np.einsum("hrq,nq->nhr", np.asarray(w_uq, dtype=np.float64), c_q)  # [n, H, 192]
    q_nope = q[..., :d_nope]
    q_pe = rope_rotate(q[..., d_nope:], np.asarray(positions)[:, None], base)
    return q_nope, q_pe


def query_batch(hidden_bits, w_dq_bits, w_uq_bits, seq_lens, q_tokens, base=ROPE_BASE):
    """Exact q_nope [B, Sq, H, 128] and q_pe [B, Sq, H, 64] for a batch (bf16
    bit inputs; positions L_b - Sq + i)."""
    h = bf16_bits_to_f64(hidden_bits)
    n_b, sq, d_h = h.shape
    pos = append_positions(seq_lens, q_tokens).reshape(-1)
    qn, qp = query_project(h.reshape(n_b * sq, d_h), bf16_bits_to_f64(w_dq_bits),
                           bf16_bits_to_f64(w_uq_bits), pos, base)
    return qn.reshape(n_b, sq, *qn.shape[1:]), qp.reshape(n_b, sq, *qp.shape[1:])
