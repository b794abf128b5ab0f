/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) Multi-head Latent Attention
 * decode library, absorbed path.
 *
 * What it computes. DeepSeek-V3's MLA caches, per layer and per token, only a
 * 512-d joint KV latent c_KV and a 64-d decoupled RoPE key k_R that all heads
 * share ("DeepSeek-V3" page at ailearn.mscapital.top, MLA section and its
 * configuration table; m.lsln.cn article, sections 2.2 and 2.3). For a decode
 * step the library computes, for every sequence b, new-token row i and head h:
 *
 *   q_abs = W_UK[h]^T q_nope[b,i,h]                          (128 -> 512)
 *   s_j   = scale * (q_abs . c_KV,j + q_pe[b,i,h] . k_R,j)    j visible to (b,i)
 *   p     = softmax_j(s)
 *   o_lat = sum_j p_j c_KV,j                                   (512)
 *   out[b,i,h] = W_UV[h] o_lat                                 (512 -> 128)
 *
 * i.e. the absorb order of the identity q^T (U c) = (U^T q)^T c given in the
 * algebra check of section 2 of the wq-win.github.io DeepSeek-V3 notes: the
 * per-head keys and values are never materialised. It equals, up to rounding,
 * softmax attention with K_h = [W_UK[h] c ; k_R] and V_h = W_UV[h] c.
 *
 * Visibility: seq_lens[b] = L_b counts every cached token of sequence b,
 * including its q_tokens new ones; new-token row i (0-based) sees positions
 * j <= L_b - q_tokens + i (itself and everything before it). A row that sees
 * no position (L_b < q_tokens) yields zeros.
 *
 * Fixed dimensions (checked at init): 128 heads, d_nope 128, d_rope 64,
 * d_latent 512, d_v 128, cache block 64 tokens, q_tokens 1 or 2.
 *
 * Data layouts (all row-major, all device memory, all borrowed):
 *   q_nope   bf16  [B, Sq, 128 heads, 128]
 *   q_pe     bf16  [B, Sq, 128 heads, 64]       already rotated
 *   w_uk     bf16  [128 heads, 128 (nope), 512 (latent)]   k_nope = W_UK[h] c
 *   w_uv     bf16  [128 heads, 128 (v), 512 (latent)]      v      = W_UV[h] c
 *   kv_cache bf16  [num_blocks, 64, 576]  each row = c_KV (512) | k_R (64),
 *                  k_R already rotated; logical token j of sequence b lives in
 *                  block block_table[b, j / 64], slot j % 64
 *   block_table int32 [B, max_blocks_per_seq]; entries past ceil(L_b/64) unread
 *   seq_lens    int32 [B]   (device memory; read only by the kernels)
 *   out         fp32  [B, Sq, 128 heads, 128]
 * Slots of a block past L_b may hold anything (NaN included): they are never
 * used. Every pointer must be 16-byte aligned.
 *
 * Numerics: bf16 inputs are consumed exactly. The absorbed query and the
 * softmax probabilities are rounded to fp16 and the latent tile is converted
 * bf16 -> fp16 for the matrix-core products. q_pe . k_R runs in bf16.
 * Accumulation, the softmax and the split merge are fp32; out is fp32.
 * Range rules of the fp16 operands (no page states value ranges; these are
 * preconditions of this implementation):
 *  - c_KV: converted exactly while |c_KV| <= 65504; a larger magnitude
 *    saturates to +-65504 (round toward zero), silently.
 *  - q_abs: stored as fp16 after an exact scaling by 2^-4 (q_pe gets the same
 *    scaling; the softmax scale undoes it), so |q_abs| <= 1048064 stays
 *    finite. A larger (or non-finite) value is detected: the call still
 *    returns MLA_OK (it never synchronises), the output may be inf/NaN, and
 *    mla_decode_range_flags reports MLA_RANGE_QABS for that workspace.
 *
 * Errors: every call returns an int status (MLA_OK = 0 or a negative code);
 * no C++ exception crosses the ABI. Faults inside kernels surface at the
 * caller's next synchronisation of the stream.
 *
 * Threading: a context is immutable after init; mla_decode_run may be called
 * concurrently on different streams as long as each call has its own
 * workspace.
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mla_decode_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,     /* null pointer, non-positive size, Sq not 1/2 */
  MLA_ERR_UNSUPPORTED = -2,     /* dims other than the compiled set, not gfx950 */
  MLA_ERR_MISALIGNED = -3,      /* a pointer not 16-byte aligned */
  MLA_ERR_WORKSPACE = -4,       /* workspace null or smaller than required */
  MLA_ERR_HIP = -5,             /* a HIP runtime call or launch failed */
  MLA_ERR_PRECONDITION = -6,    /* inputs break a documented precondition:
                                   mla_decode_check_inputs, or any entry point
                                   of the debug build (below) */
};

typedef struct mla_decode_config {
  int32_t num_heads;     /* 128 */
  int32_t d_nope;        /* 128 */
  int32_t d_rope;        /* 64 */
  int32_t d_latent;      /* 512 */
  int32_t d_v;           /* 128 */
  int32_t block_size;    /* 64 */
  int32_t max_q_tokens;  /* 1 or 2 */
  float softmax_scale;   /* <= 0 selects 1/sqrt(d_nope + d_rope) */
  int32_t split_target;  /* attention work slots that run at once (each is one
                            workgroup for Sq = 1, two for Sq = 2); the plan
                            cuts the batch into at most 4 rounds of them.
                            0 = one per compute unit (Sq = 1) or per two
                            (Sq = 2) */
} mla_decode_config;

typedef struct mla_decode_args {
  const void* q_nope;         /* bf16 [B, Sq, H, 128] */
  const void* q_pe;           /* bf16 [B, Sq, H, 64] */
  const void* w_uk;           /* bf16 [H, 128, 512] */
  const void* w_uv;           /* bf16 [H, 128, 512] */
  const void* kv_cache;       /* bf16 [num_blocks, 64, 576] */
  const int32_t* block_table; /* int32 [B, max_blocks_per_seq] */
  const int32_t* seq_lens;    /* int32 [B] */
  float* out;                 /* fp32 [B, Sq, H, 128] */
  int64_t num_blocks;         /* blocks in kv_cache */
  int32_t batch;              /* 1 <= B <= 1000000 */
  int32_t q_tokens;           /* Sq: 1 or 2, <= max_q_tokens */
  int32_t max_blocks_per_seq; /* row stride of block_table */
  int32_t max_seq_len;        /* host upper bound on every L_b;
                                 <= 64 * max_blocks_per_seq */
} mla_decode_args;

typedef struct mla_decode_ctx mla_decode_ctx;

/* Validate cfg against the compiled dimensions, check that `hip_device` is a
 * gfx950 GPU, and read its compute-unit count. Host only: no device memory is
 * allocated and nothing is launched. On success *out owns a small host object
 * released by mla_decode_destroy. */
int mla_decode_init(const mla_decode_config* cfg, int hip_device, mla_decode_ctx** out);

/* Bytes of device workspace mla_decode_run needs for a call with this batch,
 * q_tokens and max_seq_len. Pure host arithmetic. */
int mla_decode_workspace_size(const mla_decode_ctx* ctx, int32_t batch, int32_t q_tokens,
                              int32_t max_seq_len, size_t* bytes);

/* Enqueue one decode step on `stream` (a hipStream_t; NULL = default stream):
 * the split plan, the absorb product, the fused score / softmax / latent
 * accumulation over the paged cache, and the split merge with the W_UV
 * product. Never allocates, never synchronises. `workspace` is caller-owned
 * device memory of at least mla_decode_workspace_size bytes, 256-byte aligned,
 * and must not be shared by calls that may overlap. */
int mla_decode_run(const mla_decode_ctx* ctx, const mla_decode_args* args, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Host-side check of the preconditions on the decode inputs, on HOST copies
 * of seq_lens (int32 [batch]) and block_table (int32 [batch,
 * max_blocks_per_seq], row-major) with the same meaning as in
 * mla_decode_args. The layout it checks is the paged cache above: token j of
 * sequence b is row j % 64 of physical block block_table[b, j / 64]
 * ("DeepSeek-V3" page at ailearn.mscapital.top, MLA section: each cached
 * token is one 512 + 64 wide row). It requires, per sequence b:
 *   - 0 <= L_b <= max_seq_len;
 *   - block_table[b, k] in [0, num_blocks) for every block k < ceil(L_b / 64)
 *     the sequence uses (entries past them are not read), no two of them equal;
 *   - the rows of its new tokens (positions max(0, L_b - q_tokens) .. L_b - 1)
 *     in slots no other sequence's new tokens use. Blocks may be shared
 *     between sequences (a common prefix); a new token's row may not.
 * Returns MLA_OK, MLA_ERR_PRECONDITION with *first_bad = the lowest-numbered
 * sequence that breaks one (for a shared new-token slot: every sequence of
 * the group but the lowest-numbered one), or MLA_ERR_INVALID_ARG (NULL
 * arrays, batch outside 1..1000000, q_tokens < 1, max_blocks_per_seq < 1,
 * max_seq_len outside 1..64 * max_blocks_per_seq, num_blocks < 1, or host
 * memory too short for the check's lists of blocks and slots).
 * *first_bad is -1 unless the status is MLA_ERR_PRECONDITION; first_bad may
 * be NULL. Reads only seq_lens[0..batch) and, of row b, the entries the
 * sequence uses. Pure host code: no GPU needed, no context, thread-safe.
 *
 * The release kernels never read outside the cache for any input (a block id
 * out of range is clamped to [0, num_blocks), a length to [0, max_seq_len]);
 * such inputs give unspecified results. The debug build (libmla_decode_debug.so:
 * the same kernels, compiled with MLA_DEBUG_CHECKS) instead copies seq_lens
 * and block_table to the host and runs this check at the start of
 * mla_decode_run, mla_decode_run_profiled, mla_decode_run_noalloc,
 * mla_cache_append and mla_naive_run (max_seq_len = 64 * max_blocks_per_seq
 * for the append), returning MLA_ERR_PRECONDITION before any launch. Those
 * calls then synchronise `stream` and allocate host memory, so the debug
 * build is not for graph capture or tight loops. */
int mla_decode_check_inputs(const int32_t* seq_lens, const int32_t* block_table, int32_t batch,
                            int32_t q_tokens, int32_t max_blocks_per_seq, int32_t max_seq_len,
                            int64_t num_blocks, int32_t* first_bad);

/* mla_decode_run, plus timing marks for measurement tools: records the
 * hipEvent_t handles events[0] and events[1] before the preparation launch
 * (split plan and absorb product), events[2] before the attention pass,
 * events[3] before the merge and W_UV product and events[4] after it, so
 * hipEventElapsedTime(events[i], events[i+1]) is a stage's duration (stage 0
 * is empty). NULL entries are skipped. Same arguments, errors and results as
 * mla_decode_run. */
int mla_decode_run_profiled(const mla_decode_ctx* ctx, const mla_decode_args* args,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const events[5]);

/* mla_decode_run without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The workspace is a 66 MiB array inside the
 * library, one per GPU (the GPU holds it while the library is loaded); the
 * call allocates nothing, launches the same kernels on `stream` and never
 * synchronises. Its split plan is limited to one round (at most one work item
 * per attention slot), so it requires batch <= the split target (by default
 * the compute-unit count for q_tokens = 1, half of it for q_tokens = 2) and a
 * workspace layout within 66 MiB: about B * Sq * 128 KB of absorbed queries
 * plus 128 KB * Sq per attention slot of partial states, which covers every
 * batch of up to 256 sequences (Sq = 1) or 128 (Sq = 2) on a 256-CU GPU.
 * Anything larger returns MLA_ERR_WORKSPACE before any launch. Every call on
 * a GPU uses that GPU's one array (calls that may overlap on one GPU race,
 * whatever their streams); nothing in it needs clearing between calls. Same
 * arguments, results (up to rounding: the plan may cut the history
 * differently) and other errors as mla_decode_run. */
int mla_decode_run_noalloc(const mla_decode_ctx* ctx, const mla_decode_args* args, void* stream);

/* Range flags of the last decode call that used `workspace` (the q_abs rule
 * under Numerics above): enqueues a 2 KB device-to-host copy of the flags
 * region at the start of the workspace on `stream`, synchronises that stream
 * and sets *flags to 0 or MLA_RANGE_QABS. Call it after mla_decode_run on the
 * same stream; it is a debugging aid, not needed for a correct result.
 * Errors: MLA_ERR_INVALID_ARG (NULL ctx or flags), MLA_ERR_WORKSPACE (NULL,
 * misaligned or under 2 KB), MLA_ERR_HIP. */
#define MLA_RANGE_QABS 1
int mla_decode_range_flags(const mla_decode_ctx* ctx, const void* workspace, size_t workspace_bytes,
                           void* stream, int32_t* flags);

/* ---- Packed weights of the projections -----------------------------------
 *
 * The projections below (cache append, query side, output projection) are
 * weight streams: for a decode batch every weight byte is used by only a few
 * dozen tokens, so they are bound by reading the weights from HBM. They take
 * their weights in a packed layout, made once per weight (at load time) by
 * mla_pack_weight from the row-major matrix W [n][k] (bf16):
 *   the 1 KB block of column tile ct (rows 32 ct .. 32 ct + 31 of W) and
 *   k-step ks (columns 16 ks .. 16 ks + 15) sits at byte (ks * n/32 + ct) *
 *   1024; within it, 16-byte lane piece l (l = 0..63) holds
 *   W[32 ct + l % 32][16 ks + 8 (l / 32) .. 16 ks + 8 (l / 32) + 7].
 * That is the operand fragment order of the 32x32x16 bf16 matrix
 * instructions, so every load of the stream is one contiguous 1 KB. The
 * packed matrix has the same size, n * k * 2 bytes; it is a permutation of
 * the bytes (packing is exact).
 *
 * `w` and `packed`: device memory, borrowed, 16-byte aligned, not
 * overlapping; n % 32 == 0, k % 16 == 0, n * k <= 2^33. One kernel on
 * `stream`, no allocation, no synchronisation. Errors: MLA_ERR_INVALID_ARG
 * (NULL, shape, overlap), MLA_ERR_MISALIGNED, MLA_ERR_HIP. */
int mla_pack_weight(const mla_decode_ctx* ctx, const void* w, void* packed, int32_t n, int32_t k,
                    void* stream);

/* ---- Cache-append producer ------------------------------------------------
 *
 * Writes the cache rows of a decode step's new tokens: per token the short
 * joint latent c_KV = W_DKV h (7168 -> 512) and the head-shared position key
 * k_R = RoPE(W_KR h, pos) (7168 -> 64) ("DeepSeek-V3" article at m.lsln.cn,
 * sections 2.2 and 2.3: c_t^KV = W^DKV h_t, and a small decoupled key k^R
 * shared by the heads that carries the rotary position). New token i of
 * sequence b sits at pos = seq_lens[b] - q_tokens + i (the same counting as
 * mla_decode_run) and is stored, as bf16 rounded to nearest (ties to even),
 * in block block_table[b, pos / 64], slot pos % 64, as [c_KV | k_R].
 *
 * RoPE: consecutive pairs (x_2i, x_2i+1) of W_KR h turn counter-clockwise by
 * the angle pos * rope_base^(-2i/64), i = 0..31 (the pages name the rotary
 * embedding without a formula; this is its own definition, no length
 * scaling). Angles are formed in fp64.
 *
 * Layouts (device memory, borrowed, 16-byte aligned):
 *   hidden   bf16 [B, Sq, 7168] row-major
 *   w_kv     the stacked weight [W_DKV; W_KR] (576 x 7168: rows 0..511 are
 *            W_DKV, rows 512..575 W_KR) packed by mla_pack_weight
 *   kv_cache bf16 [num_blocks, 64, 576]: only the new tokens' rows are written;
 *            a token whose position or block id is out of range is skipped
 * Numerics: bf16 products exact, fp32 accumulation, one rounding to bf16 of
 * the finished value (the result is within one bf16 step of the exact one).
 * The call enqueues two kernels on `stream`, never allocates or
 * synchronises; `workspace` (fp32 partial sums, mla_cache_append_workspace_size
 * bytes, 256-byte aligned) must not be shared by overlapping calls. Errors as
 * for mla_decode_run. */
typedef struct mla_append_args {
  const void* hidden;          /* bf16 [B, Sq, 7168] */
  const void* w_kv;            /* packed [W_DKV; W_KR], 576 x 7168 */
  void* kv_cache;              /* bf16 [num_blocks, 64, 576]; rows written */
  const int32_t* block_table;  /* int32 [B, max_blocks_per_seq] */
  const int32_t* seq_lens;     /* int32 [B], counting the new tokens */
  int64_t num_blocks;          /* blocks in kv_cache */
  int32_t batch;               /* 1 <= B <= 1000000 */
  int32_t q_tokens;            /* Sq: 1 or 2, <= max_q_tokens */
  int32_t max_blocks_per_seq;  /* row stride of block_table */
  float rope_base;             /* <= 0 selects 10000 */
} mla_append_args;

/* Bytes of workspace mla_cache_append needs for B * Sq new tokens. */
int mla_cache_append_workspace_size(const mla_decode_ctx* ctx, int32_t batch, int32_t q_tokens,
                                    size_t* bytes);

/* Enqueue the cache-append producer for one decode step (see above). */
int mla_cache_append(const mla_decode_ctx* ctx, const mla_append_args* args, void* workspace,
                     size_t workspace_bytes, void* stream);

/* ---- Query side ------------------------------------------------------------
 *
 * The decode's queries from the new tokens' hidden states: the query is
 * compressed to rank 1536 and each head carries 128 non-positional and 64
 * position dimensions ("DeepSeek-V3" page at ailearn.mscapital.top,
 * configuration table); the small per-head position query is rotated like
 * the shared position key ("DeepSeek-V3" article at m.lsln.cn, section 2.3):
 *   c_Q = W_DQ h (7168 -> 1536);  q[h] = W_UQ[h] c_Q (1536 -> 192)
 *   q_nope[h] = q[h][0..127];  q_pe[h] = RoPE(q[h][128..191], pos)
 * with pos = seq_lens[b] - q_tokens + i and the RoPE of mla_cache_append. The
 * outputs are exactly mla_decode_run's q_nope and q_pe inputs.
 *
 * Layouts (device memory, borrowed, 16-byte aligned):
 *   hidden  bf16 [B, Sq, 7168] row-major
 *   w_dq    W_DQ (1536 x 7168) packed by mla_pack_weight
 *   w_uq    W_UQ (24576 x 1536: head h's 192 rows at 192 h, 128
 *           non-positional rows, then 64 position rows) packed by
 *           mla_pack_weight
 *   q_nope  bf16 [B, Sq, 128, 128] written (rounded to nearest, ties to even)
 *   q_pe    bf16 [B, Sq, 128, 64]  written
 * Numerics: bf16 products exact, fp32 accumulation; c_Q is kept in fp32 and
 * enters the second product as hi + lo bf16 halves. Three kernels on `stream`;
 * `workspace` (mla_query_project_workspace_size bytes, 256-byte aligned)
 * holds the partial sums and c_Q. Errors as for mla_decode_run. */
typedef struct mla_query_args {
  const void* hidden;         /* bf16 [B, Sq, 7168] */
  const void* w_dq;           /* packed W_DQ, 1536 x 7168 */
  const void* w_uq;           /* packed W_UQ, 24576 x 1536 */
  const int32_t* seq_lens;    /* int32 [B], counting the new tokens */
  void* q_nope;               /* bf16 [B, Sq, 128, 128], written */
  void* q_pe;                 /* bf16 [B, Sq, 128, 64], written */
  int32_t batch;              /* 1 <= B <= 1000000 */
  int32_t q_tokens;           /* Sq: 1 or 2, <= max_q_tokens */
  float rope_base;            /* <= 0 selects 10000 */
} mla_query_args;

int mla_query_project_workspace_size(const mla_decode_ctx* ctx, int32_t batch, int32_t q_tokens,
                                     size_t* bytes);

int mla_query_project(const mla_decode_ctx* ctx, const mla_query_args* args, void* workspace,
                      size_t workspace_bytes, void* stream);

/* ---- Decode-step prologue: cache append and query side together -----------
 *
 * mla_cache_append and mla_query_project for the same new tokens in one call:
 * W_DQ and [W_DKV; W_KR] both read the hidden states h, so they are streamed
 * side by side in one product and one split sum finishes both (c_Q for the
 * second query product, the cache rows). Results: the cache rows of
 * mla_cache_append and the q_nope / q_pe of mla_query_project, with the same
 * bounds (the compressed query's fp32 sums are split differently, so a q
 * value can differ from mla_query_project's in its last bit). Three kernels
 * on `stream` instead of five; the arguments and layouts are those of the two
 * calls. Errors as for mla_decode_run. */
typedef struct mla_prologue_args {
  const void* hidden;          /* bf16 [B, Sq, 7168] */
  const void* w_dq;            /* packed W_DQ, 1536 x 7168 */
  const void* w_uq;            /* packed W_UQ, 24576 x 1536 */
  const void* w_kv;            /* packed [W_DKV; W_KR], 576 x 7168 */
  void* kv_cache;              /* bf16 [num_blocks, 64, 576]; the new tokens' rows written */
  const int32_t* block_table;  /* int32 [B, max_blocks_per_seq] */
  const int32_t* seq_lens;     /* int32 [B], counting the new tokens */
  void* q_nope;                /* bf16 [B, Sq, 128, 128], written */
  void* q_pe;                  /* bf16 [B, Sq, 128, 64], written */
  int64_t num_blocks;          /* blocks in kv_cache */
  int32_t batch;               /* 1 <= B <= 1000000 */
  int32_t q_tokens;            /* Sq: 1 or 2, <= max_q_tokens */
  int32_t max_blocks_per_seq;  /* row stride of block_table */
  float rope_base;             /* <= 0 selects 10000 */
} mla_prologue_args;

int mla_project_new_tokens_workspace_size(const mla_decode_ctx* ctx, int32_t batch, int32_t q_tokens,
                                          size_t* bytes);

int mla_project_new_tokens(const mla_decode_ctx* ctx, const mla_prologue_args* args, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---- Output projection -----------------------------------------------------
 *
 * y[t, :] = W_O x_t: the attention outputs of token t (the `out` of
 * mla_decode_run, 128 heads x 128, concatenated head-major: index h * 128 + v)
 * mapped back to the model width 7168 by one output projection matrix
 * ("DeepSeek-V3" page at ailearn.mscapital.top, MLA state flow).
 *
 * Layouts (device memory, borrowed, 16-byte aligned):
 *   x    fp32 [rows, 16384] row-major (mla_decode_run's out viewed as
 *        [B * Sq, 16384])
 *   w_o  W_O (7168 x 16384) packed by mla_pack_weight
 *   y    fp32 [rows, 7168]       written
 * Numerics: x enters the bf16 matrix cores as x = hi + lo (hi = bf16(x), lo =
 * bf16(x - hi), together within 2^-17 of x); products are accumulated in fp32
 * and the four K-splits added in a fixed order. Three kernels on `stream`, no
 * allocation, no synchronisation; `workspace` (the packed input and the
 * partial sums, mla_output_project_workspace_size bytes, 256-byte aligned)
 * must not be shared by overlapping calls. Errors as for mla_decode_run. */
typedef struct mla_oproj_args {
  const float* x;    /* fp32 [rows, 16384] */
  const void* w_o;   /* packed W_O, 7168 x 16384 */
  float* y;          /* fp32 [rows, 7168] */
  int32_t rows;      /* tokens, 1 <= rows <= 2000000 */
} mla_oproj_args;

int mla_output_project_workspace_size(const mla_decode_ctx* ctx, int32_t rows, size_t* bytes);

int mla_output_project(const mla_decode_ctx* ctx, const mla_oproj_args* args, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ---- Naive path (materialised keys and values; prefill) -------------------
 *
 * The same attention as mla_decode_run, computed the other way round: per
 * head the keys K_h[j] = [W_UK[h] c_j ; k_R,j] (192 wide) and values
 * V_h[j] = W_UV[h] c_j (128) are materialised from the latent cache, then a
 * standard softmax attention runs over them ("DeepSeek-V3" page at
 * ailearn.mscapital.top, MLA paragraphs: the naive branch, which expands the
 * per-token cache to 128 x (192 + 128) = 40,960 elements; "DeepSeek-V3"
 * article at m.lsln.cn, section 2.1). Any number of query tokens: with
 * q_tokens = L every prompt token is a query (prefill, causal, quadratic in
 * L). Visibility, scale and the zero rule are those of mla_decode_run (row i
 * of sequence b sees positions j <= L_b - q_tokens + i; L_b is clamped to
 * [0, max_seq_len]).
 *
 * Layouts (device memory, borrowed, 16-byte aligned):
 *   q_nope, q_pe, kv_cache, block_table, seq_lens, out as for mla_decode_run,
 *            with any q_tokens in [1, max_seq_len]
 *   w_uk, w_uv  W_UK and W_UV ([128, 128, 512] each, viewed as 16384 x 512)
 *            packed by mla_pack_weight
 * Workspace (mla_naive_workspace_size bytes, 256-byte aligned): the
 * materialised keys and values, B * ceil(max_seq_len / 64) tiles of 4,104 KiB
 * (K_nope in bf16, V in fp16, k_R once per tile), i.e. 64 KiB + 128 B per
 * token against the latent cache's 1,152 B.
 * Numerics: K_nope and V are rounded once (bf16, fp16) from fp32 sums;
 * q . K on bf16 matrix cores, the softmax in fp32, P in fp16 against V on fp16
 * matrix cores, fp32 accumulation. |V| must stay within fp16's range (65504).
 * Two kernels on `stream`, no allocation, no synchronisation. Errors as for
 * mla_decode_run. */
typedef struct mla_naive_args {
  const void* q_nope;          /* bf16 [B, Sq, 128, 128] */
  const void* q_pe;            /* bf16 [B, Sq, 128, 64] */
  const void* w_uk;            /* packed W_UK, 16384 x 512 */
  const void* w_uv;            /* packed W_UV, 16384 x 512 */
  const void* kv_cache;        /* bf16 [num_blocks, 64, 576] */
  const int32_t* block_table;  /* int32 [B, max_blocks_per_seq] */
  const int32_t* seq_lens;     /* int32 [B] */
  float* out;                  /* fp32 [B, Sq, 128, 128] */
  int64_t num_blocks;
  int32_t batch;               /* 1 <= B <= 1000000 */
  int32_t q_tokens;            /* 1 <= Sq <= max_seq_len */
  int32_t max_blocks_per_seq;  /* >= ceil(max_seq_len / 64) */
  int32_t max_seq_len;         /* 1 <= max_seq_len <= 2^20, bounds every L_b */
} mla_naive_args;

int mla_naive_workspace_size(const mla_decode_ctx* ctx, int32_t batch, int32_t max_seq_len, size_t* bytes);

int mla_naive_run(const mla_decode_ctx* ctx, const mla_naive_args* args, void* workspace,
                  size_t workspace_bytes, void* stream);

/* Release a context (NULL is accepted). */
void mla_decode_destroy(mla_decode_ctx* ctx);

/* Static, human-readable text for a status code. */
const char* mla_decode_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
