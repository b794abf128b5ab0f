// Shared definitions of the gfx950 MLA decode kernels: fixed dimensions,
// vector types, the workspace layout and the launchers each kernel file
// provides to the C ABI in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

// DeepSeek-V3 MLA dimensions ("DeepSeek-V3" page, configuration table).
constexpr int kHeads = 128;
constexpr int kDNope = 128;
constexpr int kDRope = 64;
constexpr int kDLat = 512;
constexpr int kDV = 128;
constexpr int kRow = kDLat + kDRope;    // 576 cached elements per token
constexpr int kRowBytes = kRow * 2;     // 1152
constexpr int kBlock = 64;              // tokens per cache block
constexpr int kDHidden = 7168;          // model width, input of the cache-append producer

// Work decomposition of the attention pass.
constexpr int kTileTok = 32;            // cached tokens per LDS tile
constexpr int kRowsPerWave = 32;        // query rows (heads) per wavefront
constexpr int kWaves = 4;               // wavefronts per workgroup
constexpr int kRowsPerWg = kRowsPerWave * kWaves;   // 128
constexpr int kMinChunk = 64;           // split granularity (one cache block)
constexpr int kMaxBatch = 1000000;      // keeps the plan's packed 21-bit counters exact
constexpr int kPlanWaves = 4;           // the plan fills the positions at most this many times over
constexpr int kPlanSortMax = 1024;      // batches up to this size get the searched, sorted plan
constexpr int kAbsorbGroups = kHeads * (kDLat / 128);   // absorb workgroups: (head, 128-wide latent block)
// q_abs (fp16) and q_pe enter the score products scaled by 2^-4: exact for
// both, and it moves fp16's overflow bound for q_abs from 65504 to 2^20 - 2^9.
// The softmax multiplies the scores back by 2^4 together with its scale.
constexpr float kQScale = 0.0625f;
constexpr float kQAbsMax = 1048064.0f;  // 65504 / kQScale

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// One split of one sequence: tokens [t_begin, t_end) of sequence b (whose
// effective length is len); its partial softmax state goes to slot `slot`.
// blk0 and blk1 are the cache blocks of its first two 64-token blocks (the
// plan resolves them, so the attention pass can fetch its first tiles
// without a block-table round trip; blk1 = blk0 when the split has one block).
// slot < 0 marks an unused entry of the work list. The list is [depth][positions]:
// the attention workgroup(s) of position p run entries (0, p), (1, p), ... up to
// the first unused one.
struct WorkItem {
  int b, t_begin, t_end, slot, len, blk0, blk1, pad;
};

// Per-sequence split summary written by the plan kernel: partial slots
// [base, base + count), and the effective length used by every kernel.
struct SeqInfo {
  int base, count, len, pad;
};

// Byte offsets of each region inside the caller's workspace.
struct Layout {
  size_t range, work, seqinfo, meta, qabs, part_o, part_lse, total;
  int max_chunks;   // capacity of the partial slots
  int positions;    // work-list positions: the split target rounded up to 8
  int depth;        // work-list entries per position
  int rows;         // B * Sq query rows
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Split target P: the number of work slots the plan fills at once (one
// workgroup each for Sq = 1, two for Sq = 2), i.e. one per CU.
inline int default_split_target(int n_cu, int q_tokens) {
  return q_tokens == 1 ? n_cu : n_cu / 2;
}

// one_round: the plan is limited to one round (max_rounds = 1), which with
// batch <= split_target always finds a searched plan of at most one item per
// slot; the work list then needs depth 1 and the partial states split_target
// slots.
inline Layout make_layout(int batch, int q_tokens, int max_seq_len, int split_target, bool one_round = false) {
  Layout L{};
  const int max_blocks = (max_seq_len + kBlock - 1) / kBlock;
  // items: at most kPlanWaves * P on the searched plan (at most kPlanWaves
  // rounds), P + B on the simple one (sum_b ceil(L_b / C) <= total / C + B
  // with C >= total / P, i.e. at most 1 + ceil(B / P) rounds); either way no
  // more than one per cache block
  L.positions = (split_target + 7) / 8 * 8;
  {
    const int simple_rounds = 1 + (batch + split_target - 1) / split_target;
    L.depth = one_round ? 1 : (simple_rounds > kPlanWaves ? simple_rounds : kPlanWaves);
  }
  long long cap = (long long)L.depth * split_target;
  long long by_len = (long long)batch * max_blocks;
  L.max_chunks = (int)(cap < by_len ? cap : by_len);
  if (L.max_chunks < 1) L.max_chunks = 1;
  L.rows = batch * q_tokens;
  const size_t rows_per_chunk = (size_t)q_tokens * kHeads;
  size_t off = 0;
  // range flags first, at a fixed offset: one int per absorb workgroup,
  // written on every call (1 = a q_abs value of its tile outside kQAbsMax)
  L.range = off;   off = align_up(off + sizeof(int) * kAbsorbGroups, 256);
  L.work = off;    off = align_up(off + sizeof(WorkItem) * (size_t)L.depth * L.positions, 256);
  L.seqinfo = off; off = align_up(off + sizeof(SeqInfo) * batch, 256);
  L.meta = off;    off = align_up(off + 64, 256);
  L.qabs = off;    off = align_up(off + (size_t)L.rows * kHeads * kDLat * 2, 256);
  L.part_o = off;   off = align_up(off + (size_t)L.max_chunks * rows_per_chunk * kDLat * 2, 256);
  L.part_lse = off; off = align_up(off + (size_t)L.max_chunks * rows_per_chunk * 4, 256);
  L.total = off;
  return L;
}

// ---- launchers (each returns hipGetLastError() of its launch)
// split plan + absorb product (one launch)
hipError_t launch_prep(const int32_t* seq_lens, const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                       int batch, int max_len, int split_target,
                       int max_rounds, int positions, int depth, int max_chunks, WorkItem* work, SeqInfo* seqinfo, int* meta,
                       const uint16_t* q_nope, const uint16_t* w_uk, _Float16* q_abs, int rows,
                       int* range_flags, hipStream_t stream);
struct AttnArgs {
  const uint16_t* cache;
  const int32_t* block_table;
  const uint16_t* q_pe;
  const _Float16* q_abs;
  const WorkItem* work;
  const SeqInfo* seqinfo;
  const int* meta;
  _Float16* part_o;   // [slot][Sq * 128 rows][512] normalised partial O
  float* part_lse;    // [slot][Sq * 128 rows] m + log2 l (log2 units), -inf if empty
  long long num_blocks;
  int max_blocks_per_seq;
  int q_tokens;
  int max_chunks;
  int positions;      // work-list positions (one workgroup each; two for Sq = 2)
  int depth;          // work-list entries per position
  float scale_log2;   // softmax scale * log2(e) / kQScale (the scores arrive scaled by kQScale)
};
hipError_t launch_attn(const AttnArgs& a, hipStream_t stream);

// Weight-stream products (wstream.h); every weight in the packed layout that
// launch_pack_weight writes (n % 32 == 0, k % 16 == 0, n * k * 2 bytes).
hipError_t launch_pack_weight(const uint16_t* w, uint16_t* packed, int n, int k, hipStream_t stream);

// output projection y = W_O x (three launches): x fp32 [rows][16384], W_O
// packed [7168][16384], y fp32 [rows][7168]
size_t oproj_workspace_bytes(int rows);
hipError_t launch_oproj(const float* x, const uint16_t* w_o, float* y, int rows, void* ws, hipStream_t stream);

// query side (three launches): q_nope / q_pe of the new tokens from h
size_t qproj_workspace_bytes(int rows);
hipError_t launch_qproj(const uint16_t* hidden, const uint16_t* w_dq, const uint16_t* w_uq,
                        const int32_t* seq_lens, uint16_t* q_nope, uint16_t* q_pe, int batch,
                        int q_tokens, double rope_base, void* ws, hipStream_t stream);

// decode-step prologue (three launches): the cache append and the query side
// of the same new tokens, W_DQ and [W_DKV; W_KR] streamed side by side
size_t prologue_workspace_bytes(int rows);
hipError_t launch_prologue(const uint16_t* hidden, const uint16_t* w_dq, const uint16_t* w_uq,
                           const uint16_t* w_kv, uint16_t* cache, const int32_t* block_table,
                           const int32_t* seq_lens, long long num_blocks, int max_blocks_per_seq,
                           uint16_t* q_nope, uint16_t* q_pe, int batch, int q_tokens, double rope_base, void* ws,
                           hipStream_t stream);

// cache-append producer (two launches): the new tokens' cache rows from h
// and the packed stacked weight [W_DKV; W_KR] ([576][7168])
size_t append_workspace_bytes(int rows);
hipError_t launch_append(const uint16_t* hidden, const uint16_t* w_kv, uint16_t* cache,
                         const int32_t* block_table, const int32_t* seq_lens, long long num_blocks,
                         int max_blocks_per_seq, int batch, int q_tokens, double rope_base, void* ws,
                         hipStream_t stream);
// naive path (two launches): per-head K, V materialised into the workspace
// (naive_workspace_bytes), then causal softmax attention over them
size_t naive_workspace_bytes(int batch, int max_len);
hipError_t launch_naive(const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk, const uint16_t* w_uv,
                        const uint16_t* cache, const int32_t* block_table, const int32_t* seq_lens, float* out,
                        long long num_blocks, int batch, int q_tokens, int max_blocks_per_seq, int max_len,
                        float scale, void* ws, hipStream_t stream);

hipError_t launch_merge(const _Float16* part_o, const float* part_lse, const SeqInfo* seqinfo,
                        const uint16_t* w_uv, float* out, int batch, int q_tokens, int max_chunks,
                        hipStream_t stream);

}  // namespace mla
