// Query side of a decode step: from the new tokens' hidden states h to the
// per-head queries the decode consumes,
//   c_Q  = W_DQ h                      (7168 -> 1536, the compressed query)
//   q[h] = W_UQ[h] c_Q                 (1536 -> 192 per head)
//   q_nope[h] = q[h][0 .. 127],  q_pe[h] = RoPE(q[h][128 .. 191], pos)
// with pos = L_b - Sq + i, the token's position (the same rotation as its
// cached k_R). The query is compressed to rank 1536 and each head carries
// 128 non-positional and 64 position dimensions ("DeepSeek-V3" page,
// ailearn.mscapital.top, configuration table); the small position query is
// rotated like the shared position key ("DeepSeek-V3" article at m.lsln.cn,
// section 2.3).
//
// Three launches on the caller's stream (weight-stream products, wstream.h),
// all deterministic:
//  1. stream W_DQ: 16 column blocks of 96 x 16 K-splits = 256 workgroups,
//     each wavefront with all its 7 k-steps (3 column tiles each) in flight
//     at once (h read from its rows, once per 3 column tiles), partial sums
//     per split;
//  2. the splits added in split order; c_Q (fp32) is written straight into
//     the packed input layout of the second product;
//  3. stream W_UQ: 256 column blocks of 96, one split (each wavefront 24
//     k-steps); c_Q enters as fp32 hi + lo. Its epilogue (rows.h) finishes
//     the heads.
// The decode-step prologue (mla_project_new_tokens) runs the cache append on
// the same stream: W_DQ and [W_DKV; W_KR] both read h, so launch 1 streams
// both weights side by side (22 column blocks of 96 x 8 K-splits = 176
// workgroups, each wavefront with all its 14 k-steps in flight) and launch 2
// routes the columns past 1536 to the cache rows. The tilings of launch 1
// were chosen by measurement (a sweep of column tiles, splits and ring
// depths at 32 tokens); with 8 splits here and 16 in the query side alone,
// the two calls' c_Q sums differ in order, i.e. in the last bit.
#include "rows.h"
#include "wstream.h"

namespace mla {

namespace {

using rows::kQRank;
using rows::kQUp;
using QDownPlan = ws::Plan<false, kQRank, kDHidden, 3, 7, 16, true>;
using ProloguePlan = ws::Plan<false, kQRank + kRow, kDHidden, 3, 14, 8, true>;   // [W_DQ | W_KV] columns
using QUpPlan = ws::Plan<true, kQUp, kQRank, 3, 4, 1>;

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

// columns [0, 1536) -> packed c_Q; [1536, 2112) -> the token's cache row
struct PrologueEpi {
  ws::StorePackedF32 c_q;
  rows::CacheRowEpi cache;
  __device__ void operator()(int r, int c, f32x4 v) const {
    if (c < kQRank)
      c_q(r, c, v);
    else
      cache(r, c - kQRank, v);
  }
};

}  // namespace

size_t qproj_workspace_bytes(int rows) {
  return round256(QDownPlan::part_bytes(rows)) + round256(QUpPlan::packed_x_bytes(rows));
}

hipError_t launch_qproj(const uint16_t* hidden, const uint16_t* w_dq, const uint16_t* w_uq,
                        const int32_t* seq_lens, uint16_t* q_nope, uint16_t* q_pe, int batch,
                        int q_tokens, double rope_base, void* ws, hipStream_t stream) {
  const int rows = batch * q_tokens;
  float* part = (float*)ws;
  char* cq = (char*)ws + round256(QDownPlan::part_bytes(rows));
  // c_Q rows past the batch in its last row tile are not written: a matrix
  // product keeps tokens apart, so they only reach output rows that the
  // epilogue never stores
  const hipError_t e = QDownPlan::run(hidden, w_dq, part, rows, ws::StorePackedF32{cq, kQRank / 16}, stream);
  if (e != hipSuccess) return e;
  return QUpPlan::run(cq, w_uq, nullptr, rows, rows::HeadsEpi{seq_lens, q_nope, q_pe, q_tokens, rows::RopeFreq::make(rope_base)},
                      stream);
}

size_t prologue_workspace_bytes(int rows) {
  return round256(ProloguePlan::part_bytes(rows)) + round256(QUpPlan::packed_x_bytes(rows));
}

hipError_t launch_prologue(const uint16_t* hidden, const uint16_t* w_dq, const uint16_t* w_uq,
                           const uint16_t* w_kv, uint16_t* cache, const int32_t* block_table,
                           const int32_t* seq_lens, long long num_blocks, int max_blocks_per_seq,
                           uint16_t* q_nope, uint16_t* q_pe, int batch, int q_tokens, double rope_base, void* ws,
                           hipStream_t stream) {
  const int rows = batch * q_tokens;
  float* part = (float*)ws;
  char* cq = (char*)ws + round256(ProloguePlan::part_bytes(rows));
  const PrologueEpi epi{ws::StorePackedF32{cq, kQRank / 16},
                        rows::CacheRowEpi{seq_lens, block_table, cache, num_blocks, max_blocks_per_seq, q_tokens,
                                          rows::RopeFreq::make(rope_base)}};
  const hipError_t e = ProloguePlan::run2(hidden, w_dq, kQRank, w_kv, part, rows, epi, stream);
  if (e != hipSuccess) return e;
  return QUpPlan::run(cq, w_uq, nullptr, rows, rows::HeadsEpi{seq_lens, q_nope, q_pe, q_tokens, rows::RopeFreq::make(rope_base)},
                      stream);
}

}  // namespace mla
