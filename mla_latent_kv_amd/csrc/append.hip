// Cache-append producer: the rows a decode step's new tokens add to the paged
// latent cache,
//   c_KV = W_DKV h           (7168 -> 512)
//   k_R  = RoPE(W_KR h, pos) (7168 -> 64), pos = L_b - Sq + i
// stored as one 576-wide bf16 row [c_KV | k_R] in block
// block_table[b, pos / 64], slot pos % 64. Each token keeps only the short
// joint latent and the small head-shared position key, the latter rotated by
// its position ("DeepSeek-V3" article at m.lsln.cn, sections 2.2 and 2.3;
// "DeepSeek-V3" page at ailearn.mscapital.top, MLA paragraphs).
//
// The two projections are one product with the stacked weight [W_DKV; W_KR]
// ([576][7168], in the packed weight layout of wstream.h), two launches:
//  1. the weight stream: 18 column tiles x 14 K-splits = 252 workgroups, each
//     wavefront with all its 8 k-steps in flight at once (h read from its
//     rows), partial sums per split;
//  2. per (token, 4 columns) the splits added in split order and the cache
//     row finished (rows.h: RoPE, bf16, the paged write). No atomics: results
//     are deterministic.
#include "rows.h"
#include "wstream.h"

namespace mla {

namespace {
using AppendPlan = ws::Plan<false, kRow, kDHidden, 1, 8, 14, true>;
}  // namespace

size_t append_workspace_bytes(int rows) { return AppendPlan::part_bytes(rows); }

hipError_t launch_append(const uint16_t* hidden, const uint16_t* w_kv, uint16_t* cache,
                         const int32_t* block_table, const int32_t* seq_lens, long long num_blocks,
                         int max_blocks_per_seq, int batch, int q_tokens, double rope_base, void* ws,
                         hipStream_t stream) {
  const int rows = batch * q_tokens;
  return AppendPlan::run(hidden, w_kv, (float*)ws, rows,
                         rows::CacheRowEpi{seq_lens, block_table, cache, num_blocks, max_blocks_per_seq, q_tokens,
                                           rows::RopeFreq::make(rope_base)},
                         stream);
}

}  // namespace mla
