// Cache-append producer: the rows a decode step's new tokens add to the paged
// latent cache,
//   c_KV = W_DKV h           (7168 -> 512)
//   k_R  = RoPE(W_KR h, pos) (7168 -> 64), pos = L_b - Sq + i
// stored as one 576-wide bf16 row [c_KV | k_R] in block
// block_table[b, pos / 64], slot pos % 64. Each token keeps only the short
// joint latent and the small head-shared position key, the latter rotated by
// its position ("DeepSeek-V3" article at m.lsln.cn, sections 2.2 and 2.3;
// "DeepSeek-V3" page at ailearn.mscapital.top, MLA paragraphs). RoPE turns
// consecutive pairs (x_2i, x_2i+1) counter-clockwise by pos * base^(-2i/64).
//
// The two projections are one product with the stacked weight [W_DKV; W_KR]
// ([576][7168], in the packed weight layout of wstream.h), two launches:
//  1. the weight stream: 18 column tiles x 14 K-splits = 252 workgroups, each
//     wavefront with all its 8 k-steps in flight at once (h read from its
//     rows), partial sums per split;
//  2. per (token, 4 columns) the splits added in split order, the position
//     pairs rotated (angles in fp64, so positions up to 2^31 keep their
//     phase), rounded to bf16 (nearest, ties to even) and written as 8 bytes
//     of the token's cache row. No atomics: results are deterministic.
#include "wstream.h"

namespace mla {

namespace {

using AppendPlan = ws::Plan<false, kRow, kDHidden, 1, 8, 14, true>;

__device__ __forceinline__ unsigned int bf16_rne_bits(float x) {
  unsigned int u = __builtin_bit_cast(unsigned int, x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// [c_KV | W_KR h][r][c .. c + 3] -> the token's cache row
struct CacheRowEpi {
  const int32_t* seq_lens;
  const int32_t* block_table;
  uint16_t* cache;
  long long num_blocks;
  int max_blocks_per_seq;
  int q_tokens;
  double rope_base;
  __device__ void operator()(int r, int c, f32x4 v) const {
    const int b = r / q_tokens, i = r % q_tokens;
    const int pos = seq_lens[b] - q_tokens + i;
    // no slot for this token (a length below Sq, or past the table): nothing written
    if (pos < 0 || pos / kBlock >= max_blocks_per_seq) return;
    const long long blk = block_table[(size_t)b * max_blocks_per_seq + pos / kBlock];
    if (blk < 0 || blk >= num_blocks) return;   // an invalid block id is never written through
    unsigned int w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      float y0 = v[2 * k], y1 = v[2 * k + 1];
      if (c >= kDLat) {
        const int pair = (c - kDLat) / 2 + k;
        const double theta = pow(rope_base, -2.0 * pair / kDRope);
        double s, co;
        sincos((double)pos * theta, &s, &co);
        const double x0 = y0, x1 = y1;
        y0 = (float)(x0 * co - x1 * s);
        y1 = (float)(x0 * s + x1 * co);
      }
      w[k] = bf16_rne_bits(y0) | (bf16_rne_bits(y1) << 16);
    }
    *(u32x2*)(cache + ((size_t)blk * kBlock + pos % kBlock) * kRow + c) = u32x2{w[0], w[1]};
  }
};

}  // namespace

size_t append_workspace_bytes(int rows) { return AppendPlan::part_bytes(rows); }

hipError_t launch_append(const uint16_t* hidden, const uint16_t* w_kv, uint16_t* cache,
                         const int32_t* block_table, const int32_t* seq_lens, long long num_blocks,
                         int max_blocks_per_seq, int batch, int q_tokens, double rope_base, void* ws,
                         hipStream_t stream) {
  const int rows = batch * q_tokens;
  return AppendPlan::run(hidden, w_kv, (float*)ws, rows,
                         CacheRowEpi{seq_lens, block_table, cache, num_blocks, max_blocks_per_seq, q_tokens,
                                     rope_base},
                         stream);
}

}  // namespace mla
