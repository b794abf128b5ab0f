// Epilogues that finish a weight-stream product (wstream.h) into the rows a
// decode step consumes: the new tokens' latent cache rows and their per-head
// queries. Both rotate position pairs with RoPE at the token's position
// pos = L_b - Sq + i: consecutive pairs (x_2i, x_2i+1) turned
// counter-clockwise by pos * base^(-2i/64), angles in fp64 (positions up to
// 2^31 keep their phase), each value rounded once to bf16 (nearest, ties to
// even).
#pragma once

#include "common.h"

namespace mla {
namespace rows {

constexpr int kQRank = 1536;                     // compressed query width
constexpr int kQRow = kDNope + kDRope;           // 192 rows of W_UQ per head
constexpr int kQUp = kHeads * kQRow;             // 24576
static_assert(kQRow % 4 == 0 && kDNope % 4 == 0, "4 columns never straddle a head or the nope/rope boundary");

__device__ __forceinline__ unsigned int bf16_rne(float x) {
  unsigned int u = __builtin_bit_cast(unsigned int, x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ void rope_pair(double pos, int pair, double base, float& y0, float& y1) {
  const double theta = pow(base, -2.0 * pair / kDRope);
  double s, co;
  sincos(pos * theta, &s, &co);
  const double x0 = y0, x1 = y1;
  y0 = (float)(x0 * co - x1 * s);
  y1 = (float)(x0 * s + x1 * co);
}

// [c_KV | W_KR h][r][c .. c + 3] (c % 4 == 0, c < 576) -> token r's cache row:
// block block_table[b, pos / 64], slot pos % 64; the W_KR columns rotated.
// A token without a slot (a length below Sq, a position past the table) or
// with an invalid block id is skipped: nothing is written through it.
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
    if (pos < 0 || pos / kBlock >= max_blocks_per_seq) return;
    const long long blk = block_table[(size_t)b * max_blocks_per_seq + pos / kBlock];
    if (blk < 0 || blk >= num_blocks) return;
    float y[4] = {v[0], v[1], v[2], v[3]};
    if (c >= kDLat) {
      rope_pair((double)pos, (c - kDLat) / 2, rope_base, y[0], y[1]);
      rope_pair((double)pos, (c - kDLat) / 2 + 1, rope_base, y[2], y[3]);
    }
    const u32x2 w = {bf16_rne(y[0]) | (bf16_rne(y[1]) << 16), bf16_rne(y[2]) | (bf16_rne(y[3]) << 16)};
    *(u32x2*)(cache + ((size_t)blk * kBlock + pos % kBlock) * kRow + c) = w;
  }
};

// q[r][c .. c + 3] (c % 4 == 0, c < 24576) -> q_nope / q_pe of token r, head
// c / 192: the 128 non-positional columns rounded, the 64 position columns
// rotated and rounded.
struct HeadsEpi {
  const int32_t* seq_lens;
  uint16_t* q_nope;
  uint16_t* q_pe;
  int q_tokens;
  double rope_base;
  __device__ void operator()(int r, int c, f32x4 v) const {
    const int head = c / kQRow, j = c % kQRow;
    const size_t rh = (size_t)r * kHeads + head;
    float y[4] = {v[0], v[1], v[2], v[3]};
    if (j < kDNope) {
      *(u32x2*)(q_nope + rh * kDNope + j) =
          u32x2{bf16_rne(y[0]) | (bf16_rne(y[1]) << 16), bf16_rne(y[2]) | (bf16_rne(y[3]) << 16)};
      return;
    }
    const int b = r / q_tokens, i = r % q_tokens;
    const double pos = (double)(seq_lens[b] - q_tokens + i);
    const int jr = j - kDNope;   // first of two position pairs
    rope_pair(pos, jr / 2, rope_base, y[0], y[1]);
    rope_pair(pos, jr / 2 + 1, rope_base, y[2], y[3]);
    *(u32x2*)(q_pe + rh * kDRope + jr) =
        u32x2{bf16_rne(y[0]) | (bf16_rne(y[1]) << 16), bf16_rne(y[2]) | (bf16_rne(y[3]) << 16)};
  }
};

}  // namespace rows
}  // namespace mla
