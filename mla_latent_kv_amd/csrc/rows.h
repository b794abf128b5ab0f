// Epilogues that finish a weight-stream product (wstream.h) into the rows a
// decode step consumes: the new tokens' latent cache rows and their per-head
// queries. Both rotate position pairs with RoPE at the token's position
// pos = L_b - Sq + i: consecutive pairs (x_2i, x_2i+1) turned
// counter-clockwise by pos * base^(-2i/64), each value rounded once to bf16
// (nearest, ties to even). The 32 frequencies are computed on the host once
// per call; the angle pos * f_i is formed and reduced by pi/2 in fp64
// (positions up to 2^31 keep their phase), and only the remainder, at most
// pi/4, has its sine and cosine taken in fp32.
#pragma once

#include <cmath>

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

// base^(-2i/64) for the 32 position pairs, made on the host per call.
struct RopeFreq {
  double f[kDRope / 2];
  static RopeFreq make(double base) {
    RopeFreq r;
    for (int i = 0; i < kDRope / 2; ++i) r.f[i] = std::pow(base, -2.0 * i / kDRope);
    return r;
  }
};

// sin and cos of an fp64 angle a >= 0: a = n pi/2 + t with n = rint(a 2/pi)
// and t in [-pi/4, pi/4], taken with pi/2 split into the nearest double and
// its remainder (Cody and Waite's additive reduction; for a < 2^31, n < 2^31
// and the neglected part of n pi/2 stays below 1e-24); sin t and cos t in
// fp32, then the quadrant n mod 4 applied.
__device__ __forceinline__ void sincos_reduced(double a, float& s, float& c) {
  constexpr double kTwoOverPi = 0.636619772367581343076;
  constexpr double kHalfPiHi = 1.5707963267948966;        // pi/2 rounded to double
  constexpr double kHalfPiLo = 6.123233995736766e-17;     // pi/2 - kHalfPiHi
  const double n = rint(a * kTwoOverPi);
  const double t = fma(-n, kHalfPiLo, fma(-n, kHalfPiHi, a));
  float st, ct;
  sincosf((float)t, &st, &ct);
  switch ((long long)n & 3) {
    case 0: s = st; c = ct; break;
    case 1: s = ct; c = -st; break;
    case 2: s = -st; c = -ct; break;
    default: s = -ct; c = st; break;
  }
}

__device__ __forceinline__ void rope_pair(double pos, int pair, const RopeFreq& fr, float& y0, float& y1) {
  float s, c;
  sincos_reduced(pos * fr.f[pair], s, c);
  const float x0 = y0, x1 = y1;
  y0 = fmaf(x0, c, -x1 * s);
  y1 = fmaf(x0, s, x1 * c);
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
  RopeFreq freq;
  __device__ void operator()(int r, int c, f32x4 v) const {
    const int b = r / q_tokens, i = r % q_tokens;
    const int pos = seq_lens[b] - q_tokens + i;
    if (pos < 0 || pos / kBlock >= max_blocks_per_seq) return;
    const long long blk = block_table[(size_t)b * max_blocks_per_seq + pos / kBlock];
    if (blk < 0 || blk >= num_blocks) return;
    float y[4] = {v[0], v[1], v[2], v[3]};
    if (c >= kDLat) {
      rope_pair((double)pos, (c - kDLat) / 2, freq, y[0], y[1]);
      rope_pair((double)pos, (c - kDLat) / 2 + 1, freq, y[2], y[3]);
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
  RopeFreq freq;
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
    rope_pair(pos, jr / 2, freq, y[0], y[1]);
    rope_pair(pos, jr / 2 + 1, freq, y[2], y[3]);
    *(u32x2*)(q_pe + rh * kDRope + jr) =
        u32x2{bf16_rne(y[0]) | (bf16_rne(y[1]) << 16), bf16_rne(y[2]) | (bf16_rne(y[3]) << 16)};
  }
};

}  // namespace rows
}  // namespace mla
