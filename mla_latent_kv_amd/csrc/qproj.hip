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
// Four launches on the caller's stream, all deterministic:
//  1. split-K weight stream h -> c_Q partials (wstream.h; 48 column tiles x 7
//     K-splits = 336 workgroups, W_DQ read once);
//  2. the 7 partials summed in a fixed order -> c_Q (fp32);
//  3. weight stream c_Q -> q (768 column tiles, W_UQ read once; c_Q enters
//     as fp32 hi + lo);
//  4. epilogue: per (token, head, column pair) the non-positional pairs are
//     rounded to bf16 and the position pairs rotated (fp64 angles) and
//     rounded (nearest, ties to even).
#include "wstream.h"

namespace mla {

namespace {

constexpr int kQRank = 1536;
constexpr int kQRow = kDNope + kDRope;            // 192 rows of W_UQ per head
constexpr int kQUp = kHeads * kQRow;              // 24576
constexpr int kQDownSplit = 7;                    // K-splits of the first product
constexpr int kQDownPerWave = kDHidden / kQDownSplit / 4;   // 256
static_assert(kDHidden % (kQDownSplit * 4 * ws::kChunk) == 0, "whole chunks per split");
static_assert(kQRank % (4 * ws::kChunk) == 0 && kQRank % 32 == 0 && kQUp % 32 == 0, "tiles");

__device__ __forceinline__ unsigned int bf16_rne(float x) {
  unsigned int u = __builtin_bit_cast(unsigned int, x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__global__ __launch_bounds__(256) void qdown_sum_kernel(const float* __restrict__ part, float* __restrict__ c_q,
                                                        int rows) {
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;   // 4 values each
  if (g * 4 >= (long long)rows * kQRank) return;
  f32x4 s = *(const f32x4*)(part + g * 4);
#pragma unroll
  for (int k = 1; k < kQDownSplit; ++k) {
    const f32x4 v = *(const f32x4*)(part + (size_t)k * rows * kQRank + g * 4);
    s += v;
  }
  *(f32x4*)(c_q + g * 4) = s;
}

__global__ __launch_bounds__(256) void qfinish_kernel(const float* __restrict__ q, const int32_t* __restrict__ seq_lens,
                                                      uint16_t* __restrict__ q_nope, uint16_t* __restrict__ q_pe,
                                                      int rows, int q_tokens, double rope_base) {
  constexpr int kPairs = kQRow / 2;   // 96 per head: 64 non-positional, 32 position
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= (long long)rows * kHeads * kPairs) return;
  const int pr = (int)(g % kPairs);
  const long long rh = g / kPairs;   // row * 128 + head
  const int r = (int)(rh / kHeads);
  const f32x2 v = *(const f32x2*)(q + rh * kQRow + 2 * pr);
  float y0 = v[0], y1 = v[1];
  if (pr < kDNope / 2) {
    *(unsigned int*)(q_nope + rh * kDNope + 2 * pr) = bf16_rne(y0) | (bf16_rne(y1) << 16);
    return;
  }
  const int qq = pr - kDNope / 2;   // position pair
  const int b = r / q_tokens, i = r % q_tokens;
  const int pos = seq_lens[b] - q_tokens + i;
  const double theta = pow(rope_base, -2.0 * qq / kDRope);
  double s, c;
  sincos((double)pos * theta, &s, &c);
  const float z0 = (float)((double)y0 * c - (double)y1 * s);
  const float z1 = (float)((double)y0 * s + (double)y1 * c);
  *(unsigned int*)(q_pe + rh * kDRope + 2 * qq) = bf16_rne(z0) | (bf16_rne(z1) << 16);
}

}  // namespace

size_t qproj_workspace_bytes(int rows) {
  return ((size_t)kQDownSplit * rows * kQRank + (size_t)rows * kQRank + (size_t)rows * kQUp) * sizeof(float);
}

hipError_t launch_qproj(const uint16_t* hidden, const uint16_t* w_dq, const uint16_t* w_uq,
                        const int32_t* seq_lens, uint16_t* q_nope, uint16_t* q_pe, int batch,
                        int q_tokens, double rope_base, float* ws, hipStream_t stream) {
  const int rows = batch * q_tokens;
  float* part = ws;
  float* c_q = part + (size_t)kQDownSplit * rows * kQRank;
  float* q = c_q + (size_t)rows * kQRank;
  hipLaunchKernelGGL((ws::wstream_kernel<false, kQDownPerWave>), dim3(kQRank / 32, kQDownSplit),
                     dim3(ws::kThreads), 0, stream, (const void*)hidden, (long long)kDHidden, w_dq,
                     (long long)kDHidden, part, (long long)kQRank, (long long)rows * kQRank, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n4 = (long long)rows * kQRank / 4;
  hipLaunchKernelGGL(qdown_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, stream, part, c_q,
                     rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((ws::wstream_kernel<true, kQRank / 4>), dim3(kQUp / 32, 1), dim3(ws::kThreads), 0,
                     stream, (const void*)c_q, (long long)kQRank, w_uq, (long long)kQRank, q,
                     (long long)kQUp, 0LL, rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const long long nf = (long long)rows * kHeads * (kQRow / 2);
  hipLaunchKernelGGL(qfinish_kernel, dim3((unsigned)((nf + 255) / 256)), dim3(256), 0, stream, q, seq_lens,
                     q_nope, q_pe, rows, q_tokens, rope_base);
  return hipGetLastError();
}

}  // namespace mla
