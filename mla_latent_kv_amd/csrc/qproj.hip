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
//  1. stream W_DQ: 48 column tiles x 16 K-splits = 768 workgroups, each
//     wavefront with all its 7 k-steps in flight at once (h read from its
//     rows), partial sums per split;
//  2. the splits added in split order; c_Q (fp32) is written straight into
//     the packed input layout of the second product;
//  3. stream W_UQ: 256 column blocks of 96, one split (each wavefront 24
//     k-steps); c_Q enters as fp32 hi + lo. Its epilogue finishes the heads:
//     non-positional columns rounded to bf16, position pairs rotated (fp64
//     angles) and rounded (nearest, ties to even).
#include "wstream.h"

namespace mla {

namespace {

constexpr int kQRank = 1536;
constexpr int kQRow = kDNope + kDRope;   // 192 rows of W_UQ per head
constexpr int kQUp = kHeads * kQRow;     // 24576
using QDownPlan = ws::Plan<false, kQRank, kDHidden, 1, 7, 16, true>;
using QUpPlan = ws::Plan<true, kQUp, kQRank, 3, 4, 1>;
static_assert(kQRow % 4 == 0 && kDNope % 4 == 0, "4 columns never straddle a head or the nope/rope boundary");

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

__device__ __forceinline__ unsigned int bf16_rne(float x) {
  unsigned int u = __builtin_bit_cast(unsigned int, x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// q[r][c .. c + 3] (c % 4 == 0) -> q_nope / q_pe of token r, head c / 192
struct HeadsEpi {
  const int32_t* seq_lens;
  uint16_t* q_nope;
  uint16_t* q_pe;
  int q_tokens;
  double rope_base;
  __device__ void operator()(int r, int c, f32x4 v) const {
    const int head = c / kQRow, j = c % kQRow;
    const size_t rh = (size_t)r * kHeads + head;
    if (j < kDNope) {
      const u32x2 p = {bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16)};
      *(u32x2*)(q_nope + rh * kDNope + j) = p;
      return;
    }
    const int b = r / q_tokens, i = r % q_tokens;
    const double pos = (double)(seq_lens[b] - q_tokens + i);
    const int jr = j - kDNope;   // first of two position pairs
    unsigned int w[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int pair = jr / 2 + k;
      const double theta = pow(rope_base, -2.0 * pair / kDRope);
      double s, co;
      sincos(pos * theta, &s, &co);
      const double x0 = v[2 * k], x1 = v[2 * k + 1];
      w[k] = bf16_rne((float)(x0 * co - x1 * s)) | (bf16_rne((float)(x0 * s + x1 * co)) << 16);
    }
    *(u32x2*)(q_pe + rh * kDRope + jr) = u32x2{w[0], w[1]};
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
  return QUpPlan::run(cq, w_uq, nullptr, rows, HeadsEpi{seq_lens, q_nope, q_pe, q_tokens, rope_base}, stream);
}

}  // namespace mla
