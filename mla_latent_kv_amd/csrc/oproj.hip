// Output projection: y[t, :] = W_O x_t, x_t = the attention outputs of token t
// concatenated head-major (index h * 128 + v, 16384 values), W_O [7168][16384].
// The last step of the attention block: the heads' outputs go through one
// output projection matrix back to the model width ("DeepSeek-V3" page,
// ailearn.mscapital.top, MLA state flow).
//
// A weight stream: for a decode batch (a few dozen tokens) every W_O byte is
// used by only those tokens, so the bound is HBM (235 MB per call). One
// launch, no partial sums in memory:
// * workgroup = 32 output columns over the whole K = 16384; its 1 MB weight
//   slice crosses HBM once. 224 workgroups.
// * its 4 wavefronts split K (4096 each) and stream weight and input
//   fragments straight from global memory into registers, 8 k-steps ahead
//   (≈ 96 KB in flight per workgroup to cover HBM latency).
// * D[n, t] = sum_k W[n][k] x[t][k] on 32x32x16 bf16 MFMA: both operands are
//   row-major with k contiguous, so each fragment is one contiguous load.
//   The fp32 input is split as x = hi + lo with hi = bf16(x) and
//   lo = bf16(x - hi) (together within 2^-17 of x) and both halves are
//   multiplied (two MFMAs per k-step); the matrix cores have ample slack
//   against the weight stream.
// * the 4 wavefront tiles are summed in LDS in a fixed order and stored as
//   fp32. No atomics: results are deterministic.
// More than 32 tokens loop over row tiles with the same weight fragments
// re-read per tile (each extra 32 tokens re-streams the slice).
#include "common.h"

namespace mla {

namespace {

constexpr int kOpThreads = 256;
constexpr int kOpK = kHeads * kDV;            // 16384
constexpr int kOpKPerWave = kOpK / 4;         // 4096
constexpr int kOpSteps = kOpKPerWave / 16;    // 256 k-steps per wavefront
constexpr int kOpDepth = 8;                   // k-steps in flight per wavefront
static_assert(kOpSteps % kOpDepth == 0, "pipeline depth divides the k-steps");
static_assert(kDHidden % 32 == 0, "whole column tiles");

__device__ __forceinline__ void split_bf16(const f32x4 a, const f32x4 b, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = (__bf16)a[e];
    hi[4 + e] = (__bf16)b[e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] = (__bf16)(a[e] - (float)hi[e]);
    lo[4 + e] = (__bf16)(b[e] - (float)hi[4 + e]);
  }
}

__global__ __launch_bounds__(kOpThreads) void oproj_kernel(const float* __restrict__ x,
                                                           const uint16_t* __restrict__ w_o,
                                                           float* __restrict__ y, int rows) {
  __shared__ float red[4][32][33];   // [wave][column][token], padded
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int n0 = blockIdx.x * 32;
  const int koff = w * kOpKPerWave + 8 * (lane >> 5);   // this lane's first k
  // A operand (lane = column, 8 consecutive k)
  const uint16_t* wrow = w_o + (size_t)(n0 + (lane & 31)) * kOpK + koff;

  for (int r0 = 0; r0 < rows; r0 += 32) {
    // B operand (lane = token, 8 consecutive k). Lanes past the batch read
    // token 0: their columns of D are never stored.
    const int r = r0 + (lane & 31);
    const float* xrow = x + (size_t)(r < rows ? r : 0) * kOpK + koff;
    u32x4 wf[kOpDepth];
    f32x4 xa[kOpDepth], xb[kOpDepth];
#pragma unroll
    for (int d = 0; d < kOpDepth; ++d) {
      wf[d] = *(const u32x4*)(wrow + 16 * d);
      xa[d] = *(const f32x4*)(xrow + 16 * d);
      xb[d] = *(const f32x4*)(xrow + 16 * d + 4);
    }
    f32x16 acc = {};
    for (int ks = 0; ks < kOpSteps; ks += kOpDepth) {
#pragma unroll
      for (int d = 0; d < kOpDepth; ++d) {
        bf16x8 hi, lo;
        split_bf16(xa[d], xb[d], hi, lo);
        const bf16x8 a = __builtin_bit_cast(bf16x8, wf[d]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lo, acc, 0, 0, 0);
        const int nk = ks + d + kOpDepth;   // refill this stage with k-step nk
        if (nk < kOpSteps) {
          wf[d] = *(const u32x4*)(wrow + 16 * nk);
          xa[d] = *(const f32x4*)(xrow + 16 * nk);
          xb[d] = *(const f32x4*)(xrow + 16 * nk + 4);
        }
      }
    }
    // acc[i] is column 8 (i / 4) + 4 (lane / 32) + i % 4 of token lane % 32
#pragma unroll
    for (int i = 0; i < 16; ++i) red[w][8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)][lane & 31] = acc[i];
    __syncthreads();
    {
      const int rr = t >> 3, nq = (t & 7) * 4;   // token, first of 4 columns
      if (r0 + rr < rows) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = ((red[0][nq + e][rr] + red[1][nq + e][rr]) + red[2][nq + e][rr]) + red[3][nq + e][rr];
        *(f32x4*)(y + (size_t)(r0 + rr) * kDHidden + n0 + nq) = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_oproj(const float* x, const uint16_t* w_o, float* y, int rows, hipStream_t stream) {
  hipLaunchKernelGGL(oproj_kernel, dim3(kDHidden / 32), dim3(kOpThreads), 0, stream, x, w_o, y, rows);
  return hipGetLastError();
}

}  // namespace mla
