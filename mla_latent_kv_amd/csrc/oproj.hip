// Output projection: y[t, :] = W_O x_t, x_t = the attention outputs of token t
// concatenated head-major (index h * 128 + v, 16384 values), W_O [7168][16384].
// The last step of the attention block: the heads' outputs go through one
// output projection matrix back to the model width ("DeepSeek-V3" page,
// ailearn.mscapital.top, MLA state flow).
//
// A weight stream: for a decode batch (a few dozen tokens) every W_O byte is
// used by only those tokens, so the bound is HBM (235 MB per call). One
// launch of the weight-stream product (wstream.h), no partial sums in memory:
// * workgroup = 32 output columns over the whole K = 16384; its 1 MB weight
//   slice crosses HBM once. 224 workgroups.
// * its 4 wavefronts split K (4096 each); each streams its weight and input
//   tiles (chunks of 64 k: 4 KB of W_O rows, 8 KB of inputs) through its own
//   3-stage LDS ring with direct-to-LDS fetches laid out so that every 1 KB
//   fetch covers 8 whole cache lines (fragments loaded straight from global
//   memory would touch 32 rows per instruction and starve the load path).
//   Two chunks in flight per wavefront (≈ 96 KB per workgroup) cover HBM
//   latency; the waits are explicit and no barrier is needed in the loop.
// * D[n, t] = sum_k W[n][k] x[t][k] on 32x32x16 bf16 MFMA: both operands are
//   row-major with k contiguous, so each fragment is one contiguous load.
//   The fp32 input is split as x = hi + lo with hi = bf16(x) and
//   lo = bf16(x - hi) (together within 2^-17 of x) and both halves are
//   multiplied (two MFMAs per k-step); the matrix cores have ample slack
//   against the weight stream.
// * the 4 wavefront tiles are summed in LDS in a fixed order and stored as
//   fp32. No atomics: results are deterministic.
// More than 32 tokens loop over row tiles (each extra 32 tokens re-streams
// the slice).
#include "wstream.h"

namespace mla {

namespace {
constexpr int kOpK = kHeads * kDV;   // 16384
static_assert(kDHidden % 32 == 0, "whole column tiles");
}  // namespace

hipError_t launch_oproj(const float* x, const uint16_t* w_o, float* y, int rows, hipStream_t stream) {
  hipLaunchKernelGGL((ws::wstream_kernel<true, kOpK / 4>), dim3(kDHidden / 32, 1), dim3(ws::kThreads), 0,
                     stream, (const void*)x, (long long)kOpK, w_o, (long long)kOpK, y,
                     (long long)kDHidden, 0LL, rows);
  return hipGetLastError();
}

}  // namespace mla
