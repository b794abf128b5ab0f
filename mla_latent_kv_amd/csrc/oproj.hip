// Output projection: y[t, :] = W_O x_t, x_t = the attention outputs of token t
// concatenated head-major (index h * 128 + v, 16384 values), W_O [7168][16384].
// The last step of the attention block: the heads' outputs go through one
// output projection matrix back to the model width ("DeepSeek-V3" page,
// ailearn.mscapital.top, MLA state flow).
//
// A weight stream (wstream.h): for a decode batch (a few dozen tokens) every
// W_O byte is used by only those tokens, so the bound is HBM (235 MB per
// call). Three launches on the caller's stream:
//  1. x (fp32 rows) -> the packed input layout (2 MB for 32 tokens);
//  2. the stream: 56 column blocks of 128 x 4 K-splits = 224 workgroups, each
//     wavefront 64 k-steps (a quarter of its split); W_O in the packed weight
//     layout, read once;
//  3. the 4 splits' partial sums added in split order -> y.
#include "wstream.h"

namespace mla {

namespace {
constexpr int kOpK = kHeads * kDV;   // 16384
using OprojPlan = ws::Plan<true, kDHidden, kOpK, 4, 4, 4>;

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }
}  // namespace

size_t oproj_workspace_bytes(int rows) {
  return round256(OprojPlan::packed_x_bytes(rows)) + round256(OprojPlan::part_bytes(rows));
}

hipError_t launch_oproj(const float* x, const uint16_t* w_o, float* y, int rows, void* ws, hipStream_t stream) {
  char* xp = (char*)ws;
  float* part = (float*)(xp + round256(OprojPlan::packed_x_bytes(rows)));
  const hipError_t e = OprojPlan::pack_x(x, xp, rows, stream);
  if (e != hipSuccess) return e;
  return OprojPlan::run(xp, w_o, part, rows, ws::StoreF32{y, kDHidden}, stream);
}

}  // namespace mla
