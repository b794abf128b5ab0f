// The packed weight layout of the weight-stream products (wstream.h), made
// once per weight at load time: the 1 KB block of column tile ct (32 rows of
// W) and k-step ks (16 columns) sits at byte (ks * N/32 + ct) * 1024, lane l's
// 16 bytes being W[32 ct + l % 32][16 ks + 8 (l / 32) .. + 7], the operand
// fragment of one 32x32x16 bf16 MFMA. A pure permutation of the bytes.
#include "wstream.h"

namespace mla {

namespace {

// One thread per 16-byte piece of the packed weight.
__global__ __launch_bounds__(256) void pack_w_kernel(const uint16_t* __restrict__ w, u32x4* __restrict__ p,
                                                     int n_tiles, int k_steps) {
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= (long long)n_tiles * k_steps * 64) return;
  const int lane = (int)(g & 63);
  const long long tk = g >> 6;
  const int ct = (int)(tk % n_tiles), ks = (int)(tk / n_tiles);
  const size_t ld = (size_t)16 * k_steps;
  p[g] = *(const u32x4*)(w + (size_t)(32 * ct + (lane & 31)) * ld + 16 * ks + 8 * (lane >> 5));
}

}  // namespace

hipError_t launch_pack_weight(const uint16_t* w, uint16_t* packed, int n, int k, hipStream_t stream) {
  const long long pieces = (long long)(n / 32) * (k / 16) * 64;
  hipLaunchKernelGGL(pack_w_kernel, dim3((unsigned)((pieces + 255) / 256)), dim3(256), 0, stream, w,
                     (u32x4*)packed, n / 32, k / 16);
  return hipGetLastError();
}

}  // namespace mla
