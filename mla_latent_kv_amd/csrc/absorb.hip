// Absorb product: q_abs[r, h, :] = W_UK[h]^T q_nope[r, h, :]  (128 -> 512).
//
// This is the query side of the identity q^T (U c) = (U^T q)^T c (the algebra
// check in section 2 of the wq-win.github.io DeepSeek-V3 notes, U = W_UK[h]):
// transforming the query once lets every cached latent be used as it is
// ("DeepSeek-V3" page, MLA section: q_nope x W_UK, then dot products with all
// cached c_KV). One workgroup per (head, 128-wide latent block) reads its
// 128 x 128 slice of W_UK once and applies it to every query row of the batch,
// so W_UK crosses HBM exactly once per call.
//
// Matrix cores: D[c, r] = sum_k W_UK[h][k][c] * q_nope[r][h][k], bf16 inputs
// (exact products), fp32 accumulation, 32x32x16 MFMA. W_UK is stored with the
// latent index contiguous, so its k-major operand fragments come from LDS
// through transposing reads (ds_read_b64_tr_b16). The result is rounded to
// fp16 and written in the fragment order the attention kernel loads it in:
//   q_abs[((r * 4 + h / 32) * 32 + c / 16) * 64 + (h % 32) + 32 * ((c % 16) / 8)][c % 8]
// so that each wavefront there reads its 32 heads x 512 values as one
// contiguous 32 KB run.
#include "common.h"

namespace mla {

namespace {

constexpr int kWStride = 288;   // LDS row stride (bytes) of the W_UK slice: 256 + 32 pad

__global__ __launch_bounds__(256) void absorb_kernel(const uint16_t* __restrict__ q_nope,
                                                     const uint16_t* __restrict__ w_uk,
                                                     _Float16* __restrict__ q_abs, int rows) {
  __shared__ __attribute__((aligned(16))) char wl[kDNope * kWStride];
  const int h = blockIdx.x;
  const int cb = blockIdx.y;          // latent block of 128
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;

  // W_UK[h][k][cb*128 .. +128] -> LDS rows k (16-byte granules, coalesced)
  const uint16_t* wsrc = w_uk + ((size_t)h * kDNope) * kDLat + cb * 128;
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int G = t + 256 * n;
    const int k = G >> 4, g = G & 15;
    u32x4 v = *(const u32x4*)(wsrc + (size_t)k * kDLat + g * 8);
    *(u32x4*)(wl + k * kWStride + g * 16) = v;
  }
  __syncthreads();

  // A fragments (W_UK^T[c][k], lane = c) for all 8 k-steps, via transposing reads.
  // Lane group gg = lane / 16 covers columns 16 * (gg % 2) + (0..15) and the
  // k-half hh = gg / 2; source lane L addresses row k = 16 ks + 8 hh + 4 q + L / 4
  // at column 4 * (L % 4), so the read returns, per lane, 4 consecutive k of its
  // own column.
  const int gg = lane >> 4, L = lane & 15, hh = gg >> 1;
  const int cw = 32 * w + 16 * (gg & 1) + 4 * (L & 3);
  bf16x8 a[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    s16x4 p0, p1;
    const int k0 = 16 * ks + 8 * hh + (L >> 2);
    p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(wl + k0 * kWStride + cw * 2));
    p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(wl + (k0 + 4) * kWStride + cw * 2));
    a[ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  const int hg = h >> 5, hj = h & 31;
  const int c0 = cb * 128 + 32 * w;           // first latent column of this wave
  const int half = lane >> 5;
  for (int r0 = 0; r0 < rows; r0 += 32) {
    const int r = r0 + (lane & 31);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      u32x4 bv = {0, 0, 0, 0};
      if (r < rows)
        bv = *(const u32x4*)(q_nope + ((size_t)r * kHeads + h) * kDNope + 16 * ks + 8 * half);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], __builtin_bit_cast(bf16x8, bv), acc,
                                                    0, 0, 0);
    }
    if (r < rows) {
      // acc[4 q + e] holds column c0 + 8 q + 4 half + e of row r
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + 8 * q + 4 * half;
        f16x4 v = {(_Float16)acc[4 * q], (_Float16)acc[4 * q + 1], (_Float16)acc[4 * q + 2],
                   (_Float16)acc[4 * q + 3]};
        const size_t frag = (((size_t)r * 4 + hg) * 32 + (c >> 4)) * 64 + hj + 32 * ((c & 15) >> 3);
        *(f16x4*)(q_abs + frag * 8 + (c & 7)) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_absorb(const uint16_t* q_nope, const uint16_t* w_uk, _Float16* q_abs, int rows,
                         hipStream_t stream) {
  hipLaunchKernelGGL(absorb_kernel, dim3(kHeads, kDLat / 128), dim3(256), 0, stream, q_nope, w_uk,
                     q_abs, rows);
  return hipGetLastError();
}

}  // namespace mla
