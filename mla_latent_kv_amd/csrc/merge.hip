// Split merge and value projection: for each query row r = (b, i) and head h
//   o_lat = sum_s w_s O_s / sum_s w_s l_s,   w_s = 2^(m_s - max_s m_s)
//   out[r, h, :] = W_UV[h] o_lat                              (512 -> 128)
//
// The merge is the log-sum-exp regrouping of one softmax over the whole
// history; the projection is the output side of the absorb order (the latent
// is aggregated first and W_UV applied once: "DeepSeek-V3" page,
// ailearn.mscapital.top, MLA section; m.lsln.cn article, section 2.2).
//
// One workgroup per (head, 32 query rows): phase 1 merges the partial states
// of its rows into LDS as bf16 hi + lo pairs (hi = bf16(x), lo = bf16(x - hi),
// together within 2^-16 of x); phase 2 is a 32x32x16 bf16 MFMA product with
// W_UV[h] (exact bf16 operand, read straight from HBM with the latent index
// contiguous), hi and lo accumulated in fp32. Each workgroup reads W_UV[h]
// (128 KB) once for its 32 rows.
#include "common.h"

namespace mla {

namespace {

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float x) {
  unsigned int u = __builtin_bit_cast(unsigned int, x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __builtin_bit_cast(float, (unsigned int)h << 16);
}

__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_o,
                                                    const float* __restrict__ part_ml,
                                                    const SeqInfo* __restrict__ seqinfo,
                                                    const uint16_t* __restrict__ w_uv,
                                                    float* __restrict__ out, int rows,
                                                    int q_tokens) {
  // o_lat of 32 rows, bf16 hi and lo, 1 KB per row each; granule swizzle
  // g ^ (row % 8) keeps the MFMA operand reads conflict-free.
  __shared__ __attribute__((aligned(16))) unsigned short lat_hi[32 * kDLat];
  __shared__ __attribute__((aligned(16))) unsigned short lat_lo[32 * kDLat];
  const int h = blockIdx.x;
  const int r0 = blockIdx.y * 32;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const size_t rows_per_chunk = (size_t)q_tokens * kHeads;

  // ---- phase 1: wave w merges rows r0 + 8 w .. +8; lane owns latent 8 lane .. +8
  for (int j = 0; j < 8; ++j) {
    const int rl = 8 * w + j;
    const int r = r0 + rl;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (r < rows) {
      const int b = r / q_tokens, i = r % q_tokens;
      const SeqInfo si = seqinfo[b];
      const size_t prow = (size_t)i * kHeads + h;
      float mx = -INFINITY;
      for (int s = 0; s < si.count; ++s)
        mx = fmaxf(mx, part_ml[((size_t)(si.base + s) * rows_per_chunk + prow) * 2]);
      float den = 0.f;
      if (mx != -INFINITY) {
        for (int s = 0; s < si.count; ++s) {
          const size_t pr = (size_t)(si.base + s) * rows_per_chunk + prow;
          const float ms = part_ml[pr * 2];
          if (ms == -INFINITY) continue;
          const float ws = exp2f(ms - mx);
          den += ws * part_ml[pr * 2 + 1];
          const f32x4* src = (const f32x4*)(part_o + pr * kDLat + 8 * lane);
          f32x4 v0 = src[0], v1 = src[1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[e] += ws * v0[e];
            acc[4 + e] += ws * v1[e];
          }
        }
      }
      const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] *= inv;
    }
    unsigned short hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = f32_to_bf16_rne(acc[e]);
      lo[e] = f32_to_bf16_rne(acc[e] - bf16_to_f32(hi[e]));
    }
    const int off = rl * kDLat + 8 * (lane ^ (rl & 7));
    u32x4 vh, vl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vh[e] = (unsigned int)hi[2 * e] | ((unsigned int)hi[2 * e + 1] << 16);
      vl[e] = (unsigned int)lo[2 * e] | ((unsigned int)lo[2 * e + 1] << 16);
    }
    *(u32x4*)(lat_hi + off) = vh;
    *(u32x4*)(lat_lo + off) = vl;
  }
  __syncthreads();

  // ---- phase 2: D[v, row] = sum_c W_UV[h][v][c] o_lat[row][c]; wave w: v in 32 w .. +32
  const int half = lane >> 5, l32 = lane & 31;
  const uint16_t* wrow = w_uv + ((size_t)h * kDV + 32 * w + l32) * kDLat + 8 * half;
  f32x16 acc = {};
#pragma unroll 8
  for (int ks = 0; ks < kDLat / 16; ++ks) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(wrow + 16 * ks));
    const int g = (2 * ks + half) ^ (l32 & 7);
    const bf16x8 bh = __builtin_bit_cast(bf16x8, *(const u32x4*)(lat_hi + l32 * kDLat + 8 * g));
    const bf16x8 bl = __builtin_bit_cast(bf16x8, *(const u32x4*)(lat_lo + l32 * kDLat + 8 * g));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bl, acc, 0, 0, 0);
  }
  const int r = r0 + l32;
  if (r < rows) {
    float* dst = out + ((size_t)r * kHeads + h) * kDV + 32 * w + 4 * half;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(f32x4*)(dst + 8 * q) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
  }
}

}  // namespace

hipError_t launch_merge(const float* part_o, const float* part_ml, const SeqInfo* seqinfo,
                        const uint16_t* w_uv, float* out, int batch, int q_tokens,
                        hipStream_t stream) {
  const int rows = batch * q_tokens;
  hipLaunchKernelGGL(merge_kernel, dim3(kHeads, (rows + 31) / 32), dim3(256), 0, stream, part_o,
                     part_ml, seqinfo, w_uv, out, rows, q_tokens);
  return hipGetLastError();
}

}  // namespace mla
