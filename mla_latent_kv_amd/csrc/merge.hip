// Split merge and value projection: for each query row r = (b, i) and head h
//   o_lat = sum_s w_s o_hat_s,   w_s = 2^(lse_s - M) / sum_s 2^(lse_s - M),
//   M = max_s lse_s,  out[r, h, :] = W_UV[h] o_lat               (512 -> 128)
// where o_hat_s = O_s / l_s is split s's normalised partial and
// lse_s = m_s + log2 l_s. The merge is the log-sum-exp regrouping of one
// softmax over the whole history; the projection is the output side of the
// absorb order (the latent is aggregated first and W_UV applied once:
// "DeepSeek-V3" page, ailearn.mscapital.top, MLA section; m.lsln.cn article,
// section 2.2).
//
// One workgroup of 16 wavefronts per (head, 32 query rows), so W_UV[h] is read
// once per 32 rows:
//  1a. per row: M and 1 / sum 2^(lse - M) by wavefront reductions;
//  1b. per (row, 8-column chunk) unit: the weighted sum over splits, streamed
//      as 16-byte loads; when the workgroup has few rows, the splits of a unit
//      are spread over up to 8 thread groups and summed afterwards in a fixed
//      order (deterministic); o_lat goes to LDS as bf16 hi + lo pairs
//      (hi = bf16(x), lo = bf16(x - hi), together within 2^-16 of x);
//  2.  out = W_UV[h] o_lat on 32x32x16 bf16 MFMA (W_UV exact, hi and lo
//      accumulated in fp32): 4 value tiles x 4 latent quarters over the 16
//      wavefronts, quarter sums added in a fixed order.
#include "common.h"

namespace mla {

namespace {

constexpr int kMThreads = 1024;
constexpr int kMRows = 32;
constexpr int kUnits = kMRows * (kDLat / 8);   // 2048 (row, 8-column) units

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float x) {
  unsigned int u = __builtin_bit_cast(unsigned int, x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __builtin_bit_cast(float, (unsigned int)h << 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

__global__ __launch_bounds__(kMThreads) void merge_kernel(const _Float16* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          const SeqInfo* __restrict__ seqinfo,
                                                          const uint16_t* __restrict__ w_uv,
                                                          float* __restrict__ out, int rows,
                                                          int q_tokens) {
  __shared__ __attribute__((aligned(16))) unsigned short lat_hi[kMRows * kDLat];
  __shared__ __attribute__((aligned(16))) unsigned short lat_lo[kMRows * kDLat];
  __shared__ __attribute__((aligned(16))) float red[16 * 64 * 16];   // 64 KB of partial sums
  __shared__ float row_m[kMRows], row_inv[kMRows];
  __shared__ int row_base[kMRows], row_cnt[kMRows], row_prow[kMRows];

  const int h = blockIdx.x;
  const int r0 = blockIdx.y * kMRows;
  const int rt = min(kMRows, rows - r0);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const size_t rpc = (size_t)q_tokens * kHeads;   // partial rows per split slot

  // W_UV fragments for phase 2, issued first so they arrive during the merge:
  // wave w covers value tile vt = w % 4 (32 values) and latent quarter kq = w / 4.
  const int vt = w & 3, kq = w >> 2;
  bf16x8 wa[8];
  {
    const uint16_t* src = w_uv + ((size_t)h * kDV + 32 * vt + l32) * kDLat + 128 * kq + 8 * half;
#pragma unroll
    for (int k = 0; k < 8; ++k) wa[k] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + 16 * k));
  }

  // ---- 1a: per-row max and normaliser
  for (int rl = w; rl < kMRows; rl += 16) {
    float mx = -INFINITY, den = 0.f;
    int base = 0, cnt = 0;
    size_t prow = 0;
    if (rl < rt) {
      const int r = r0 + rl;
      const SeqInfo si = seqinfo[r / q_tokens];
      prow = (size_t)(r % q_tokens) * kHeads + h;
      base = si.base;
      cnt = si.count;
      for (int s = lane; s < cnt; s += 64) mx = fmaxf(mx, part_lse[(base + s) * rpc + prow]);
      mx = wave_max(mx);
      if (mx != -INFINITY) {
        for (int s = lane; s < cnt; s += 64)
          den += __builtin_amdgcn_exp2f(part_lse[(base + s) * rpc + prow] - mx);
        den = wave_sum(den);
      }
    }
    if (lane == 0) {
      row_m[rl] = mx == -INFINITY ? 0.f : mx;
      row_inv[rl] = den > 0.f ? 1.f / den : 0.f;
      row_base[rl] = base;
      row_cnt[rl] = den > 0.f ? cnt : 0;
      row_prow[rl] = (int)prow;
    }
  }
  __syncthreads();

  // ---- 1b: weighted sums over splits. g split groups of kMThreads / g threads;
  // group sg takes splits sg, sg + g, ...
  const int active = rt * (kDLat / 8);
  int g = 1;
  while (g < 8 && g * 2 * active <= kMThreads) g *= 2;
  const int per = kMThreads / g;
  const int sg = t / per, u0 = t % per;
  // with g > 1 every active unit is below `per` (g * active <= kMThreads), so
  // one pass covers them; red holds exactly g * per units
  const int u_end = g > 1 ? per : kUnits;
  for (int u = u0; u < u_end; u += per) {
    const int rl = u >> 6, c = u & 63;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const int cnt = row_cnt[rl];
    if (cnt > 0) {
      const float mr = row_m[rl], inv = row_inv[rl];
      const size_t prow = (size_t)row_prow[rl];
      const int base = row_base[rl];
#pragma unroll 4
      for (int s = sg; s < cnt; s += g) {
        const size_t pr = (base + s) * rpc + prow;
        const float ws = __builtin_amdgcn_exp2f(part_lse[pr] - mr) * inv;
        const f16x8 v = __builtin_bit_cast(f16x8, *(const u32x4*)(part_o + pr * kDLat + 8 * c));
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += ws * (float)v[e];
      }
    }
    if (g == 1) {
      unsigned short hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = f32_to_bf16_rne(acc[e]);
        lo[e] = f32_to_bf16_rne(acc[e] - bf16_to_f32(hi[e]));
      }
      u32x4 vh, vl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vh[e] = (unsigned int)hi[2 * e] | ((unsigned int)hi[2 * e + 1] << 16);
        vl[e] = (unsigned int)lo[2 * e] | ((unsigned int)lo[2 * e + 1] << 16);
      }
      const int off = rl * kDLat + 8 * (c ^ (rl & 7));
      *(u32x4*)(lat_hi + off) = vh;
      *(u32x4*)(lat_lo + off) = vl;
    } else {
      float* dstp = red + ((size_t)sg * per + u) * 8;
      *(f32x4*)dstp = f32x4{acc[0], acc[1], acc[2], acc[3]};
      *(f32x4*)(dstp + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
  }
  if (g > 1) {
    __syncthreads();
    for (int u = t; u < kUnits; u += kMThreads) {
      const int rl = u >> 6, c = u & 63;
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (u < per) {
        for (int k = 0; k < g; ++k) {
          const float* srcp = red + ((size_t)k * per + u) * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += srcp[e];
        }
      }
      unsigned short hi[8], lo[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        hi[e] = f32_to_bf16_rne(acc[e]);
        lo[e] = f32_to_bf16_rne(acc[e] - bf16_to_f32(hi[e]));
      }
      u32x4 vh, vl;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vh[e] = (unsigned int)hi[2 * e] | ((unsigned int)hi[2 * e + 1] << 16);
        vl[e] = (unsigned int)lo[2 * e] | ((unsigned int)lo[2 * e + 1] << 16);
      }
      const int off = rl * kDLat + 8 * (c ^ (rl & 7));
      *(u32x4*)(lat_hi + off) = vh;
      *(u32x4*)(lat_lo + off) = vl;
    }
  }
  __syncthreads();

  // ---- 2: D[v, row] = sum_c W_UV[h][v][c] o_lat[row][c] over this wave's
  // latent quarter; B fragments (lane = row, 8 consecutive c) from LDS
  f32x16 acc = {};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int gi = (16 * kq + 2 * k + half) ^ (l32 & 7);
    const bf16x8 bh = __builtin_bit_cast(bf16x8, *(const u32x4*)(lat_hi + l32 * kDLat + 8 * gi));
    const bf16x8 bl = __builtin_bit_cast(bf16x8, *(const u32x4*)(lat_lo + l32 * kDLat + 8 * gi));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[k], bh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[k], bl, acc, 0, 0, 0);
  }
  {
    float* dstp = red + ((size_t)(kq * 4 + vt) * 64 + lane) * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(f32x4*)(dstp + 4 * q) = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
  }
  __syncthreads();
  if (w < 4) {
    f32x16 sum = {};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float* srcp = red + ((size_t)(k * 4 + w) * 64 + lane) * 16;
#pragma unroll
      for (int e = 0; e < 16; ++e) sum[e] += srcp[e];
    }
    const int r = r0 + l32;
    if (l32 < rt) {
      // sum[4 q + e] is value 32 w + 8 q + 4 half + e of row r
      float* dst = out + ((size_t)r * kHeads + h) * kDV + 32 * w + 4 * half;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(f32x4*)(dst + 8 * q) = f32x4{sum[4 * q], sum[4 * q + 1], sum[4 * q + 2], sum[4 * q + 3]};
    }
  }
}

}  // namespace

hipError_t launch_merge(const _Float16* part_o, const float* part_lse, const SeqInfo* seqinfo,
                        const uint16_t* w_uv, float* out, int batch, int q_tokens,
                        hipStream_t stream) {
  const int rows = batch * q_tokens;
  hipLaunchKernelGGL(merge_kernel, dim3(kHeads, (rows + kMRows - 1) / kMRows), dim3(kMThreads), 0,
                     stream, part_o, part_lse, seqinfo, w_uv, out, rows, q_tokens);
  return hipGetLastError();
}

}  // namespace mla
