// Weight-stream product for a few dozen tokens:
//   D[t][n] = sum_k W[n][k] x[t][k]
// with W bf16 [N][K] and x bf16 or fp32 [tokens][K]. Every weight byte is used
// by only the batch's tokens, so the bound is HBM on W.
//
// Layouts. The matrix cores take 32x32x16 bf16 steps: operand A (the weight)
// is one 16-byte fragment per lane, lane l holding row n = l % 32 and the 8
// consecutive k at 8 (l / 32) of a 16-wide k-step. Both operands are stored
// in that fragment order, so that every wavefront load is one contiguous
// 1 KB (8 whole cache lines) and goes straight into registers:
//  * packed weight (made once, at load time, by pack_w_kernel): the 1 KB block
//    of column tile ct (32 rows of W) and k-step ks sits at byte
//    (ks * N/32 + ct) * 1024; lane l's 16 bytes are W[32 ct + l % 32][16 ks +
//    8 (l / 32) .. + 7]. The k-step is the outer index: the wavefronts that
//    stream one K range at the same time read one compact address window.
//  * packed input (per call, pack_x_kernel, or written in this order by the
//    producing epilogue): row tile rt (32 tokens), k-step ks; bf16: 1 KB at
//    (rt * K/16 + ks) * 1024, lane l: x[32 rt + l % 32][16 ks + 8 (l / 32) ..
//    + 7]; fp32: 2 KB at (rt * K/16 + ks) * 2048, half q at + 1024 q, lane l:
//    x[32 rt + l % 32][16 ks + 8 (l / 32) + 4 q .. + 3]. Tokens past the batch
//    are zero.
//
// stream_kernel: workgroup = kCT column tiles (32 kCT columns) x one K range
// of one row tile; its 4 wavefronts split the range (ks_per_wave k-steps
// each). Each wavefront keeps kDepth k-steps of fragments in flight in a
// register ring (weights with non-temporal loads, so that they do not evict
// the inputs that every column block re-reads), no LDS and no barrier in the
// loop. fp32 inputs enter as x = hi + lo (hi = bf16(x), lo = bf16(x - hi),
// together within 2^-17 of x), two MFMAs per k-step; accumulation in fp32.
// The 4 wavefront tiles are summed in LDS in a fixed order. With one K split
// the epilogue receives the finished values; with several each split stores
// its partial tile and sum_kernel adds the splits in split order and calls the
// epilogue. No atomics: results are deterministic. (A split-K finish inside
// the stream, the last workgroup of a column block adding the others' tiles,
// needs device-scope release/acquire fences between workgroups on different
// XCDs; they write back and invalidate the whole L2 and measured slower than
// the separate sum.)
#pragma once

#include "common.h"

namespace mla {
namespace ws {

constexpr int kThreads = 256;

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

// Byte offset of the 16-byte piece holding x[r][c .. c + 3] (c % 4 == 0) in
// the packed fp32 input layout of a K-wide input (k_steps = K / 16).
__device__ __forceinline__ size_t packed_f32_piece(int r, int c, int k_steps) {
  const int rt = r >> 5, n = r & 31, ks = c >> 4, h = (c >> 3) & 1, q = (c >> 2) & 1;
  return (((size_t)rt * k_steps + ks) * 2 + q) * 1024 + 16 * (n + 32 * h);
}

// Packs the input: workgroup = one row tile x kPackSteps k-steps. The 32
// rows' slices are read with whole-row-segment loads into LDS, then written
// out in the packed order (one contiguous block of kPackSteps pieces of 1 or
// 2 KB). Tokens past `rows` are written as zeros.
constexpr int kPackSteps = 8;
template <bool kXF32>
__global__ __launch_bounds__(256) void pack_x_kernel(const void* __restrict__ x, u32x4* __restrict__ p, int rows,
                                                     int k_steps) {
  constexpr int kEl = kXF32 ? 4 : 2;                       // bytes per element
  constexpr int kRowBytes = kPackSteps * 16 * kEl;         // a row's slice: 512 or 256 bytes
  constexpr int kPieces = 32 * kRowBytes / 16;             // 16-byte pieces in the tile
  __shared__ u32x4 tile[32][kRowBytes / 16 + 1];           // padded rows
  const int rt = blockIdx.y, ks0 = blockIdx.x * kPackSteps, t = threadIdx.x;
  const size_t ld = (size_t)16 * k_steps * kEl;            // bytes per input row
  for (int i = t; i < kPieces; i += 256) {
    const int row = i / (kRowBytes / 16), pc = i % (kRowBytes / 16);
    const int r = 32 * rt + row;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows) v = *(const u32x4*)((const char*)x + (size_t)r * ld + (size_t)ks0 * 16 * kEl + 16 * pc);
    tile[row][pc] = v;
  }
  __syncthreads();
  // piece i of the output block: k-step j, (half q), lane l = n + 32 h
  for (int i = t; i < kPieces; i += 256) {
    const int per = kXF32 ? 128 : 64;
    const int j = i / per, rem = i % per, q = kXF32 ? rem / 64 : 0, lane = rem % 64;
    const int n = lane & 31, h = lane >> 5;
    const int pc = (j * 16 + 8 * h + 4 * q) * kEl / 16;   // 16-byte piece within the row slice
    p[((size_t)rt * k_steps + ks0) * per + i] = tile[n][pc];
  }
}

struct StreamArgs {
  const u32x4* xp;    // packed input
  const u32x4* wp;    // packed weight
  int n_tiles;        // its column tiles (its N / 32)
  int k_steps;        // K / 16
  int rows;           // tokens
  int ks_per_wave;    // k-steps per wavefront (a multiple of kDepth, >= kDepth)
  // optional second weight with the same K, packed on its own: column blocks
  // cb >= cb2 stream wp2 (column block cb - cb2 of it); their outputs follow
  // the first weight's columns
  const u32x4* wp2;
  int n_tiles2;
  int cb2;
};

template <bool kXF32, int kCT>
struct Step {
  u32x4 w[kCT];
  u32x4 x[kXF32 ? 2 : 1];
};

// Grid (n_tiles / kCT, splits, row tiles). Wavefront w of workgroup (cb, s)
// covers k-steps [(4 s + w) * ks_per_wave, + ks_per_wave). Epi is called as
// epi(r, c, v) with v = D[r][c .. c + 3], c % 4 == 0, only for r < rows.
// kXRows: a bf16 input read straight from its row-major rows (lane (n, h)
// loads its 16 bytes from row n: 32 rows per load instead of 8 cache lines,
// which costs little where the input is small and L2-resident and the stream
// is short, and saves the packing launch); rows past the batch read row 0.
template <bool kXF32, int kCT, int kDepth, bool kXRows, class Epi>
__global__ __launch_bounds__(kThreads, 1) void stream_kernel(StreamArgs a, Epi epi) {
  static_assert(!(kXF32 && kXRows), "row-major input only for bf16");
  __shared__ float red[4][kCT * 32][33];   // [wave][column][token], padded
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int cb = blockIdx.x, rt = blockIdx.z;
  const int ks0 = (blockIdx.y * 4 + wv) * a.ks_per_wave;
  const int n = lane & 31, h = lane >> 5;
  constexpr int kXPer = kXF32 ? 128 : 64;   // 16-byte pieces per input k-step
  const bool second = cb >= a.cb2;
  const u32x4* wbase = (second ? a.wp2 + (size_t)(cb - a.cb2) * kCT * 64 : a.wp + (size_t)cb * kCT * 64) + lane;
  const size_t wstep = (size_t)(second ? a.n_tiles2 : a.n_tiles) * 64;
  const u32x4* xbase =
      kXRows ? (const u32x4*)((const uint16_t*)a.xp +
                              (size_t)(32 * rt + n < a.rows ? 32 * rt + n : 0) * (16 * (size_t)a.k_steps) +
                              16 * (size_t)ks0 + 8 * h)
             : a.xp + ((size_t)rt * a.k_steps + ks0) * kXPer + lane;
  constexpr int kXStep = kXRows ? 2 : kXPer;   // 16-byte units from one k-step to the next

  Step<kXF32, kCT> ring[kDepth];
  auto load = [&](Step<kXF32, kCT>& st, int s) {
    const u32x4* wb = wbase + (size_t)(ks0 + s) * wstep;
#pragma unroll
    for (int j = 0; j < kCT; ++j) st.w[j] = __builtin_nontemporal_load(wb + 64 * j);
    const u32x4* xb = xbase + (size_t)s * kXStep;
    st.x[0] = xb[0];
    if constexpr (kXF32) st.x[1] = xb[64];
  };
  f32x16 acc[kCT];
#pragma unroll
  for (int j = 0; j < kCT; ++j) acc[j] = f32x16{};
  auto compute = [&](const Step<kXF32, kCT>& st) {
    if constexpr (kXF32) {
      bf16x8 hi, lo;
      split_bf16(__builtin_bit_cast(f32x4, st.x[0]), __builtin_bit_cast(f32x4, st.x[1]), hi, lo);
#pragma unroll
      for (int j = 0; j < kCT; ++j) {
        const bf16x8 wf = __builtin_bit_cast(bf16x8, st.w[j]);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, hi, acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, lo, acc[j], 0, 0, 0);
      }
    } else {
      const bf16x8 b = __builtin_bit_cast(bf16x8, st.x[0]);
#pragma unroll
      for (int j = 0; j < kCT; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, st.w[j]), b, acc[j], 0, 0,
                                                         0);
    }
  };
  // The scheduling barriers keep every step's loads in issue order (the
  // compiler otherwise sinks the refills to the end of the unrolled round and
  // drains the ring): each step's wait leaves the kDepth - 1 younger steps in
  // flight.
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    load(ring[d], d);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int s = 0; s < a.ks_per_wave - kDepth; s += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      compute(ring[d]);
      __builtin_amdgcn_sched_barrier(0);
      load(ring[d], s + d + kDepth);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int d = 0; d < kDepth; ++d) compute(ring[d]);

  // acc[j][i] is column 32 j + 8 (i / 4) + 4 h + i % 4 of token n
#pragma unroll
  for (int j = 0; j < kCT; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wv][32 * j + 8 * (i >> 2) + 4 * h + (i & 3)][n] = acc[j][i];
  __syncthreads();
  const int c0 = cb * kCT * 32;
  for (int e = t; e < 32 * kCT * 8; e += kThreads) {   // (token, 4 columns)
    const int rr = e / (kCT * 8), c4 = (e % (kCT * 8)) * 4;
    const int r = 32 * rt + rr;
    if (r >= a.rows) continue;
    f32x4 v;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = ((red[0][c4 + q][rr] + red[1][c4 + q][rr]) + red[2][c4 + q][rr]) + red[3][c4 + q][rr];
    epi(r, c0 + c4, v);
  }
}

// A K split's partial sums: [split][rows][n] fp32, split = blockIdx.y.
struct StorePartial {
  float* part;
  int rows, n;
  __device__ void operator()(int r, int c, f32x4 v) const {
    *(f32x4*)(part + ((size_t)blockIdx.y * rows + r) * n + c) = v;
  }
};

// Sums the K splits in split order: one thread per (token, 4 columns); all
// of a thread's loads are issued before the first add.
template <int kSplits, class Epi>
__global__ __launch_bounds__(256) void sum_kernel(const float* __restrict__ part, int rows, int n, Epi epi) {
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= (long long)rows * (n / 4)) return;
  const int r = (int)(g / (n / 4)), c = (int)(g % (n / 4)) * 4;
  const size_t split = (size_t)rows * n;
  f32x4 u[kSplits];
#pragma unroll
  for (int s = 0; s < kSplits; ++s) u[s] = *(const f32x4*)(part + s * split + (size_t)r * n + c);
  f32x4 v = u[0];
#pragma unroll
  for (int s = 1; s < kSplits; ++s) v += u[s];
  epi(r, c, v);
}

// Host side: a product's shape and tiling, fixed at compile time. kXRows:
// the (bf16) input is passed row-major, without the packing launch.
template <bool kXF32, int kN, int kK, int kCT, int kDepth, int kSplits, bool kXRows = false>
struct Plan {
  static constexpr int kNTiles = kN / 32, kKSteps = kK / 16;
  static constexpr int kKsPerWave = kKSteps / (4 * kSplits);
  static_assert(kN % (32 * kCT) == 0, "whole column blocks");
  static_assert(kKSteps % (4 * kSplits) == 0, "whole k-steps per wavefront");
  static_assert(kKsPerWave % kDepth == 0 && kKsPerWave >= kDepth, "whole ring rounds");
  static_assert(4 * kCT * 32 * 33 * 4 <= 160 * 1024, "LDS of one gfx950 workgroup");

  static size_t packed_x_bytes(int rows) {
    return kXRows ? 0 : (size_t)((rows + 31) / 32) * 32 * kK * (kXF32 ? 4 : 2);
  }
  static size_t part_bytes(int rows) { return kSplits > 1 ? (size_t)kSplits * rows * kN * sizeof(float) : 0; }

  static hipError_t pack_x(const void* x, void* xp, int rows, hipStream_t stream) {
    static_assert(!kXRows, "a row-major input is not packed");
    static_assert(kKSteps % kPackSteps == 0, "whole packing tiles");
    hipLaunchKernelGGL(pack_x_kernel<kXF32>, dim3(kKSteps / kPackSteps, (rows + 31) / 32), dim3(256), 0, stream, x,
                       (u32x4*)xp, rows, kKSteps);
    return hipGetLastError();
  }
  // The product of the input xp (packed, or row-major with kXRows) and the
  // packed weight wp, finished by
  // epi: one launch with one split, else the stream into `part`
  // (part_bytes(rows)) and the split-order sum.
  template <class Epi>
  static hipError_t run(const void* xp, const void* wp, float* part, int rows, Epi epi, hipStream_t stream) {
    return run2(xp, wp, kN, nullptr, part, rows, epi, stream);
  }
  // The same with two weights of this K side by side: wp's n1 columns, then
  // wp2's kN - n1 (n1 a multiple of 32 kCT).
  template <class Epi>
  static hipError_t run2(const void* xp, const void* wp, int n1, const void* wp2, float* part, int rows, Epi epi,
                         hipStream_t stream) {
    const StreamArgs a{(const u32x4*)xp, (const u32x4*)wp, n1 / 32,          kKSteps,
                       rows,             kKsPerWave,       (const u32x4*)wp2, (kN - n1) / 32,
                       n1 / (32 * kCT)};
    const dim3 grid(kNTiles / kCT, kSplits, (rows + 31) / 32);
    if (kSplits > 1 && part == nullptr) return hipErrorInvalidValue;   // split sums need their buffer
    if (n1 % (32 * kCT) != 0 || n1 > kN || (n1 < kN && wp2 == nullptr)) return hipErrorInvalidValue;
    if constexpr (kSplits == 1) {
      hipLaunchKernelGGL((stream_kernel<kXF32, kCT, kDepth, kXRows, Epi>), grid, dim3(kThreads), 0, stream, a,
                         epi);
      return hipGetLastError();
    } else {
      hipLaunchKernelGGL((stream_kernel<kXF32, kCT, kDepth, kXRows, StorePartial>), grid, dim3(kThreads), 0,
                         stream, a, StorePartial{part, rows, kN});
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const long long items = (long long)rows * (kN / 4);
      hipLaunchKernelGGL((sum_kernel<kSplits, Epi>), dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream,
                         part, rows, kN, epi);
      return hipGetLastError();
    }
  }
};

// fp32 rows of `ld` floats.
struct StoreF32 {
  float* out;
  long long ld;
  __device__ void operator()(int r, int c, f32x4 v) const { *(f32x4*)(out + (size_t)r * ld + c) = v; }
};

// The packed fp32 input layout of a following product with k_steps = N / 16.
struct StorePackedF32 {
  char* out;
  int k_steps;
  __device__ void operator()(int r, int c, f32x4 v) const { *(f32x4*)(out + packed_f32_piece(r, c, k_steps)) = v; }
};

}  // namespace ws
}  // namespace mla
