// Weight-stream product for a few dozen tokens:
//   D[split][t][n] = sum_{k in the split's K range} W[n][k] x[t][k]
// W bf16 [N][ldw] row-major, x bf16 or fp32 [tokens][ldx] row-major, D fp32.
// Every W byte is used by only the batch's tokens, so the bound is HBM on W.
//
// Workgroup = 32 columns (n) x one K range; its 4 wavefronts split the range
// (kKPerWave each) and each streams its weight and input tiles (chunks of 64
// k) through its own 3-stage LDS ring with direct-to-LDS fetches laid out so
// that every 1 KB fetch covers 8 whole cache lines (fragments loaded straight
// from global memory touch 32 rows per instruction and starve the load path).
// Two chunks stay in flight per wavefront; the waits are explicit and the
// loop has no barrier. 32x32x16 bf16 MFMA, fp32 accumulation; an fp32 input
// enters as x = hi + lo (hi = bf16(x), lo = bf16(x - hi): within 2^-17 of x),
// two MFMAs per k-step. The 4 wavefront tiles are summed in LDS in a fixed
// order (deterministic) and stored as fp32 at
//   out + blockIdx.y * out_split + t * ldo + n.
// Grid: (N / 32, number of K splits); split s covers k in
// [s * 4 * kKPerWave, (s + 1) * 4 * kKPerWave). More than 32 tokens loop over
// row tiles (each re-streams the slice).
#pragma once

#include "common.h"

namespace mla {
namespace ws {

constexpr int kThreads = 256;
constexpr int kChunk = 64;                     // k per staged chunk (4 k-steps)
constexpr int kRing = 3;                       // chunks resident per wavefront
constexpr int kWTile = 32 * kChunk * 2;        // 4 KB: 32 weight rows x 64 bf16

template <bool kXF32>
struct Tiles {
  static constexpr int kXTile = 32 * kChunk * (kXF32 ? 4 : 2);   // inputs of 32 tokens
  static constexpr int kStage = kWTile + kXTile;
  static constexpr int kWaveLds = kRing * kStage;
  static constexpr int kLds = 4 * kWaveLds;
  static constexpr int kDmaPerChunk = (kWTile + kXTile) / 1024;
};

#define WS_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")
#define WS_WAIT_LGKM0() asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory")

// One direct-to-LDS fetch: 64 lanes x 16 bytes from base + voff (per lane) to
// LDS bytes [lds, lds + 1024), lane l at lds + 16 l. Inline asm so that the
// compiler does not drain it before every LDS read; the kernel orders it with
// its own waits. No VGPR result.
__device__ __forceinline__ void dma16(const char* lds, const char* base, unsigned voff) {
  const unsigned m0 = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(base)
               : "m0");
}

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

template <bool kXF32, int kKPerWave>
__global__ __launch_bounds__(kThreads, 1) void wstream_kernel(const void* __restrict__ x, long long ldx,
                                                              const uint16_t* __restrict__ w,
                                                              long long ldw, float* __restrict__ out,
                                                              long long ldo, long long out_split,
                                                              int rows) {
  using T = Tiles<kXF32>;
  constexpr int kChunks = kKPerWave / kChunk;
  constexpr int kXBytes = kXF32 ? 4 : 2;
  static_assert(kKPerWave % kChunk == 0, "whole chunks");
  static_assert(T::kLds <= 160 * 1024, "LDS of one gfx950 workgroup");
  __shared__ __attribute__((aligned(1024))) char smem[T::kLds];
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n0 = blockIdx.x * 32;
  const long long kw = (long long)blockIdx.y * 4 * kKPerWave + (long long)wv * kKPerWave;
  char* ring = smem + wv * T::kWaveLds;

  // Weight tile, fetch i (0..3): lane = (row 8 i + lane / 8, 16-byte piece
  // lane % 8 of the row's 128 bytes): 8 whole cache lines per fetch. Offsets
  // are relative to the tile's first row and the wavefront's first k, which
  // go into the scalar base with the chunk advance.
  unsigned voff_w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff_w[i] = (unsigned)(((8 * i + (lane >> 3)) * ldw + 8 * (lane & 7)) * 2);
  const char* w_tile = (const char*)(w + (size_t)n0 * ldw + kw);

  for (int r0 = 0; r0 < rows; r0 += 32) {
    // Input tile: fp32 rows are 256 bytes per chunk (fetch i: token
    // 4 i + lane / 16, piece lane % 16), bf16 rows 128 bytes (fetch i: token
    // 8 i + lane / 8, piece lane % 8). Tokens past the batch read the tile's
    // first token: their columns of D are never stored.
    constexpr int kXFetch = T::kXTile / 1024;
    unsigned voff_x[kXFetch];
#pragma unroll
    for (int i = 0; i < kXFetch; ++i) {
      const int tt = kXF32 ? 4 * i + (lane >> 4) : 8 * i + (lane >> 3);
      const int piece = kXF32 ? (lane & 15) : (lane & 7);
      voff_x[i] = (unsigned)(((r0 + tt < rows ? tt : 0) * ldx) * kXBytes + 16 * piece);
    }
    const char* x_tile = (const char*)x + ((size_t)r0 * ldx + kw) * kXBytes;
    auto fetch = [&](int c) {   // chunk c (clamped to the last) into its ring stage
      const int cc = c < kChunks ? c : kChunks - 1;
      char* st = ring + (c % kRing) * T::kStage;
      const char* wb = w_tile + (size_t)cc * kChunk * 2;
      const char* xb = x_tile + (size_t)cc * kChunk * kXBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) dma16(st + 1024 * i, wb, voff_w[i]);
#pragma unroll
      for (int i = 0; i < kXFetch; ++i) dma16(st + kWTile + 1024 * i, xb, voff_x[i]);
    };
#pragma unroll
    for (int c = 0; c < kRing; ++c) fetch(c);

    // fragments: A (lane = column n, half h): row n, k 16 j + 8 h; B (lane =
    // token, half h): token, k 16 j + 8 h
    const int n = lane & 31, h = lane >> 5;
    const int a_off = (n >> 3) * 1024 + (n & 7) * 128 + 16 * h;
    const int b_off = kXF32 ? kWTile + (n >> 2) * 1024 + (n & 3) * 256 + 32 * h
                            : kWTile + (n >> 3) * 1024 + (n & 7) * 128 + 16 * h;
    f32x16 acc = {};
    for (int c = 0; c < kChunks; ++c) {
      // chunk c is in: at most the two younger chunks' fetches remain
      if constexpr (kXF32) {
        WS_WAIT_VM(24);
      } else {
        WS_WAIT_VM(16);
      }
      const char* st = ring + (c % kRing) * T::kStage;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(st + a_off + 32 * j));
        if constexpr (kXF32) {
          const f32x4 xa = *(const f32x4*)(st + b_off + 64 * j);
          const f32x4 xb = *(const f32x4*)(st + b_off + 64 * j + 16);
          bf16x8 hi, lo;
          split_bf16(xa, xb, hi, lo);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hi, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lo, acc, 0, 0, 0);
        } else {
          const bf16x8 b = __builtin_bit_cast(bf16x8, *(const u32x4*)(st + b_off + 32 * j));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
        }
      }
      WS_WAIT_LGKM0();        // this stage's reads are done before its refill lands
      fetch(c + kRing);       // past the end: the last chunk again, into a spent stage
    }
    WS_WAIT_VM(0);
    __syncthreads();   // every wavefront is done with its ring: reuse it for the sum
    float(*red)[32][33] = (float(*)[32][33])smem;   // [wave][column][token]
    // acc[i] is column 8 (i / 4) + 4 (lane / 32) + i % 4 of token lane % 32
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wv][8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)][lane & 31] = acc[i];
    __syncthreads();
    {
      const int rr = t >> 3, nq = (t & 7) * 4;   // token, first of 4 columns
      if (r0 + rr < rows) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = ((red[0][nq + e][rr] + red[1][nq + e][rr]) + red[2][nq + e][rr]) + red[3][nq + e][rr];
        *(f32x4*)(out + (size_t)blockIdx.y * out_split + (size_t)(r0 + rr) * ldo + n0 + nq) = v;
      }
    }
    __syncthreads();
  }
}

}  // namespace ws
}  // namespace mla
