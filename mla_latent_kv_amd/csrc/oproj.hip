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
#include "common.h"

namespace mla {

namespace {

constexpr int kOpThreads = 256;
constexpr int kOpK = kHeads * kDV;                  // 16384
constexpr int kOpKPerWave = kOpK / 4;               // 4096
constexpr int kOpChunk = 64;                        // k per staged chunk (4 k-steps)
constexpr int kOpChunks = kOpKPerWave / kOpChunk;   // 64 chunks per wavefront
constexpr int kOpRing = 3;                          // chunks resident per wavefront
constexpr int kOpWTile = 32 * kOpChunk * 2;         // 4 KB: 32 weight rows x 64 bf16
constexpr int kOpXTile = 32 * kOpChunk * 4;         // 8 KB: 32 tokens x 64 fp32
constexpr int kOpStage = kOpWTile + kOpXTile;       // 12 KB
constexpr int kOpWaveLds = kOpRing * kOpStage;      // 36 KB per wavefront
constexpr int kOpLds = 4 * kOpWaveLds;              // 144 KB
constexpr int kOpDmaPerChunk = kOpWTile / 1024 + kOpXTile / 1024;   // 12
static_assert(kDHidden % 32 == 0 && kOpKPerWave % kOpChunk == 0, "tiling");
static_assert(kOpLds <= 160 * 1024, "LDS of one gfx950 workgroup");

#define OP_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")
#define OP_WAIT_LGKM0() asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory")

// One direct-to-LDS fetch: 64 lanes x 16 bytes from base + voff (per lane) to
// LDS bytes [lds, lds + 1024), lane l at lds + 16 l. Inline asm so that the
// compiler does not drain it before every LDS read; the kernel orders it with
// its own waits. No VGPR result.
__device__ __forceinline__ void op_dma16(const char* lds, const char* base, unsigned voff) {
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

__global__ __launch_bounds__(kOpThreads, 1) void oproj_kernel(const float* __restrict__ x,
                                                              const uint16_t* __restrict__ w_o,
                                                              float* __restrict__ y, int rows) {
  __shared__ __attribute__((aligned(1024))) char smem[kOpLds];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n0 = blockIdx.x * 32;
  char* ring = smem + w * kOpWaveLds;

  // DMA lanes. Weight tile, fetch i (0..3): lane = (row 8 i + lane / 8, 16-byte
  // piece lane % 8 of the row's 128 bytes), so each fetch reads 8 whole cache
  // lines. Byte offsets within W_O (< 2^32: 235 MB); the chunk advance goes
  // into the scalar base.
  unsigned voff_w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    voff_w[i] = (unsigned)(((size_t)(n0 + 8 * i + (lane >> 3)) * kOpK + w * kOpKPerWave + 8 * (lane & 7)) * 2);

  for (int r0 = 0; r0 < rows; r0 += 32) {
    // Input tile, fetch i (0..7): lane = (token 4 i + lane / 16, 16-byte piece
    // lane % 16 of the token's 256 bytes). Tokens past the batch read the
    // tile's first token: their columns of D are never stored.
    // Offsets are relative to the tile's first token (< 2 MB), whose address
    // goes into the scalar base with the chunk advance.
    unsigned voff_x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tt = 4 * i + (lane >> 4);
      voff_x[i] = (unsigned)(((r0 + tt < rows ? tt : 0) * kOpK + w * kOpKPerWave + 4 * (lane & 15)) * 4);
    }
    const char* x_tile = (const char*)(x + (size_t)r0 * kOpK);
    auto fetch = [&](int c) {   // chunk c (clamped to the last) into its ring stage
      const int cc = c < kOpChunks ? c : kOpChunks - 1;
      char* st = ring + (c % kOpRing) * kOpStage;
      const char* wb = (const char*)w_o + (size_t)cc * kOpChunk * 2;
      const char* xb = x_tile + (size_t)cc * kOpChunk * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) op_dma16(st + 1024 * i, wb, voff_w[i]);
#pragma unroll
      for (int i = 0; i < 8; ++i) op_dma16(st + kOpWTile + 1024 * i, xb, voff_x[i]);
    };
    for (int c = 0; c < kOpRing; ++c) fetch(c);

    // fragment reads: A (lane = column n, half h): row n, k 16 j + 8 h;
    // B (lane = token t, half h): token t, k 16 j + 8 h (8 fp32 = 2 reads)
    const int n = lane & 31, h = lane >> 5;
    const int a_off = (n >> 3) * 1024 + (n & 7) * 128 + 16 * h;
    const int b_off = kOpWTile + (n >> 2) * 1024 + (n & 3) * 256 + 32 * h;
    f32x16 acc = {};
    for (int c = 0; c < kOpChunks; ++c) {
      OP_WAIT_VM(24);   // chunk c is in: at most the two younger chunks' 24 fetches remain
      const char* st = ring + (c % kOpRing) * kOpStage;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)(st + a_off + 32 * j));
        const f32x4 xa = *(const f32x4*)(st + b_off + 64 * j);
        const f32x4 xb = *(const f32x4*)(st + b_off + 64 * j + 16);
        bf16x8 hi, lo;
        split_bf16(xa, xb, hi, lo);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, hi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, lo, acc, 0, 0, 0);
      }
      OP_WAIT_LGKM0();   // this stage's reads are done before its refill lands
      fetch(c + kOpRing);   // past the end: the last chunk again, into a spent stage
    }
    OP_WAIT_VM(0);
    __syncthreads();   // every wavefront is done with its ring: reuse it for the sum
    float(*red)[32][33] = (float(*)[32][33])smem;   // [wave][column][token]
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
