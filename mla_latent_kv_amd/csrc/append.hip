// Cache-append producer: the rows a decode step's new tokens add to the paged
// latent cache,
//   c_KV = W_DKV h           (7168 -> 512)
//   k_R  = RoPE(W_KR h, pos) (7168 -> 64), pos = L_b - Sq + i
// stored as one 576-wide bf16 row [c_KV | k_R] in block
// block_table[b, pos / 64], slot pos % 64. Each token keeps only the short
// joint latent and the small head-shared position key, the latter rotated by
// its position ("DeepSeek-V3" article at m.lsln.cn, sections 2.2 and 2.3;
// "DeepSeek-V3" page at ailearn.mscapital.top, MLA paragraphs). RoPE turns
// consecutive pairs (x_2i, x_2i+1) counter-clockwise by pos * base^(-2i/64).
//
// Two launches:
//  1. split-K product on the matrix cores. The weights are one logical
//     [576][7168] matrix (W_DKV rows, then W_KR rows): 18 column tiles of 32 x
//     16 K-chunks of 448 = 288 workgroups, each reading its 28 KB weight slice
//     once (the whole 8.3 MB crosses HBM once) and applying it to every new
//     token. D[n, r] = sum_k W[n][k] h[r][k] on 32x32x16 bf16 MFMA: both
//     operands are row-major with k contiguous, so every fragment is one
//     16-byte load from global memory. The 4 wavefronts split the chunk's 28
//     k-steps and their partial tiles are summed in LDS in a fixed order; the
//     workgroup writes one fp32 partial per (chunk, token, column).
//  2. finish: each thread sums one column pair over the 16 chunks in a fixed
//     order, rotates it (RoPE pairs; angles in fp64, so positions up to 2^31
//     keep their phase), rounds to bf16 (nearest, ties to even) and writes 4
//     bytes of the token's cache row. No atomics: results are deterministic.
#include "common.h"

namespace mla {

namespace {

constexpr int kAppThreads = 256;
constexpr int kAppNTiles = kRow / 32;                  // 18 column tiles
constexpr int kAppKSteps = kDHidden / 16;              // 448 k-steps of 16
constexpr int kAppStepsPerWg = kAppKSteps / kAppKSplit;   // 28
constexpr int kAppStepsPerWave = kAppStepsPerWg / 4;      // 7
static_assert(kAppKSteps % kAppKSplit == 0 && kAppStepsPerWg % 4 == 0, "K split");
static_assert(kDLat % 32 == 0, "a column tile is all latent or all RoPE");

__device__ __forceinline__ unsigned int bf16_rne_bits(float x) {
  unsigned int u = __builtin_bit_cast(unsigned int, x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__global__ __launch_bounds__(kAppThreads) void append_gemm_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ w_dkv,
    const uint16_t* __restrict__ w_kr, float* __restrict__ part, int rows) {
  __shared__ float red[4][32][33];   // [wave][column][token], padded
  const int nt = blockIdx.x % kAppNTiles, ks = blockIdx.x / kAppNTiles;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int n0 = nt * 32;
  // A operand (lane = column, 8 consecutive k): weight row n0 + lane % 32
  const uint16_t* wrow = n0 < kDLat ? w_dkv + (size_t)(n0 + (lane & 31)) * kDHidden
                                    : w_kr + (size_t)(n0 - kDLat + (lane & 31)) * kDHidden;
  const int kb = (ks * kAppStepsPerWg + w * kAppStepsPerWave) * 16 + 8 * (lane >> 5);
  bf16x8 a[kAppStepsPerWave];
#pragma unroll
  for (int j = 0; j < kAppStepsPerWave; ++j)
    a[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(wrow + kb + 16 * j));

  for (int r0 = 0; r0 < rows; r0 += 32) {
    // B operand (lane = token, 8 consecutive k); tokens past the batch are 0
    const int r = r0 + (lane & 31);
    bf16x8 bq[kAppStepsPerWave];
#pragma unroll
    for (int j = 0; j < kAppStepsPerWave; ++j)
      bq[j] = r < rows ? __builtin_bit_cast(bf16x8, *(const u32x4*)(hidden + (size_t)r * kDHidden + kb + 16 * j))
                       : bf16x8{};
    f32x16 acc = {};
#pragma unroll
    for (int j = 0; j < kAppStepsPerWave; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], bq[j], acc, 0, 0, 0);
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
        *(f32x4*)(part + ((size_t)ks * rows + r0 + rr) * kRow + n0 + nq) = v;
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kAppThreads) void append_finish_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ block_table, uint16_t* __restrict__ cache, long long num_blocks,
    int max_blocks_per_seq, int rows, int q_tokens, double rope_base) {
  const long long g = (long long)blockIdx.x * kAppThreads + threadIdx.x;
  if (g >= (long long)rows * (kRow / 2)) return;
  const int r = (int)(g / (kRow / 2)), pr = (int)(g % (kRow / 2));   // token, column pair
  float x0 = 0.f, x1 = 0.f;
#pragma unroll
  for (int ks = 0; ks < kAppKSplit; ++ks) {
    // (a bit cast applied directly to a vector element reads element 0 with
    // this compiler, so the pair is loaded as float lanes and used as is)
    const f32x2 v = *(const f32x2*)(part + ((size_t)ks * rows + r) * kRow + 2 * pr);
    x0 += v[0];
    x1 += v[1];
  }
  const int b = r / q_tokens, i = r % q_tokens;
  const int pos = seq_lens[b] - q_tokens + i;
  // no slot for this token (a length below Sq, or past the table): nothing written
  if (pos < 0 || pos / kBlock >= max_blocks_per_seq) return;
  const long long blk = block_table[(size_t)b * max_blocks_per_seq + pos / kBlock];
  if (blk < 0 || blk >= num_blocks) return;   // an invalid block id is never written through
  float y0 = x0, y1 = x1;
  if (pr >= kDLat / 2) {
    const int q = pr - kDLat / 2;   // RoPE pair
    const double theta = pow(rope_base, -2.0 * q / kDRope);
    double s, c;
    sincos((double)pos * theta, &s, &c);
    y0 = (float)((double)x0 * c - (double)x1 * s);
    y1 = (float)((double)x0 * s + (double)x1 * c);
  }
  const unsigned int packed = bf16_rne_bits(y0) | (bf16_rne_bits(y1) << 16);
  *(unsigned int*)(cache + ((size_t)blk * kBlock + pos % kBlock) * kRow + 2 * pr) = packed;
}

}  // namespace

size_t append_workspace_bytes(int rows) { return (size_t)kAppKSplit * rows * kRow * sizeof(float); }

hipError_t launch_append(const uint16_t* hidden, const uint16_t* w_dkv, const uint16_t* w_kr,
                         uint16_t* cache, const int32_t* block_table, const int32_t* seq_lens,
                         long long num_blocks, int max_blocks_per_seq, int batch, int q_tokens,
                         double rope_base, float* part, hipStream_t stream) {
  const int rows = batch * q_tokens;
  hipLaunchKernelGGL(append_gemm_kernel, dim3(kAppNTiles * kAppKSplit), dim3(kAppThreads), 0, stream,
                     hidden, w_dkv, w_kr, part, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = (long long)rows * (kRow / 2);
  hipLaunchKernelGGL(append_finish_kernel, dim3((unsigned)((n + kAppThreads - 1) / kAppThreads)),
                     dim3(kAppThreads), 0, stream, part, seq_lens, block_table, cache, num_blocks,
                     max_blocks_per_seq, rows, q_tokens, rope_base);
  return hipGetLastError();
}

}  // namespace mla
