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
// One workgroup of 8 wavefronts per (head, kR query rows), kR = 16, or 32
// when there are more than 32 rows (each workgroup loads all of W_UV[h], so
// wider groups load it fewer times; up to 32 rows the narrow groups keep at
// least one workgroup per CU, which measured faster). The row groups of one head run on one
// XCD (ids 8 apart), so W_UV[h] crosses HBM once and is then served by that
// XCD's L2.
//  1. thread (row, slot) sums 64 / (512 / kR) units of 8 latent values over
//     the row's splits, several splits per round trip (their lse values and
//     16-byte partial loads together; the slots of a row read contiguous
//     bytes of a partial row), with a running max across rounds; o_lat goes
//     to LDS as bf16 hi + lo (hi = bf16(x), lo = bf16(x - hi), together
//     within 2^-16 of x).
//  2. out^T[v, r] = W_UV[h][v, :] . o_lat[r, :] on 16x16x32 bf16 MFMA (W_UV
//     exact, hi and lo accumulated in fp32), 16 rows per MFMA: wavefront w owns
//     value tile w (16 values); up to 128 rows its W_UV fragments are loaded
//     at the start and arrive while phase 1 runs. Above 128 rows (four or more
//     workgroups per CU) they are loaded after phase 1, which keeps the
//     workgroup within 128 VGPRs so that two share a CU and one's loads are in
//     flight while the other computes (256 rows: 51.7 -> 42.1 us).
// No atomics: every output is written once, so results are deterministic.
#include "common.h"

namespace mla {

namespace {

constexpr int kMThreads = 512;
constexpr int kKSteps = kDLat / 32;   // 16 k-steps of 32 latent values

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float x) {
  unsigned int u = __builtin_bit_cast(unsigned int, x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __builtin_bit_cast(float, (unsigned int)h << 16);
}

// kLate: the W_UV fragments are loaded after phase 1 instead of at entry, so
// the two phases' registers do not overlap and two workgroups fit on a CU
// (one's loads in flight while the other computes): for batches of many
// workgroups per CU.
template <int kR, bool kEarly, bool kLate>
__global__ __launch_bounds__(kMThreads) __attribute__((amdgpu_waves_per_eu(kLate ? 4 : 1))) void merge_kernel(const _Float16* __restrict__ part_o,
                                                          const float* __restrict__ part_lse,
                                                          const SeqInfo* __restrict__ seqinfo,
                                                          const uint16_t* __restrict__ w_uv,
                                                          float* __restrict__ out, int rows,
                                                          int q_tokens, int groups, int max_chunks) {
  static_assert(kR == 16 || kR == 32, "16 or 32 rows per workgroup");
  constexpr int kSlots = kMThreads / kR;    // threads per row: 32 or 16
  constexpr int kUnits = 64 / kSlots;       // 16-byte units per thread and split: 2 or 4
  constexpr int kChunk = 16 / kUnits;       // splits whose loads are in flight together: 8 or 4
  // o_lat of the workgroup's rows as bf16 hi / lo: [row][64 granules of 8],
  // granule g of row r stored at g ^ (r % 16) (16 rows: 16 different bank groups)
  __shared__ __attribute__((aligned(16))) unsigned short lat[2][kR * kDLat];

  // heads x, x + 8, ... run on XCD x; the row groups of a head are consecutive there
  const int xcd = blockIdx.x & 7, seat = blockIdx.x >> 3;
  const int h = (seat / groups) * 8 + xcd;
  const int r0 = (seat % groups) * kR;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const size_t rpc = (size_t)q_tokens * kHeads;   // partial rows per split slot

  // W_UV fragments for phase 2 (A operand: lane = value, 8 consecutive latent
  // values): value tile w, k-step kk
  bf16x8 wa[kKSteps];
  auto load_wa = [&]() {
    const uint16_t* src = w_uv + ((size_t)h * kDV + 16 * w + (lane & 15)) * kDLat + 8 * (lane >> 4);
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk)
      wa[kk] = __builtin_bit_cast(bf16x8, *(const u32x4*)(src + 32 * kk));
  };
  // Loads return in order. By default the fragments go out first, under the
  // round trip of the sequence's split range. With kEarly the first chunk of
  // partials goes first and the fragments arrive while it is summed: measured
  // faster at 256 query rows (55.6 -> 51.3 us), slower at 32 and 64.
  if constexpr (!kEarly && !kLate) load_wa();

  // ---- 1: weighted sum over splits; thread = (row rl, slot g32), units g32 + kSlots k
  const int rl = t / kSlots, g32 = t % kSlots;
  const int r = r0 + rl;
  const bool live = r < rows;
  int base = 0, cnt = 0;
  size_t prow = 0;
  if (live) {
    const SeqInfo si = seqinfo[r / q_tokens];
    prow = (size_t)(r % q_tokens) * kHeads + h;
    // the slot range stays inside the partial states (memory safety only: the
    // plan never writes a range past them)
    base = min(max(si.base, 0), max_chunks);
    cnt = min(max(si.count, 0), max_chunks - base);
  }
  // chunks of kChunk splits: the lse values and the partial rows of a chunk
  // are loaded in one round trip; a running max M rescales what earlier
  // chunks added (the same regrouping as the online softmax)
  float lv[kChunk];
  f16x8 v[kChunk][kUnits];
  auto load_chunk = [&](int s0) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int s = min(s0 + i, cnt - 1);   // past the end: re-read, weight 0
      const size_t pr = (base + s) * rpc + prow;
      // unconditional load (s is a valid split; splits past the end are
      // masked where the values are used): a load under a branch makes the
      // compiler drain the queue where it rejoins
      lv[i] = part_lse[pr];
      const _Float16* src = part_o + pr * kDLat + 8 * g32;
#pragma unroll
      for (int k = 0; k < kUnits; ++k) v[i][k] = __builtin_bit_cast(f16x8, *(const u32x4*)(src + 8 * kSlots * k));
    }
  };

  if (cnt > 0) load_chunk(0);
  if constexpr (kEarly && !kLate) {
    load_wa();
    __builtin_amdgcn_sched_barrier(0);   // keeps the chunk's max below these loads
  }

  float acc[kUnits][8];
#pragma unroll
  for (int k = 0; k < kUnits; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.f;
  float mrun = -INFINITY, den = 0.f;
  for (int s0 = 0; s0 < cnt; s0 += kChunk) {
    if (s0 > 0) load_chunk(s0);
#pragma unroll
    for (int i = 1; i < kChunk; ++i)
      if (s0 + i >= cnt) lv[i] = -INFINITY;   // past the end: weight 0
    float cm = lv[0];
#pragma unroll
    for (int i = 1; i < kChunk; ++i) cm = fmaxf(cm, lv[i]);
    const float mnew = fmaxf(mrun, cm);
    // no branch on "nothing visible yet" (a branch here lets the compiler
    // sink the partial loads behind the lse values): with every lse so far
    // -inf the reference is 0, so every weight and the rescale are 0 and
    // acc and den stay 0 (the partial states are finite)
    const float mref = mnew == -INFINITY ? 0.f : mnew;
    const float sc = __builtin_amdgcn_exp2f(mrun - mref);   // 0 when mrun = -inf
    den *= sc;
#pragma unroll
    for (int k = 0; k < kUnits; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[k][e] *= sc;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const float wi = __builtin_amdgcn_exp2f(lv[i] - mref);   // 0 for -inf
      den += wi;
#pragma unroll
      for (int k = 0; k < kUnits; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[k][e] += wi * (float)v[i][k][e];
    }
    mrun = mnew;
  }
  {
    const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int k = 0; k < kUnits; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[k][e] *= inv;
  }
#pragma unroll
  for (int k = 0; k < kUnits; ++k) {
    unsigned short hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = f32_to_bf16_rne(acc[k][e]);
      lo[e] = f32_to_bf16_rne(acc[k][e] - bf16_to_f32(hi[e]));
    }
    u32x4 vh, vl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vh[e] = (unsigned int)hi[2 * e] | ((unsigned int)hi[2 * e + 1] << 16);
      vl[e] = (unsigned int)lo[2 * e] | ((unsigned int)lo[2 * e + 1] << 16);
    }
    const int g = g32 + kSlots * k;
    const int off = rl * kDLat + 8 * (g ^ (rl & 15));
    *(u32x4*)(&lat[0][off]) = vh;
    *(u32x4*)(&lat[1][off]) = vl;
  }
  if constexpr (kLate) load_wa();
  __syncthreads();

  // ---- 2: D[v, r] over 16 k-steps per 16-row tile; B fragment: lane = row
  // (lane % 16), 8 consecutive latent values from granule 4 kk + lane / 16
  const int br = lane & 15;
#pragma unroll
  for (int rt = 0; rt < kR / 16; ++rt) {
    f32x4 d = {0, 0, 0, 0};
    const int row = 16 * rt + br;
#pragma unroll
    for (int kk = 0; kk < kKSteps; ++kk) {
      const int off = row * kDLat + 8 * ((4 * kk + (lane >> 4)) ^ br);
      const bf16x8 bh = __builtin_bit_cast(bf16x8, *(const u32x4*)(&lat[0][off]));
      const bf16x8 bl = __builtin_bit_cast(bf16x8, *(const u32x4*)(&lat[1][off]));
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[kk], bh, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[kk], bl, d, 0, 0, 0);
    }
    // d[e] is value 16 w + 4 (lane / 16) + e of row r0 + row
    const int ro = r0 + row;
    if (ro < rows)
      *(f32x4*)(out + ((size_t)ro * kHeads + h) * kDV + 16 * w + 4 * (lane >> 4)) = d;
  }
}

}  // namespace

hipError_t launch_merge(const _Float16* part_o, const float* part_lse, const SeqInfo* seqinfo,
                        const uint16_t* w_uv, float* out, int batch, int q_tokens, int max_chunks,
                        hipStream_t stream) {
  const int rows = batch * q_tokens;
  if (rows <= 32) {
    // 16-row groups: at least one workgroup per CU for 32 rows
    const int groups = (rows + 15) / 16;
    hipLaunchKernelGGL((merge_kernel<16, false, false>), dim3(kHeads * groups), dim3(kMThreads), 0, stream, part_o,
                       part_lse, seqinfo, w_uv, out, rows, q_tokens, groups, max_chunks);
  } else {
    const int groups = (rows + 31) / 32;
    if (rows <= 128)
      hipLaunchKernelGGL((merge_kernel<32, false, false>), dim3(kHeads * groups), dim3(kMThreads), 0, stream, part_o,
                         part_lse, seqinfo, w_uv, out, rows, q_tokens, groups, max_chunks);
    else
      hipLaunchKernelGGL((merge_kernel<32, false, true>), dim3(kHeads * groups), dim3(kMThreads), 0, stream, part_o,
                         part_lse, seqinfo, w_uv, out, rows, q_tokens, groups, max_chunks);
  }
  return hipGetLastError();
}

}  // namespace mla
