// Preparation launch with the wide absorb tile: workgroup 0 computes the
// split plan (plan.h), every other workgroup one (4 heads, 64-wide latent
// block) tile of the absorb product q_abs[r, h, :] = W_UK[h]^T q_nope[r, h, :]
// ("DeepSeek-V3" page, ailearn.mscapital.top, MLA section; the algebra check
// in section 2 of the wq-win.github.io DeepSeek-V3 notes), in the same
// fragment order and range-flag convention as prep.hip's narrow tile. Used
// from 128 query rows on, where each q_nope row read by 8 workgroups instead
// of 16 pays for the later-arriving 128-byte W_UK pieces.
#include "common.h"
#include "plan.h"

namespace mla {

namespace {

// ---- the wide tile for many query rows: 4 heads x 64 latent columns per
// workgroup (wavefront w owns head 4 g4 + w, both 32-column tiles), half as
// many workgroups. Each workgroup applies a 64 KB slice of W_UK to every
// query row, so each q_nope row is read by 8 workgroups instead of 4 x 4
// (launch_prep in prep.hip picks the tile by row count).
constexpr int kAbsWideHeads = 4;                                // heads per wide workgroup
constexpr int kAbsWideCols = 64;                                // latent columns per wide workgroup
constexpr int kAbsWideRowBytes = kAbsWideCols * 2;              // 128: one k row of a head's slice
constexpr int kAbsWideHeadBytes = kDNope * kAbsWideRowBytes;    // 16 KB: one head's slice
constexpr int kAbsWideBytes = kAbsWideHeads * kAbsWideHeadBytes;   // 64 KB
constexpr int kAbsWideGroups = (kHeads / kAbsWideHeads) * (kDLat / kAbsWideCols);   // 256
static_assert(2 * kAbsWideGroups == kAbsorbGroups, "a wide workgroup covers two narrow ones' flags");
// one 32-row tile of the workgroup's results: 32 rows x 4 column groups of 16
// x 2 halves of 8 columns x 4 heads, 16 bytes each
constexpr int kStageGranules = 32 * 4 * 2 * kAbsWideHeads;      // 1024
constexpr int kStageBytes = kStageGranules * 16;                // 16 KB, two of them
static_assert(kStageGranules == 4 * kPrepThreads, "four granules per thread");

// Staging granule of (row in tile rl, column group c16l, half sel, head h4):
// the index runs in the order of q_abs's fragment layout (the 4 heads of the
// workgroup are 4 consecutive 16-byte slots of one line), XOR-swizzled in its
// low 4 bits by the row so that the 32 rows one staging write covers spread
// over the LDS banks.
__device__ __forceinline__ int stage_off(int g) { return 16 * (g ^ ((g >> 5) & 15)); }

// LDS byte offset of 16-byte granule g (0..7) of row k of head h4's slice.
// Rows are 128 bytes; where bit 1 of k is set the row's two 64-byte halves
// trade places, so the four consecutive rows a transposing read covers
// (32 columns each) fill all 64 banks once.
__device__ __forceinline__ int wl_off_wide(int h4, int k, int g) {
  return h4 * kAbsWideHeadBytes + k * kAbsWideRowBytes + 16 * (g ^ (4 * ((k >> 1) & 1)));
}

// One wide workgroup: heads 4 g4 .. 4 g4 + 3 x latent columns [64 cb, 64 cb +
// 64), every query row. Its slice is read as whole 128-byte lines; the 4
// heads' results fill half of each 128-byte line of q_abs (8 consecutive heads
// x 8 values), and the workgroup with the other 4 heads runs on the same XCD,
// so the halves meet in its L2. Each 32-row tile's results go through LDS
// (two 16 KB buffers in the slice's space, free once every wavefront holds
// its A fragments) so that the 4 heads leave as 64-byte runs, four
// consecutive lanes' 16-byte stores: written straight from the accumulators
// every 16-byte fragment slot was a separate piece of a different 128-byte
// line, and at 256 query rows those scattered stores took over a third of
// the launch (29 against 18 us without them).
__device__ __forceinline__ void absorb_block_wide(const uint16_t* __restrict__ q_nope,
                                                  const uint16_t* __restrict__ w_uk, _Float16* __restrict__ q_abs,
                                                  int rows, int g4, int cb, char* wl,
                                                  int* __restrict__ range_flag) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int half = lane >> 5;
  const int h = kAbsWideHeads * g4 + w;   // this wavefront's head

  // W_UK[4 g4 + h4][k][64 cb .. + 64] -> LDS: granule G = t + 256 n is
  // (h4, k, g) = (G / 1024, (G / 8) % 128, G % 8); 8 threads per 128-byte row
  constexpr int kWLoads = kAbsWideBytes / 16 / kPrepThreads;   // 16
  const uint16_t* wsrc = w_uk + ((size_t)(kAbsWideHeads * g4) * kDNope) * kDLat + cb * kAbsWideCols;
  u32x4 wv[kWLoads];
#pragma unroll
  for (int n = 0; n < kWLoads; ++n) {
    const int G = t + kPrepThreads * n;
    wv[n] = *(const u32x4*)(wsrc + ((size_t)(G >> 10) * kDNope + ((G >> 3) & 127)) * kDLat + 8 * (G & 7));
  }
  // B fragments (lane = query row r0 + lane % 32, 8 consecutive k per k-step)
  // of three 32-row tiles, loaded in the same round trip as the slice
  auto load_q = [&](int r0, u32x4 (&bq)[8]) {
    const int r = r0 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      bq[ks] = r < rows ? *(const u32x4*)(q_nope + ((size_t)r * kHeads + h) * kDNope + 16 * ks + 8 * half)
                        : u32x4{0, 0, 0, 0};
  };
  u32x4 bq0[8], bq1[8], bq2[8];
  load_q(0, bq0);
  load_q(32, bq1);
  load_q(64, bq2);
#pragma unroll
  for (int n = 0; n < kWLoads; ++n) {
    const int G = t + kPrepThreads * n;
    *(u32x4*)(wl + wl_off_wide(G >> 10, (G >> 3) & 127, G & 7)) = wv[n];
  }
  __syncthreads();

  // A fragments (W_UK^T[c][k], lane = column) of the two 32-column tiles ct
  // for all 8 k-steps, through transposing reads: lane group gg = lane / 16
  // covers columns 32 ct + 16 (gg % 2) + (0..15) and the k-half hh = gg / 2;
  // source lane L addresses row k = 16 ks + 8 hh + 4 q + L / 4 at column
  // 32 ct + 16 (gg % 2) + 4 (L % 4), so the read returns, per lane, 4
  // consecutive k of its own column.
  const int gg = lane >> 4, L = lane & 15, hh = gg >> 1;
  bf16x8 a[2][8];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int k0 = 16 * ks + 8 * hh + (L >> 2);
      const int g = 4 * ct + 2 * (gg & 1) + ((L & 3) >> 1);
      const int sub = 8 * (L & 1);
      const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(wl + wl_off_wide(w, k0, g) + sub));
      const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(wl + wl_off_wide(w, k0 + 4, g) + sub));
      a[ct][ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
    }

  // the slice's LDS becomes the staging space once every wavefront holds its
  // A fragments (one workgroup then fits beside the plan's on a CU)
  static_assert(2 * kStageBytes <= kAbsWideBytes, "staging fits the slice buffer");
  char* const stage = wl;
  __syncthreads();
  const int hg = h >> 5;                  // the 4 heads share their 32-head group
  const int hj0 = (kAbsWideHeads * g4) & 31;   // the first one's place in it
  bool out_of_range = false;   // a value past kQAbsMax (or not finite)
  // one 32-row tile; its buffer then loads the tile three further on
  auto tile = [&](int r0, u32x4 (&bt)[8]) {
    const int rl = lane & 31, r = r0 + rl;
    f32x16 acc[2] = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ct][ks], __builtin_bit_cast(bf16x8, bt[ks]), acc[ct], 0,
                                                          0, 0);
    if (r0 + 96 < rows) load_q(r0 + 96, bt);
    // tiles alternate between the two staging buffers: the barrier below
    // also orders this tile's writes after every read of the tile two back
    char* stg = stage + ((r0 >> 5) & 1) * kStageBytes;
    if (r < rows) {
      // acc[ct][4 q + e] holds column 64 cb + 32 ct + 8 q + 4 half + e of row
      // r; stored scaled by kQScale (a power of two: the rounding to fp16 is
      // the same)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int e = 0; e < 16; ++e) out_of_range |= !(__builtin_fabsf(acc[ct][e]) <= kQAbsMax);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          // column group 2 ct + q / 2 of the tile's four, half q % 2 of it
          const int g = rl * 32 + ((2 * ct + (q >> 1)) * 2 + (q & 1)) * kAbsWideHeads + w;
          f16x4 v = {(_Float16)(acc[ct][4 * q] * kQScale), (_Float16)(acc[ct][4 * q + 1] * kQScale),
                     (_Float16)(acc[ct][4 * q + 2] * kQScale), (_Float16)(acc[ct][4 * q + 3] * kQScale)};
          *(f16x4*)(stg + stage_off(g) + 8 * half) = v;
        }
    }
    __syncthreads();
    // granule G = 4 run + head: run (rl, c16l, sel) is 64 contiguous bytes of
    // q_abs, fragment slots hj0 .. hj0 + 3 (+ 32 sel) of the 1 KB fragment
    // block (row, hg, column group 4 cb + c16l)
#pragma unroll
    for (int n = 0; n < kStageGranules / kPrepThreads; ++n) {
      const int G = t + kPrepThreads * n;
      const int run = G >> 2, hq = G & 3;
      const int rr = r0 + (run >> 3);
      if (rr < rows) {
        const u32x4 v = *(const u32x4*)(stg + stage_off(G));
        const int c16 = 4 * cb + ((run >> 1) & 3);
        const size_t frag = (((size_t)rr * 4 + hg) * 32 + c16) * 64 + hj0 + hq + 32 * (run & 1);
        *(u32x4*)(q_abs + frag * 8) = v;
      }
    }
  };
  for (int r0 = 0; r0 < rows; r0 += 96) {
    tile(r0, bq0);
    if (r0 + 32 < rows) tile(r0 + 32, bq1);
    if (r0 + 64 < rows) tile(r0 + 64, bq2);
  }
  // this workgroup's flag, and the second flag of the pair that the narrow
  // layout's twice as many workgroups would write, on every call
  const int any = __syncthreads_or(out_of_range ? 1 : 0);
  if (t == 0) {
    range_flag[0] = any ? 1 : 0;
    range_flag[kAbsWideGroups] = 0;
  }
}

// the same launch with the wide absorb tile (from kAbsWideRows query rows on)
__global__ __launch_bounds__(kPrepThreads, 2) void prep_wide_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ block_table, int mbps, int num_blocks, int batch, int max_len, int split_target, int max_rounds, int positions,
    int depth, int max_chunks, WorkItem* __restrict__ work, SeqInfo* __restrict__ seqinfo,
    int* __restrict__ meta, const uint16_t* __restrict__ q_nope,
    const uint16_t* __restrict__ w_uk, _Float16* __restrict__ q_abs, int rows, int* __restrict__ range_flags) {
  __shared__ __attribute__((aligned(16))) char wl[kAbsWideBytes];
  static_assert(128 + 7 * 4 * kPlanSortMax <= kAbsWideBytes, "plan scratch fits the LDS buffer");
  if (blockIdx.x == 0) {
    // the plan is a short serial chain of barriers and reductions that must
    // not wait behind the absorb wavefronts sharing its SIMDs
    __builtin_amdgcn_s_setprio(3);
    plan_block(seq_lens, block_table, mbps, num_blocks, batch, max_len, split_target, max_rounds, positions, depth, max_chunks, work, seqinfo, meta,
               wl);
  } else {
    // workgroups are dealt to the 8 XCDs round-robin by id (XCD = id % 8)
    const int j = blockIdx.x - 1;
    const int x = blockIdx.x & 7, s = j >> 3;
    // XCD x takes heads [16 x, 16 x + 16) as head groups 4 x .. 4 x + 3 with
    // all 8 column blocks of each (seat s: group 4 x + s / 8, block s % 8)
    absorb_block_wide(q_nope, w_uk, q_abs, rows, 4 * x + (s >> 3), s & 7, wl, range_flags + j);
  }
}

}  // namespace

hipError_t launch_prep_wide(const int32_t* seq_lens, const int32_t* block_table, int max_blocks_per_seq,
                            int num_blocks, int batch, int max_len, int split_target, int max_rounds, int positions,
                            int depth, int max_chunks, WorkItem* work, SeqInfo* seqinfo, int* meta,
                            const uint16_t* q_nope, const uint16_t* w_uk, _Float16* q_abs, int rows,
                            int* range_flags, hipStream_t stream) {
  hipLaunchKernelGGL(prep_wide_kernel, dim3(1 + kAbsWideGroups), dim3(kPrepThreads), 0, stream,
                     seq_lens, block_table, max_blocks_per_seq, num_blocks, batch, max_len, split_target, max_rounds,
                     positions, depth, max_chunks, work, seqinfo, meta, q_nope, w_uk, q_abs, rows, range_flags);
  return hipGetLastError();
}

}  // namespace mla
