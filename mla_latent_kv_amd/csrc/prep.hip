// Preparation kernel, one launch: workgroup 0 computes the split plan, every
// other workgroup one (head, 128-wide latent block) tile of the absorb
// product (prep_wide.hip holds the 4-head tile used from 128 query rows on).
//
// Split plan: cut every sequence's cached tokens into pieces (multiples of
// the 64-token cache block) that `split_target` attention slots run in at
// most kPlanWaves rounds, and emit the work list the attention pass walks
// plus, per sequence, the range of partial-state slots the merge pass reads
// (plan_block below says how the piece length is chosen).
// The pages describe one softmax over the whole history ("DeepSeek-V3" page,
// ailearn.mscapital.top, MLA section: every step still scores every cached
// position); cutting it into chunks and merging by log-sum-exp is an exact
// regrouping of that sum.
//
// Absorb product: q_abs[r, h, :] = W_UK[h]^T q_nope[r, h, :]  (128 -> 512), the
// query side of the identity q^T (U c) = (U^T q)^T c (the algebra check in
// section 2 of the wq-win.github.io DeepSeek-V3 notes, U = W_UK[h]):
// transforming the query once lets every cached latent be used as it is. Each
// absorb workgroup reads its 128 x 128 slice of W_UK once and applies it
// to every query row of the batch, so W_UK crosses HBM once per call.
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
#include "plan.h"

namespace mla {

namespace {

// ---------------------------------------------------------------- absorb

constexpr int kAbsCols = 128;                           // latent columns per absorb workgroup (32 per wavefront)
constexpr int kAbsRowBytes = kAbsCols * 2;              // 256: one k row of the head's W_UK slice
constexpr int kAbsBytes = kDNope * kAbsRowBytes;        // 32 KB
static_assert(kAbsorbGroups == kHeads * (kDLat / kAbsCols), "absorb workgroup count");

// LDS byte offset of 16-byte granule g (0..15) of row k of the W_UK slice.
// Rows are 256 bytes, four 64-byte quarters (32 columns each); quarter q of
// row k is stored at q ^ (k % 4), so the four consecutive rows a transposing
// read covers (32 columns each) fill all 64 banks once.
__device__ __forceinline__ int wl_off(int k, int g) { return k * kAbsRowBytes + 16 * (g ^ (4 * (k & 3))); }

// One absorb workgroup: head h x latent columns [128 cb, 128 cb + 128), every
// query row; wavefront w owns the 32 columns 128 cb + 32 w + (0..31). Its W_UK
// slice (32 KB) is read as 256-byte row pieces, and its results fill 16 bytes
// of each 128-byte line of q_abs (8 consecutive heads x 8 values); the
// workgroups with the other 7 heads of the line run on the same XCD, so the
// pieces meet in its L2.
__device__ __forceinline__ void absorb_block(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ w_uk,
                                             _Float16* __restrict__ q_abs, int rows, int h, int cb, char* wl,
                                             int* __restrict__ range_flag) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int half = lane >> 5;

  // W_UK[h][k][128 cb .. + 128] -> LDS: granule G = t + 256 n is
  // (k, g) = (G / 16, G % 16); 16 threads per 256-byte row piece
  constexpr int kWLoads = kAbsBytes / 16 / kPrepThreads;   // 8
  const uint16_t* wsrc = w_uk + ((size_t)h * kDNope) * kDLat + cb * kAbsCols;
  u32x4 wv[kWLoads];
#pragma unroll
  for (int n = 0; n < kWLoads; ++n) {
    const int G = t + kPrepThreads * n;
    wv[n] = *(const u32x4*)(wsrc + (size_t)(G >> 4) * kDLat + 8 * (G & 15));
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
    *(u32x4*)(wl + wl_off(G >> 4, G & 15)) = wv[n];
  }
  __syncthreads();

  // A fragments (W_UK^T[c][k], lane = column) of the wavefront's 32 columns
  // for all 8 k-steps, through transposing reads. Lane group gg = lane / 16
  // covers columns 32 w + 16 (gg % 2) + (0..15) and the k-half hh = gg / 2;
  // source lane L addresses row k = 16 ks + 8 hh + 4 q + L / 4 at column
  // 32 w + 16 (gg % 2) + 4 (L % 4), so the read returns, per lane, 4
  // consecutive k of its own column.
  const int gg = lane >> 4, L = lane & 15, hh = gg >> 1;
  const int g = 4 * w + 2 * (gg & 1) + ((L & 3) >> 1);   // granule of the lane's 4 columns
  const int sub = 8 * (L & 1);                            // byte offset inside it
  bf16x8 a[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int k0 = 16 * ks + 8 * hh + (L >> 2);
    const s16x4 p0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(wl + wl_off(k0, g) + sub));
    const s16x4 p1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(wl + wl_off(k0 + 4, g) + sub));
    a[ks] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  const int hg = h >> 5, hj = h & 31;
  bool out_of_range = false;   // a value past kQAbsMax (or not finite)
  // one 32-row tile; its buffer then loads the tile three further on
  auto tile = [&](int r0, u32x4 (&bt)[8]) {
    const int r = r0 + (lane & 31);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], __builtin_bit_cast(bf16x8, bt[ks]), acc, 0, 0, 0);
    if (r0 + 96 < rows) load_q(r0 + 96, bt);
    if (r < rows) {
      // acc[4 q + e] holds column 128 cb + 32 w + 8 q + 4 half + e of row r;
      // stored scaled by kQScale (a power of two: the rounding to fp16 is the
      // same)
#pragma unroll
      for (int e = 0; e < 16; ++e) out_of_range |= !(__builtin_fabsf(acc[e]) <= kQAbsMax);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c16 = 8 * cb + 2 * w + (q >> 1);   // column / 16
        f16x4 v = {(_Float16)(acc[4 * q] * kQScale), (_Float16)(acc[4 * q + 1] * kQScale),
                   (_Float16)(acc[4 * q + 2] * kQScale), (_Float16)(acc[4 * q + 3] * kQScale)};
        const size_t frag = (((size_t)r * 4 + hg) * 32 + c16) * 64 + hj + 32 * (q & 1);
        *(f16x4*)(q_abs + frag * 8 + 4 * half) = v;
      }
    }
  };
  for (int r0 = 0; r0 < rows; r0 += 96) {
    tile(r0, bq0);
    if (r0 + 32 < rows) tile(r0 + 32, bq1);
    if (r0 + 64 < rows) tile(r0 + 64, bq2);
  }
  // this workgroup's flag, written on every call (no clearing needed)
  const int any = __syncthreads_or(out_of_range ? 1 : 0);
  if (t == 0) *range_flag = any ? 1 : 0;
}

__global__ __launch_bounds__(kPrepThreads) void prep_kernel(
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ block_table, int mbps, int num_blocks, int batch, int max_len, int split_target, int max_rounds, int positions,
    int depth, int max_chunks, WorkItem* __restrict__ work, SeqInfo* __restrict__ seqinfo,
    int* __restrict__ meta, const uint16_t* __restrict__ q_nope,
    const uint16_t* __restrict__ w_uk, _Float16* __restrict__ q_abs, int rows, int* __restrict__ range_flags) {
  __shared__ __attribute__((aligned(16))) char wl[kAbsBytes];
  static_assert(128 + 7 * 4 * kPlanSortMax <= kAbsBytes, "plan scratch fits the LDS buffer");
  if (blockIdx.x == 0) {
    // the plan is a short serial chain of barriers and reductions that must
    // not wait behind the absorb wavefronts sharing its SIMDs
    __builtin_amdgcn_s_setprio(3);
    plan_block(seq_lens, block_table, mbps, num_blocks, batch, max_len, split_target, max_rounds, positions, depth, max_chunks, work, seqinfo, meta,
               wl);
  } else {
    // workgroups are dealt to the 8 XCDs round-robin by id (XCD = id % 8):
    // XCD x takes heads [16 x, 16 x + 16) with all 4 column blocks of each
    // (seat s: head 16 x + s / 4, column block s % 4), so the 8 heads sharing
    // a q_abs line and the column blocks sharing q_nope rows meet in one L2
    const int j = blockIdx.x - 1;
    const int x = blockIdx.x & 7, s = j >> 3;
    absorb_block(q_nope, w_uk, q_abs, rows, 16 * x + (s >> 2), s & 3, wl, range_flags + j);
  }
}

}  // namespace

// the same launch with the wide absorb tile (prep_wide.hip), from this many
// query rows on: at 256 query rows the launch measured 29.1 us against 33.9
// with the narrow tile, at 64 rows 0.5-0.9 us slower and at 32 rows 0.4-0.6 us
// slower. It is a separate code object: built into this one, its presence
// alone made the narrow launch ~0.9 us slower per call (same code, measured).
constexpr int kAbsWideRows = 128;
hipError_t launch_prep_wide(const int32_t* seq_lens, const int32_t* block_table, int max_blocks_per_seq,
                            int num_blocks, int batch, int max_len, int split_target, int max_rounds, int positions,
                            int depth, int max_chunks, WorkItem* work, SeqInfo* seqinfo, int* meta,
                            const uint16_t* q_nope, const uint16_t* w_uk, _Float16* q_abs, int rows,
                            int* range_flags, hipStream_t stream);

hipError_t launch_prep(const int32_t* seq_lens, const int32_t* block_table, int max_blocks_per_seq, int num_blocks,
                       int batch, int max_len, int split_target, int max_rounds,
                       int positions, int depth, int max_chunks, WorkItem* work, SeqInfo* seqinfo, int* meta,
                       const uint16_t* q_nope, const uint16_t* w_uk, _Float16* q_abs, int rows,
                       int* range_flags, hipStream_t stream) {
  if (rows >= kAbsWideRows)
    return launch_prep_wide(seq_lens, block_table, max_blocks_per_seq, num_blocks, batch, max_len, split_target,
                            max_rounds, positions, depth, max_chunks, work, seqinfo, meta, q_nope, w_uk, q_abs, rows,
                            range_flags, stream);
  hipLaunchKernelGGL(prep_kernel, dim3(1 + kAbsorbGroups), dim3(kPrepThreads), 0, stream,
                     seq_lens, block_table, max_blocks_per_seq, num_blocks, batch, max_len, split_target, max_rounds,
                     positions, depth, max_chunks, work, seqinfo, meta, q_nope, w_uk, q_abs, rows, range_flags);
  return hipGetLastError();
}

}  // namespace mla
