// Preparation kernel, one launch: workgroup 0 computes the split plan, every
// other workgroup one (head, 128-wide latent block) tile of the absorb product.
//
// Split plan: cut every sequence's cached tokens into chunks of one common
// length C (a multiple of the 64-token cache block) so that the batch yields
// about `split_target` chunks, and emit the work list the attention pass walks
// plus, per sequence, the range of partial-state slots the merge pass reads.
// The pages describe one softmax over the whole history ("DeepSeek-V3" page,
// ailearn.mscapital.top, MLA section: every step still scores every cached
// position); cutting it into chunks and merging by log-sum-exp is an exact
// regrouping of that sum.
//
// Absorb product: q_abs[r, h, :] = W_UK[h]^T q_nope[r, h, :]  (128 -> 512), the
// query side of the identity q^T (U c) = (U^T q)^T c (the algebra check in
// section 2 of the wq-win.github.io DeepSeek-V3 notes, U = W_UK[h]):
// transforming the query once lets every cached latent be used as it is. Each
// absorb workgroup reads its 128 x 128 slice of W_UK once and applies it to
// every query row of the batch, so W_UK crosses HBM once per call.
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

constexpr int kPrepThreads = 256;

// ---------------------------------------------------------------- split plan

// Inclusive scan over the workgroup of one packed 64-bit value per thread
// (three 21-bit counters side by side; no field can carry into the next).
__device__ unsigned long long block_scan(unsigned long long v, unsigned long long* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    unsigned long long o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  if (lane == 63) sh[w] = v;
  __syncthreads();
  unsigned long long add = 0;
  for (int k = 0; k < w; ++k) add += sh[k];
  __syncthreads();
  return v + add;
}

__device__ __forceinline__ void plan_block(const int32_t* __restrict__ seq_lens, int batch, int max_len,
                           int split_target, int max_chunks, WorkItem* __restrict__ work,
                           SeqInfo* __restrict__ seqinfo, int* __restrict__ meta,
                           unsigned long long* sh) {
  const int t = threadIdx.x;
  const int per = (batch + kPrepThreads - 1) / kPrepThreads;
  const int b0 = t * per;
  const int b1 = min(batch, b0 + per);
  // Lengths are clamped to [0, max_len] (max_len = min(host bound, block-table
  // reach)); with C >= total / target this keeps sum_b ceil(L_b / C) within
  // min(target + B, B * ceil(max_len / 64)) = max_chunks, so every slot fits.
  long long mine = 0;
  for (int b = b0; b < b1; ++b) mine += min(max(seq_lens[b], 0), max_len);
  const long long total = (long long)block_scan((unsigned long long)mine, sh);   // inclusive
  __shared__ long long total_sh;
  if (t == kPrepThreads - 1) total_sh = total;
  __syncthreads();
  long long c = (total_sh + split_target - 1) / split_target;
  c = (c + kMinChunk - 1) / kMinChunk * kMinChunk;
  if (c < kMinChunk) c = kMinChunk;
  const int C = (int)c;

  // per-sequence chunk counts; full-length chunks are listed first so that the
  // longest work is dispatched first, the shorter tails last
  unsigned long long cnt = 0;   // n_all | n_full << 21 | n_tail << 42
  for (int b = b0; b < b1; ++b) {
    const int L = min(max(seq_lens[b], 0), max_len);
    cnt += (unsigned long long)((L + C - 1) / C) | ((unsigned long long)(L / C) << 21) |
           ((unsigned long long)((L % C) ? 1 : 0) << 42);
  }
  const unsigned long long inc = block_scan(cnt, sh);
  const unsigned long long mask = (1ull << 21) - 1;
  __shared__ unsigned long long all_sh;
  if (t == kPrepThreads - 1) all_sh = inc;
  __syncthreads();
  const int tot_all = (int)(all_sh & mask), tot_full = (int)((all_sh >> 21) & mask);
  if (t == 0) {
    meta[0] = min(tot_all, max_chunks);   // chunks in the work list
    meta[1] = C;
    meta[2] = tot_all;
  }
  const unsigned long long exc = inc - cnt;
  int slot = (int)(exc & mask);
  int full_idx = (int)((exc >> 21) & mask);
  int tail_idx = tot_full + (int)((exc >> 42) & mask);
  // Work item k goes to position (k % n) * 8 + k / n, n = ceil(n_work / 8):
  // the attention workgroup with id p (dealt to XCD p % 8) reads position p,
  // so XCD x runs items [x n, x n + n), consecutive splits of the same
  // sequences.
  const int n_work = min(tot_all, max_chunks);
  const int per_xcd = (n_work + 7) / 8;
  auto pos = [&](int kk) { return (kk % per_xcd) * 8 + kk / per_xcd; };
  for (int b = b0; b < b1; ++b) {
    const int L = min(max(seq_lens[b], 0), max_len);
    const int nb = (L + C - 1) / C;
    const int nf = L / C;
    seqinfo[b] = SeqInfo{slot, nb, L, 0};
    for (int s = 0; s < nf; ++s, ++full_idx)
      if (full_idx < max_chunks) work[pos(full_idx)] = WorkItem{b, s * C, (s + 1) * C, slot + s, L, 0, 0, 0};
    if (nb > nf) {
      if (tail_idx < max_chunks) work[pos(tail_idx)] = WorkItem{b, nf * C, L, slot + nf, L, 0, 0, 0};
      ++tail_idx;
    }
    slot += nb;
  }
  // every other position of the list's capacity is marked unused, so no
  // workgroup ever reads an entry left from an earlier call
  const int cap = (max_chunks + 7) / 8 * 8;
  for (int q = t; q < cap; q += kPrepThreads) {
    if (q >= 8 * per_xcd || (q % 8) * per_xcd + q / 8 >= n_work)
      work[q] = WorkItem{0, 0, 0, -1, 0, 0, 0, 0};
  }
}

// ---------------------------------------------------------------- absorb

constexpr int kWStride = 288;   // LDS row stride (bytes) of the W_UK slice: 256 + 32 pad

__device__ __forceinline__ void absorb_block(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ w_uk,
                             _Float16* __restrict__ q_abs, int rows, int h, int cb, char* wl) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;

  // W_UK[h][k][cb*128 .. +128] -> LDS rows k (16-byte granules, coalesced);
  // the first 32 query rows' B fragments are loaded in the same round trip
  const uint16_t* wsrc = w_uk + ((size_t)h * kDNope) * kDLat + cb * 128;
  u32x4 wv[8];
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int G = t + 256 * n;
    const int k = G >> 4, g = G & 15;
    wv[n] = *(const u32x4*)(wsrc + (size_t)k * kDLat + g * 8);
  }
  const int half = lane >> 5;
  auto load_q = [&](int r0, u32x4 (&bq)[8]) {
    const int r = r0 + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      bq[ks] = r < rows ? *(const u32x4*)(q_nope + ((size_t)r * kHeads + h) * kDNope + 16 * ks + 8 * half)
                        : u32x4{0, 0, 0, 0};
  };
  u32x4 bq[8];
  load_q(0, bq);
#pragma unroll
  for (int n = 0; n < 8; ++n) {
    const int G = t + 256 * n;
    const int k = G >> 4, g = G & 15;
    *(u32x4*)(wl + k * kWStride + g * 16) = wv[n];
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
  for (int r0 = 0; r0 < rows; r0 += 32) {
    const int r = r0 + (lane & 31);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], __builtin_bit_cast(bf16x8, bq[ks]), acc,
                                                    0, 0, 0);
    if (r0 + 32 < rows) load_q(r0 + 32, bq);   // next 32 rows in flight under the stores
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


__global__ __launch_bounds__(kPrepThreads) void prep_kernel(
    const int32_t* __restrict__ seq_lens, int batch, int max_len, int split_target,
    int max_chunks, WorkItem* __restrict__ work, SeqInfo* __restrict__ seqinfo,
    int* __restrict__ meta, const uint16_t* __restrict__ q_nope,
    const uint16_t* __restrict__ w_uk, _Float16* __restrict__ q_abs, int rows) {
  __shared__ __attribute__((aligned(16))) char wl[kDNope * kWStride];
  if (blockIdx.x == 0) {
    plan_block(seq_lens, batch, max_len, split_target, max_chunks, work, seqinfo, meta,
               (unsigned long long*)wl);
  } else {
    const int id = blockIdx.x - 1;
    absorb_block(q_nope, w_uk, q_abs, rows, id >> 2, id & 3, wl);
  }
}

}  // namespace

hipError_t launch_prep(const int32_t* seq_lens, int batch, int max_len, int split_target,
                       int max_chunks, WorkItem* work, SeqInfo* seqinfo, int* meta,
                       const uint16_t* q_nope, const uint16_t* w_uk, _Float16* q_abs, int rows,
                       hipStream_t stream) {
  hipLaunchKernelGGL(prep_kernel, dim3(1 + kHeads * (kDLat / 128)), dim3(kPrepThreads), 0, stream,
                     seq_lens, batch, max_len, split_target, max_chunks, work, seqinfo, meta,
                     q_nope, w_uk, q_abs, rows);
  return hipGetLastError();
}

}  // namespace mla
