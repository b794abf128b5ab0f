// Split plan: cut every sequence's cached tokens into chunks of one common
// length C (a multiple of the 64-token cache block) so that the batch yields
// about `split_target` chunks, and emit the work list the attention pass
// walks plus, per sequence, the range of partial-state slots the merge pass
// reads. Integer work only; one workgroup.
//
// The pages describe a single softmax over the whole history (the "DeepSeek-V3"
// page, MLA section: every step still scores every cached position); cutting it
// into chunks and merging by log-sum-exp is an exact regrouping of that sum.
#include "common.h"

namespace mla {

namespace {

constexpr int kPlanThreads = 1024;

// Inclusive block-wide scan of one int per thread (Hillis-Steele in LDS).
__device__ int block_inclusive_scan(int v, int* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int d = 1; d < kPlanThreads; d <<= 1) {
    int add = t >= d ? sh[t - d] : 0;
    __syncthreads();
    sh[t] += add;
    __syncthreads();
  }
  int r = sh[t];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ seq_lens, int batch, int max_len, int split_target,
    int max_chunks, WorkItem* __restrict__ work,
    SeqInfo* __restrict__ seqinfo, int* __restrict__ meta) {
  __shared__ int sh[kPlanThreads];
  __shared__ long long total_sh;
  const int t = threadIdx.x;
  const int per = (batch + kPlanThreads - 1) / kPlanThreads;
  const int b0 = t * per;
  const int b1 = min(batch, b0 + per);
  // Lengths are clamped to [0, max_len] (max_len = min(host bound, block-table
  // reach)); with C >= total / target this keeps sum_b ceil(L_b / C) within
  // min(target + B, B * ceil(max_len / 64)) = max_chunks, so every slot fits.
  const int cap = max_len;

  // 1. total cached tokens
  long long mine = 0;
  for (int b = b0; b < b1; ++b) mine += min(max(seq_lens[b], 0), cap);
  if (t == 0) total_sh = 0;
  __syncthreads();
  atomicAdd((unsigned long long*)&total_sh, (unsigned long long)mine);
  __syncthreads();
  const long long total = total_sh;

  // 2. common chunk length: >= total/target, a multiple of one block
  long long c = (total + split_target - 1) / split_target;
  c = (c + kMinChunk - 1) / kMinChunk * kMinChunk;
  if (c < kMinChunk) c = kMinChunk;
  const int C = (int)c;

  // 3. per-sequence chunk counts; full-length chunks are listed first so that
  //    the longest work is dispatched first, the shorter tails last.
  int n_all = 0, n_full = 0, n_tail = 0;
  for (int b = b0; b < b1; ++b) {
    int L = min(max(seq_lens[b], 0), cap);
    n_all += (L + C - 1) / C;
    n_full += L / C;
    n_tail += (L % C) ? 1 : 0;
  }
  const int inc_all = block_inclusive_scan(n_all, sh);
  const int inc_full = block_inclusive_scan(n_full, sh);
  const int inc_tail = block_inclusive_scan(n_tail, sh);
  if (t == kPlanThreads - 1) {
    meta[0] = min(inc_all, max_chunks);   // chunks in the work list
    meta[1] = C;
    meta[2] = inc_all;                    // before clamping (diagnostic)
  }
  __shared__ int total_full;
  if (t == kPlanThreads - 1) total_full = inc_full;
  __syncthreads();

  int slot = inc_all - n_all;
  int full_idx = inc_full - n_full;
  int tail_idx = total_full + inc_tail - n_tail;
  for (int b = b0; b < b1; ++b) {
    int L = min(max(seq_lens[b], 0), cap);
    int nb = (L + C - 1) / C;
    int nf = L / C;
    seqinfo[b] = SeqInfo{slot, nb, L, 0};
    for (int s = 0; s < nf; ++s, ++full_idx)
      if (full_idx < max_chunks) work[full_idx] = WorkItem{b, s * C, (s + 1) * C, slot + s};
    if (nb > nf) {
      if (tail_idx < max_chunks) work[tail_idx] = WorkItem{b, nf * C, L, slot + nf};
      ++tail_idx;
    }
    slot += nb;
  }
}

}  // namespace

hipError_t launch_plan(const int32_t* seq_lens, int batch, int max_len, int split_target,
                       int max_chunks, WorkItem* work, SeqInfo* seqinfo, int* meta,
                       hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, batch,
                     max_len, split_target, max_chunks, work, seqinfo, meta);
  return hipGetLastError();
}

}  // namespace mla
