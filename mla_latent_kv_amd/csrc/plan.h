// Split plan of the preparation launch (workgroup 0 of prep_kernel and of
// prep_wide_kernel): device code shared by the two absorb layouts' files.
#pragma once

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

// Wavefront-wide sum (kMax: maximum) of a 32-bit value in the VALU's
// cross-lane (DPP) moves, no LDS access: xor 1 and xor 2 inside each quad,
// then the mirrors inside each half-row and row of 16 lanes (every lane then
// holds its row's result), then rows 1 and 3 take the last lane of rows 0
// and 2, and rows 2 and 3 the last lane of row 1; lane 63 ends with the
// wavefront's result.
template <bool kMax>
__device__ __forceinline__ unsigned wave_reduce(unsigned v) {
  auto op = [](unsigned a, unsigned b) { return kMax ? (a > b ? a : b) : a + b; };
  const unsigned id = 0u;   // identity of both (values are unsigned) for the lanes a broadcast skips
  v = op(v, (unsigned)__builtin_amdgcn_update_dpp((int)id, (int)v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  v = op(v, (unsigned)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  v = op(v, (unsigned)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = op(v, (unsigned)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  v = op(v, (unsigned)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x142, 0xA, 0xF, false));   // row_bcast:15
  v = op(v, (unsigned)__builtin_amdgcn_update_dpp((int)id, (int)v, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}

// ceil(x / d) for 32-bit x and d >= 1 through the fp64 reciprocal: the
// truncated product is the quotient or one below it (x / d < 2^32 and the
// product's relative error is a few units of 2^-53), and one integer test
// settles which.
__device__ __forceinline__ unsigned ceil_div(unsigned x, unsigned d, double inv_d) {
  const unsigned n = x + d - 1;   // callers keep x + d < 2^32
  unsigned q = (unsigned)((double)n * inv_d);
  if ((unsigned long long)(q + 1) * d <= n) ++q;
  return q;
}

constexpr int kItemCostTiles = 6;   // per-item fixed cost of the attention pass, in tiles

// The split plan. Every sequence's cached tokens [0, L_b) are cut into pieces
// (multiples of 64 tokens but the last) that the attention pass runs as
// independent items; P = split_target slots run at once (one per CU), and
// item k of the list goes to slot k % P as its (k / P)-th item, so a slot
// runs its items back to back.
//
// For a batch of at most kPlanSortMax sequences that fits in kPlanWaves rounds
// of P, the plan searches the piece length: for k = 1 .. kPlanWaves rounds,
// C_k = the smallest multiple of 64 with sum_b ceil(L_b / C_k) <= k P, at an
// estimated cost of k (ceil(C_k / 32) + kItemCostTiles) tiles per slot; the
// cheapest k wins. Each sequence is then cut into ceil(L_b / C) pieces of
// equal length (rounded up to 64), and the sequences are listed longest piece
// first, so that every round holds pieces of similar length (a static
// longest-first schedule). Otherwise the simple plan: C = total / P rounded up
// to 64, every sequence's full C-chunks first, the shorter tails last.
//
// Slot i of a round is position (i % (P8 / 8)) * 8 + i / (P8 / 8) of the list
// (P8 = P rounded up to 8): the attention workgroup at position p runs on XCD
// p % 8, so XCD x runs slots [x P8 / 8, (x + 1) P8 / 8), consecutive items and
// therefore the pieces of the same sequences, which share one L2.
//
// The plan is one workgroup's short chain of reductions; it keeps the
// barriers few (each costs a round trip of every wavefront) and runs the
// kPlanWaves searches side by side, one per wavefront.
__device__ __forceinline__ void plan_block(const int32_t* __restrict__ seq_lens,
                                           const int32_t* __restrict__ block_table, int mbps, int num_blocks,
                                           int batch, int max_len,
                                           int split_target, int max_rounds, int positions, int depth, int max_chunks,
                                           WorkItem* __restrict__ work, SeqInfo* __restrict__ seqinfo,
                                           int* __restrict__ meta, char* shm) {
  static_assert(kPlanWaves == kPrepThreads / 64, "one wavefront per searched round count");
  const int t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int P = split_target;
  const int per_xcd = positions / 8;
  const int per = (batch + kPrepThreads - 1) / kPrepThreads;
  const int b0 = t * per;
  const int b1 = min(batch, b0 + per);
  // LDS map: [0, 64) totals exchange; [64, 96) scan exchange; [96, 112)
  // search results; then the per-sequence arrays of the searched plan
  unsigned* sh_tot = (unsigned*)shm;                          // 4 waves x 4 words
  unsigned long long* shu = (unsigned long long*)(shm + 64);  // scans, 4 entries
  unsigned* lo_sh = (unsigned*)(shm + 96);                    // kPlanWaves
  unsigned* key = (unsigned*)(shm + 128);                     // [kPlanSortMax] sort keys
  unsigned* skey = key + kPlanSortMax;                        // [kPlanSortMax] keys in sorted order
  int* s_n = (int*)(skey + kPlanSortMax);                     // per sequence: pieces
  int* s_base = s_n + kPlanSortMax;                           //   piece length
  int* s_slot = s_base + kPlanSortMax;                        //   first partial slot
  int* s_start = s_slot + kPlanSortMax;                       // per sorted entry: first item
  int* s_len = s_start + kPlanSortMax;                        // lengths (batches up to kPlanSortMax)
  // batches of at most kPlanSortMax keep their lengths in LDS: every later
  // pass (the search's counts above all) reads them there, not from memory
  const bool cached = batch <= kPlanSortMax;
  for (int b = b0; b < b1 && cached; ++b) s_len[b] = min(max(seq_lens[b], 0), max_len);
  auto len_of = [&](int b) { return cached ? s_len[b] : min(max(seq_lens[b], 0), max_len); };

  // ---- totals: sum, nonempty count and maximum of the lengths (clamped to
  // [0, max_len], max_len = min(host bound, block-table reach)), one barrier.
  // A thread's sum stays below 2^21 * 2^31 (batch <= kMaxBatch); it is
  // reduced as two 21-bit-aligned halves, whose wavefront sums fit 32 bits.
  unsigned long long mine = 0;
  unsigned ne = 0, mx = 0;
  for (int b = b0; b < b1; ++b) {
    const unsigned L = (unsigned)len_of(b);
    mine += L;
    ne += L > 0;
    mx = L > mx ? L : mx;
  }
  {
    const unsigned lo21 = wave_reduce<false>((unsigned)(mine & 0x1fffffu));
    const unsigned hi = wave_reduce<false>((unsigned)(mine >> 21));
    const unsigned nes = wave_reduce<false>(ne);
    const unsigned mxs = wave_reduce<true>(mx);
    if (lane == 0) {
      sh_tot[4 * wv] = lo21;
      sh_tot[4 * wv + 1] = hi;
      sh_tot[4 * wv + 2] = nes;
      sh_tot[4 * wv + 3] = mxs;
    }
  }
  __syncthreads();
  unsigned long long total = 0;
  long long n_ne = 0, max_l = 0;
#pragma unroll
  for (int q = 0; q < kPrepThreads / 64; ++q) {
    total += (unsigned long long)sh_tot[4 * q] + ((unsigned long long)sh_tot[4 * q + 1] << 21);
    n_ne += sh_tot[4 * q + 2];
    max_l = max(max_l, (long long)sh_tot[4 * q + 3]);
  }
  auto up64 = [](long long x) { return (x + kMinChunk - 1) / kMinChunk * kMinChunk; };
  // max_rounds (1 .. kPlanWaves) bounds the rounds the search may choose
  const bool search = total > 0 && batch <= kPlanSortMax && n_ne <= (long long)max_rounds * P;

  // The search works in 64-token blocks: lb = ceil(L / 64) < 2^26, and
  // ceil(L / C) = ceil(lb / (C / 64)) for C a multiple of 64, so every count
  // is 32-bit arithmetic. A block count mb is feasible for k rounds when
  // N(mb) = sum_b ceil(lb_b / mb) <= k P; N never grows with mb.
  const unsigned max_lb = (unsigned)((max_l + kMinChunk - 1) / kMinChunk);
  unsigned mb;   // the chosen piece length C = 64 mb
  if (search) {
    const bool uniform = max_l * n_ne == (long long)total;   // every nonempty sequence of length max_l
    auto feasible = [&](int k) { return k < max_rounds && (long long)(k + 1) * P >= n_ne; };
    // this wavefront's search: round count wv + 1, smallest feasible mb
    if (!uniform && feasible(wv)) {
      const double tb = (double)total / kMinChunk;   // sum_b lb_b lies in [tb, tb + n_ne]
      const double cap = (double)(wv + 1) * P;
      // below tb / cap nothing fits (N >= sum lb / mb); from (tb + n_ne) /
      // (cap - n_ne) on everything fits (N <= sum lb / mb + n_ne); the
      // search returns the smallest feasible mb whatever the bracket
      const double l = floor(tb / cap) - 1.0;
      unsigned hi = max_lb;
      if (cap > (double)n_ne) {
        const double u = ceil((tb + (double)n_ne) / (cap - (double)n_ne)) + 1.0;
        if (u < (double)hi) hi = (unsigned)u;
      }
      hi = max(hi, 1u);
      unsigned lo = l < 1.0 ? 1u : (l >= (double)hi ? hi : (unsigned)l);
      // lane i counts sequences i, i + 64, ... (block counts held in VGPRs);
      // every count fits 32 bits: N(mid) <= N(lo) <= k P + n_ne, or n_ne where
      // mid is the longest sequence's block count
      constexpr int kPerLane = kPlanSortMax / 64;
      unsigned lbv[kPerLane];
#pragma unroll
      for (int j = 0; j < kPerLane; ++j) {
        const int b = lane + 64 * j;
        lbv[j] = b < batch ? ((unsigned)s_len[b] + kMinChunk - 1) / kMinChunk : 0u;
      }
      const unsigned capu = (unsigned)(wv + 1) * (unsigned)P;
      while (lo < hi) {   // lo and hi are wavefront-uniform
        const unsigned mid = lo + (hi - lo) / 2;
        const double inv = 1.0 / (double)mid;
        unsigned cnt = 0;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j)
          if (64 * j < batch) cnt += lbv[j] ? ceil_div(lbv[j], mid, inv) : 0u;
        if (wave_reduce<false>(cnt) <= capu)
          hi = mid;
        else
          lo = mid + 1;
      }
      if (lane == 0) lo_sh[wv] = lo;
    }
    __syncthreads();
    long long best_cost = -1;
    mb = max(max_lb, 1u);
#pragma unroll
    for (int k = 0; k < kPlanWaves; ++k) {
      if (!feasible(k)) continue;
      unsigned lk;
      if (uniform) {
        // equal lengths (lb blocks each): n_ne ceil(lb / mb) <= cap exactly when
        // ceil(lb / mb) <= floor(cap / n_ne), i.e. mb >= ceil(lb / floor(cap / n_ne))
        const unsigned m = (unsigned)min((long long)(k + 1) * P / n_ne, (long long)max_lb);
        lk = (max_lb + m - 1) / m;
      } else {
        lk = lo_sh[k];
      }
      // k + 1 rounds of items of up to 2 lk tiles (64 lk tokens) each
      const long long cost = (long long)(k + 1) * (2LL * lk + kItemCostTiles);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        mb = lk;
      }
    }
  } else {
    // C = total / P rounded up to 64, no longer than the longest sequence
    // needs (any C of at least max L leaves every sequence one piece)
    const long long c = max(up64((long long)((total + P - 1) / P)), (long long)kMinChunk) / kMinChunk;
    mb = (unsigned)min(c, (long long)max(max_lb, 1u));
  }
  const long long C = (long long)mb * kMinChunk;

  // pieces of a sequence: count n, length `base` (the last one may be shorter)
  auto pieces = [&](unsigned L, int& n, int& base) {
    if (L == 0) {
      n = 0;
      base = kMinChunk;
      return;
    }
    const unsigned lb = (L + kMinChunk - 1) / kMinChunk;
    const unsigned nb = (lb + mb - 1) / mb;
    if (search) {
      const unsigned bb = (lb + nb - 1) / nb;   // blocks per piece
      base = (int)(bb * kMinChunk);
      n = (int)((lb + bb - 1) / bb);
    } else {
      base = (int)min(C, (long long)0x7fffffff);
      n = (int)nb;
    }
  };

  // partial slots in sequence order; item counts: all | full-length | tails
  // (the simple plan lists full chunks first)
  unsigned long long cnt = 0;   // n_all | n_full << 21 | n_tail << 42
  for (int b = b0; b < b1; ++b) {
    const unsigned L = (unsigned)len_of(b);
    int n, base;
    pieces(L, n, base);
    const unsigned nf = search ? 0u : (unsigned)(L / (unsigned long long)C);
    cnt += (unsigned long long)n | ((unsigned long long)nf << 21) | ((unsigned long long)(n - nf) << 42);
  }
  const unsigned long long inc = block_scan(cnt, shu);
  const unsigned long long mask = (1ull << 21) - 1;
  __shared__ unsigned long long all_sh;
  if (t == kPrepThreads - 1) all_sh = inc;
  __syncthreads();
  const int n_items = (int)(all_sh & mask), tot_full = (int)((all_sh >> 21) & mask);
  if (t == 0) {
    meta[0] = n_items;
    meta[1] = (int)min(C, (long long)0x7fffffff);
    meta[2] = (n_items + P - 1) / P;   // rounds
    meta[3] = search ? 1 : 0;
  }
  const unsigned long long exc = inc - cnt;

  // list entry of item k (k < n_items < 2^21: 32-bit index arithmetic)
  auto entry = [&](int k) -> int {
    const int i = k % P;
    return (k / P) * positions + (i % per_xcd) * 8 + i / per_xcd;
  };
  // the cache block holding token tt of sequence b (tt < max_len: inside the
  // table row), clamped like every cache access
  auto blk_at = [&](int b, int tt) -> int {
    const int v = block_table[(size_t)b * mbps + tt / kMinChunk];
    return v < 0 ? 0 : (v >= num_blocks ? num_blocks - 1 : v);
  };
  auto put = [&](int k, int b, int t0, int t1, int slot, int L) {
    if (slot < max_chunks && k / P < depth) {
      const int bk0 = blk_at(b, t0);
      const int bk1 = t1 - t0 > kMinChunk ? blk_at(b, t0 + kMinChunk) : bk0;
      work[entry(k)] = WorkItem{b, t0, t1, slot, L, bk0, bk1, 0};
    }
  };

  if (!search) {
    int slot = (int)(exc & mask);
    int full_idx = (int)((exc >> 21) & mask);
    int tail_idx = tot_full + (int)((exc >> 42) & mask);
    for (int b = b0; b < b1; ++b) {
      const int L = len_of(b);
      int n, base;
      pieces((unsigned)L, n, base);
      // C may be 2^31 (one piece per sequence); every full chunk ends at or
      // below L < 2^31
      const int nf = (int)(L / C);
      seqinfo[b] = SeqInfo{slot, n, L, 0};
      for (int q = 0; q < nf; ++q, ++full_idx)
        put(full_idx, b, (int)(q * C), (int)((q + 1) * C), slot + q, L);
      if (n > nf) put(tail_idx++, b, (int)(nf * C), L, slot + nf, L);
      slot += n;
    }
  } else {
    // sequences ordered longest piece first (ties: lower b first), then each
    // item finds its sequence by binary search over the sorted prefix of item
    // counts
    int slot = (int)(exc & mask);
    for (int b = b0; b < b1; ++b) {
      const int L = s_len[b];
      int n, base;
      pieces((unsigned)L, n, base);
      seqinfo[b] = SeqInfo{slot, n, L, 0};
      s_n[b] = n;
      s_base[b] = base;
      s_slot[b] = slot;
      slot += n;
    }
    __syncthreads();
    // one round (every slot runs at most one item): sequence order, which
    // keeps a sequence's pieces on one XCD; no sort
    const bool one_round = n_items <= P;
    if (one_round) {
      // a sequence's first item is its first partial slot
      for (int e = t; e < batch; e += kPrepThreads) {
        skey[e] = (unsigned)e;
        s_start[e] = s_slot[e];
      }
    } else {
      // rank sort of the distinct keys (bucket of the piece length, b): the
      // rank of a key is the number of smaller keys
      for (int q = t; q < batch; q += kPrepThreads)
        key[q] = ((4095u - (unsigned)min(s_base[q] / kMinChunk, 4095)) << 20) | (unsigned)q;
      __syncthreads();
      for (int q = t; q < batch; q += kPrepThreads) {
        const unsigned kq = key[q];
        int rank = 0;
        int j = 0;
        for (; j + 4 <= batch; j += 4) {
          const u32x4 k4 = *(const u32x4*)(key + j);
          rank += (k4[0] < kq) + (k4[1] < kq) + (k4[2] < kq) + (k4[3] < kq);
        }
        for (; j < batch; ++j) rank += key[j] < kq;
        skey[rank] = kq;
      }
      __syncthreads();
      // exclusive prefix of item counts in sorted order: thread t owns sorted
      // entries [e0, e1)
      const int eper = (batch + kPrepThreads - 1) / kPrepThreads;
      const int e0 = min(batch, t * eper), e1 = min(batch, e0 + eper);
      unsigned long long own = 0;
      for (int e = e0; e < e1; ++e) own += (unsigned long long)s_n[skey[e] & 0xfffffu];
      unsigned long long run = block_scan(own, shu) - own;
      for (int e = e0; e < e1; ++e) {
        s_start[e] = (int)run;
        run += (unsigned long long)s_n[skey[e] & 0xfffffu];
      }
    }
    __syncthreads();
    for (int k = t; k < n_items; k += kPrepThreads) {
      int lo_e = 0, hi_e = batch - 1;   // the last sorted entry with s_start <= k
      while (lo_e < hi_e) {
        const int m = (lo_e + hi_e + 1) >> 1;
        if (s_start[m] <= k)
          lo_e = m;
        else
          hi_e = m - 1;
      }
      const int b = (int)(skey[lo_e] & 0xfffffu);
      const int q = k - s_start[lo_e];
      const int L = s_len[b];
      const int base = s_base[b];
      put(k, b, q * base, min((q + 1) * base, L), s_slot[b] + q, L);
    }
  }
  // a position runs its entries up to the first unused one: that entry is
  // marked, so no workgroup ever reads past it into entries left from an
  // earlier call
  for (int pos = t; pos < positions; pos += kPrepThreads) {
    const int i = (pos % 8) * per_xcd + pos / 8;   // the slot at this position
    const int count = i < P && n_items > i ? (n_items - 1 - i) / P + 1 : 0;
    if (count < depth) work[count * positions + pos] = WorkItem{0, 0, 0, -1, 0, 0, 0, 0};
  }
}

}  // namespace

}  // namespace mla
