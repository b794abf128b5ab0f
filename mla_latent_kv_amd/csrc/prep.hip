// Preparation kernel, one launch: workgroup 0 computes the split plan, every
// other workgroup one (head, 128-wide latent block) tile of the absorb product.
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

// Workgroup-wide sums (kMax: maxima) of kN 32-bit values per thread: the
// wavefronts reduce in DPP moves, their results meet in LDS (`sh`: 4 kN
// entries). Every thread gets the results; all threads must call it.
template <int kN, bool kMax = false>
__device__ void block_sums(unsigned (&v)[kN], unsigned* sh) {
#pragma unroll
  for (int k = 0; k < kN; ++k) v[k] = wave_reduce<kMax>(v[k]);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0)
#pragma unroll
    for (int k = 0; k < kN; ++k) sh[w * kN + k] = v[k];
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kN; ++k) {
    unsigned r = sh[k];
#pragma unroll
    for (int q = 1; q < kPrepThreads / 64; ++q) r = kMax ? (sh[q * kN + k] > r ? sh[q * kN + k] : r) : r + sh[q * kN + k];
    v[k] = r;
  }
  __syncthreads();
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
__device__ __forceinline__ void plan_block(const int32_t* __restrict__ seq_lens, int batch, int max_len,
                                           int split_target, int max_rounds, int positions, int depth, int max_chunks,
                                           WorkItem* __restrict__ work, SeqInfo* __restrict__ seqinfo,
                                           int* __restrict__ meta, char* shm) {
  const int t = threadIdx.x;
  const int P = split_target;
  const int per_xcd = positions / 8;
  const int per = (batch + kPrepThreads - 1) / kPrepThreads;
  const int b0 = t * per;
  const int b1 = min(batch, b0 + per);
  unsigned* shs = (unsigned*)shm;                              // sums, 4 x 4 entries
  unsigned long long* shu = (unsigned long long*)(shm + 64);   // scans, 4 entries
  // batches of at most kPlanSortMax keep their lengths in LDS: every later
  // pass (the search's counts above all) reads them there, not from memory
  int* s_len = (int*)(shm + 128 + 20 * kPlanSortMax);
  const bool cached = batch <= kPlanSortMax;
  for (int b = b0; b < b1 && cached; ++b) s_len[b] = min(max(seq_lens[b], 0), max_len);
  auto len_of = [&](int b) { return cached ? s_len[b] : min(max(seq_lens[b], 0), max_len); };

  // lengths are clamped to [0, max_len] (max_len = min(host bound, block-table reach))
  long long mine = 0, ne = 0, mx = 0;
  for (int b = b0; b < b1; ++b) {
    const long long L = len_of(b);
    mine += L;
    ne += L > 0;
    mx = L > mx ? L : mx;
  }
  // the total needs 64 bits: the block scan's inclusive value of the last thread
  __shared__ unsigned long long total_sh;
  const unsigned long long inc_total = block_scan((unsigned long long)mine, shu);
  if (t == kPrepThreads - 1) total_sh = inc_total;
  unsigned nm[1] = {(unsigned)ne};
  block_sums<1>(nm, shs);
  unsigned ml[1] = {(unsigned)mx};
  block_sums<1, true>(ml, shs);
  const long long total = (long long)total_sh, n_ne = nm[0], max_l = ml[0];
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
    unsigned lo[kPlanWaves], hi[kPlanWaves];
    bool feas[kPlanWaves];
    const bool uniform = max_l * n_ne == total;   // every nonempty sequence of length max_l
#pragma unroll
    for (int k = 0; k < kPlanWaves; ++k) {
      feas[k] = k < max_rounds && (long long)(k + 1) * P >= n_ne;
      lo[k] = hi[k] = max(max_lb, 1u);
    }
    if (!uniform) {
      const double tb = (double)total / kMinChunk;   // sum_b lb_b lies in [tb, tb + n_ne]
#pragma unroll
      for (int k = 0; k < kPlanWaves; ++k) {
        const double cap = (double)(k + 1) * P;
        // below tb / cap nothing fits (N >= sum lb / mb); from (tb + n_ne) /
        // (cap - n_ne) on everything fits (N <= sum lb / mb + n_ne); the
        // search returns the smallest feasible mb whatever the bracket
        const double l = floor(tb / cap) - 1.0;
        unsigned h = max_lb;
        if (cap > (double)n_ne) {
          const double u = ceil((tb + (double)n_ne) / (cap - (double)n_ne)) + 1.0;
          if (u < (double)h) h = (unsigned)u;
        }
        hi[k] = max(h, 1u);
        lo[k] = l < 1.0 ? 1u : (l >= (double)hi[k] ? hi[k] : (unsigned)l);
      }
    }
    __shared__ unsigned lo_sh[kPlanWaves];
    if (uniform) {
      // equal lengths (lb blocks each): n_ne ceil(lb / mb) <= cap exactly when
      // ceil(lb / mb) <= floor(cap / n_ne), i.e. mb >= ceil(lb / floor(cap / n_ne))
#pragma unroll
      for (int k = 0; k < kPlanWaves; ++k)
        if (feas[k]) {
          const unsigned m = (unsigned)min((long long)(k + 1) * P / n_ne, (long long)max_lb);
          lo[k] = hi[k] = (max_lb + m - 1) / m;
        }
    } else if (t < 64) {
      // one wavefront runs the kPlanWaves binary searches: lane i counts
      // sequences i, i + 64, ... and the cross-lane sums take no barrier
      for (;;) {
        bool any = false;
        unsigned mid[kPlanWaves];
        bool open[kPlanWaves];
#pragma unroll
        for (int k = 0; k < kPlanWaves; ++k) {
          open[k] = feas[k] && lo[k] < hi[k];
          any |= open[k];
          mid[k] = open[k] ? lo[k] + (hi[k] - lo[k]) / 2 : hi[k];
        }
        if (!any) break;   // uniform across the wavefront
        // every count fits 32 bits: N(mid) <= N(lo_k) <= k P + n_ne, or n_ne
        // where mid is the longest sequence's block count
        unsigned cnt[kPlanWaves] = {};
        for (int b = t; b < batch; b += 64) {
          const unsigned lb = ((unsigned)s_len[b] + kMinChunk - 1) / kMinChunk;
#pragma unroll
          for (int k = 0; k < kPlanWaves; ++k)
            if (open[k]) cnt[k] += (lb + mid[k] - 1) / mid[k];   // only the searches still open
        }
#pragma unroll
        for (int k = 0; k < kPlanWaves; ++k) {
          if (!open[k]) continue;
          const unsigned n = wave_reduce<false>(cnt[k]);
          {
            if ((double)n <= (double)(k + 1) * P)
              hi[k] = mid[k];
            else
              lo[k] = mid[k] + 1;
          }
        }
      }
      if (t == 0)
#pragma unroll
        for (int k = 0; k < kPlanWaves; ++k) lo_sh[k] = lo[k];
    }
    if (!uniform) {
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kPlanWaves; ++k) lo[k] = hi[k] = lo_sh[k];
    }
    long long best_cost = -1;
    mb = hi[kPlanWaves - 1];
#pragma unroll
    for (int k = 0; k < kPlanWaves; ++k) {
      if (!feas[k]) continue;
      // k + 1 rounds of items of up to 2 lo tiles (64 lo tokens) each
      const long long cost = (long long)(k + 1) * (2LL * lo[k] + kItemCostTiles);
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        mb = lo[k];
      }
    }
  } else {
    // C = total / P rounded up to 64, no longer than the longest sequence
    // needs (any C of at least max L leaves every sequence one piece)
    const long long c = max(up64((total + P - 1) / P), (long long)kMinChunk) / kMinChunk;
    mb = (unsigned)min(c, (long long)max(max_lb, 1u));
  }
  const long long C = (long long)mb * kMinChunk;

  // pieces of a sequence: count n, length `base` (the last one may be shorter)
  auto pieces = [&](long long L, long long& n, long long& base) {
    if (L <= 0) {
      n = 0;
      base = kMinChunk;
      return;
    }
    const unsigned lb = ((unsigned)L + kMinChunk - 1) / kMinChunk;
    const unsigned nb = (lb + mb - 1) / mb;
    if (search) {
      const unsigned bb = (lb + nb - 1) / nb;   // blocks per piece
      base = (long long)bb * kMinChunk;
      n = (lb + bb - 1) / bb;
    } else {
      base = C;
      n = nb;
    }
  };

  // partial slots in sequence order; item counts: all | full-length | tails
  // (the simple plan lists full chunks first)
  unsigned long long cnt = 0;   // n_all | n_full << 21 | n_tail << 42
  for (int b = b0; b < b1; ++b) {
    const long long L = len_of(b);
    long long n, base;
    pieces(L, n, base);
    const long long nf = search ? 0 : L / C;
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

  // list entry of item k
  auto entry = [&](long long k) -> size_t {
    const int i = (int)(k % P);
    return (size_t)(k / P) * positions + (size_t)((i % per_xcd) * 8 + i / per_xcd);
  };
  auto put = [&](long long k, int b, long long t0, long long t1, int slot, int L) {
    if (slot < max_chunks && k / P < depth) work[entry(k)] = WorkItem{b, (int)t0, (int)t1, slot, L, 0, 0, 0};
  };

  if (!search) {
    int slot = (int)(exc & mask);
    long long full_idx = (long long)((exc >> 21) & mask);
    long long tail_idx = tot_full + (long long)((exc >> 42) & mask);
    for (int b = b0; b < b1; ++b) {
      const long long L = len_of(b);
      long long n, base;
      pieces(L, n, base);
      const long long nf = L / C;
      seqinfo[b] = SeqInfo{slot, (int)n, (int)L, 0};
      for (long long q = 0; q < nf; ++q, ++full_idx) put(full_idx, b, q * C, (q + 1) * C, slot + (int)q, (int)L);
      if (n > nf) put(tail_idx++, b, nf * C, L, slot + (int)nf, (int)L);
      slot += (int)n;
    }
  } else {
    // sequences ordered longest piece first (ties: lower b first): bitonic
    // sort of (piece-length bucket, b) keys in LDS, then each item finds its
    // sequence by binary search over the sorted prefix of item counts
    unsigned* key = (unsigned*)(shm + 128);                 // [kPlanSortMax]
    int* s_n = (int*)(shm + 128 + 4 * kPlanSortMax);       // per sequence: pieces
    int* s_base = s_n + kPlanSortMax;                      //   piece length
    int* s_slot = s_base + kPlanSortMax;                   //   first partial slot
    int* s_start = s_slot + kPlanSortMax;                  // per sorted entry: first item
    int slot = (int)(exc & mask);
    for (int b = b0; b < b1; ++b) {
      const long long L = len_of(b);
      long long n, base;
      pieces(L, n, base);
      seqinfo[b] = SeqInfo{slot, (int)n, (int)L, 0};
      s_n[b] = (int)n;
      s_base[b] = (int)base;
      s_slot[b] = slot;
      slot += (int)n;
    }
    int ns = 1;
    while (ns < batch) ns <<= 1;
    __syncthreads();
    // one round (every slot runs at most one item): sequence order, which
    // keeps a sequence's pieces on one XCD; no sort
    const bool one_round = n_items <= P;
    for (int q = t; q < ns; q += kPrepThreads) {
      if (q < batch) {
        const unsigned bucket = one_round ? 4095u : (unsigned)min(s_base[q] / kMinChunk, 4095);
        key[q] = ((4095u - bucket) << 20) | (unsigned)q;
      } else {
        key[q] = 0xffffffffu;
      }
    }
    __syncthreads();
    if (!one_round)
    for (int size = 2; size <= ns; size <<= 1)
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int q = t; q < ns / 2; q += kPrepThreads) {
          const int a = 2 * q - (q & (stride - 1)), c = a + stride;
          const unsigned ka = key[a], kc = key[c];
          if ((ka > kc) == ((a & size) == 0)) {
            key[a] = kc;
            key[c] = ka;
          }
        }
        __syncthreads();
      }
    // exclusive prefix of item counts in sorted order: thread t owns sorted
    // entries [e0, e1)
    if (one_round) {
      // sequence order: a sequence's first item is its first partial slot
      for (int e = t; e < ns; e += kPrepThreads) s_start[e] = e < batch ? s_slot[e] : n_items;
    } else {
      const int eper = (ns + kPrepThreads - 1) / kPrepThreads;
      const int e0 = min(ns, t * eper), e1 = min(ns, e0 + eper);
      unsigned long long own = 0;
      for (int e = e0; e < e1; ++e) own += key[e] == 0xffffffffu ? 0 : (unsigned long long)s_n[key[e] & 0xfffffu];
      unsigned long long run = block_scan(own, shu) - own;
      for (int e = e0; e < e1; ++e) {
        s_start[e] = (int)run;
        run += key[e] == 0xffffffffu ? 0 : (unsigned long long)s_n[key[e] & 0xfffffu];
      }
    }
    __syncthreads();
    for (int k = t; k < n_items; k += kPrepThreads) {
      int lo_e = 0, hi_e = ns - 1;   // the last sorted entry with s_start <= k
      while (lo_e < hi_e) {
        const int m = (lo_e + hi_e + 1) >> 1;
        if (s_start[m] <= k)
          lo_e = m;
        else
          hi_e = m - 1;
      }
      const int b = (int)(key[lo_e] & 0xfffffu);
      const long long q = k - s_start[lo_e];
      const long long L = len_of(b);
      const long long base = s_base[b];
      put(k, b, q * base, min((q + 1) * base, L), s_slot[b] + (int)q, (int)L);
    }
  }
  // a position runs its entries up to the first unused one: that entry is
  // marked, so no workgroup ever reads past it into entries left from an
  // earlier call
  for (int pos = t; pos < positions; pos += kPrepThreads) {
    const int i = (pos % 8) * per_xcd + pos / 8;   // the slot at this position
    const long long count = i < P && n_items > i ? (n_items - 1 - i) / P + 1 : 0;
    if (count < depth) work[(size_t)count * positions + pos] = WorkItem{0, 0, 0, -1, 0, 0, 0, 0};
  }
}

// ---------------------------------------------------------------- absorb

constexpr int kWStride = 288;   // LDS row stride (bytes) of the W_UK slice: 256 + 32 pad

__device__ __forceinline__ void absorb_block(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ w_uk,
                             _Float16* __restrict__ q_abs, int rows, int h, int cb, char* wl,
                             int* __restrict__ range_flag) {
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
  bool out_of_range = false;                  // a value past kQAbsMax (or not finite)
  // row tiles of 32 in pairs, two tiles' loads in flight: tile i + 2 loads
  // into the buffer tile i just used, under tile i's stores
  auto tile = [&](int r0, u32x4 (&bt)[8]) {
    const int r = r0 + (lane & 31);
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], __builtin_bit_cast(bf16x8, bt[ks]), acc, 0, 0, 0);
    if (r0 + 64 < rows) load_q(r0 + 64, bt);
    if (r < rows) {
      // acc[4 q + e] holds column c0 + 8 q + 4 half + e of row r; stored
      // scaled by kQScale (a power of two: the rounding to fp16 is the same)
#pragma unroll
      for (int e = 0; e < 16; ++e) out_of_range |= !(__builtin_fabsf(acc[e]) <= kQAbsMax);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + 8 * q + 4 * half;
        f16x4 v = {(_Float16)(acc[4 * q] * kQScale), (_Float16)(acc[4 * q + 1] * kQScale),
                   (_Float16)(acc[4 * q + 2] * kQScale), (_Float16)(acc[4 * q + 3] * kQScale)};
        const size_t frag = (((size_t)r * 4 + hg) * 32 + (c >> 4)) * 64 + hj + 32 * ((c & 15) >> 3);
        *(f16x4*)(q_abs + frag * 8 + (c & 7)) = v;
      }
    }
  };
  u32x4 bq2[8];
  if (32 < rows) load_q(32, bq2);
  for (int r0 = 0; r0 < rows; r0 += 64) {
    tile(r0, bq);
    if (r0 + 32 < rows) tile(r0 + 32, bq2);
  }
  // this workgroup's flag, written on every call (no clearing needed)
  const int any = __syncthreads_or(out_of_range ? 1 : 0);
  if (t == 0) *range_flag = any ? 1 : 0;
}


__global__ __launch_bounds__(kPrepThreads) void prep_kernel(
    const int32_t* __restrict__ seq_lens, int batch, int max_len, int split_target, int max_rounds, int positions,
    int depth,
    int max_chunks, WorkItem* __restrict__ work, SeqInfo* __restrict__ seqinfo,
    int* __restrict__ meta, const uint16_t* __restrict__ q_nope,
    const uint16_t* __restrict__ w_uk, _Float16* __restrict__ q_abs, int rows, int* __restrict__ range_flags) {
  __shared__ __attribute__((aligned(16))) char wl[kDNope * kWStride];
  static_assert(128 + 6 * 4 * kPlanSortMax <= kDNope * kWStride, "plan scratch fits the LDS buffer");
  if (blockIdx.x == 0) {
    // the plan is a short serial chain of barriers and reductions that must
    // not wait behind the absorb wavefronts sharing its SIMDs
    __builtin_amdgcn_s_setprio(3);
    plan_block(seq_lens, batch, max_len, split_target, max_rounds, positions, depth, max_chunks, work, seqinfo, meta,
               wl);
  } else {
    const int id = blockIdx.x - 1;
    absorb_block(q_nope, w_uk, q_abs, rows, id >> 2, id & 3, wl, range_flags + id);
  }
}

}  // namespace

hipError_t launch_prep(const int32_t* seq_lens, int batch, int max_len, int split_target, int max_rounds,
                       int positions, int depth, int max_chunks, WorkItem* work, SeqInfo* seqinfo, int* meta,
                       const uint16_t* q_nope, const uint16_t* w_uk, _Float16* q_abs, int rows,
                       int* range_flags, hipStream_t stream) {
  hipLaunchKernelGGL(prep_kernel, dim3(1 + kAbsorbGroups), dim3(kPrepThreads), 0, stream,
                     seq_lens, batch, max_len, split_target, max_rounds, positions, depth, max_chunks, work, seqinfo, meta,
                     q_nope, w_uk, q_abs, rows, range_flags);
  return hipGetLastError();
}

}  // namespace mla
