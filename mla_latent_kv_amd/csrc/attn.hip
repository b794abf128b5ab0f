// Fused score / online softmax / latent accumulation over the paged cache.
//
// For one split (sequence b, cached tokens [t_begin, t_end)) and 128 query
// rows, stream the 576-wide cached rows through LDS once and compute, per row:
//   s_j  = scale * (q_abs . c_KV,j + q_pe . k_R,j)
//   running max m, running sum l, O = sum_j exp(s_j - m) c_KV,j   (512 wide)
// then write the normalised partial O / l (fp16) and lse = m + log2 l for the
// merge pass. This is the absorb
// order of the "DeepSeek-V3" page (ailearn.mscapital.top), MLA section: the
// query side already carries W_UK, the RoPE part is multiplied separately and
// added, and the latent is aggregated before W_UV, so per-head keys and values
// never exist; k_R is one key per token shared by all heads (m.lsln.cn
// article, section 2.3).
//
// Mapping on gfx950 (wave64, 32x32x16 MFMA, 160 KB LDS):
// * workgroup = 4 wavefronts = 128 query rows. For the scores and the softmax
//   wavefront w owns 32 rows (32 heads of one new token); for the latent
//   accumulation it owns latent columns [128 w, 128 w + 128) of all 128 rows.
//   All wavefronts share each cache tile in LDS, so every cached byte crosses
//   HBM once per split (Sq = 2 runs two workgroups per split, one per 64-head
//   half, on the same XCD so the second read hits L2).
// * scores: D[token, row] = C_tile[token, :] . Q[row, :] -- the cache tile is
//   the A operand (lane = token, 8 consecutive latent values per k-step, one
//   16-byte LDS read), the wavefront's queries are the B operand and stay in
//   VGPRs for the whole split (32 fp16 k-steps of the latent part, 4 bf16
//   k-steps of the RoPE part). The chain accumulates in VGPRs (inline MFMAs)
//   so O owns all 256 AGPRs.
// * softmax: each lane owns one row (lane % 32) and 16 of the tile's 32
//   tokens, so row max and row sum are 16 in-lane steps plus one exchange with
//   lane ^ 32 (v_permlane32_swap, a VALU op: no LDS round trip, no wait on
//   the LDS queue). The running max is moved only when it grows by more than 2^15
//   (log2 units; p stays inside fp16); otherwise the stale max is kept, which
//   is exact because the final normalisation uses the same reference for O
//   and l. P (fp16) and the rare rescale factors go through LDS.
// * latent accumulation: D[latent col, row] += C_tile^T[col, token] P^T[token,
//   row]; the A operand comes from transposing LDS reads (ds_read_b64_tr_b16,
//   half the bytes per cycle of a 16-byte read, so each wavefront reads only
//   its quarter of the columns), the B operand (P) from LDS. O lives in 16
//   accumulator tiles (4 column tiles x 4 row tiles, 256 registers per lane).
// * cache tiles: 32 tokens, contiguous inside one 64-token block. The c_KV
//   part (32 KB) goes to a ring of four LDS buffers, the k_R part (4 KB) to a
//   ring of three, with direct-to-LDS loads (global_load_lds_dwordx4: no VGPRs
//   in flight). Each lane converts the c_KV granules it fetched from bf16 to
//   fp16 in place (exact in fp16's range). Rows past the split re-read its
//   last row, so NaN padding never reaches the latent MFMAs (their zero
//   softmax weights cancel them; masked scores become -inf with a select).
//   Granules are stored under a row-dependent permutation (S(r) below) that
//   keeps the score reads, the transposed reads and the P buffer free of
//   bank conflicts on gfx950's 64-bank LDS; the fetch addresses apply the
//   inverse permutation.
// * software pipeline, one barrier per tile, one MFMA per issue slot.
//   Iteration i runs phase A, the score chain of tile i + 1 with the fetch of
//   tile i + 3 and the conversion of tile i + 2 beside it, then phase B, the
//   latent MFMAs of tile i with the softmax of tile i + 1 cut into small
//   stages between them. sched_barrier fixes each slot's contents so the
//   operand reads stay ahead of their MFMAs. The barrier, three MFMAs before
//   the end of phase B, publishes P and the converted tile for the next
//   iteration, whose first score operands are read under those last MFMAs.
#include "common.h"

namespace mla {

namespace {

constexpr int kThreads = kWaves * 64;                     // 256
constexpr int kKvBytes = kTileTok * kDLat * 2;            // 32 KB: c_KV of a tile, 1 KB rows
constexpr int kKrBytes = kTileTok * kDRope * 2;           // 4 KB: k_R of a tile, 128 B rows
constexpr int kNKv = 4;                                   // c_KV ring: tiles i .. i + 3
constexpr int kNKr = 3;                                   // k_R ring: tiles i + 1 .. i + 3
constexpr int kColsPerWave = kDLat / kWaves;              // 128
constexpr int kPBytes = kRowsPerWg * kTileTok * 2;        // 8 KB of P per tile
// LDS map
constexpr int kOffKr = kNKv * kKvBytes;                          // 131072
constexpr int kOffP = kOffKr + kNKr * kKrBytes;                  // 143360: P, 2 parities
constexpr int kOffAlpha = kOffP + 2 * kPBytes;                   // 159744: rescale, 2 parities
constexpr int kOffFlag = kOffAlpha + 2 * kRowsPerWg * 4;         // 160768: per-wave flags
constexpr int kLdsBytes = kOffFlag + 2 * kWaves * 4;             // 160800
constexpr int kEpiBytes = kWaves * kRowsPerWg * kColsPerWave * 2;   // 131072 transpose space
static_assert(kEpiBytes <= kOffKr, "epilogue space is the c_KV ring");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
constexpr float kRescaleLog2 = 15.0f;   // lazy max threshold: p = 2^(x - m) < 2^15

#define MLA_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")
#define MLA_WAIT_LGKM0() asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory")
#define MLA_BARRIER() asm volatile("s_barrier" ::: "memory")

__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float lo = __builtin_bit_cast(float, v[i] << 16);
    float hi = __builtin_bit_cast(float, v[i] & 0xffff0000u);
    // exact for values representable in fp16, so the rounding mode is moot
    auto p = __builtin_amdgcn_cvt_pkrtz(lo, hi);
    r[i] = __builtin_bit_cast(unsigned int, p);
  }
  return r;
}

// One direct-to-LDS fetch: 64 lanes x 16 bytes from base + voff (per lane) to
// LDS bytes [lds, lds + 1024). Issued as inline asm so that the compiler does
// not treat every later LDS read as a possible alias of the in-flight write
// (it would otherwise drain all fetches before each read); the kernel orders
// these writes itself with explicit vmcnt waits and barriers. No VGPR result.
__device__ __forceinline__ void dma16(const char* lds, const char* base, unsigned voff) {
  const unsigned m0 = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(base)
               : "m0");
}

// x and x of lane l ^ 32, as the two halves of v_permlane32_swap: result 0
// holds [a lanes 0-31 | b lanes 0-31], result 1 [a lanes 32-63 | b lanes 32-63],
// so with a = b = x lane l sees x[l] in one and x[l ^ 32] in the other. The
// second copy goes through an empty asm so the two operands are distinct
// values to the optimizer.
struct Pair32 {
  float a, b;
};
__device__ __forceinline__ Pair32 pair32(float x) {
  float y = x;
  asm volatile("" : "+v"(y));
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, y), false, false);
  return Pair32{__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
}

// The same fetch with the LDS address given as a wave-uniform base plus an
// immediate, added straight into m0 (one scalar instruction per fetch).
__device__ __forceinline__ void dma16i(unsigned lds_base, int imm, const char* base, unsigned voff) {
  asm volatile("s_add_u32 m0, %0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3"
               :
               : "s"(lds_base), "i"(imm), "v"(voff), "s"(base)
               : "m0");
}

// max of three / two scores in one instruction each. fmaxf on values the
// compiler cannot prove canonical (MFMA results from inline asm) costs an
// extra canonicalizing instruction per operand; the scores are never
// signalling NaNs, so the plain instructions give the same maxima.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

template <typename T>
__device__ __forceinline__ T lds_read16(const char* base, int off) {
  return __builtin_bit_cast(T, *(const u32x4*)(base + off));
}

__device__ __forceinline__ f16x8 lds_read_tr(const char* p0, const char* p1) {
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
  return __builtin_bit_cast(f16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// score-chain MFMAs: accumulator in VGPRs, issued in program order
#define S_MFMA_FIRST(acc, a, b) \
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b))
#define S_MFMA(acc, a, b) \
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))
#define S_MFMA_BF16(acc, a, b) \
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))

__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  // ---- which position / which half of the heads. Workgroups are dealt to
  // the 8 XCDs round-robin by id (XCD = id % 8); the plan stores the work list
  // so that position p holds items of XCD p % 8 and each XCD runs a
  // contiguous run of slots (consecutive splits of the same sequences share
  // one L2 and their queries are fetched into it once). With Sq = 2 the two
  // head halves of a position are ids 8 apart: same XCD, dispatched together.
  // A workgroup runs the entries of its position one after another.
  int pos, grp;
  if (p.q_tokens == 1) {
    pos = blockIdx.x;
    grp = 0;
  } else {
    pos = ((blockIdx.x >> 4) << 3) + (blockIdx.x & 7);
    grp = (blockIdx.x >> 3) & 1;
  }
  if (pos >= p.positions) return;
  for (int item = 0; item < p.depth; ++item) {
  const WorkItem wi = p.work[(size_t)item * p.positions + pos];
  if (wi.slot < 0 || wi.slot >= p.max_chunks || wi.t_end <= wi.t_begin) break;
  const int b = wi.b;
  const int L = wi.len;

  // the thread index is made opaque per item, so that nothing derived from it
  // is hoisted out of the item loop (its registers would stay live across the
  // whole body, which already fills the register file)
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform (SGPR)
  const int half = lane >> 5;
  const int l32 = lane & 31;
  // rows of the workgroup: rr = 32 g + j is (new token qi(g), head hg(g) * 32 + j)
  auto row_qi = [&](int g) { return p.q_tokens == 1 ? 0 : (g >> 1); };
  auto row_hg = [&](int g) { return p.q_tokens == 1 ? g : 2 * grp + (g & 1); };
  const int qi = row_qi(w), hg = row_hg(w);                   // this wave's score rows
  const int r = b * p.q_tokens + qi;                          // query row of the batch
  const int n_vis = L - p.q_tokens + qi + 1;                  // visible positions
  const int lim = min(wi.t_end, n_vis);                       // tokens this wave may use
  const int rr = 32 * w + l32;                                // this lane's score row

  // ---- tile buffers
  auto kvb = [&](int i) -> char* { return smem + (i & (kNKv - 1)) * kKvBytes; };
  auto krb = [&](int i) -> char* { return smem + kOffKr + (i % kNKr) * kKrBytes; };

  // ---- fetch plan. c_KV rows are 1 KB, 64 granules of 16 bytes; logical
  // granule g of row r is stored at g ^ S(r), S(r) = sw(r % 8) + 8 ((r / 8) % 2)
  // with sw(x) the 3-bit rotate left of x (S is a permutation of 0..15 over any
  // 16 consecutive rows; why, below). Fetch j (0..7) of wave w moves row
  // 4 j + w: LDS slot `lane` of it holds logical granule lane ^ S(4 j + w),
  // and S(4 j + w) = 2 w + (j % 2) + 8 ((j / 2) % 2). The k_R fetch moves rows
  // 8 w .. 8 w + 7 (128 B rows of 8 granules, stored at g ^ ((r / 2) % 8)):
  // lane holds row 8 w + lane / 8, slot lane % 8, logical granule
  // (lane % 8) ^ ((4 w + lane / 16) % 8).
  // The row of fetch j is folded into the lane offset: fetch j reads
  // src + 16 rows * (j / 4) + voff_row[j % 4] (the granule permutation
  // repeats with period 4 in j), so a full tile's fetch needs no scalar
  // address arithmetic.
  const unsigned voff_base = 16u * (unsigned)(lane ^ (2 * w));
  unsigned voff_row[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj)
    voff_row[jj] = (voff_base ^ (16u * (jj & 1)) ^ (128u * ((jj >> 1) & 1))) + (unsigned)((4 * jj + w) * kRowBytes);
  const unsigned voff_kr = (unsigned)((8 * w + (lane >> 3)) * kRowBytes + kDLat * 2 +
                                      16 * ((lane & 7) ^ ((4 * w + (lane >> 4)) & 7)));
  // block ids of this split, 64 per window: lane i holds the id of block
  // blk_base + i; a tile reads its id with one lane read
  const int32_t* btab = p.block_table + (size_t)b * p.max_blocks_per_seq;
  const int blk_first = wi.t_begin / kBlock;
  const int blk_last = (wi.t_end - 1) / kBlock;
  int blk_base = blk_first;
  // issued before the query loads below, consumed from tile 3 on
  int blk_lane = blk_first + lane <= blk_last ? btab[blk_first + lane] : 0;
  const int blk_max = (int)min(p.num_blocks - 1, (long long)0x7fffffff);
  auto tile_src = [&](int ts) -> const char* {   // ts >= 0
    const int bi = (int)((unsigned)ts / kBlock);
    if (bi >= blk_base + 64) {   // next window (splits longer than 4096 tokens)
      blk_base += 64;
      blk_lane = blk_base + lane <= blk_last ? btab[blk_base + lane] : 0;
      asm volatile("" : "+v"(blk_lane));
    }
    const int blk = min(max(__builtin_amdgcn_readlane(blk_lane, bi - blk_base), 0), blk_max);   // memory safety
    return (const char*)p.cache + (size_t)(unsigned)blk * (kBlock * kRowBytes) +
           ((unsigned)ts % kBlock) * kRowBytes;
  };
  // c_KV fetch j of a tile with `valid` rows inside the split: rows at or past
  // it re-read the last valid row, so they hold finite values that the zero
  // softmax weights of their (masked) positions cancel; the choice is
  // wave-uniform (scalar address arithmetic)
  auto fetch_kv = [&](const char* src, int i, int j, int valid) {
    const int srow = min(4 * j + w, valid - 1);
    dma16(kvb(i) + 1024 * (4 * j + w), src + (srow - 4 * (j & 3) - w) * kRowBytes, voff_row[j & 3]);
  };
  auto fetch_kr = [&](const char* src, int i) { dma16(krb(i) + 1024 * w, src, voff_kr); };
  // in-place bf16 -> fp16 of the c_KV granules this lane fetched (rows 4 j + w);
  // all reads first, then the conversions and writes
  auto convert_tile = [&](char* tb) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = *(const u32x4*)(tb + 1024 * (4 * j + w) + 16 * lane);
#pragma unroll
    for (int j = 0; j < 8; ++j) *(u32x4*)(tb + 1024 * (4 * j + w) + 16 * lane) = bf16x8_to_f16x8(v[j]);
  };

  // ---- queries: latent part and RoPE part -> VGPRs (B operands: lane = row,
  // 8 consecutive k), in flight together with the block ids
  f16x8 qa[32];
  bf16x8 qp[4];
  {
    const u32x4* src = (const u32x4*)(p.q_abs + ((size_t)(r * 4 + hg) * 32) * 64 * 8);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qa[ks] = __builtin_bit_cast(f16x8, src[ks * 64 + lane]);
    const uint16_t* qsrc = p.q_pe + ((size_t)r * kHeads + hg * 32 + l32) * kDRope + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qp[ks] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qsrc + 16 * ks));
  }

  // ---- prologue fetch of tile 0 (tiles 1 and 2 follow once the queries are
  // in). Tiles 0 and 1 lie in the split's first cache block and tile 2 in
  // its second (splits start on a block boundary); the plan resolved both
  // block ids, so these fetches need no block-table round trip.
  const int n_tiles = (wi.t_end - wi.t_begin + kTileTok - 1) / kTileTok;
  const int t0 = wi.t_begin;
  auto fetch_tile = [&](int i) {
    const long long blk = i < 2 ? wi.blk0 : wi.blk1;
    const long long bl = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);   // memory safety
    const char* src = (const char*)p.cache + ((size_t)bl * kBlock + (i & 1) * kTileTok) * kRowBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) fetch_kv(src, i, j, wi.t_end - (t0 + i * kTileTok));
    fetch_kr(src, i);
  };
  fetch_tile(0);
  // the compiler waits for the queries (and so for tile 0) here: a wait inside
  // the loop would also drain the fetches
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) asm volatile("" : "+v"(qa[ks]));
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(qp[ks]));
  MLA_WAIT_VM(0);
  // the block ids (the oldest load) are in as well; the empty asm keeps the
  // load ahead of this point, so the loop's first lookups do not wait
  asm volatile("" : "+v"(blk_lane));
  // q_pe enters the score scaled by kQScale like q_abs (exact: a power of
  // two on bf16 values; the products and the softmax scale undo it)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    u32x4 v = __builtin_bit_cast(u32x4, qp[ks]);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float lo = __builtin_bit_cast(float, v[d] << 16) * kQScale;
      const float hi = __builtin_bit_cast(float, v[d] & 0xffff0000u) * kQScale;
      v[d] = (__builtin_bit_cast(unsigned int, lo) >> 16) | (__builtin_bit_cast(unsigned int, hi) & 0xffff0000u);
    }
    qp[ks] = __builtin_bit_cast(bf16x8, v);
  }
  // the score chain reads qp through inline MFMAs, whose operand hazards the
  // compiler does not cover: two wait states after the last VALU write
  asm volatile("s_nop 1" : "+v"(qp[0]), "+v"(qp[1]), "+v"(qp[2]), "+v"(qp[3]));
  // tiles 1 and 2 land under the conversion, scores and softmax of tile 0
  for (int i = 1; i < 3 && i < n_tiles; ++i) fetch_tile(i);

  // ---- per-lane LDS offsets. gfx950's LDS serves a 16-byte read 16 lanes at
  // a time across 64 banks; a pass is free of bank conflicts when its 16
  // addresses fall in 16 different 16-byte bank groups of a 256-byte window
  // (measured: a 128-byte window, the 32-bank layout, doubles the time of a
  // score read). S(r) does that for 16 consecutive rows that read one logical
  // granule (score reads); sw(x) = ((x & 3) << 1) | (x >> 2) also puts the
  // granule pair {2 m, 2 m + 1} of rows 4 k .. 4 k + 3 in 8 different groups
  // (transposed reads). Rows are 1 KB apart, so every row starts in the same
  // bank.
  auto sw = [](int x) { return ((x & 3) << 1) | (x >> 2); };
  // scores: row = l32, logical granule 2 ks + half, stored at
  // l32 * 1024 + 16 ((2 ks + half) ^ S(l32)): the low 3 bits move by sw(l32 % 8)
  // and the 128-byte block ks / 4 becomes (ks / 4) ^ b3, b3 = (l32 / 8) % 2,
  // i.e. + b3 for even blocks and - b3 for odd ones (s_at). k_R k-step ks
  // reads r_off[ks] in the k_R buffer.
  int s_offE[4], s_offO[4], r_off[4];
  {
    const int b3 = (l32 >> 3) & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int base = l32 * 1024 + 16 * ((2 * j + half) ^ sw(l32 & 7));
      s_offE[j] = base + 128 * b3;
      s_offO[j] = base - 128 * b3;
      r_off[j] = l32 * 128 + 16 * ((2 * j + half) ^ ((l32 >> 1) & 7));
    }
  }
  auto s_at = [&](int ks) { return (((ks >> 2) & 1) ? s_offO : s_offE)[ks & 3] + 128 * (ks >> 2); };
  // transposed reads of this wave's columns. MFMA k-slot (hh, e) of k-step st
  // is token 16 st + 8 (e / 4) + 4 hh + e % 4 (the score accumulator's token
  // order). Group gg = lane / 16 (k-half hh = gg / 2, 16-column half gg % 2);
  // for read q source lane L addresses token 16 st + 8 q + 4 hh + L / 4 at
  // column 128 w + 32 ct + 16 (gg % 2) + 4 (L % 4). For q = 0 the row's
  // swizzle is sw(row % 8) for every st, so one base per column tile serves
  // all k-steps; rows of q = 1 add 8 to S, which flips bit 3 of the granule:
  // bit 6 of the column, i.e. ct / 2 (tr_pair).
  const int gg = lane >> 4, Lq = lane & 15, hh = gg >> 1;
  // the low-3-bit swizzle flips bit 2 of the granule at most, and a column
  // tile is 4 granules: tiles 2 and 3 sit 8 granules (128 bytes) past tiles 0
  // and 1, so two registers serve all four (tr_at)
  int tr_off2[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int row = 4 * hh + (Lq >> 2);
    const int col = kColsPerWave * w + 32 * ct + 16 * (gg & 1) + 4 * (Lq & 3);
    tr_off2[ct] = row * 1024 + 16 * ((col >> 3) ^ sw(row & 7)) + 2 * (col & 7);
  }
  auto tr_at = [&](int ct) { return tr_off2[ct & 1] + 128 * (ct >> 1); };
  // A operand of column tile ct, k-step st, from the tile at `tb`
  auto tr_pair = [&](const char* tb, int ct, int st) {
    const char* p0 = tb + tr_at(ct) + 1024 * 16 * st;
    return lds_read_tr(p0, p0 + 1024 * 8 + ((ct >> 1) ? -128 : 128));
  };
  // P: [row][32 positions] fp16, 64 B per row, 16-byte chunk c stored at
  // c ^ ((row / 4) % 4) (16 consecutive rows reading one chunk fill 16 bank
  // groups). Position 16 st + 8 hh + e holds the token of k-slot (hh, e) of
  // k-step st, so a B fragment is one 16-byte chunk (2 st + hh).
  auto p_chunk = [](int row, int c) { return row * 64 + 16 * (c ^ ((row >> 2) & 3)); };

  f32x16 o[4][4];   // [column tile][row tile]
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int h = 0; h < 4; ++h) o[c][h] = f32x16{};
  float m = -INFINITY, l = 0.f;   // statistics of this lane's score row
  const float scale_log2 = p.scale_log2;

  // softmax of one tile's scores (tile start ts, parity par): P and the rescale
  // factor to LDS, the running statistics updated. Straight-line code, so it
  // can be interleaved with independent MFMAs.
  auto softmax_tile = [&](f32x16 s, int ts, int par) {
    // s[i] is token ts + 8 (i / 4) + 4 half + i % 4
    const int nv = lim - ts - 4 * half;   // tokens of this lane's k-half below lim
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = (8 * (i >> 2) + (i & 3)) < nv ? s[i] : -INFINITY;
    float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                     fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mt = fmaxf(mt, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                         fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
    {
      const Pair32 pm = pair32(mt);
      mt = fmaxf(pm.a, pm.b) * scale_log2;
    }
    const bool grow = mt > m + kRescaleLog2;
    const float m_new = grow ? mt : m;
    // O rows hold earlier tiles relative to m; they scale by 2^(m - m_new)
    const bool rescale = grow && m != -INFINITY;
    const float alpha = rescale ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
    const int any_rescale = __ballot(rescale) != 0ull;
    m = m_new;
    const float neg_m = (m == -INFINITY) ? 0.f : -m;
    float rs = 0.f;
    f16x4 pq[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], scale_log2, neg_m));
      rs += e;
      pq[i >> 2][i & 3] = (_Float16)e;
    }
    {
      const Pair32 ps = pair32(rs);
      rs = ps.a + ps.b;
    }
    l = l * alpha + rs;
    // registers 4 q .. 4 q + 3 are tokens 8 q + 4 half + 0..3, i.e. k-step
    // q / 2, k-half `half`, slots 4 (q % 2) .. + 3: chunk 2 (q / 2) + half,
    // 8 bytes in at 8 (q % 2)
    char* pbuf = smem + kOffP + par * kPBytes;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(f16x4*)(pbuf + p_chunk(rr, 2 * (q >> 1) + half) + 8 * (q & 1)) = pq[q];
    // both half-waves store the same values (no divergent branch)
    ((float*)(smem + kOffAlpha + par * kRowsPerWg * 4))[rr] = alpha;
    ((int*)(smem + kOffFlag + par * kWaves * 4))[w] = any_rescale;
  };

  // rescale O rows whose reference moved (rare); flags / factors of parity par
  // always inlined: an out-of-line copy would take O out of the registers
  auto rescale_o = [&](int par, int4 fl) __attribute__((always_inline)) {
    {
      const float* al = (const float*)(smem + kOffAlpha + par * kRowsPerWg * 4);
      float ah[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int fh = h == 0 ? fl.x : h == 1 ? fl.y : h == 2 ? fl.z : fl.w;
        ah[h] = fh ? al[32 * h + l32] : 1.f;
      }
      // O *= alpha in place in the accumulator registers (read / multiply /
      // write per element, so O never leaves the AGPRs); the s_nops cover
      // the MFMA -> accumulator-read and write -> MFMA distances.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = o[c][h][i], tmp;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                : "+a"(x), "=&v"(tmp)
                : "v"(ah[h]));
            o[c][h][i] = x;
          }
      asm volatile("s_nop 7" ::: "memory");
    }
  };

  // latent MFMAs of one k-step (16 tokens) of tile `cur` with P of parity par
  auto pv_step = [&](const char* cur, const char* pbuf, int st) {
    f16x8 pb[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) pb[h] = lds_read16<f16x8>(pbuf, p_chunk(32 * h + l32, 2 * st + half));
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const f16x8 a = tr_pair(cur, ct, st);
#pragma unroll
      for (int h = 0; h < 4; ++h)
        o[ct][h] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[h], o[ct][h], 0, 0, 0);
    }
  };

  // ---- prologue: convert tile 0; scores and softmax of tile 0; convert tile 1
  convert_tile(kvb(0));
  MLA_WAIT_LGKM0();
  MLA_BARRIER();
  {
    const char* kv = kvb(0);
    const char* kr = krb(0);
    f32x16 s;
    f16x8 sa[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sa[j] = lds_read16<f16x8>(kv, s_at(j));
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) {
      if (ks == 0) {
        S_MFMA_FIRST(s, sa[0], qa[0]);
      } else {
        S_MFMA(s, sa[ks & 3], qa[ks]);
      }
      const int nk = ks + 4;
      if (nk < 32) sa[ks & 3] = lds_read16<f16x8>(kv, s_at(nk));
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 a = lds_read16<bf16x8>(kr, r_off[ks]);
      S_MFMA_BF16(s, a, qp[ks]);
    }
    asm volatile("s_nop 15" : "+v"(s));
    softmax_tile(s, t0, 0);
  }
  if (n_tiles > 1) {
    // tile 1 has landed once at most tile 2's 9 fetches are outstanding
    if (n_tiles > 2) {
      MLA_WAIT_VM(9);
    } else {
      MLA_WAIT_VM(0);
    }
    convert_tile(kvb(1));
  }
  MLA_WAIT_LGKM0();
  MLA_BARRIER();

  // ---- main loop: iteration i = latent pass of tile i, scores and softmax of
  // tile i + 1, conversion of tile i + 2, fetch of tile i + 3. The body is one
  // straight-line MFMA stream, compiled four ways: with the fetch of a full
  // tile and the conversion (three instructions per fetch: the row is in the
  // lane offset), with the fetch of the split's last tile (rows past the
  // split clamped to its last row) and the conversion (i = n - 4), with the
  // conversion only (i = n - 3: tile i + 3 does not exist) and with neither
  // (i = n - 2), so the last iterations do no dead work; all fetches are
  // drained before the epilogue.
  const int t_last = t0 + (n_tiles - 1) * kTileTok;
  // One issue slot = one MFMA plus the loads, stores and VALU work placed
  // beside it; sched_barrier keeps every slot's work where it is written, so
  // the operand loads stay several MFMAs ahead of their use (the compiler
  // would otherwise pull them next to the MFMA and wait for each one).
#define MLA_SLOT() __builtin_amdgcn_sched_barrier(0)
  // Only about four VALU instructions issue under one 32x32x16 MFMA of the
  // same wave (measured on gfx950: 8 VALU per MFMA take 42-47 cycles instead of
  // 32), so the VALU work of an iteration (the conversion's 96 instructions,
  // the softmax's ~90) is spread at most ~4 per slot.
  // kFetch: tile i + 3 exists; kFull: it is not the split's last tile, so all
  // its 32 rows lie inside the split and need no clamp; kConv: tile i + 2
  // exists. Every call passes constants, so each inlined copy keeps only its
  // own work.
  f16x8 sa_pre[2];
  auto iteration = [&](int i, const char* fsrc, const bool kFetch, const bool kFull, const bool kConv)
                       __attribute__((always_inline)) -> const char* {
    const int ts = t0 + i * kTileTok;
    const char* cur = kvb(i);
    const char* pbuf = smem + kOffP + (i & 1) * kPBytes;
    const char* kv1 = kvb(i + 1);
    const char* kr1 = krb(i + 1);
    const int fts = min(ts + 3 * kTileTok, t_last);
    const int fvalid = wi.t_end - fts;
    char* cbuf = kvb(i + 2);
    // LDS address of this wave's first c_KV row of tile i + 3
    const unsigned f_lds = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)(kvb(i + 3) + 1024 * w);
    // the rescale flags of tile i, read now and tested before its latent
    // MFMAs (phase B), so the read's latency hides behind the score chain;
    // the first two score operands of tile i + 1 were read by the previous
    // iteration (or before the loop) right after its barrier, under its last
    // latent MFMAs
    const int4 flags = *(const int4*)(smem + kOffFlag + (i & 1) * kWaves * 4);

    // in-place bf16 -> fp16 of granule g (rows 4 g + w) of tile i + 2, read 4
    // slots before its first dword is converted; its fetch was issued in the
    // previous iteration, ahead of tile i + 3's fetches (vmcnt counts loads in
    // issue order; the nine fetches of tile i + 3 go out in slots 0-8, each
    // before the granule read of its slot), so granule g read in slot 4 g
    // waits for all but (8 - g) + min(4 g + 1, 9) younger loads; without the
    // fetch of tile i + 3 only tile i + 2's own later fetches (8 - g) are younger
    auto conv_read = [&](int g) -> u32x4 {
      if (kFetch) {
        switch (g) {   // vmcnt takes an immediate
          case 0: MLA_WAIT_VM(9); break;
          case 1: MLA_WAIT_VM(12); break;
          case 2: MLA_WAIT_VM(15); break;
          case 3: MLA_WAIT_VM(14); break;
          case 4: MLA_WAIT_VM(13); break;
          case 5: MLA_WAIT_VM(12); break;
          case 6: MLA_WAIT_VM(11); break;
          default: MLA_WAIT_VM(10); break;
        }
      } else {
        switch (g) {
          case 0: MLA_WAIT_VM(8); break;
          case 1: MLA_WAIT_VM(7); break;
          case 2: MLA_WAIT_VM(6); break;
          case 3: MLA_WAIT_VM(5); break;
          case 4: MLA_WAIT_VM(4); break;
          case 5: MLA_WAIT_VM(3); break;
          case 6: MLA_WAIT_VM(2); break;
          default: MLA_WAIT_VM(1); break;
        }
      }
      return *(const u32x4*)(cbuf + 1024 * (4 * g + w) + 16 * lane);
    };
    auto conv_dword = [&](u32x4& v, int d) {   // 3 VALU: exact in fp16's range
      const float lo = __builtin_bit_cast(float, v[d] << 16);
      const float hi = __builtin_bit_cast(float, v[d] & 0xffff0000u);
      v[d] = __builtin_bit_cast(unsigned int, __builtin_amdgcn_cvt_pkrtz(lo, hi));
    };
    auto conv_store = [&](int g, u32x4 v) { *(u32x4*)(cbuf + 1024 * (4 * g + w) + 16 * lane) = v; };

    // ---- phase A: the score chain of tile i + 1 (32 fp16 + 4 bf16 MFMAs,
    // operands read 4 k-steps ahead). Slots 0-8 issue the nine fetches of
    // tile i + 3; granule g of tile i + 2 is read in slot 4 g, converted a
    // dword per slot in slots 4 g + 4 .. 4 g + 7 and written back in the last
    // of them; slots 32-35 read phase B's first operands.
    auto s_frag = [&](int ks) -> f16x8 {
      return ks < 32 ? lds_read16<f16x8>(kv1, s_at(ks))
                     : lds_read16<f16x8>(kr1, r_off[ks - 32]);
    };
    f16x8 sa[4];
    sa[0] = sa_pre[0];
    sa[1] = sa_pre[1];
#pragma unroll
    for (int j = 2; j < 4; ++j) sa[j] = s_frag(j);
    MLA_SLOT();
    f32x16 s;
    u32x4 cv[2];
    f16x8 pb[4], ta[2];
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      // inline MFMAs keep the chain's accumulator in VGPRs (O holds the AGPRs)
      if (ks == 0) {
        S_MFMA_FIRST(s, sa[0], qa[0]);
      } else if (ks < 32) {
        S_MFMA(s, sa[ks & 3], qa[ks]);
      } else {
        S_MFMA_BF16(s, __builtin_bit_cast(bf16x8, sa[ks & 3]), qp[ks - 32]);
      }
      if (ks + 4 < 36) sa[ks & 3] = s_frag(ks + 4);
      if (kFetch && !kFull && ks < 8) fetch_kv(fsrc, i + 3, ks, fvalid);
      if (kFetch && kFull && ks < 8)
        dma16i(f_lds, 4096 * ks, ks < 4 ? fsrc : fsrc + 16 * kRowBytes, voff_row[ks & 3]);
      if (kFetch && ks == 8) fetch_kr(fsrc, i + 3);
      if (kConv && ks < 32 && (ks & 3) == 0) cv[(ks >> 2) & 1] = conv_read(ks >> 2);
      if (kConv && ks >= 4) {
        const int g = (ks - 4) >> 2, d = (ks - 4) & 3;
        conv_dword(cv[g & 1], d);
        if (d == 3) conv_store(g, cv[g & 1]);
      }
      // phase B's first operands, in the registers the chain's last k-steps free
      if (ks >= 32) pb[ks - 32] = lds_read16<f16x8>(pbuf, p_chunk(32 * (ks - 32) + l32, half));
      if (ks == 33) ta[0] = tr_pair(cur, 0, 0);
      MLA_SLOT();
    }

    // ---- phase B: the latent MFMAs of tile i (2 k-steps x 4 column tiles x 4
    // row tiles) with the softmax of tile i + 1 cut into stages of at most
    // about four VALU instructions, one per slot
    const int sts = ts + kTileTok;
    const int par1 = (i + 1) & 1;
    float mx[5], mt = 0.f, alpha = 1.f, neg_m = 0.f, rsum[2] = {0.f, 0.f};
    bool grow = false, rescale = false;
    int any_rescale = 0;
    f16x4 pq[4];
    // tokens of this lane's k-half below lim; a full tile needs no mask
    const int nv = lim - sts - 4 * half;
    const bool full = sts + kTileTok <= lim;   // wave-uniform
    // the tile's 16 scores of this lane: five max3 of 15 scores, then the
    // five partial maxima and the 16th score
    auto mx3 = [&](int q) { mx[q] = max3f(s[3 * q], s[3 * q + 1], s[3 * q + 2]); };
    auto stage = [&](int k) {
      if (k == 0) {
        // the chain's last MFMA (inline asm: the compiler does not count its
        // latency) has written s at least 16 wait states before this read
        asm volatile("s_nop 15" : "+v"(s));
        if (!full) {
#pragma unroll
          for (int e = 0; e < 16; ++e) s[e] = (8 * (e >> 2) + (e & 3)) < nv ? s[e] : -INFINITY;
        }
      } else if (k == 1) {
        mx3(0);
        mx3(1);
        mx3(2);
      } else if (k == 2) {
        mx3(3);
        mx3(4);
      } else if (k == 3) {
        mt = max2f(max3f(mx[0], mx[1], mx[2]), max3f(mx[3], mx[4], s[15]));
      } else if (k == 4) {
        const Pair32 pm = pair32(mt);
        mt = max2f(pm.a, pm.b) * scale_log2;
      } else if (k == 5) {
        grow = mt > m + kRescaleLog2;
        rescale = grow && m != -INFINITY;
      } else if (k == 6) {
        const float m_new = grow ? mt : m;
        alpha = rescale ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
        m = m_new;
      } else if (k == 7) {
        any_rescale = __ballot(rescale) != 0ull;
        neg_m = (m == -INFINITY) ? 0.f : -m;
      } else if (k >= 8 && k < 24) {   // one exponential per stage
        const int e = k - 8;
        const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], scale_log2, neg_m));
        rsum[e & 1] += x;
        pq[e >> 2][e & 3] = (_Float16)x;
      } else if (k == 24) {
        const Pair32 ps = pair32(rsum[0] + rsum[1]);
        l = l * alpha + (ps.a + ps.b);
      } else if (k == 25) {
        char* pdst = smem + kOffP + par1 * kPBytes;
#pragma unroll
        for (int q = 0; q < 4; ++q) *(f16x4*)(pdst + p_chunk(rr, 2 * (q >> 1) + half) + 8 * (q & 1)) = pq[q];
      } else if (k == 26) {
        ((float*)(smem + kOffAlpha + par1 * kRowsPerWg * 4))[rr] = alpha;
        ((int*)(smem + kOffFlag + par1 * kWaves * 4))[w] = any_rescale;
      }
    };

    if (flags.x | flags.y | flags.z | flags.w) rescale_o(i & 1, flags);
    MLA_SLOT();
    const char* fsrc_next = fsrc;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int st = k >> 4, ct = (k >> 2) & 3, rt = k & 3;
      o[ct][rt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ta[ct & 1], pb[rt], o[ct][rt], 0, 0, 0);
      // next column tile's transposed operand, 3 MFMAs ahead of its first use
      if (rt == 1 && k + 3 < 32) {
        const int nst = (k + 3) >> 4, nct = ((k + 3) >> 2) & 3;
        ta[nct & 1] = tr_pair(cur, nct, nst);
      }
      // P of k-step 1 replaces k-step 0's once its last MFMA has issued
      if (st == 0 && ct == 3) pb[rt] = lds_read16<f16x8>(pbuf, p_chunk(32 * rt + l32, 2 + half));
      // softmax stages 0-26 in slots 1-27
      if (k >= 1 && k <= 27) stage(k - 1);
      // the next iteration's fetch source (scalar work, off the first slot)
      if (kFetch && k == 29) fsrc_next = tile_src(min(ts + 4 * kTileTok, t_last));
      if (k == 28) {
        // The barrier goes here, three MFMAs before the end: P, the rescale
        // flags (stages 25-26) and the converted tile i + 2 are written, every
        // operand read of tile i has been issued (the last at slot 25) and
        // is waited for, so tile i's buffer is free for the next fetch; the
        // last three MFMAs need registers only.
        // Tile i + 2's k_R fetch has landed too (its nine fetches are all in).
        if (kFetch) {
          MLA_WAIT_VM(9);
        } else {
          MLA_WAIT_VM(0);
        }
        MLA_WAIT_LGKM0();
        MLA_BARRIER();
      }
      // the next iteration's first score operands (tile i + 2, published by
      // the barrier) under the last MFMAs
      if (kConv && k == 29) sa_pre[0] = lds_read16<f16x8>(kvb(i + 2), s_at(0));
      if (kConv && k == 30) sa_pre[1] = lds_read16<f16x8>(kvb(i + 2), s_at(1));
      MLA_SLOT();
    }
    return fsrc_next;
  };
  {
    const char* fsrc = tile_src(min(t0 + 3 * kTileTok, t_last));
    sa_pre[0] = lds_read16<f16x8>(kvb(1), s_at(0));
    sa_pre[1] = lds_read16<f16x8>(kvb(1), s_at(1));
    int i = 0;
    for (; i + 4 < n_tiles; ++i) fsrc = iteration(i, fsrc, true, true, true);
    if (i + 3 < n_tiles) fsrc = iteration(i++, fsrc, true, false, true);
    if (i + 2 < n_tiles) iteration(i++, fsrc, false, false, true);
    if (i + 1 < n_tiles) iteration(i, fsrc, false, false, false);
  }
  // last tile: latent pass only. The statistics are final (the last softmax
  // ran in the previous iteration): 1/l of this wave's rows goes to the
  // rescale slot of parity (i + 1) & 1, which no wave reads again, and the
  // barrier after the latent pass publishes it
  float* stat = (float*)(smem + kOffAlpha + (n_tiles & 1) * kRowsPerWg * 4);
  {
    const int i = n_tiles - 1;
    const int4 fl = *(const int4*)(smem + kOffFlag + (i & 1) * kWaves * 4);
    if (half == 0) stat[rr] = l > 0.f ? 1.f / l : 0.f;
    {
      // lse = m + log2 l per score row, -inf when the row saw no position
      const size_t rows_per_chunk = (size_t)p.q_tokens * kHeads;
      const size_t row0 = (size_t)wi.slot * rows_per_chunk + qi * kHeads + hg * 32;
      if (half == 0) p.part_lse[row0 + l32] = l > 0.f ? m + __log2f(l) : -INFINITY;
    }
    if (fl.x | fl.y | fl.z | fl.w) rescale_o(i & 1, fl);
    const char* cur = kvb(i);
    const char* pbuf = smem + kOffP + (i & 1) * kPBytes;
    pv_step(cur, pbuf, 0);
    pv_step(cur, pbuf, 1);
  }

  // the epilogue reuses the c_KV ring: no fetch may still be landing, and
  // every wave must be past its last read (and its 1/l written)
  MLA_WAIT_VM(0);
  MLA_WAIT_LGKM0();
  MLA_BARRIER();
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // ---- partial state: o_hat = O / l rounded to fp16, rows (qi, head) of 512
  // contiguous values; this wave writes columns [128 w, 128 w + 128) of all
  // 128 rows. The accumulator layout (lane = row, registers = columns) is
  // turned row-major through this wave's 32 KB of LDS (the c_KV ring is free
  // after the last barrier): 8-byte units of 4 columns, unit ^ 2 (row % 16).
  float inv_l[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) inv_l[h] = stat[32 * h + l32];
  char* tw = smem + w * (kRowsPerWg * kColsPerWave * 2);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 32 * h + l32;
        const int u = 8 * c + 2 * q + half;   // columns 32 c + 8 q + 4 half .. + 3
        const float il = inv_l[h];
        f16x4 v = {(_Float16)(o[c][h][4 * q] * il), (_Float16)(o[c][h][4 * q + 1] * il),
                   (_Float16)(o[c][h][4 * q + 2] * il), (_Float16)(o[c][h][4 * q + 3] * il)};
        *(f16x4*)(tw + row * (kColsPerWave * 2) + 8 * (u ^ (2 * (row & 15)))) = v;
      }
  MLA_WAIT_LGKM0();   // this wave's own LDS writes only: no barrier needed
  const size_t rows_per_chunk = (size_t)p.q_tokens * kHeads;
  _Float16* dst = p.part_o + (size_t)wi.slot * rows_per_chunk * kDLat + kColsPerWave * w;
#pragma unroll 8
  for (int i = 0; i < kRowsPerWg / 4; ++i) {
    const int row = 4 * i + (lane >> 4), c16 = lane & 15;   // 16 lanes x 16 B per row
    const int x = 2 * (row & 15);
    const u32x4 v = *(const u32x4*)(tw + row * (kColsPerWave * 2) + 8 * ((2 * c16) ^ x));
    const int g = row >> 5, j = row & 31;
    const size_t prow = (size_t)row_qi(g) * kHeads + row_hg(g) * 32 + j;
    *(u32x4*)(dst + prow * kDLat + 8 * c16) = v;
  }
  // the next item's fetches refill the buffers this epilogue read
  MLA_WAIT_LGKM0();
  MLA_BARRIER();
  }   // item
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  // one workgroup per work-list position (two for Sq = 2)
  const int grid = a.q_tokens == 1 ? a.positions : 2 * a.positions;
  hipLaunchKernelGGL(attn_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
