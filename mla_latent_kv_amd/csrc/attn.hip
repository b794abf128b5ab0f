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
//   k-steps of the RoPE part). The chain accumulates in VGPRs (inline MFMAs,
//   the result-to-VALU distance covered by s_nop) so O owns all 256 AGPRs.
// * softmax: each lane owns one row (lane % 32) and 16 of the tile's 32
//   tokens, so row max and row sum are 16 in-lane steps plus one exchange with
//   lane ^ 32. The running max is moved only when it grows by more than 2^15
//   (log2 units; p stays inside fp16); otherwise the stale max is kept, which
//   is exact because the final normalisation uses the same reference for O
//   and l. P (fp16) and the rare rescale factors go through LDS.
// * latent accumulation: D[latent col, row] += C_tile^T[col, token] P^T[token,
//   row]; the A operand comes from transposing LDS reads (ds_read_b64_tr_b16,
//   half the bytes per cycle of a 16-byte read, so each wavefront reads only
//   its quarter of the columns), the B operand (P) from LDS. O lives in 16
//   accumulator tiles (4 column tiles x 4 row tiles, 256 registers per lane).
// * cache tiles: 32 tokens x 1152 B = 36 KB, contiguous inside one 64-token
//   block, in a ring of three LDS buffers. Tiles are fetched two ahead with
//   direct-to-LDS loads (global_load_lds_dwordx4: no VGPRs in flight), issued
//   under the latent MFMAs; once a tile has landed each lane converts the
//   c_KV granules it fetched from bf16 to fp16 in place (exact in fp16's
//   range) and zeroes rows past the split, so NaN padding never reaches the
//   latent MFMAs (masked scores become -inf with a select). The granule
//   swizzle g ^ (row % 8) keeps the score reads, the transposed reads and the
//   conversion pass free of bank conflicts; the fetch addresses apply the
//   inverse permutation.
// * per tile, one barrier: scores, softmax, P to LDS, conversion of the next
//   tile | barrier | rescale (rare), latent accumulation, fetch of the tile
//   after next.
#include "common.h"

namespace mla {

namespace {

constexpr int kGranPerRow = kRowBytes / 16;               // 72
constexpr int kTileBytes = kTileTok * kRowBytes;          // 36864
constexpr int kThreads = kWaves * 64;                     // 256
constexpr int kFetch = kTileBytes / 16 / kThreads;        // 9 granules per lane per tile
constexpr int kNBuf = 3;                                  // LDS tile ring
constexpr int kColsPerWave = kDLat / kWaves;              // 128
constexpr int kQpWaveBytes = kRowsPerWave * kDRope * 2;   // 4 KB of q_pe per wavefront
constexpr int kPBytes = kRowsPerWg * kTileTok * 2;        // 8 KB of P per tile
// LDS map
constexpr int kOffQp = kNBuf * kTileBytes;                       // 110592
constexpr int kOffP = kOffQp + kWaves * kQpWaveBytes;            // 126976: P, 2 parities
constexpr int kOffAlpha = kOffP + 2 * kPBytes;                   // 143360: rescale, 2 parities
constexpr int kOffFlag = kOffAlpha + 2 * kRowsPerWg * 4;         // 144384: per-wave flags
constexpr int kOffStat = kOffFlag + 2 * kWaves * 4;              // 144416: 1/l per row
constexpr int kLdsBytes = kOffStat + kRowsPerWg * 4;             // 144928
constexpr int kEpiBytes = kWaves * kRowsPerWg * kColsPerWave * 2;   // 131072 transpose space
static_assert(kEpiBytes <= kOffAlpha, "epilogue space must not reach the statistics");
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

template <typename T>
__device__ __forceinline__ T lds_read16(const char* base, int off) {
  return __builtin_bit_cast(T, *(const u32x4*)(base + off));
}

__device__ __forceinline__ f16x8 lds_read_tr(const char* p0, const char* p1) {
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
  return __builtin_bit_cast(f16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Scores of one tile for this wavefront's 32 rows: D[token, row] over 32 fp16
// k-steps (latent) and 4 bf16 k-steps (RoPE), accumulated in VGPRs; dependent
// MFMAs on one accumulator issue back to back, s_nop 15 covers the
// MFMA-result -> VALU-read distance. A fragments are read 4 MFMAs ahead.
__device__ __forceinline__ f32x16 score_tile(const char* cur, const int (&s_off)[4],
                                             const f16x8 (&qa)[32], const char* qp_row,
                                             int qp_x) {
  constexpr int kPre = 4;
  f16x8 a[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) a[j] = lds_read16<f16x8>(cur, s_off[j & 3] + 128 * (j >> 2));
  f32x16 s;
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=v"(s) : "v"(a[0]), "v"(qa[0]));
  a[0] = lds_read16<f16x8>(cur, s_off[0] + 128);
#pragma unroll
  for (int ks = 1; ks < 32; ++ks) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                 : "+v"(s)
                 : "v"(a[ks % kPre]), "v"(qa[ks]));
    const int nk = ks + kPre;
    if (nk < 32) a[ks % kPre] = lds_read16<f16x8>(cur, s_off[nk & 3] + 128 * (nk >> 2));
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 ar = lds_read16<bf16x8>(cur, s_off[ks] + 128 * 8);
    const bf16x8 br = lds_read16<bf16x8>(qp_row, 16 * ((2 * ks + (qp_x >> 3)) ^ (qp_x & 7)));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(ar), "v"(br));
  }
  asm volatile("s_nop 15" : "+v"(s));
  return s;
}

__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  // ---- which split / which half of the heads. Workgroups are dealt to the 8
  // XCDs round-robin by id (XCD = id % 8); XCD x takes the contiguous run of
  // work items [x n, x n + n), n = ceil(n_work / 8), so the splits of one
  // sequence share one L2 and its queries are fetched into it once. The grid
  // has at least n seats per XCD (2 n for Sq = 2); spare seats exit. With
  // Sq = 2 the two head halves of a split are ids 8 apart: same XCD,
  // dispatched together.
  const int n_work = p.meta[0];
  const int xcd = blockIdx.x & 7, seat = blockIdx.x >> 3;
  const int per_xcd = (n_work + 7) >> 3;
  int k, grp;
  if (p.q_tokens == 1) {
    if (seat >= per_xcd) return;
    k = xcd * per_xcd + seat;
    grp = 0;
  } else {
    if ((seat >> 1) >= per_xcd) return;
    k = xcd * per_xcd + (seat >> 1);
    grp = seat & 1;
  }
  if (k >= n_work) return;
  const WorkItem wi = p.work[k];
  if (wi.slot < 0 || wi.slot >= p.max_chunks || wi.t_end <= wi.t_begin) return;
  const int b = wi.b;
  const int L = p.seqinfo[b].len;

  const int t = threadIdx.x;
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

  // ---- fetch plan: wave w, fetch j moves LDS granule slots P = 256 j + 64 w +
  // lane; slot P holds logical granule (P % 72) ^ (row % 8) of row P / 72
  // (P / 72 == (P * 3641) >> 18 for P < 2304). Offsets are recomputed per use.
  int t_f = t;   // re-materialised each tile so the offsets are not hoisted
  auto slot_row = [&](int j) { return ((kThreads * j + t_f) * 3641) >> 18; };
  auto fetch_off = [&](int j) -> unsigned {
    const int P = kThreads * j + t_f, row = slot_row(j);
    return row * kRowBytes + 16 * ((P - row * kGranPerRow) ^ (row & 7));
  };
  // block ids of this split, 64 per window: lane i holds the id of block
  // blk_base + i; a tile reads its id with one lane read
  const int32_t* btab = p.block_table + (size_t)b * p.max_blocks_per_seq;
  const int blk_first = wi.t_begin / kBlock;
  const int blk_last = (wi.t_end - 1) / kBlock;
  int blk_base = blk_first;
  int blk_lane = blk_first + lane <= blk_last ? btab[blk_first + lane] : 0;
  asm volatile("" : "+v"(blk_lane));   // consume the load here: later waits stay local
  auto buf = [&](int i) -> char* { return smem + (i % kNBuf) * kTileBytes; };
  auto tile_src = [&](int ts) -> const char* {
    const int bi = ts / kBlock;
    if (bi >= blk_base + 64) {   // next window (splits longer than 4096 tokens)
      blk_base += 64;
      blk_lane = blk_base + lane <= blk_last ? btab[blk_base + lane] : 0;
      asm volatile("" : "+v"(blk_lane));
    }
    long long blk = __builtin_amdgcn_readlane(blk_lane, bi - blk_base);
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);   // memory safety
    return (const char*)p.cache + ((size_t)blk * kBlock + (ts % kBlock)) * kRowBytes;
  };
  auto fetch_one = [&](const char* src, char* dst, int j) {
    dma16(dst + 1024 * (4 * j + w), src, fetch_off(j));
  };
  // in-place bf16 -> fp16 of the c_KV granules this lane fetched; rows past the
  // split become zeros. Reads first, then conversions and writes.
  auto convert_tile = [&](char* tb, int ts) {
    const int valid = wi.t_end - ts;
    u32x4 v[kFetch];
#pragma unroll
    for (int j = 0; j < kFetch; ++j) {
      const int row = slot_row(j);
      if (kThreads * j + t_f - row * kGranPerRow < kDLat / 8)
        v[j] = *(const u32x4*)(tb + 16 * (kThreads * j + t_f));
    }
#pragma unroll
    for (int j = 0; j < kFetch; ++j) {
      const int row = slot_row(j);
      if (kThreads * j + t_f - row * kGranPerRow < kDLat / 8)
        *(u32x4*)(tb + 16 * (kThreads * j + t_f)) =
            row < valid ? bf16x8_to_f16x8(v[j]) : u32x4{0, 0, 0, 0};
    }
  };

  // ---- queries: latent part -> VGPRs (B operands: lane = row, 8 consecutive
  // k), RoPE part -> this wave's LDS slice (rows, granule ^ row % 8)
  f16x8 qa[32];
  {
    const u32x4* src = (const u32x4*)(p.q_abs + ((size_t)(r * 4 + hg) * 32) * 64 * 8);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qa[ks] = __builtin_bit_cast(f16x8, src[ks * 64 + lane]);
    // wait for them here: a wait inside the loop would also drain the fetches
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) asm volatile("" : "+v"(qa[ks]));
  }
  char* qp_lds = smem + kOffQp + w * kQpWaveBytes;
  {
    const uint16_t* src = p.q_pe + ((size_t)r * kHeads + hg * 32) * kDRope;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int G = lane + 64 * n, row = G >> 3, g = G & 7;
      *(u32x4*)(qp_lds + row * 128 + 16 * (g ^ (row & 7))) = *(const u32x4*)(src + 8 * G);
    }
  }
  const char* qp_row = qp_lds + l32 * 128;
  const int qp_x = 8 * half + (l32 & 7);   // k-half of the B fragment, row swizzle

  // ---- per-lane LDS offsets
  // scores: row = l32, logical granule 2 ks + half (+64 for k_R)
  int s_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s_off[j] = l32 * kRowBytes + 16 * ((2 * j + half) ^ (l32 & 7));
  // transposed reads of this wave's columns. MFMA k-slot (hh, e) of k-step st
  // is token 16 st + 8 (e / 4) + 4 hh + e % 4 (the score accumulator's token
  // order). Group gg = lane / 16 (k-half hh = gg / 2, 16-column half gg % 2);
  // for read q source lane L addresses token 16 st + 8 q + 4 hh + L / 4 at
  // column 128 w + 32 ct + 16 (gg % 2) + 4 (L % 4). The row swizzle (row % 8)
  // is the same for every st and q, so one base per column tile serves them
  // all (st and q add immediates).
  const int gg = lane >> 4, Lq = lane & 15, hh = gg >> 1;
  int tr_off[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int row = 4 * hh + (Lq >> 2);
    const int col = kColsPerWave * w + 32 * ct + 16 * (gg & 1) + 4 * (Lq & 3);
    tr_off[ct] = row * kRowBytes + 16 * ((col >> 3) ^ (row & 7)) + 2 * (col & 7);
  }
  // P: [row][32 positions] fp16, 64 B per row, 16-byte chunk c stored at
  // c ^ ((row / 2) % 4). Position 16 st + 8 hh + e holds the token of k-slot
  // (hh, e) of k-step st, so a B fragment is one 16-byte chunk (2 st + hh).
  auto p_chunk = [](int row, int c) { return row * 64 + 16 * (c ^ ((row >> 1) & 3)); };

  f32x16 o[4][4];   // [column tile][row tile]
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int h = 0; h < 4; ++h) o[c][h] = f32x16{};
  float m = -INFINITY, l = 0.f;   // statistics of this lane's score row
  const float scale_log2 = p.scale_log2;

  // ---- prologue: tile 0 converted, tile 1 in flight
  const int n_tiles = (wi.t_end - wi.t_begin + kTileTok - 1) / kTileTok;
  const int t0 = wi.t_begin;
  {
    const char* src = tile_src(t0);
#pragma unroll
    for (int j = 0; j < kFetch; ++j) fetch_one(src, buf(0), j);
    if (n_tiles > 1) {
      src = tile_src(t0 + kTileTok);
#pragma unroll
      for (int j = 0; j < kFetch; ++j) fetch_one(src, buf(1), j);
      MLA_WAIT_VM(9);
    } else {
      MLA_WAIT_VM(0);
    }
  }
  convert_tile(buf(0), t0);
  MLA_WAIT_LGKM0();
  MLA_BARRIER();

  for (int it = 0; it < n_tiles; ++it) {
    asm volatile("" : "+v"(t_f));
    const int ts = t0 + it * kTileTok;
    const int par = it & 1;
    const char* cur = buf(it);
    char* pbuf = smem + kOffP + par * kPBytes;

    // -- scores and softmax of this wave's rows
    f32x16 s = score_tile(cur, s_off, qa, qp_row, qp_x);
    // s[i] is token 8 (i/4) + 4 half + i%4; masking only on a split's last
    // tile or a query's last visible one
    if (ts + kTileTok > lim) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tok = ts + 8 * (i >> 2) + 4 * half + (i & 3);
        s[i] = tok < lim ? s[i] : -INFINITY;
      }
    }
    float mt = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])),
                     fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
    mt = fmaxf(mt, fmaxf(fmaxf(fmaxf(s[8], s[9]), fmaxf(s[10], s[11])),
                         fmaxf(fmaxf(s[12], s[13]), fmaxf(s[14], s[15]))));
    mt = fmaxf(mt, __shfl_xor(mt, 32)) * scale_log2;
    const bool grow = mt > m + kRescaleLog2;
    const float m_new = grow ? mt : m;
    // O rows hold earlier tiles relative to m; they scale by 2^(m - m_new)
    const bool rescale = grow && m != -INFINITY;
    const float alpha = rescale ? __builtin_amdgcn_exp2f(m - m_new) : 1.f;
    const unsigned long long any_rescale = __ballot(rescale);
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
    rs += __shfl_xor(rs, 32);
    l = l * alpha + rs;
    // P rows to LDS: registers 4 q .. 4 q + 3 are tokens 8 q + 4 half + 0..3,
    // i.e. k-step q / 2, k-half `half`, slots 4 (q % 2) .. + 3: chunk
    // 2 (q / 2) + half, 8 bytes in at 8 (q % 2)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *(f16x4*)(pbuf + p_chunk(rr, 2 * (q >> 1) + half) + 8 * (q & 1)) = pq[q];
    if (any_rescale) {
      if (half == 0) ((float*)(smem + kOffAlpha + par * kRowsPerWg * 4))[rr] = alpha;
    }
    if (lane == 0) ((int*)(smem + kOffFlag + par * kWaves * 4))[w] = any_rescale ? 1 : 0;

    // -- the next tile has landed (its fetch was issued one tile ago): convert
    if (it + 1 < n_tiles) {
      MLA_WAIT_VM(0);
      convert_tile(buf(it + 1), ts + kTileTok);
    }
    MLA_WAIT_LGKM0();
    MLA_BARRIER();

    // -- rescale O rows whose reference moved (rare)
    {
      const int4 fl = *(const int4*)(smem + kOffFlag + par * kWaves * 4);
      if (fl.x | fl.y | fl.z | fl.w) {
        const float* al = (const float*)(smem + kOffAlpha + par * kRowsPerWg * 4);
        float ah[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const int4 f4 = fl;
          const int fh = h == 0 ? f4.x : h == 1 ? f4.y : h == 2 ? f4.z : f4.w;
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
    }

    // -- latent accumulation of this wave's 128 columns, all 128 rows; the
    // fetch of the tile after next (into the buffer tile it - 1 used) is
    // issued under the MFMAs
    const bool far = it + 2 < n_tiles;
    const char* fsrc = far ? tile_src(ts + 2 * kTileTok) : nullptr;
    char* fdst = buf(it + 2);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f16x8 pb[4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        pb[h] = lds_read16<f16x8>(pbuf, p_chunk(32 * h + l32, 2 * st + half));
      f16x8 a_next = lds_read_tr(cur + tr_off[0] + 16 * kRowBytes * st,
                                 cur + tr_off[0] + 16 * kRowBytes * st + 8 * kRowBytes);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const f16x8 a = a_next;
        if (ct + 1 < 4)
          a_next = lds_read_tr(cur + tr_off[ct + 1] + 16 * kRowBytes * st,
                               cur + tr_off[ct + 1] + 16 * kRowBytes * st + 8 * kRowBytes);
#pragma unroll
        for (int h = 0; h < 4; ++h)
          o[ct][h] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[h], o[ct][h], 0, 0, 0);
        const int j = 4 * st + ct;   // 8 of the 9 fetches here, the last after the loop
        if (far) fetch_one(fsrc, fdst, j);
      }
    }
    if (far) fetch_one(fsrc, fdst, 8);
  }
  if (half == 0) ((float*)(smem + kOffStat))[rr] = l > 0.f ? 1.f / l : 0.f;
  {
    // lse = m + log2 l per score row, -inf when the row saw no position
    const size_t rows_per_chunk = (size_t)p.q_tokens * kHeads;
    const size_t row0 = (size_t)wi.slot * rows_per_chunk + qi * kHeads + hg * 32;
    if (half == 0) p.part_lse[row0 + l32] = l > 0.f ? m + __log2f(l) : -INFINITY;
  }
  MLA_WAIT_LGKM0();
  MLA_BARRIER();
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // ---- partial state: o_hat = O / l rounded to fp16, rows (qi, head) of 512
  // contiguous values; this wave writes columns [128 w, 128 w + 128) of all
  // 128 rows. The accumulator layout (lane = row, registers = columns) is
  // turned row-major through this wave's 32 KB of LDS (the tile ring is free
  // after the last barrier): 8-byte units of 4 columns, unit ^ 2 (row % 16).
  float inv_l[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) inv_l[h] = ((const float*)(smem + kOffStat))[32 * h + l32];
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
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  // a multiple of 8 work items per XCD row (see the mapping in the kernel)
  const int per = (a.max_chunks + 7) / 8 * 8;
  const int grid = a.q_tokens == 1 ? per : 2 * per;
  hipLaunchKernelGGL(attn_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
