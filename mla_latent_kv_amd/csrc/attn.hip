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
// * workgroup = 4 wavefronts = 128 query rows; wavefront = 32 rows (heads) of
//   one new token. All 4 wavefronts share each cache tile in LDS, so every
//   cached byte crosses HBM once per split (Sq = 2 runs two workgroups per
//   split, one per 64-head half, on the same XCD so the second read hits L2).
// * scores: D[token, head] = C_tile[token, :] . Q[head, :] -- the cache tile is
//   the A operand (lane = token, 8 consecutive latent values per k-step, one
//   16-byte LDS read), the wavefront's queries are the B operand and stay in
//   VGPRs for the whole split (32 fp16 k-steps of the latent part, 4 bf16
//   k-steps of the RoPE part).
// * softmax: each lane owns one head (lane % 32) and 16 of the tile's 32
//   tokens, so row max and row sum are 16 in-lane steps plus one exchange with
//   lane ^ 32. The running max is moved only when it grows by more than 2^8
//   (in log2 units); otherwise the stale max is kept, which is exact because
//   the final normalisation uses the same reference for O and l.
// * latent accumulation: D[latent col, head] += C_tile^T[col, token] P^T[token,
//   head] -- the probabilities stay in the score accumulator's registers (its
//   token order defines the k order) and become the B operand; the cache tile
//   is read transposed with ds_read_b64_tr_b16 as the A operand. O lives in
//   16 accumulator tiles (256 registers per lane).
// * cache tiles: 32 tokens x 1152 B = 36 KB, contiguous inside one 64-token
//   block, in a ring of three LDS buffers. Tiles are fetched two ahead with
//   direct-to-LDS loads (global_load_lds_dwordx4: no VGPRs in flight); once a
//   tile has landed, each lane converts the c_KV granules it fetched from bf16
//   to fp16 in place (exact in fp16's range) and zeroes rows past the split, so
//   NaN padding never reaches the latent MFMAs (masked scores are replaced by
//   -inf with a select). A granule swizzle g ^ f(row) keeps the score reads,
//   the transposed reads and the conversion pass free of bank conflicts; the
//   fetch addresses apply the inverse permutation.
// * per tile, one barrier: scores (36 MFMAs); row max and the first half of
//   the exponentials; then the P.C product in two 16-token halves, the second
//   half's exponentials and the conversion of the next tile running on the
//   VALU/LDS under the first half's MFMAs. The score chain accumulates in VGPRs
//   (issued as inline MFMAs, the result-to-VALU distance covered by s_nop) so
//   that O owns all 256 accumulator registers.
#include "common.h"

namespace mla {

namespace {

constexpr int kGranPerRow = kRowBytes / 16;               // 72
constexpr int kTileBytes = kTileTok * kRowBytes;          // 36864
constexpr int kThreads = kWaves * 64;                     // 256
constexpr int kFetch = kTileBytes / 16 / kThreads;        // 9 granules per lane per tile
constexpr int kNBuf = 3;                                  // LDS tile ring
constexpr int kQpWaveBytes = kRowsPerWave * kDRope * 2;   // 4 KB of q_pe per wavefront
constexpr int kRingBytes = kNBuf * kTileBytes + kWaves * kQpWaveBytes;
constexpr int kEpiBytes = kWaves * kRowsPerWave * kDLat * 2;   // fp16 transpose space
constexpr int kLdsBytes = kRingBytes > kEpiBytes ? kRingBytes : kEpiBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget of one gfx950 workgroup");
constexpr float kRescaleLog2 = 15.0f;                     // lazy max threshold (p < 2^15 in fp16)

#define MLA_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")
#define MLA_WAIT_LGKM0() asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory")
#define MLA_BARRIER() asm volatile("s_barrier" ::: "memory")

// Swizzle of the 16-byte granule index within a row: a permutation of 0..7
// applied to the low three bits. Rows r..r+7 (r % 8 == 0) map one logical
// granule to eight distinct bank groups; rows r..r+3 (r % 4 == 0) map the
// granule pair {2m, 2m+1} to eight distinct bank groups.
__device__ __forceinline__ int swz(int row) { return 2 * (row & 3) + ((row >> 2) & 1); }

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

template <typename T>
__device__ __forceinline__ T lds_read16(const char* base, int off) {
  return __builtin_bit_cast(T, *(const u32x4*)(base + off));
}

__device__ __forceinline__ f16x8 lds_read_tr(const char* p0, const char* p1) {
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p0);
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p1);
  return __builtin_bit_cast(f16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Scores of one tile: D[token, head] over 32 fp16 k-steps (latent) and 4 bf16
// k-steps (RoPE). Accumulates in VGPRs: dependent MFMAs on one accumulator
// issue back to back; s_nop 15 covers the MFMA-result -> VALU-read distance.
// fetch(j), j = 0..8, is called after every fourth MFMA so that the next
// tile's direct-to-LDS loads issue under the matrix work instead of in a burst.
template <typename Fetch>
__device__ __forceinline__ f32x16 score_tile(const char* cur, const int (&s_off)[4],
                                             const f16x8 (&qa)[32], const char* qp_row,
                                             int qp_x, Fetch&& fetch) {
  constexpr int kPre = 4;
  f16x8 a[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) a[j] = lds_read16<f16x8>(cur, s_off[j & 3] + 128 * (j >> 2));
  f32x16 s;
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=v"(s) : "v"(a[0]), "v"(qa[0]));
  fetch(0);
  a[0] = lds_read16<f16x8>(cur, s_off[0] + 128);
#pragma unroll
  for (int ks = 1; ks < 32; ++ks) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0"
                 : "+v"(s)
                 : "v"(a[ks % kPre]), "v"(qa[ks]));
    if (ks % 4 == 0) fetch(ks / 4);
    const int nk = ks + kPre;
    if (nk < 32) a[ks % kPre] = lds_read16<f16x8>(cur, s_off[nk & 3] + 128 * (nk >> 2));
  }
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const bf16x8 ar = lds_read16<bf16x8>(cur, s_off[ks] + 128 * 8);
    const bf16x8 br = lds_read16<bf16x8>(qp_row, 16 * ((2 * ks + (qp_x >> 3)) ^ (qp_x & 7)));
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(ar), "v"(br));
    if (ks == 0) fetch(8);
  }
  asm volatile("s_nop 15" : "+v"(s));
  return s;
}

__global__ __launch_bounds__(kThreads, 1) void attn_kernel(AttnArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[kLdsBytes];

  // ---- which split / which half of the heads
  int k, grp;
  if (p.q_tokens == 1) {
    k = blockIdx.x;
    grp = 0;
  } else {
    // pairs (k, 0), (k, 1) land 8 ids apart: same XCD, dispatched together
    k = 8 * (blockIdx.x >> 4) + (blockIdx.x & 7);
    grp = (blockIdx.x >> 3) & 1;
  }
  const int n_work = p.meta[0];
  if (k >= n_work) return;
  const WorkItem wi = p.work[k];
  if (wi.slot < 0 || wi.slot >= p.max_chunks || wi.t_end <= wi.t_begin) return;
  const int b = wi.b;
  const int L = p.seqinfo[b].len;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int qi = (p.q_tokens == 1) ? 0 : (w >> 1);          // new-token index of this wave
  const int hg = (p.q_tokens == 1) ? w : 2 * grp + (w & 1);  // 32-head group
  const int r = b * p.q_tokens + qi;                          // query row
  const int n_vis = L - p.q_tokens + qi + 1;                  // visible positions
  const int lim = min(wi.t_end, n_vis);                       // tokens this wave may use

  // ---- fetch plan: wave w, fetch j moves LDS granule slots P = 256 j + 64 w +
  // lane; slot P holds logical granule (P % 72) ^ swz(row) of row P / 72
  // (P / 72 == (P * 3641) >> 18 for P < 2304). Offsets are recomputed per use
  // rather than held in registers.
  int t_f = t;   // re-materialised each tile (see the loop) so offsets are not hoisted
  auto slot_row = [&](int j) { return ((kThreads * j + t_f) * 3641) >> 18; };
  auto fetch_off = [&](int j) {
    const int P = kThreads * j + t_f, row = slot_row(j);
    return row * kRowBytes + 16 * ((P - row * kGranPerRow) ^ swz(row));
  };
  // block ids of this split, 64 per window: lane i holds the id of block
  // blk_base + i; a tile reads its id with one lane read
  const int32_t* btab = p.block_table + (size_t)b * p.max_blocks_per_seq;
  const int blk_first = wi.t_begin / kBlock;
  const int blk_last = (wi.t_end - 1) / kBlock;
  int blk_base = blk_first;
  int blk_lane = blk_first + lane <= blk_last ? btab[blk_first + lane] : 0;
  // consume the load here, so no later wait on it can also drain the fetches
  asm volatile("" : "+v"(blk_lane));
  auto buf = [&](int i) -> char* { return smem + (i % kNBuf) * kTileBytes; };
  // global address of the first row of the tile starting at token ts
  auto tile_src = [&](int ts) -> const char* {
    const int bi = ts / kBlock;
    if (bi >= blk_base + 64) {   // next window (chunks longer than 4096 tokens)
      blk_base += 64;
      blk_lane = blk_base + lane <= blk_last ? btab[blk_base + lane] : 0;
      asm volatile("" : "+v"(blk_lane));
    }
    long long blk = __builtin_amdgcn_readlane(blk_lane, bi - blk_base);
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);   // memory safety
    return (const char*)p.cache + ((size_t)blk * kBlock + (ts % kBlock)) * kRowBytes;
  };
  // fetch j (of 9) of a tile into LDS buffer dst
  auto fetch_one = [&](const char* src, char* dst, int j) {
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(src + (unsigned)fetch_off(j)),
        (__attribute__((address_space(3))) void*)(dst + 1024 * (4 * j + w)), 16, 0, 0);
  };
  auto issue_tile = [&](int ts, char* dst) {
    const char* src = tile_src(ts);
#pragma unroll
    for (int j = 0; j < kFetch; ++j) fetch_one(src, dst, j);
  };
  // in-place bf16 -> fp16 of the c_KV granules this lane fetched; rows past the
  // split become zeros (k_R granules are rewritten unchanged). Reads first,
  // then conversions, then writes, so the LDS latency is paid once.
  auto convert_tile = [&](char* tb, int ts) {
    const int valid = wi.t_end - ts;
    u32x4 v[kFetch];
#pragma unroll
    for (int j = 0; j < kFetch; ++j) {
      const int row = slot_row(j);
      if (kThreads * j + t - row * kGranPerRow < kDLat / 8)
        v[j] = *(const u32x4*)(tb + 16 * (kThreads * j + t));
    }
#pragma unroll
    for (int j = 0; j < kFetch; ++j) {
      const int row = slot_row(j);
      if (kThreads * j + t - row * kGranPerRow < kDLat / 8)
        *(u32x4*)(tb + 16 * (kThreads * j + t)) =
            row < valid ? bf16x8_to_f16x8(v[j]) : u32x4{0, 0, 0, 0};
    }
  };

  // ---- queries: latent part -> VGPRs (B operands: lane = head, 8 consecutive
  // k), RoPE part -> this wave's LDS slice (rows = heads, granule ^ row % 8)
  f16x8 qa[32];
  {
    const u32x4* src = (const u32x4*)(p.q_abs + ((size_t)(r * 4 + hg) * 32) * 64 * 8);
#pragma unroll
    for (int ks = 0; ks < 32; ++ks) qa[ks] = __builtin_bit_cast(f16x8, src[ks * 64 + lane]);
  }
  char* qp_lds = smem + kNBuf * kTileBytes + w * kQpWaveBytes;
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

  // ---- per-lane LDS read offsets
  // scores: row = l32, logical granule 2 ks + half (+64 for k_R)
  int s_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s_off[j] = l32 * kRowBytes + 16 * ((2 * j + half) ^ swz(l32));
  // transposed reads: group gg = lane / 16 (k-half hh = gg / 2, 16-col half
  // gg % 2), source lane L: token 16 st + 8 q + 4 hh + L / 4, column
  // 32 ct + 16 (gg % 2) + 4 (L % 4). swz(row) is the same for every (st, q),
  // so two bases (ct parity) serve all reads; st, q and ct / 2 are immediates.
  const int gg = lane >> 4, Lq = lane & 15, hh = gg >> 1;
  int tr_off[2];
#pragma unroll
  for (int cp = 0; cp < 2; ++cp) {
    const int row = 4 * hh + (Lq >> 2);
    const int col = 32 * cp + 16 * (gg & 1) + 4 * (Lq & 3);
    tr_off[cp] = row * kRowBytes + 16 * ((col >> 3) ^ swz(row)) + 2 * (col & 7);
  }

  f32x16 o[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) o[c] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const float scale_log2 = p.scale_log2;
  // Row max of the tile starting at token ts (raw scores s, masked in place)
  // and the running reference m: moved (with O and l rescaled) only when the
  // tile max exceeds it by more than 2^kRescaleLog2, so p stays below 2^15.
  auto tile_max = [&](f32x16& s, int ts) {
    // s[i] is token 8 (i/4) + 4 half + i%4 of the tile; masking only on a
    // split's last tile or a query's last visible one
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
    if (__any(grow)) {
      const float m_new = grow ? mt : m;
      if (__any(grow && m != -INFINITY)) {
        // O *= 2^(m - m_new) in place in the accumulator registers (one read /
        // multiply / write per element, so O never leaves the AGPRs); the
        // s_nops cover the MFMA -> accumulator-read and write -> MFMA distances.
        const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - m_new);
        l *= alpha;
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int c = 0; c < 16; ++c)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float x = o[c][i], tmp;
            asm volatile(
                "v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                : "+a"(x), "=&v"(tmp)
                : "v"(alpha));
            o[c][i] = x;
          }
        asm volatile("s_nop 7" ::: "memory");
      }
      m = m_new;
    }
  };
  // p = 2^(s * scale * log2 e - m) for tokens 16 h16 .. 16 h16 + 15 of the tile
  // (registers 8 h16 .. 8 h16 + 7), packed as the B fragment of that half;
  // returns their sum over the lane's 8 values
  auto tile_exp = [&](const f32x16& s, int h16, f16x8& pbh) -> float {
    const float neg_m = (m == -INFINITY) ? 0.f : -m;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h16 + i], scale_log2, neg_m));
      rs += e;
      pbh[i] = (_Float16)e;
    }
    return rs;
  };
  // o[ct] += C^T[32 ct .., 16 tokens of half st] * P^T for the tile in `tb`:
  // 16 MFMAs, the transposed A fragments read three MFMAs ahead
  auto accumulate_half = [&](const char* tb, int st, const f16x8& pbh) {
    auto tr = [&](int ct) {
      const char* base = tb + tr_off[ct & 1] + 128 * (ct >> 1) + 16 * kRowBytes * st;
      return lds_read_tr(base, base + 8 * kRowBytes);
    };
    constexpr int kPPre = 3;
    f16x8 a[kPPre];
#pragma unroll
    for (int j = 0; j < kPPre; ++j) a[j] = tr(j);
#pragma unroll
    for (int ct = 0; ct < 16; ++ct) {
      o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ct % kPPre], pbh, o[ct], 0, 0, 0);
      if (ct + kPPre < 16) a[ct % kPPre] = tr(ct + kPPre);
    }
  };

  // ---- prologue: tile 0 converted, tile 1 in flight
  const int n_tiles = (wi.t_end - wi.t_begin + kTileTok - 1) / kTileTok;
  const int t0 = wi.t_begin;
  issue_tile(t0, buf(0));
  if (n_tiles > 1) {
    issue_tile(t0 + kTileTok, buf(1));
    MLA_WAIT_VM(9);
  } else {
    MLA_WAIT_VM(0);
  }
  convert_tile(buf(0), t0);
  MLA_WAIT_LGKM0();
  MLA_BARRIER();

  // ---- tile `it`: fetch tile it + 2 into the buffer tile it - 1 used, scores,
  // softmax and accumulation of tile it, conversion of tile it + 1
  for (int it = 0; it < n_tiles; ++it) {
    asm volatile("" : "+v"(t_f));
    const int ts = t0 + it * kTileTok;
    const bool far = it + 2 < n_tiles, next = it + 1 < n_tiles;
    const char* fsrc = far ? tile_src(ts + 2 * kTileTok) : nullptr;
    char* fdst = buf(it + 2);
    f32x16 s = score_tile(buf(it), s_off, qa, qp_row, qp_x, [&](int j) {
      if (far) fetch_one(fsrc, fdst, j);
    });
    tile_max(s, ts);
    f16x8 pb0, pb1;
    float rs = tile_exp(s, 0, pb0);
    if (next) {
      if (far) {
        MLA_WAIT_VM(9);
      } else {
        MLA_WAIT_VM(0);
      }
    }
    accumulate_half(buf(it), 0, pb0);
    rs += tile_exp(s, 1, pb1);
    if (next) convert_tile(buf(it + 1), ts + kTileTok);
    rs += __shfl_xor(rs, 32);
    l += rs;
    accumulate_half(buf(it), 1, pb1);
    MLA_WAIT_LGKM0();
    MLA_BARRIER();
  }
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // ---- partial state: o_hat = O / l rounded to fp16 (the merge only needs
  // the normalised partial and lse = m + log2 l), rows (qi, head) of 512
  // contiguous values. The accumulator layout (lane = head, registers =
  // columns) is turned head-major through this wave's 32 KB of LDS (the tile
  // ring is free after the last barrier): 8-byte column units, unit index
  // XOR 2 (head % 16) so rows of equal bank phase spread over the banks.
  const float inv_l = l > 0.f ? 1.f / l : 0.f;
  const float lse = l > 0.f ? m + __log2f(l) : -INFINITY;
  char* tw = smem + w * (kRowsPerWave * kDLat * 2);
  const int xr = 2 * (l32 & 15);
#pragma unroll
  for (int ct = 0; ct < 16; ++ct)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int u = 8 * ct + 2 * q + half;   // 4-column unit of columns 32 ct + 8 q + 4 half
      f16x4 v = {(_Float16)(o[ct][4 * q] * inv_l), (_Float16)(o[ct][4 * q + 1] * inv_l),
                 (_Float16)(o[ct][4 * q + 2] * inv_l), (_Float16)(o[ct][4 * q + 3] * inv_l)};
      *(f16x4*)(tw + l32 * (kDLat * 2) + 8 * (u ^ xr)) = v;
    }
  const size_t rows_per_chunk = (size_t)p.q_tokens * kHeads;
  const size_t row0 = (size_t)wi.slot * rows_per_chunk + qi * kHeads + hg * 32;
  if (half == 0) p.part_lse[row0 + l32] = lse;
  MLA_WAIT_LGKM0();   // this wave's own LDS writes only: no barrier needed
  _Float16* dst = p.part_o + row0 * kDLat;
#pragma unroll 8
  for (int j = 0; j < kRowsPerWave; ++j) {
    const int xj = 2 * (j & 15);
    const u32x4 v = *(const u32x4*)(tw + j * (kDLat * 2) + 8 * ((2 * lane) ^ xj));
    *(u32x4*)(dst + (size_t)j * kDLat + 8 * lane) = v;
  }
}

}  // namespace

hipError_t launch_attn(const AttnArgs& a, hipStream_t stream) {
  int grid;
  if (a.q_tokens == 1) {
    grid = a.max_chunks;
  } else {
    grid = 2 * ((a.max_chunks + 7) / 8) * 8;
  }
  hipLaunchKernelGGL(attn_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
