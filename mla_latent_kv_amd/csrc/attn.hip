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
constexpr float kRescaleLog2 = 8.0f;                      // lazy max threshold

// s_waitcnt immediates (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; an all-ones field means "do not wait on this counter".
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

  // ---- fetch plan: wave w, fetch j moves LDS granule slots 256 j + 64 w + lane;
  // slot P holds logical granule (P % 72) ^ swz(row) of row P / 72.
  int plan[kFetch];   // byte offset in the global tile | row << 16 | is_c_kv << 23
#pragma unroll
  for (int j = 0; j < kFetch; ++j) {
    const int P = kThreads * j + t;
    const int row = P / kGranPerRow;
    const int g = (P % kGranPerRow) ^ swz(row);
    plan[j] = (row * kRowBytes + 16 * g) | (row << 16) | ((g < kDLat / 8) ? (1 << 23) : 0);
  }
  const int32_t* btab = p.block_table + (size_t)b * p.max_blocks_per_seq;
  auto issue_tile = [&](int ts, char* buf) {
    long long blk = btab[ts / kBlock];
    blk = blk < 0 ? 0 : (blk >= p.num_blocks ? p.num_blocks - 1 : blk);   // memory safety
    const char* src = (const char*)p.cache + ((size_t)blk * kBlock + (ts % kBlock)) * kRowBytes;
#pragma unroll
    for (int j = 0; j < kFetch; ++j)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src + (plan[j] & 0xffff)),
          (__attribute__((address_space(3))) void*)(buf + 1024 * (4 * j + w)), 16, 0, 0);
  };
  auto convert_tile = [&](char* buf, int ts) {
    const int valid = wi.t_end - ts;   // rows of this tile inside the split
#pragma unroll
    for (int j = 0; j < kFetch; ++j) {
      if (plan[j] & (1 << 23)) {
        u32x4* a = (u32x4*)(buf + 16 * (kThreads * j + t));
        const int row = (plan[j] >> 16) & 31;
        u32x4 v = *a;
        *a = row < valid ? bf16x8_to_f16x8(v) : u32x4{0, 0, 0, 0};
      }
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

  // ---- per-lane LDS read offsets
  // scores: row = l32, logical granule 2 ks + half (+64 for k_R)
  int s_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s_off[j] = l32 * kRowBytes + 16 * ((2 * j + half) ^ swz(l32));
  // transposed reads: group gg = lane / 16 (k-half hh = gg / 2, 16-col half
  // gg % 2), source lane L: token 16 st + 8 q + 4 hh + L / 4, column
  // 32 ct + 16 (gg % 2) + 4 (L % 4). Offsets for ct = 0 and ct = 1; ct + 2
  // adds one 128-byte block of 8 granules.
  const int gg = lane >> 4, Lq = lane & 15, hh = gg >> 1;
  int tr_off[2][2][2];   // [st][q][ct parity]
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = 16 * st + 8 * q + 4 * hh + (Lq >> 2);
#pragma unroll
      for (int cp = 0; cp < 2; ++cp) {
        const int col = 32 * cp + 16 * (gg & 1) + 4 * (Lq & 3);
        tr_off[st][q][cp] = row * kRowBytes + 16 * ((col >> 3) ^ swz(row)) + 2 * (col & 7);
      }
    }
  const int qp_off = l32 * 128;

  f32x16 o[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) o[c] = f32x16{};
  float m = -INFINITY, l = 0.f;

  // ---- prologue: tiles 0 and 1 in flight, tile 0 converted
  const int n_tiles = (wi.t_end - wi.t_begin + kTileTok - 1) / kTileTok;
  issue_tile(wi.t_begin, smem);
  if (n_tiles > 1) {
    issue_tile(wi.t_begin + kTileTok, smem + kTileBytes);
    MLA_WAIT_VM(9);
  } else {
    MLA_WAIT_VM(0);
  }
  convert_tile(smem, wi.t_begin);
  MLA_WAIT_LGKM0();
  MLA_BARRIER();

  int cur_i = 0;   // ring index of tile `it`
  for (int it = 0; it < n_tiles; ++it) {
    const int ts = wi.t_begin + it * kTileTok;
    const int nxt_i = cur_i == kNBuf - 1 ? 0 : cur_i + 1;
    const int far_i = nxt_i == kNBuf - 1 ? 0 : nxt_i + 1;
    const bool far = it + 2 < n_tiles;
    // tile it + 2 -> the buffer tile it - 1 used (every wave is past it)
    if (far) issue_tile(ts + 2 * kTileTok, smem + far_i * kTileBytes);
    const char* cur = smem + cur_i * kTileBytes;

    // -- scores: 36 MFMAs; the A fragments are read from LDS kSPre steps ahead
    // (sched_barrier keeps that order so LDS latency hides behind the MFMAs)
    f32x16 s = {};
    {
      constexpr int kSPre = 4;
      f16x8 a[kSPre];
#pragma unroll
      for (int j = 0; j < kSPre; ++j) a[j] = lds_read16<f16x8>(cur, s_off[j & 3] + 128 * (j >> 2));
#pragma unroll
      for (int ks = 0; ks < 32; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[ks % kSPre], qa[ks], s, 0, 0, 0);
        const int nk = ks + kSPre;
        if (nk < 32) a[ks % kSPre] = lds_read16<f16x8>(cur, s_off[nk & 3] + 128 * (nk >> 2));
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8 ar[4], br[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ar[ks] = lds_read16<bf16x8>(cur, s_off[ks] + 128 * 8);
        br[ks] = lds_read16<bf16x8>(qp_lds, qp_off + 16 * ((2 * ks + half) ^ (l32 & 7)));
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ar[ks], br[ks], s, 0, 0, 0);
    }

    // -- online softmax in log2 units: m is the running reference (scaled),
    // p = 2^(s * scale * log2 e - m). s[i] is token 8 (i/4) + 4 half + i%4.
    // Masking is needed only on a split's last tile or a query's last visible one.
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
    mt = fmaxf(mt, __shfl_xor(mt, 32)) * p.scale_log2;
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
    const float neg_m = (m == -INFINITY) ? 0.f : -m;
    float rs = 0.f;
    f16x8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], p.scale_log2, neg_m));
      rs += e;
      pb[i >> 3][i & 7] = (_Float16)e;
    }
    rs += __shfl_xor(rs, 32);
    l += rs;

    // -- latent accumulation: o[ct] += C^T[32 ct .., tokens] * P^T, 32 MFMAs;
    // transposed A fragments are read two MFMAs ahead
    {
      auto tr = [&](int idx) {
        const int ct = idx >> 1, st = idx & 1;
        const int blk = 128 * (ct >> 1);
        return lds_read_tr(cur + tr_off[st][0][ct & 1] + blk, cur + tr_off[st][1][ct & 1] + blk);
      };
      constexpr int kPPre = 3;
      f16x8 a[kPPre];
#pragma unroll
      for (int j = 0; j < kPPre; ++j) a[j] = tr(j);
#pragma unroll
      for (int idx = 0; idx < 32; ++idx) {
        o[idx >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[idx % kPPre], pb[idx & 1], o[idx >> 1], 0, 0, 0);
        if (idx + kPPre < 32) a[idx % kPPre] = tr(idx + kPPre);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // -- tile it + 1 has landed (only tile it + 2's fetches may be pending):
    // convert this lane's part of it, then one barrier publishes it and frees
    // tile it's buffer for the fetch two tiles ahead.
    if (it + 1 < n_tiles) {
      if (far) {
        MLA_WAIT_VM(9);
      } else {
        MLA_WAIT_VM(0);
      }
      convert_tile(smem + nxt_i * kTileBytes, ts + kTileTok);
    }
    MLA_WAIT_LGKM0();
    MLA_BARRIER();
    cur_i = nxt_i;
  }

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
