// Naive-path attention: the per-head keys and values are materialised from the
// latent cache,
//   K_h[j] = [W_UK[h] c_j ; k_R,j]  (192 wide),   V_h[j] = W_UV[h] c_j  (128),
// and a standard causal softmax attention runs over them, out[b,i,h] =
// softmax(scale * q_h K_h^T) V_h with row i seeing positions
// j <= L_b - Sq + i. This is the branch the "DeepSeek-V3" page
// (ailearn.mscapital.top, MLA paragraphs) contrasts with the absorb order: it
// expands every cached token to 128 x (192 + 128) = 40,960 elements instead
// of keeping 576 ("DeepSeek-V3" article at m.lsln.cn, section 2.1: the
// attention softmax(Q K^T) V over the cached keys and values). With every
// prompt token as a query (Sq = L, prefill) the work is quadratic in L and
// bound by the matrix cores.
//
// Two launches:
//  1. expand_kernel, workgroup = one head x a range of 64-token tiles of one
//     sequence, 4 wavefronts of 64 output columns: each holds its columns of
//     W_UK[h] (2 wavefronts) or W_UV[h] (2) in registers, loaded once from
//     the packed layout (wstream.h), while the tiles' c_KV rows stream
//     through a 2-deep LDS ring:
//       K_nope^T[n][token] = W_UK[h] C^T  (MFMA: A = W_UK rows, B = C rows)
//       V[token][v]        = C W_UV[h]^T  (MFMA: A = C rows, B = W_UV rows)
//     In both the accumulator of a lane already holds one fragment of the
//     attention pass (lane = token for K, lane = v for V^T), so each result
//     is rounded (K_nope to bf16, V to fp16) and stored straight from the
//     registers as whole 1 KB fragments. The head-shared k_R is copied once
//     per tile (by the head-0 workgroups). Tokens at or past L are written as
//     zeros.
//  2. attend_kernel, workgroup = 256 queries of one sequence x one head (64
//     per wavefront): per 64-key tile, one barrier, the next tile's 40 KB
//     fetched straight into LDS while this one is used; S^T = K Q^T on bf16
//     MFMA (lane = query, so every query's softmax state stays in its lane
//     pair), online softmax in fp32, P rounded to fp16 and O^T += V^T P^T on
//     fp16 MFMA. Causal masking only in the tiles that cross the diagonal.
//
// Expanded buffer, per sequence b and 64-token tile j (kTileBytes):
//   [k_R: 8 fragments][head 0: K 16 fragments | V^T 16 fragments][head 1 ...]
// Fragment = 1 KB, lane piece l (16 bytes) at 16 l:
//   K   (kt, s), kt < 2, s < 8:  bf16 K_nope[32 kt + l%32][16 s + n(e)], e < 8,
//        n(e) = 4 (l/32) + e for e < 4 and 8 + 4 (l/32) + e - 4 after: a
//        permutation of the step's 16 dims (the query fragments take the
//        same one; a dot product does not depend on the order of its terms)
//   k_R (kt, s), kt < 2, s < 4:  bf16 k_R[32 kt + l%32][16 s + 8 (l/32) .. + 7]
//   V^T (vt, g), vt < 4, g < 4:  fp16 V[t][32 vt + l%32] for the 8 tokens
//        t = 16 g + 4 (l/32) + {0,1,2,3} and 16 g + 8 + 4 (l/32) + {0,1,2,3}
// (the token order of V^T matches the accumulator layout of S^T, so the
// probabilities feed the P V product without a shuffle).
#include "common.h"

namespace mla {

namespace {

constexpr int kFrag = 1024;
constexpr int kRFrags = 8, kKFrags = 16, kVFrags = 16;
constexpr size_t kHeadTileBytes = (size_t)(kKFrags + kVFrags) * kFrag;            // 32 KB
constexpr size_t kRTileBytes = (size_t)kRFrags * kFrag;                            // 8 KB
constexpr size_t kTileBytes = kRTileBytes + (size_t)kHeads * kHeadTileBytes;       // per (b, 64 tokens)
constexpr int kQPerWg = 256;                      // queries per attention workgroup
constexpr int kPackedTiles = kHeads * kDNope / 32;   // 512 column tiles of the packed W_UK / W_UV

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

// One direct-to-LDS fetch: 64 lanes x 16 bytes from base + voff (per lane) to
// LDS bytes [lds, lds + 1024). Inline asm so that the compiler does not drain
// it before every LDS read; the kernels order it with explicit waits and
// barriers. No VGPR result.
__device__ __forceinline__ void dma16(const char* lds, const char* base, unsigned voff) {
  const unsigned m0 = (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char*)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(m0), "v"(voff), "s"(base)
               : "m0");
}

// Max and sum of x over the lane pair (l, l ^ 32): v_permlane32_swap with
// both operands x hands each lane its own and its partner's value (the second
// copy passes an empty asm so the optimizer sees two values). Each element is
// converted to a scalar before its bit cast (a bit cast applied directly to a
// vector element reads element 0 with this compiler).
struct PairF {
  float a, b;
};
__device__ __forceinline__ PairF with_partner(float x) {
  float y = x;
  asm volatile("" : "+v"(y));
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                  false, false);
  const unsigned r0 = r[0], r1 = r[1];
  return PairF{__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1)};
}
__device__ __forceinline__ float pair_max(float x) {
  const PairF p = with_partner(x);
  return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float pair_sum(float x) {
  const PairF p = with_partner(x);
  return p.a + p.b;
}

__device__ __forceinline__ unsigned short bf16_rne(float x) {
  unsigned int u = __builtin_bit_cast(unsigned int, x);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// ---------------------------------------------------------------- expansion

struct ExpandArgs {
  const uint16_t* cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const u32x4* w_uk;   // packed W_UK, [16384][512]
  const u32x4* w_uv;   // packed W_UV, [16384][512]
  char* exp;
  long long num_blocks;
  int max_blocks_per_seq;
  int t64;             // 64-token tiles per sequence in the expanded buffer
  int max_len;
};

constexpr int kXThreads = 256;                   // 4 wavefronts: 64 output columns each
constexpr int kCRow = kDLat * 2;                 // 1024 bytes of c_KV per token in LDS
constexpr int kCTile = kBlock * kCRow;           // 64 KB: the c_KV of one 64-token tile
constexpr int kLatSteps = kDLat / 16;            // 32 k-steps over the latent

__device__ __forceinline__ long long clamp_block(const ExpandArgs& a, int b, int j) {
  const long long blk = a.block_table[(size_t)b * a.max_blocks_per_seq + j];
  return blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);   // memory safety
}

// One 64-token tile of one head for a wavefront: 32 k-steps x 2 token tiles
// x 2 column tiles. kV: D[token][v] = C rows x W_UV rows -- lane = v, the
// accumulator runs over tokens, which is the V^T fragment order. Else
// D[n][token] = W_UK rows x C rows -- lane = token, the accumulator runs over
// n, which is the K fragment order with the n order of each 16-wide k-step
// permuted (see K_nope above). The weight fragments wf stay in registers for
// the whole workgroup; C fragments come from LDS (row r's piece p at
// p ^ (r % 64)), each used for both column tiles.
template <bool kV>
__device__ __forceinline__ void expand_tile(const char* buf, const u32x4 (&wf)[kLatSteps][2],
                                            f32x16 (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, n = lane & 31, half = lane >> 5;
  auto cfrag = [&](int ks, int tt) {
    const int r = 32 * tt + n;
    return *(const u32x4*)(buf + r * kCRow + 16 * ((2 * ks + half) ^ (r & 63)));
  };
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) acc[tt][0] = acc[tt][1] = f32x16{};
  // the C fragments of k-step ks + 1 are read while step ks multiplies; the
  // scheduling barriers keep the reads from all being hoisted to the top
  u32x4 cur[2] = {cfrag(0, 0), cfrag(0, 1)};
#pragma unroll
  for (int ks = 0; ks < kLatSteps; ++ks) {
    u32x4 nxt[2];
    if (ks + 1 < kLatSteps) {
      nxt[0] = cfrag(ks + 1, 0);
      nxt[1] = cfrag(ks + 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 cf = __builtin_bit_cast(bf16x8, cur[tt]);
        const bf16x8 wv = __builtin_bit_cast(bf16x8, wf[ks][c]);
        acc[tt][c] = kV ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(cf, wv, acc[tt][c], 0, 0, 0)
                        : __builtin_amdgcn_mfma_f32_32x32x16_bf16(wv, cf, acc[tt][c], 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
    if (ks + 1 < kLatSteps) {
      cur[0] = nxt[0];
      cur[1] = nxt[1];
    }
  }
}

// grid (token splits, 128 heads, B). Workgroup (s, h, b) covers the 64-token
// tiles [j0, j1) of sequence b for head h: wavefront w loads its 64 columns
// of W_UK[h] (w < 2) or W_UV[h] (w >= 2) once (64 fragments, 256 registers),
// then the tiles' c_KV rows stream through a 2-deep LDS ring (direct-to-LDS
// fetches, the next tile in flight while this one multiplies) and every
// wavefront writes its 8 fragments of the tile straight from its
// accumulators.
__global__ __launch_bounds__(kXThreads, 1) void expand_kernel(ExpandArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kCTile];   // 128 KB
  const int b = blockIdx.z, h = blockIdx.y;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int T = (L + kBlock - 1) / kBlock;
  const int j0 = (int)((long long)T * blockIdx.x / gridDim.x), j1 = (int)((long long)T * (blockIdx.x + 1) / gridDim.x);
  if (j0 >= j1) return;
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n = lane & 31, half = lane >> 5;
  const bool is_v = w >= 2;
  const int c0 = 2 * (w & 1);        // first of the wavefront's two column tiles within the head
  const u32x4* wp = (is_v ? a.w_uv : a.w_uk) + (size_t)(4 * h + c0) * 64 + lane;
  u32x4 wf[kLatSteps][2];
#pragma unroll
  for (int ks = 0; ks < kLatSteps; ++ks)
#pragma unroll
    for (int c = 0; c < 2; ++c) wf[ks][c] = wp[(size_t)ks * kPackedTiles * 64 + 64 * c];

  auto fetch = [&](int j, char* buf) {   // rows 16 w .. 16 w + 15 of tile j
    const char* blk = (const char*)(a.cache + (size_t)clamp_block(a, b, j) * kBlock * kRow);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * w + i;
      dma16(buf + r * kCRow, blk + (size_t)r * kRow * 2, (unsigned)(16 * (lane ^ (r & 63))));
    }
  };
  fetch(j0, smem);
  for (int j = j0; j < j1; ++j) {
    const char* buf = smem + ((j - j0) & 1) * kCTile;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // own share of tile j (and the weights) in
    __syncthreads();                                   // everyone's; the other buffer is free
    if (j + 1 < j1) fetch(j + 1, smem + ((j + 1 - j0) & 1) * kCTile);
    f32x16 acc[2][2];
    if (is_v)
      expand_tile<true>(buf, wf, acc);
    else
      expand_tile<false>(buf, wf, acc);

    char* tile = a.exp + ((size_t)b * a.t64 + j) * kTileBytes;
    char* head = tile + kRTileBytes + (size_t)h * kHeadTileBytes;
    const int tok0 = kBlock * j;
    if (!is_v) {
      // K fragment (kt = tt, s = 2 (c0 + c) + s2): lane (token n, half) takes
      // acc[tt][c][8 s2 + e] = K_nope[token][16 s + {4 half + e, 8 + 4 half + e - 4}]
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bool live = tok0 + 32 * tt + n < L;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[e] = live ? ((unsigned)bf16_rne(acc[tt][c][8 * s2 + 2 * e]) |
                             ((unsigned)bf16_rne(acc[tt][c][8 * s2 + 2 * e + 1]) << 16))
                          : 0u;
            *(u32x4*)(head + (8 * tt + 2 * (c0 + c) + s2) * kFrag + 16 * lane) = v;
          }
      }
    } else {
      // V^T fragment (vt = c0 + c, g): lane (v n, half) takes acc[g / 2][c][8 (g % 2) + e]
      // = V[16 g + {4 half + e, 8 + 4 half + e - 4}][v]
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f16x8_t o;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tok = tok0 + 16 * g + (e < 4 ? 4 * half + e : 8 + 4 * half + (e - 4));
            o[e] = tok < L ? (_Float16)acc[g >> 1][c][8 * (g & 1) + e] : (_Float16)0.f;
          }
          *(f16x8_t*)(head + (kKFrags + 4 * (c0 + c) + g) * kFrag + 16 * lane) = o;
        }
    }
    if (h == 0) {   // k_R fragments (kt, s) of the tile from the cache rows: 2 per wavefront
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int rf = 2 * w + f, kt = rf >> 2, s = rf & 3;
        const int tok = tok0 + 32 * kt + n;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (tok < L)
          v = *(const u32x4*)((const char*)(a.cache + ((size_t)clamp_block(a, b, j) * kBlock + tok % kBlock) * kRow) +
                              2 * (kDLat + 16 * s + 8 * half));
        *(u32x4*)(tile + rf * kFrag + 16 * lane) = v;
      }
    }
  }
}

// ---------------------------------------------------------------- attention

struct AttendArgs {
  const uint16_t* q_nope;
  const uint16_t* q_pe;
  const char* exp;
  const int32_t* seq_lens;
  float* out;
  int q_tokens;
  int t64;
  int max_len;
  float scale_log2;   // softmax scale * log2(e)
};

constexpr int kTileLds = (kRFrags + kKFrags + kVFrags) * kFrag;   // 40 KB per key tile
constexpr int kAQT = 1;                                 // 32-query tiles per wavefront
constexpr int kAWaves = kQPerWg / (32 * kAQT);         // 8 wavefronts, two per SIMD
static_assert((kRFrags + kKFrags + kVFrags) % kAWaves == 0, "whole fetch shares");

// Rescaling of the running output is deferred until a row's maximum grows by
// more than 2^kLazy (in log2 units): until then the probabilities are formed
// against the older maximum and stay below 2^kLazy, well inside fp16.
constexpr float kLazy = 8.f;

// One 64-key tile for the wavefront's 64 queries (2 query tiles of 32):
// S^T = K Q^T (bf16 MFMA, 12 k-steps of 16 dims: 8 of K_nope, 4 of k_R), the
// online softmax (per lane = query; its 64 keys split over the lane pair),
// then O^T += V^T P^T (fp16 MFMA, 4 groups of 16 keys). kMasked: the tile
// crosses some row's last visible key.
template <bool kMasked, int kQT>
__device__ __forceinline__ void attend_tile(const char* buf, const u32x4 (&qf)[kQT][12], const int (&vis)[kQT],
                                            int nt, float scale_log2, float (&m)[kQT], float (&l)[kQT],
                                            f32x16 (&oacc)[4][kQT]) {
  const int lane = threadIdx.x & 63, half = lane >> 5;
  // The key fragments of k-step s + 1 are read while step s multiplies; the
  // scheduling barriers keep the compiler from hoisting every LDS read of the
  // tile to its top (which would leave no room for the query fragments).
  auto kfrag = [&](int s, int kt) {
    const int f = s < 8 ? kRFrags + 8 * kt + s : 4 * kt + (s - 8);
    return *(const u32x4*)(buf + f * kFrag + 16 * lane);
  };
  f32x16 sacc[2][kQT];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) sacc[kt][qt] = f32x16{};
  u32x4 kcur[2] = {kfrag(0, 0), kfrag(0, 1)};
#pragma unroll
  for (int s = 0; s < 12; ++s) {
    u32x4 knext[2];
    if (s + 1 < 12) {
      knext[0] = kfrag(s + 1, 0);
      knext[1] = kfrag(s + 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt)
        sacc[kt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kcur[kt]),
                                                               __builtin_bit_cast(bf16x8, qf[qt][s]), sacc[kt][qt],
                                                               0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < 12) {
      kcur[0] = knext[0];
      kcur[1] = knext[1];
    }
  }
  f16x8_t pf[kQT][4];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    if constexpr (kMasked) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kBlock * nt + 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key > vis[qt]) sacc[kt][qt][r] = -INFINITY;
        }
    }
    float tmax = -INFINITY;   // of the raw scores (the scale is positive)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[kt][qt][r]);
    tmax = pair_max(tmax) * scale_log2;
    // wave-uniform decision: some row's maximum grew by more than 2^kLazy
    if (__builtin_amdgcn_ballot_w64(tmax > m[qt] + kLazy) != 0) {
      const float m_new = fmaxf(m[qt], tmax);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[qt] - m_new);
      m[qt] = m_new;
      l[qt] *= alpha;
      // O *= alpha in place in the accumulator registers (read / multiply /
      // write per element, so O never leaves the AGPRs and the compiler keeps
      // no VGPR copy of it); the s_nops cover the MFMA -> accumulator-read and
      // write -> MFMA distances.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int vt = 0; vt < 4; ++vt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = oacc[vt][qt][i], tmp;
          asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                       : "+a"(x), "=&v"(tmp)
                       : "v"(alpha));
          oacc[vt][qt][i] = x;
        }
      asm volatile("s_nop 7" ::: "memory");
    }
    const float neg_m = m[qt] == -INFINITY ? 0.f : -m[qt];   // a row that sees nothing yet: p = 0
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][qt][r], scale_log2, neg_m));
        psum += p;
        pf[qt][2 * kt + (r >> 3)][r & 7] = (_Float16)p;
      }
    l[qt] += psum;
  }
  // O^T += V^T P^T; the value fragments of group g + 1 are read while group
  // g multiplies
  auto vfrag = [&](int g, int vt) { return *(const u32x4*)(buf + (kRFrags + kKFrags + 4 * vt + g) * kFrag + 16 * lane); };
  u32x4 vcur[4];
#pragma unroll
  for (int vt = 0; vt < 4; ++vt) vcur[vt] = vfrag(0, vt);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    u32x4 vnext[4];
    if (g + 1 < 4) {
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) vnext[vt] = vfrag(g + 1, vt);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int vt = 0; vt < 4; ++vt)
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt)
        oacc[vt][qt] =
            __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, vcur[vt]), pf[qt][g], oacc[vt][qt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (g + 1 < 4) {
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) vcur[vt] = vnext[vt];
    }
  }
}

// grid (ceil(Sq / 256) * 128, 1, B). Workgroup id i runs on XCD i % 8 (the
// dispatcher's round robin); the mapping below gives each XCD whole heads, all
// query tiles of a head in consecutive slots, so the head's key and value
// tiles are re-read from that XCD's L2. Within a head the query tiles run
// last-first (the causal tail has the most key tiles). Results do not depend
// on where a workgroup runs.
__global__ __launch_bounds__(kAWaves * 64, 1) void attend_kernel(AttendArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kTileLds];
  const int nq = gridDim.x / kHeads;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int b = blockIdx.z, h = xcd + 8 * (slot / nq);
  const int qtile = nq - 1 - slot % nq;
  const int Sq = a.q_tokens;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n = lane & 31, half = lane >> 5;
  const int i0 = kQPerWg * qtile;
  // the workgroup's last visible key, and the key tiles it needs
  const int vis_max = L - Sq + min(i0 + kQPerWg - 1, Sq - 1);
  const int n_tiles = vis_max < 0 ? 0 : vis_max / kBlock + 1;
  const int mask_from = L - Sq + i0 < 0 ? 0 : (L - Sq + i0 + 1) / kBlock;   // first tile that needs masking

  // queries of this lane: rows i = i0 + 32 kAQT w + 32 qt + n
  int qi[kAQT], vis[kAQT];
  u32x4 qf[kAQT][12];
#pragma unroll
  for (int qt = 0; qt < kAQT; ++qt) {
    qi[qt] = i0 + 32 * kAQT * w + 32 * qt + n;
    vis[qt] = L - Sq + qi[qt];
    const bool ok = qi[qt] < Sq;
    const size_t row = ((size_t)b * Sq + (ok ? qi[qt] : 0)) * kHeads + h;
#pragma unroll
    for (int s = 0; s < 12; ++s) {
      u32x4 v;
      if (s < 8) {   // the K_nope steps' permuted n order: 16 s + {4 half + 0..3, 8 + 4 half + 0..3}
        const u32x2 lo = *(const u32x2*)(a.q_nope + row * kDNope + 16 * s + 4 * half);
        const u32x2 hi = *(const u32x2*)(a.q_nope + row * kDNope + 16 * s + 8 + 4 * half);
        v = u32x4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        v = *(const u32x4*)(a.q_pe + row * kDRope + 16 * (s - 8) + 8 * half);
      }
      qf[qt][s] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const size_t seq_base = (size_t)b * a.t64 * kTileBytes;
  constexpr int kFetch = (kRFrags + kKFrags + kVFrags) / kAWaves;   // fragments per wavefront
  auto fetch = [&](int nt, char* buf) {
#pragma unroll
    for (int k = 0; k < kFetch; ++k) {
      const int f = kFetch * w + k;
      const char* src = a.exp + seq_base + (size_t)nt * kTileBytes +
                        (f < kRFrags ? (size_t)f * kFrag
                                     : kRTileBytes + (size_t)h * kHeadTileBytes + (size_t)(f - kRFrags) * kFrag);
      dma16(buf + f * kFrag, src, (unsigned)(16 * lane));
    }
  };

  f32x16 oacc[4][kAQT];
  float m[kAQT], l[kAQT];
#pragma unroll
  for (int qt = 0; qt < kAQT; ++qt) {
#pragma unroll
    for (int vt = 0; vt < 4; ++vt) oacc[vt][qt] = f32x16{};
    m[qt] = -INFINITY;
    l[qt] = 0.f;
  }

  // per tile: this tile's fragments are in (own share: vmcnt; everyone's: the
  // barrier, after which the other buffer is free too), then the next tile's
  // fetch goes out while this one is used
  auto next = [&](int nt) -> const char* {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (nt + 1 < n_tiles) fetch(nt + 1, smem + ((nt + 1) & 1) * kTileLds);
    return smem + (nt & 1) * kTileLds;
  };
  if (n_tiles > 0) fetch(0, smem);
  const int n_plain = min(mask_from, n_tiles);   // tiles every row sees whole
  int nt = 0;
  for (; nt < n_plain; ++nt) attend_tile<false, kAQT>(next(nt), qf, vis, nt, a.scale_log2, m, l, oacc);
  for (; nt < n_tiles; ++nt) attend_tile<true, kAQT>(next(nt), qf, vis, nt, a.scale_log2, m, l, oacc);

  // out[b, i, h, v] = O / l; a row that sees no position yields zeros
#pragma unroll
  for (int qt = 0; qt < kAQT; ++qt) {
    const float lt = pair_sum(l[qt]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qi[qt] >= Sq) continue;
    float* o = a.out + (((size_t)b * Sq + qi[qt]) * kHeads + h) * kDV;
#pragma unroll
    for (int vt = 0; vt < 4; ++vt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v = {oacc[vt][qt][4 * g4] * inv, oacc[vt][qt][4 * g4 + 1] * inv, oacc[vt][qt][4 * g4 + 2] * inv,
                         oacc[vt][qt][4 * g4 + 3] * inv};
        *(f32x4*)(o + 32 * vt + 8 * g4 + 4 * half) = v;
      }
  }
}

}  // namespace

size_t naive_workspace_bytes(int batch, int max_len) {
  return (size_t)batch * ((max_len + kBlock - 1) / kBlock) * kTileBytes;
}

hipError_t launch_naive(const uint16_t* q_nope, const uint16_t* q_pe, const uint16_t* w_uk, const uint16_t* w_uv,
                        const uint16_t* cache, const int32_t* block_table, const int32_t* seq_lens, float* out,
                        long long num_blocks, int batch, int q_tokens, int max_blocks_per_seq, int max_len,
                        float scale, void* ws, hipStream_t stream) {
  const int t64 = (max_len + kBlock - 1) / kBlock;
  const ExpandArgs ea{cache, block_table, seq_lens, (const u32x4*)w_uk, (const u32x4*)w_uv, (char*)ws,
                      num_blocks, max_blocks_per_seq, t64, max_len};
  // enough workgroups for the chip: one per head and sequence, two per head
  // for a single sequence
  const int splits = batch == 1 ? 2 : 1;
  hipLaunchKernelGGL(expand_kernel, dim3(splits, kHeads, batch), dim3(kXThreads), 0, stream, ea);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const AttendArgs aa{q_nope, q_pe, (const char*)ws, seq_lens, out, q_tokens, t64, max_len,
                      scale * 1.4426950408889634f};
  static_assert(kHeads % 8 == 0, "whole heads per XCD");
  hipLaunchKernelGGL(attend_kernel, dim3((q_tokens + kQPerWg - 1) / kQPerWg * kHeads, 1, batch),
                     dim3(kAWaves * 64), 0, stream, aa);
  return hipGetLastError();
}

}  // namespace mla
