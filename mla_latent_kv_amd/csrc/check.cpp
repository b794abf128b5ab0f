// Host-side check of the decode inputs' preconditions (declared in
// include/mla_decode.h as mla_decode_check_inputs). Plain C++ with no HIP
// dependency: the library exports it for callers, its debug build runs it on
// host copies before every launch, and the CPU tests build it on its own under
// AddressSanitizer and UndefinedBehaviorSanitizer.
//
// The conditions restate the paged-cache layout of the "DeepSeek-V3" page at
// ailearn.mscapital.top (MLA section: one 512 + 64 wide row per cached token,
// here stored in 64-token blocks that a per-sequence table maps to physical
// blocks) and the decode step's counting: L_b counts every cached token of
// sequence b, its new ones included.
#include <stdint.h>

#include <algorithm>
#include <new>
#include <vector>

#include "../../include/mla_decode.h"

namespace {

constexpr int32_t kBlockTokens = 64;
constexpr int32_t kMaxBatchRows = 1000000;

struct Use {
  int64_t key;   // a physical block, or a physical block * 64 + slot
  int32_t seq;
};

bool by_key_then_seq(const Use& x, const Use& y) { return x.key != y.key ? x.key < y.key : x.seq < y.seq; }

}  // namespace

extern "C" int mla_decode_check_inputs(const int32_t* seq_lens, const int32_t* block_table,
                                       int32_t batch, int32_t q_tokens, int32_t max_blocks_per_seq,
                                       int32_t max_seq_len, int64_t num_blocks, int32_t* first_bad) {
  if (first_bad) *first_bad = -1;
  if (!seq_lens || !block_table || batch < 1 || batch > kMaxBatchRows || q_tokens < 1 ||
      max_blocks_per_seq < 1 || max_seq_len < 1 || num_blocks < 1 ||
      (int64_t)max_seq_len > (int64_t)kBlockTokens * max_blocks_per_seq)
    return MLA_ERR_INVALID_ARG;

  int32_t bad = batch;   // lowest violating sequence so far (batch = none)
  // pass 1: lengths and block ranges; count what pass 2 collects
  std::vector<char> ok((size_t)batch, 1);
  size_t n_blocks = 0, n_slots = 0;
  try {
    for (int32_t b = 0; b < batch; ++b) {
      const int32_t len = seq_lens[b];
      // 0 <= L_b <= max_seq_len; this also keeps every table read below inside
      // row b, since max_seq_len <= 64 * max_blocks_per_seq
      if (len < 0 || len > max_seq_len) {
        ok[b] = 0;
        bad = std::min(bad, b);
        continue;
      }
      const int32_t* row = block_table + (int64_t)b * max_blocks_per_seq;
      const int32_t used = (len + kBlockTokens - 1) / kBlockTokens;
      for (int32_t k = 0; k < used && ok[b]; ++k)
        if (row[k] < 0 || (int64_t)row[k] >= num_blocks) ok[b] = 0;
      if (!ok[b]) {
        bad = std::min(bad, b);
        continue;
      }
      n_blocks += (size_t)used;
      n_slots += (size_t)std::min(len, q_tokens);
    }
    // pass 2: the blocks each sequence uses, and its new tokens' slots
    // (positions max(0, L_b - Sq) .. L_b - 1)
    std::vector<Use> blocks, slots;
    blocks.reserve(n_blocks);
    slots.reserve(n_slots);
    for (int32_t b = 0; b < batch; ++b) {
      if (!ok[b]) continue;
      const int32_t len = seq_lens[b];
      const int32_t* row = block_table + (int64_t)b * max_blocks_per_seq;
      for (int32_t k = 0; k < (len + kBlockTokens - 1) / kBlockTokens; ++k) blocks.push_back(Use{row[k], b});
      for (int32_t j = std::max(0, len - q_tokens); j < len; ++j)
        slots.push_back(Use{(int64_t)row[j / kBlockTokens] * kBlockTokens + j % kBlockTokens, b});
    }
    // a sequence maps two of its own blocks to one physical block: its
    // history would repeat rows (blocks of different sequences may coincide,
    // as a shared prefix would)
    std::sort(blocks.begin(), blocks.end(), by_key_then_seq);
    for (size_t i = 1; i < blocks.size(); ++i)
      if (blocks[i].key == blocks[i - 1].key && blocks[i].seq == blocks[i - 1].seq)
        bad = std::min(bad, blocks[i].seq);
    // two sequences' new tokens stored in one slot: every sequence of such a
    // group but the lowest-numbered one breaks the layout
    std::sort(slots.begin(), slots.end(), by_key_then_seq);
    for (size_t i = 1; i < slots.size(); ++i)
      if (slots[i].key == slots[i - 1].key && slots[i].seq != slots[i - 1].seq)
        bad = std::min(bad, slots[i].seq);
  } catch (const std::bad_alloc&) {
    return MLA_ERR_INVALID_ARG;   // the host cannot hold the check's lists
  }
  if (bad == batch) return MLA_OK;
  if (first_bad) *first_bad = bad;
  return MLA_ERR_PRECONDITION;
}
