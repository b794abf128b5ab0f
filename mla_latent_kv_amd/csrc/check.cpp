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

struct Slot {
  int64_t key;   // physical block * 64 + slot
  int32_t seq;
};

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
  std::vector<Slot> slots;
  try {
    slots.reserve((size_t)batch * (size_t)std::min(q_tokens, max_seq_len));
  } catch (const std::bad_alloc&) {
    return MLA_ERR_INVALID_ARG;
  }
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t len = seq_lens[b];
    // 0 <= L_b <= max_seq_len; this also keeps every table read below inside
    // row b, since max_seq_len <= 64 * max_blocks_per_seq
    if (len < 0 || len > max_seq_len) {
      bad = std::min(bad, b);
      continue;
    }
    const int32_t* row = block_table + (int64_t)b * max_blocks_per_seq;
    const int32_t used = (len + kBlockTokens - 1) / kBlockTokens;
    bool ok = true;
    for (int32_t k = 0; k < used; ++k)
      if (row[k] < 0 || (int64_t)row[k] >= num_blocks) {
        ok = false;
        break;
      }
    if (!ok) {
      bad = std::min(bad, b);
      continue;
    }
    // the slots of the new tokens, positions max(0, L_b - Sq) .. L_b - 1
    for (int32_t j = std::max(0, len - q_tokens); j < len; ++j)
      slots.push_back(Slot{(int64_t)row[j / kBlockTokens] * kBlockTokens + j % kBlockTokens, b});
  }
  // two new tokens stored in one slot: every sequence of such a group but
  // the lowest-numbered one violates the layout (the older prefix blocks may
  // be shared; a new token's row may not)
  std::sort(slots.begin(), slots.end(), [](const Slot& x, const Slot& y) {
    return x.key != y.key ? x.key < y.key : x.seq < y.seq;
  });
  for (size_t i = 1; i < slots.size(); ++i)
    if (slots[i].key == slots[i - 1].key && slots[i].seq != slots[i - 1].seq)
      bad = std::min(bad, slots[i].seq);
  if (bad == batch) return MLA_OK;
  if (first_bad) *first_bad = bad;
  return MLA_ERR_PRECONDITION;
}
