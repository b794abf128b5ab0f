// Randomised run of mla_decode_check_inputs for the sanitizer test: every
// case gets heap arrays of exactly the documented sizes (seq_lens [batch],
// block_table [batch * max_blocks_per_seq]), so a read past either is an
// AddressSanitizer error, and every status is compared with a direct
// restatement of the documented conditions (quadratic, no sorting).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "../../include/mla_decode.h"

namespace {

int expected(const int32_t* lens, const int32_t* table, int batch, int sq, int mbps, int max_len,
             int64_t nblk, int* bad) {
  *bad = -1;
  if (batch < 1 || sq < 1 || mbps < 1 || max_len < 1 || nblk < 1 || (int64_t)max_len > 64LL * mbps)
    return MLA_ERR_INVALID_ARG;
  std::vector<char> ok(batch, 1);
  for (int b = 0; b < batch; ++b) {
    if (lens[b] < 0 || lens[b] > max_len) {
      ok[b] = 0;
      continue;
    }
    for (int k = 0; k < (lens[b] + 63) / 64; ++k)
      if (table[(int64_t)b * mbps + k] < 0 || table[(int64_t)b * mbps + k] >= nblk) ok[b] = 0;
  }
  // the blocks of one sequence are distinct
  for (int b = 0; b < batch; ++b) {
    if (!ok[b]) continue;
    const int used = (lens[b] + 63) / 64;
    for (int k = 0; k < used; ++k)
      for (int k2 = k + 1; k2 < used; ++k2)
        if (table[(int64_t)b * mbps + k] == table[(int64_t)b * mbps + k2]) ok[b] = 0;
  }
  std::vector<char> clash(batch, 0);
  auto slot = [&](int b, int j) { return (int64_t)table[(int64_t)b * mbps + j / 64] * 64 + j % 64; };
  // a new-token slot already used by a lower-numbered sequence whose lengths
  // and block ids are in range (its own block repeats do not exempt it)
  auto in_range = [&](int a) {
    if (lens[a] < 0 || lens[a] > max_len) return false;
    for (int k = 0; k < (lens[a] + 63) / 64; ++k)
      if (table[(int64_t)a * mbps + k] < 0 || table[(int64_t)a * mbps + k] >= nblk) return false;
    return true;
  };
  for (int b = 0; b < batch; ++b) {
    if (!in_range(b)) continue;
    for (int a = 0; a < b && !clash[b]; ++a) {
      if (!in_range(a)) continue;
      for (int j = lens[b] - sq > 0 ? lens[b] - sq : 0; j < lens[b]; ++j)
        for (int i = lens[a] - sq > 0 ? lens[a] - sq : 0; i < lens[a]; ++i)
          if (slot(b, j) == slot(a, i)) clash[b] = 1;
    }
  }
  for (int b = 0; b < batch; ++b)
    if (!ok[b] || clash[b]) {
      *bad = b;
      return MLA_ERR_PRECONDITION;
    }
  return MLA_OK;
}

}  // namespace

int main(int argc, char** argv) {
  const int n_cases = argc > 1 ? atoi(argv[1]) : 20000;
  std::mt19937_64 rng(12345);
  auto uni = [&](int64_t lo, int64_t hi) { return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1)); };
  int32_t bad = 0;
  // argument errors never read the arrays (NULL arrays included)
  if (mla_decode_check_inputs(nullptr, nullptr, 4, 1, 2, 64, 10, &bad) != MLA_ERR_INVALID_ARG || bad != -1)
    return fprintf(stderr, "null arrays\n"), 1;
  int32_t one_len = 5, one_id = 0;
  if (mla_decode_check_inputs(&one_len, &one_id, 1, 1, 1, 65, 1, nullptr) != MLA_ERR_INVALID_ARG)
    return fprintf(stderr, "max_seq_len past the table\n"), 1;
  if (mla_decode_check_inputs(&one_len, &one_id, 1, 1, 1, 64, 1, nullptr) != MLA_OK)
    return fprintf(stderr, "one valid sequence\n"), 1;
  int counts[3] = {0, 0, 0};
  for (int c = 0; c < n_cases; ++c) {
    const int batch = (int)uni(1, 24), sq = (int)uni(1, 3), mbps = (int)uni(1, 6);
    const int max_len = (int)uni(1, 64 * mbps + (uni(0, 9) == 0 ? 40 : 0));
    const int64_t nblk = uni(1, 3 * batch * mbps);
    int32_t* lens = new int32_t[batch];
    int32_t* table = new int32_t[(size_t)batch * mbps];
    const int mode = (int)uni(0, 3);   // 0: mostly valid, distinct blocks; 1..3: noisier
    std::vector<int32_t> perm(nblk);
    for (int64_t i = 0; i < nblk; ++i) perm[i] = (int32_t)i;
    std::shuffle(perm.begin(), perm.end(), rng);
    for (int b = 0; b < batch; ++b) {
      lens[b] = (int32_t)(mode == 0 ? uni(0, max_len) : uni(-3, max_len + 70));
      for (int k = 0; k < mbps; ++k) {
        const int64_t i = (int64_t)b * mbps + k;
        table[i] = mode == 0 || uni(0, 7) ? perm[i % nblk] : (int32_t)uni(-2, nblk + 2);
      }
    }
    const int32_t* cl = lens;
    const int32_t* ct = table;
    int want_bad = 0;
    const int want = expected(cl, ct, batch, sq, mbps, max_len, nblk, &want_bad);
    const int got = mla_decode_check_inputs(cl, ct, batch, sq, mbps, max_len, nblk, &bad);
    if (got != want || bad != want_bad) {
      fprintf(stderr, "case %d: status %d (want %d), first_bad %d (want %d)\n", c, got, want, bad, want_bad);
      return 1;
    }
    counts[want == MLA_OK ? 0 : (want == MLA_ERR_PRECONDITION ? 1 : 2)]++;
    delete[] lens;
    delete[] table;
  }
  printf("cases ok: %d valid, %d precondition, %d invalid-arg\n", counts[0], counts[1], counts[2]);
  return 0;
}
