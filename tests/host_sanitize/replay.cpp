// Replays segmenter and validator cases through the host-only part of the
// library (segment.cpp), for a build under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The validator exists to turn malformed
// metadata into an error instead of a crash or an out-of-bounds access
// (Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences", key property 4), so every case -- good or malformed -- must run
// clean under both sanitizers.
//
// Input (stdin), one case per line:
//   S batch seq_len row_offset q_len capacity n_docs[batch] doc_lens[...]
//   V n batch seq_len row_offset q_len cu_q[n+1] cu_k[n+1] k_begin[n]
// Output (stdout), one line per case: the status, then for S with status 0
// n_seg max_q max_k cu_q cu_k k_begin; for S with capacity status the
// reported need.
#include <cstdio>
#include <vector>

#include "blockdiag.h"

static bool read_ints(int n, std::vector<int32_t>& out) {
  out.resize(n > 0 ? n : 0);
  for (int i = 0; i < n; ++i)
    if (scanf("%d", &out[i]) != 1) return false;
  return true;
}

int main() {
  char kind[4];
  while (scanf("%3s", kind) == 1) {
    if (kind[0] == 'S') {
      int batch, seq_len, r0, q_len, cap;
      if (scanf("%d %d %d %d %d", &batch, &seq_len, &r0, &q_len, &cap) != 5) return 2;
      std::vector<int32_t> per, lens;
      if (!read_ints(batch, per)) return 2;
      long total = 0;
      for (int b = 0; b < batch; ++b) total += per[b] > 0 ? per[b] : 0;
      if (!read_ints(static_cast<int>(total), lens)) return 2;
      // exact-size output arrays, so an overrun is caught
      std::vector<int32_t> cu_q(cap + 1), cu_k(cap + 1), kb(cap > 0 ? cap : 1);
      int32_t n = -1, mq = -1, mk = -1;
      const bd_status st = blockdiag_segment(lens.empty() ? nullptr : lens.data(), per.empty() ? nullptr : per.data(),
                                             batch, seq_len, r0, q_len, cap, cu_q.data(), cu_k.data(), kb.data(),
                                             &n, &mq, &mk);
      printf("%d", static_cast<int>(st));
      if (st == BD_OK) {
        printf(" %d %d %d", n, mq, mk);
        for (int i = 0; i <= n; ++i) printf(" %d", cu_q[i]);
        for (int i = 0; i <= n; ++i) printf(" %d", cu_k[i]);
        for (int i = 0; i < n; ++i) printf(" %d", kb[i]);
      } else if (st == BD_ERR_CAPACITY) {
        printf(" %d", n);
      }
      printf("\n");
    } else if (kind[0] == 'V') {
      int n, batch, seq_len, r0, q_len;
      if (scanf("%d %d %d %d %d", &n, &batch, &seq_len, &r0, &q_len) != 5) return 2;
      std::vector<int32_t> cu_q, cu_k, kb;
      if (!read_ints(n + 1, cu_q) || !read_ints(n + 1, cu_k) || !read_ints(n, kb)) return 2;
      const bd_status st = blockdiag_validate(cu_q.data(), cu_k.data(), kb.empty() ? nullptr : kb.data(), n,
                                              batch, seq_len, r0, q_len);
      printf("%d\n", static_cast<int>(st));
    } else {
      return 2;
    }
  }
  return 0;
}
