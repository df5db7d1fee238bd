// Host-only, integer-only planner of the needed-only K/V exchange of
// context-parallel block-diagonal attention (no HIP dependency).
//
// Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences":
//   - Summary: besides the fused [K;V] all-gather, needed-only exchanges --
//     a point-to-point halo from the left neighbour, or an all-to-all-v when
//     a document spans more than two ranks -- cut a rank's K/V from the whole
//     row to its own chunk plus the straddling prefix;
//   - Design overview, batch.py: the row is padded to a multiple of cp and
//     every rank holds a contiguous slice; exchange.py: left-halo p2p and the
//     needed-only all-to-all-v;
//   - Proof: the CPU tests check the halo / all-to-all-v plan geometry.
// Rank r holds rows [r0, r1) = [r * S / cp, (r + 1) * S / cp).  A row i
// attends keys [doc_start(i), i], so the chunk's rows of batch row b attend
// exactly the keys [doc_start(r0), min(r1, end of documents)) -- contiguous,
// since documents are contiguous -- of which the part left of r0 is owned by
// lower ranks (the halo).
#include <vector>

#include "blockdiag.h"
#include "internal.h"

using bd::fail;

namespace {

// Keys of batch row b needed by rank r: [*lo, *hi) (empty: lo == hi).
void row_need(const int32_t* lens, int32_t n_docs, int64_t r0, int64_t r1, int64_t* lo, int64_t* hi) {
  *lo = r0;
  int64_t pos = 0;
  for (int32_t d = 0; d < n_docs; ++d) {
    const int64_t e = pos + lens[d];
    if (lens[d] > 0 && r0 >= pos && r0 < e) {  // the document holding the chunk's first row
      *lo = pos;
      break;
    }
    pos = e;
  }
  int64_t total = 0;
  for (int32_t d = 0; d < n_docs; ++d) total += lens[d];
  if (r0 >= total) {  // the chunk is padding in this row: it attends nothing
    *lo = *hi = r0;
    return;
  }
  *hi = r1 < total ? r1 : total;
}

}  // namespace

extern "C" bd_status blockdiag_kv_plan(const int32_t* doc_lens, const int32_t* docs_per_row, int32_t batch,
                                       int32_t seq_len, int32_t cp, int32_t rank, int32_t align,
                                       int32_t* kv_begin, int32_t* kv_end, int32_t capacity, bd_kv_range* recv,
                                       int32_t* n_recv, bd_kv_range* send, int32_t* n_send, int32_t* rank_mode,
                                       int32_t* step_mode) {
  bd::clear_error();
  if (batch < 0 || seq_len < 0 || capacity < 0) return fail(BD_ERR_INVALID_ARG, "negative size");
  if (cp <= 0 || rank < 0 || rank >= cp) return fail(BD_ERR_INVALID_ARG, "rank %d of cp %d", rank, cp);
  if (seq_len % cp != 0) return fail(BD_ERR_INVALID_ARG, "seq_len %d is not a multiple of cp %d", seq_len, cp);
  if (align <= 0) return fail(BD_ERR_INVALID_ARG, "align must be positive");
  if (!kv_begin || !kv_end || !n_recv || !n_send || !rank_mode || !step_mode || (batch > 0 && !docs_per_row))
    return fail(BD_ERR_INVALID_ARG, "null pointer");
  // Document lengths: as for blockdiag_segment.
  std::vector<int64_t> first(batch + 1, 0);
  for (int32_t b = 0; b < batch; ++b) {
    if (docs_per_row[b] < 0) return fail(BD_ERR_INVALID_ARG, "docs_per_row[%d] < 0", b);
    if (docs_per_row[b] > 0 && doc_lens == nullptr) return fail(BD_ERR_INVALID_ARG, "null doc_lens");
    first[b + 1] = first[b] + docs_per_row[b];
    int64_t total = 0;
    for (int64_t d = first[b]; d < first[b + 1]; ++d) {
      if (doc_lens[d] < 0) return fail(BD_ERR_BAD_METADATA, "row %d has a negative document length", b);
      total += doc_lens[d];
    }
    if (total > seq_len) return fail(BD_ERR_BAD_METADATA, "row %d: document lengths sum past seq_len %d", b, seq_len);
  }
  const int64_t C = seq_len / cp;
  auto need = [&](int32_t b, int32_t r, int64_t* lo, int64_t* hi) {
    row_need(doc_lens + first[b], docs_per_row[b], r * C, (r + 1) * C, lo, hi);
  };
  // Mode of rank r: 0 no halo, 1 every halo key from rank r - 1, 2 some from
  // a rank further left (a document spans more than two ranks).
  auto mode_of = [&](int32_t r) {
    int m = 0;
    for (int32_t b = 0; b < batch; ++b) {
      int64_t lo, hi;
      need(b, r, &lo, &hi);
      if (lo < r * C) m = lo < (r - 1) * C ? 2 : (m > 1 ? m : 1);
    }
    return m;
  };
  const int64_t r0 = rank * C, r1 = r0 + C;
  int64_t wlo = r0;
  int32_t nr = 0, ns = 0;
  bool over = false;
  auto put = [&](bd_kv_range* arr, int32_t* cnt, int32_t row, int32_t peer, int64_t a, int64_t e) {
    if (*cnt < capacity && arr != nullptr) arr[*cnt] = bd_kv_range{row, peer, static_cast<int32_t>(a), static_cast<int32_t>(e)};
    else over = true;
    ++*cnt;
  };
  for (int32_t b = 0; b < batch; ++b) {
    int64_t lo, hi;
    need(b, rank, &lo, &hi);
    if (lo < wlo) wlo = lo;
    // receive: the halo [lo, r0), split by owning rank, lowest rank first
    for (int64_t q = lo / C; lo < r0 && q < rank; ++q) {
      const int64_t a = lo > q * C ? lo : q * C, e = (q + 1) * C;
      put(recv, &nr, b, static_cast<int32_t>(q), a, e);
    }
    // send: the part of each higher rank's halo inside this chunk
    for (int32_t q = rank + 1; q < cp; ++q) {
      int64_t qlo, qhi;
      need(b, q, &qlo, &qhi);
      if (qlo < r1) put(send, &ns, b, q, qlo > r0 ? qlo : r0, r1);
    }
  }
  *n_recv = nr;
  *n_send = ns;
  if (over) return fail(BD_ERR_CAPACITY, "plan needs %d receive and %d send ranges, capacity %d", nr, ns, capacity);
  *kv_begin = static_cast<int32_t>((wlo / align) * align);
  *kv_end = static_cast<int32_t>(r1);
  *rank_mode = mode_of(rank);
  int sm = 0;
  for (int32_t r = 0; r < cp; ++r) {
    const int m = mode_of(r);
    sm = m > sm ? m : sm;
  }
  *step_mode = sm;
  return BD_OK;
}
