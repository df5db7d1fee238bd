// Launch sequence of the bf16 matrix-core backward for gfx950: the dQ kernel
// (bwd_dq.hip), which also writes the row statistics, then the dK/dV kernel
// (bwd_dkdv.h; head_dim 64 from bwd_dkdv64.hip, 256 from bwd_dkdv256.hip);
// or, when no segment has more than 128 keys (head_dim 64 / 128), the
// short-document kernel alone (bwd_short.hip).
//
// Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences", Proof section (forward/backward parity, input gradients).
#include "bwd_dkdv.h"

namespace bd {

bool bwd_mfma_fits(int64_t q_len, int64_t h_q, int64_t head_dim) {
  // a (batch row, head)'s Q / dO rows, including the last tile's rows past
  // the chunk, must be addressable with 31-bit buffer offsets
  return dkdv_rows_fit(q_len, h_q, head_dim);
}

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t st) {
  if (a.head_dim != 64 && a.head_dim != 128 && a.head_dim != 256) return hipErrorInvalidValue;
  // Packings of short documents: one kernel over the metadata's bins.
  if (bwd_short_applies(a)) return launch_bwd_short(a, st);
  // The dQ kernel runs first: it also writes the row statistics.
  const hipError_t e = launch_bwd_dq(a, st);
  if (e != hipSuccess) return e;
  switch (a.head_dim) {
    case 64: return launch_bwd_dkdv64(a, st);
    case 128: return a.drop.thr != 0 ? launch_dkdv_t<128, true>(a, st) : launch_dkdv_t<128, false>(a, st);
    default: return launch_bwd_dkdv256(a, st);
  }
}

}  // namespace bd
