// head_dim 64 instantiation of the bf16 matrix-core dK/dV kernel (bwd_dkdv.h).
// It is a translation unit of its own because it is built with the
// backend's max-ILP instruction scheduler, which at head_dim 64 (183 -> 229
// registers, still two waves per SIMD) shortens the kernel by about 7 % on
// a 32768-token row with a 24576-token document; at head_dim 128 the same
// scheduler is slower.  The arithmetic is that of the header: only the
// instruction order differs.
#include "bwd_dkdv.h"

namespace bd {

hipError_t launch_bwd_dkdv64(const BwdArgs& a, hipStream_t st) {
  return a.drop.thr != 0 ? launch_dkdv_t<64, true>(a, st) : launch_dkdv_t<64, false>(a, st);
}

}  // namespace bd
