// Expansion of a validated varlen segment table into per-row and per-key
// mask bounds, once per step on the device.
//
// Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences": Summary (per-step precomputed cu_seqlens, zero per-layer host
// syncs) and key property 2 (a straddling document's first segment has more
// keys than queries, bottom-right aligned).  Row t of segment s attends keys
// k_begin[s] .. k_begin[s] + t + (k_len - q_len); the kernels below write,
// for each local row, that key interval, and for each key position, the
// interval of local rows attending it.
#include "device_common.h"
#include "launch.h"

namespace bd {
namespace {

// Largest s in [0, n) with a[s] <= x (0 if none); bounded loop.
__device__ __forceinline__ int upper_index(const int32_t* a, int n, int64_t x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ void meta_rows_kernel(const int32_t* __restrict__ table, int n_seg, int batch,
                                 int seq_len, int row_offset, int q_len, int32_t* __restrict__ row_lo,
                                 int32_t* __restrict__ row_hi) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n_rows = static_cast<int64_t>(batch) * q_len;
  if (idx >= n_rows) return;
  const int32_t* cu_q = table;
  const int32_t* cu_k = table + n_seg + 1;
  const int32_t* kb = table + 2 * (n_seg + 1);
  const int b = static_cast<int>(idx / q_len);
  const int t = static_cast<int>(idx % q_len);
  const int pos = row_offset + t;
  int lo = 0, hi = 0;
  if (n_seg > 0) {
    const int s = upper_index(cu_q, n_seg, idx);
    const int qn = cu_q[s + 1] - cu_q[s];
    const int kn = cu_k[s + 1] - cu_k[s];
    if (kn > 0) {
      const int64_t begin = static_cast<int64_t>(kb[s]) - static_cast<int64_t>(b) * seq_len;
      const int64_t end = begin + (idx - cu_q[s]) + (kn - qn) + 1;
      // Clamp into [0, pos + 1] so no later kernel can read past the row.
      const int64_t cl = begin < 0 ? 0 : (begin > pos + 1 ? pos + 1 : begin);
      const int64_t ch = end < cl ? cl : (end > pos + 1 ? pos + 1 : end);
      lo = static_cast<int>(cl);
      hi = static_cast<int>(ch);
    }
  }
  row_lo[idx] = lo;
  row_hi[idx] = hi;
}

__global__ void meta_keys_kernel(const int32_t* __restrict__ table, int n_seg, int batch,
                                 int seq_len, int row_offset, int q_len, int32_t* __restrict__ key_qlo,
                                 int32_t* __restrict__ key_qhi) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t n_keys = static_cast<int64_t>(batch) * seq_len;
  if (idx >= n_keys) return;
  const int32_t* cu_q = table;
  const int32_t* cu_k = table + n_seg + 1;
  const int32_t* kb = table + 2 * (n_seg + 1);
  const int b = static_cast<int>(idx / seq_len);
  const int j = static_cast<int>(idx % seq_len);
  int qlo = 0, qhi = 0;
  if (n_seg > 0) {
    const int s = upper_index(kb, n_seg, idx);
    const int qn = cu_q[s + 1] - cu_q[s];
    const int kn = cu_k[s + 1] - cu_k[s];
    const int64_t begin = static_cast<int64_t>(kb[s]) - static_cast<int64_t>(b) * seq_len;
    if (kn > 0 && j >= begin && j < begin + kn) {
      // Row tt of the segment attends keys up to begin + tt + kn - qn.
      int64_t first = j - begin - (kn - qn);
      if (first < 0) first = 0;
      const int64_t row0 = static_cast<int64_t>(cu_q[s]) - static_cast<int64_t>(b) * q_len;
      int64_t lo = row0 + first, hi = row0 + qn;
      lo = lo < 0 ? 0 : (lo > q_len ? q_len : lo);
      hi = hi < lo ? lo : (hi > q_len ? q_len : hi);
      qlo = static_cast<int>(lo);
      qhi = static_cast<int>(hi);
      if (qlo == qhi) qlo = qhi = 0;
    }
  }
  key_qlo[idx] = qlo;
  key_qhi[idx] = qhi;
}

}  // namespace

hipError_t launch_meta_build(const int32_t* d_table, int n_seg, int batch, int seq_len,
                             int row_offset, int q_len, int32_t* d_meta, hipStream_t stream) {
  MetaView m = meta_view(d_meta, batch, seq_len, q_len);
  const int64_t n_rows = static_cast<int64_t>(batch) * q_len;
  const int64_t n_keys = static_cast<int64_t>(batch) * seq_len;
  if (n_rows > 0) {
    dim3 grid(static_cast<unsigned>((n_rows + 255) / 256));
    meta_rows_kernel<<<grid, 256, 0, stream>>>(d_table, n_seg, batch, seq_len, row_offset, q_len,
                                               const_cast<int32_t*>(m.row_lo),
                                               const_cast<int32_t*>(m.row_hi));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (n_keys > 0) {
    dim3 grid(static_cast<unsigned>((n_keys + 255) / 256));
    meta_keys_kernel<<<grid, 256, 0, stream>>>(d_table, n_seg, batch, seq_len, row_offset, q_len,
                                               const_cast<int32_t*>(m.key_qlo),
                                               const_cast<int32_t*>(m.key_qhi));
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace bd
