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

// Row idx (of batch * q_len): the key interval [lo, hi) it attends.
__device__ __forceinline__ void row_bounds(const int32_t* table, int n_seg, int seq_len, int row_offset,
                                           int q_len, int64_t idx, int32_t* lo_out, int32_t* hi_out) {
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
  *lo_out = lo;
  *hi_out = hi;
}

// Key idx (of batch * seq_len): the interval [qlo, qhi) of local rows
// attending it.
__device__ __forceinline__ void key_bounds(const int32_t* table, int n_seg, int seq_len, int q_len,
                                           int64_t idx, int32_t* qlo_out, int32_t* qhi_out) {
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
  *qlo_out = qlo;
  *qhi_out = qhi;
}

// One launch for both halves: threads [0, n_rows) write row bounds, the
// rest key bounds.
__device__ __forceinline__ void meta_one(const int32_t* table, int n_seg, int seq_len, int row_offset,
                                         int q_len, int64_t n_rows, int64_t n_keys, MetaView m) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx < n_rows) {
    row_bounds(table, n_seg, seq_len, row_offset, q_len, idx, const_cast<int32_t*>(m.row_lo) + idx,
               const_cast<int32_t*>(m.row_hi) + idx);
  } else if (idx < n_rows + n_keys) {
    const int64_t kidx = idx - n_rows;
    key_bounds(table, n_seg, seq_len, q_len, kidx, const_cast<int32_t*>(m.key_qlo) + kidx,
               const_cast<int32_t*>(m.key_qhi) + kidx);
  }
}

__global__ void meta_kernel(const int32_t* __restrict__ table, int n_seg, int seq_len, int row_offset,
                            int q_len, int64_t n_rows, int64_t n_keys, MetaView m) {
  meta_one(table, n_seg, seq_len, row_offset, q_len, n_rows, n_keys, m);
}

// The table passed by value in the kernel arguments (small tables): no
// host-to-device copy before the launch.  Each block stages it in LDS.
struct InlineTable {
  int32_t v[kInlineTableInts];
};

__global__ void meta_inline_kernel(InlineTable tab, int n_seg, int seq_len, int row_offset, int q_len,
                                   int64_t n_rows, int64_t n_keys, MetaView m) {
  __shared__ int32_t sh[kInlineTableInts];
  const int n_int = 3 * n_seg + 2;
  for (int i = threadIdx.x; i < n_int; i += blockDim.x) sh[i] = tab.v[i];
  __syncthreads();
  meta_one(sh, n_seg, seq_len, row_offset, q_len, n_rows, n_keys, m);
}

}  // namespace

hipError_t launch_meta_build(const int32_t* table, bool host_table, int n_seg, int batch, int seq_len,
                             int row_offset, int q_len, int32_t* d_meta, hipStream_t stream) {
  MetaView m = meta_view(d_meta, batch, seq_len, q_len);
  const int64_t n_rows = static_cast<int64_t>(batch) * q_len;
  const int64_t n_keys = static_cast<int64_t>(batch) * seq_len;
  const int64_t n = n_rows + n_keys;
  if (n == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>((n + 255) / 256));
  if (host_table) {
    InlineTable tab;
    const int n_int = 3 * n_seg + 2;
    for (int i = 0; i < kInlineTableInts; ++i) tab.v[i] = i < n_int ? table[i] : 0;
    meta_inline_kernel<<<grid, 256, 0, stream>>>(tab, n_seg, seq_len, row_offset, q_len, n_rows, n_keys, m);
  } else {
    meta_kernel<<<grid, 256, 0, stream>>>(table, n_seg, seq_len, row_offset, q_len, n_rows, n_keys, m);
  }
  return hipGetLastError();
}

}  // namespace bd
