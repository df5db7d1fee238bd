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

// Row idx (of batch * q_len) in segment s (the largest s with
// cu_q[s] <= idx): the key interval [lo, hi) it attends.
__device__ __forceinline__ void row_bounds_in(const int32_t* table, int n_seg, int seq_len, int row_offset,
                                              int q_len, int64_t idx, int s, int32_t* lo_out, int32_t* hi_out) {
  const int32_t* cu_q = table;
  const int32_t* cu_k = table + n_seg + 1;
  const int32_t* kb = table + 2 * (n_seg + 1);
  const int b = static_cast<int>(idx / q_len);
  const int t = static_cast<int>(idx % q_len);
  const int pos = row_offset + t;
  int lo = 0, hi = 0;
  if (n_seg > 0) {
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

// Row idx (of batch * q_len): the key interval [lo, hi) it attends.
__device__ __forceinline__ void row_bounds(const int32_t* table, int n_seg, int seq_len, int row_offset,
                                           int q_len, int64_t idx, int32_t* lo_out, int32_t* hi_out) {
  const int s = n_seg > 0 ? upper_index(table, n_seg, idx) : 0;
  row_bounds_in(table, n_seg, seq_len, row_offset, q_len, idx, s, lo_out, hi_out);
}

// From a segment s with cu_q[s] <= idx, the largest such s (a forward walk:
// one thread visits increasing rows).
__device__ __forceinline__ int walk_index(const int32_t* cu_q, int n_seg, int64_t idx, int s) {
  while (s + 1 < n_seg && cu_q[s + 1] <= idx) ++s;
  return s;
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

// Work bin of a tile that visits w tiles of the other kind: exact below 128,
// then 16 bins per octave (bins rise with w; 255 from 2^15 up).
__device__ __forceinline__ int work_bin(int w) {
  if (w < 128) return w < 0 ? 0 : w;
  const int e = 31 - __builtin_clz(static_cast<unsigned>(w));
  const int bin = 128 + (e - 7) * 16 + ((w >> (e - 4)) & 15);
  return bin > 255 ? 255 : bin;
}

// Number of bytes of x equal to zero (exact: no borrow between bytes).
__device__ __forceinline__ int zero_bytes(uint32_t x, uint32_t keep) {
  const uint32_t z = ~(((x & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x | 0x7F7F7F7Fu);
  return __builtin_popcount(z & keep);
}

// The query-tile order and its statistics, built by one workgroup of 256
// threads from the segment table.  Query tile (b, qt) covers local rows
// [32 qt, 32 qt + 32); its rows attend keys from doc_start of its first row
// to the position of its last real row (padding rows are the tail of a
// chunk), so it visits last/32 - lo/32 + 1 key tiles of 32 (none when its
// first row is padding).  A stable counting sort on the visit bins
// (descending) places the codes b * n_qt + qt: ties keep ascending order.
struct OrderLds {
  alignas(16) uint8_t bin[kOrderCap];
  int hist[256];
  int scan[256];
  int vmax;
  unsigned long long vsum;
};

__device__ void build_q_order(const int32_t* table, int n_seg, int batch, int seq_len, int row_offset,
                              int q_len, MetaView m, OrderLds& ol) {
  const int tid = threadIdx.x;
  uint8_t* bins = ol.bin;
  int* hist = ol.hist;
  int* scan = ol.scan;
  const int32_t* cu_q = table;
  const int32_t* cu_k = table + n_seg + 1;
  const int n_qt = (q_len + kOrderQB - 1) / kOrderQB;
  const int nq = batch * n_qt;
  hist[tid] = 0;
  if (tid == 0) {
    ol.vmax = 0;
    ol.vsum = 0;
  }
  __syncthreads();
  int vmax = 0;
  unsigned long long vsum = 0;
  // Each thread takes a contiguous run of tile codes: their rows increase,
  // so one binary search and then a forward walk find every segment.
  const int per = (nq + 255) / 256;
  const int i0 = min(nq, tid * per), i1 = min(nq, i0 + per);
  int seg = (n_seg > 0 && i0 < i1)
                ? upper_index(cu_q, n_seg, static_cast<int64_t>(i0 / n_qt) * q_len + (i0 % n_qt) * kOrderQB)
                : 0;
  for (int i = i0; i < i1; ++i) {
    const int b = i / n_qt, qt = i % n_qt;
    int tiles = 0;
    if (n_seg > 0) {
      const int t0 = qt * kOrderQB, t1 = min(q_len, t0 + kOrderQB);
      const int64_t r0 = static_cast<int64_t>(b) * q_len + t0;
      seg = walk_index(cu_q, n_seg, r0, seg);
      int lo, hi;
      row_bounds_in(table, n_seg, seq_len, row_offset, q_len, r0, seg, &lo, &hi);
      if (hi > lo) {
        const int s1 = walk_index(cu_q, n_seg, static_cast<int64_t>(b) * q_len + t1 - 1, seg);
        const int last = cu_k[s1 + 1] - cu_k[s1] > 0
                             ? row_offset + t1 - 1
                             : row_offset + static_cast<int>(cu_q[s1] - static_cast<int64_t>(b) * q_len) - 1;
        tiles = max(0, last / kOrderQB - lo / kOrderQB + 1);
      }
    }
    const int bin = work_bin(tiles);
    bins[i] = static_cast<uint8_t>(bin);
    atomicAdd(&hist[bin], 1);
    vmax = max(vmax, tiles);
    vsum += static_cast<unsigned long long>(tiles);
  }
  atomicMax(&ol.vmax, vmax);
  atomicAdd(&ol.vsum, vsum);
  __syncthreads();
  if (tid == 0) {
    int32_t* st = const_cast<int32_t*>(m.q_stats);
    st[0] = ol.vmax;
    st[1] = static_cast<int32_t>(ol.vsum < 0x7FFFFFFFull ? ol.vsum : 0x7FFFFFFFull);  // saturated
  }
  // Exclusive scan over the bins in descending order: thread t holds bin
  // 255 - t; its tiles start after those of every higher bin.  Inclusive
  // scan inside each wave (shuffles), then the totals of the waves before.
  const int v = hist[255 - tid];
  const int lane = tid & 63, wv = tid >> 6;
  int inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int x = __shfl_up(inc, off, 64);
    if (lane >= off) inc += x;
  }
  if (lane == 63) scan[wv] = inc;
  __syncthreads();
  int before = 0;
  for (int k = 0; k < wv; ++k) before += scan[k];
  hist[255 - tid] = before + inc - v;  // first position of each bin
  __syncthreads();
  // Stable placement, 256 codes at a time: a code's position is its bin's
  // next free position plus the number of earlier codes of this chunk in
  // the same bin (bins compared four bytes at a time).
  int32_t* out = const_cast<int32_t*>(m.q_order);
  for (int c0 = 0; c0 < nq; c0 += 256) {
    const int i = c0 + tid;
    const bool has = i < nq;
    const int bin = has ? bins[i] : 0;
    int rank = 0;
    if (has) {
      // all 256 bytes of the chunk in 16 reads of 16 bytes, issued together;
      // only bytes before this code's count
      const uint4* w = reinterpret_cast<const uint4*>(bins + c0);
      const uint32_t rep = static_cast<uint32_t>(bin) * 0x01010101u;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint4 q = w[k];
        const uint32_t words[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int wi = 4 * k + e;  // bytes 4 wi .. 4 wi + 3 of the chunk
          const uint32_t keep = wi < (tid >> 2)    ? 0xFFFFFFFFu
                                : wi == (tid >> 2) ? (1u << (8 * (tid & 3))) - 1u
                                                   : 0u;
          rank += zero_bytes(words[e] ^ rep, keep);
        }
      }
      out[hist[bin] + rank] = i;
    }
    __syncthreads();  // every position of this chunk read before the bins advance
    if (has) atomicAdd(&hist[bin], 1);
    __syncthreads();
  }
}

// The short-document bins (see kBinCap) of a table staged in LDS, built in
// parallel by one workgroup of 256 threads.  The greedy walk in table order
// (a document joins the open bin when it lies in the same batch row and the
// bin's keys, with it, span at most kBinCap positions; otherwise it opens a
// new bin) is a chain: from a bin's first segment s, the next bin starts at
// next(s), the first later segment that lies in another batch row, is
// padding, or ends more than kBinCap keys after s's first key (a binary
// search: a row's documents are contiguous, so their key ends increase).
// The bins start at the segments the chains from each row's first segment
// reach; pointer doubling (log2 n rounds: reached nodes reach their 2^r-th
// successor, and successors double) marks them, and a prefix count places
// them in table order.  A segment of more than kBinCap keys, or more bins
// than the bound, leaves the count at 0: no bins.
struct BinLds {
  int32_t jmp[2][kBinMaxSeg + 1];
  uint8_t reach[kBinMaxSeg + 1];
  int32_t wsum[4];
  int flag;
};

__device__ void build_bins(const int32_t* table, int n_seg, int q_len, int64_t cap, int32_t* bins, BinLds& bl) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int32_t* cu_q = table;
  const int32_t* cu_k = table + n_seg + 1;
  const int32_t* kb = table + 2 * (n_seg + 1);
  auto kn = [&](int s) { return cu_k[s + 1] - cu_k[s]; };
  auto row = [&](int s) { return cu_q[s] / q_len; };
  // 2 * (batch row) + (padding): within a batch row the documents come
  // first, then at most one padding segment.
  auto order_key = [&](int s) { return s >= n_seg ? INT_MAX : 2 * row(s) + (kn(s) == 0 ? 1 : 0); };
  auto next_of = [&](int s) {
    const int key = 2 * row(s);
    int lo = s + 1, hi = n_seg;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (order_key(mid) > key) hi = mid; else lo = mid + 1;
    }
    const int stop = lo;
    const int64_t lim = static_cast<int64_t>(kb[s]) + kBinCap;
    lo = s + 1;
    hi = stop;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (static_cast<int64_t>(kb[mid]) + kn(mid) > lim) hi = mid; else lo = mid + 1;
    }
    return lo;
  };
  if (tid == 0) bl.flag = 0;
  __syncthreads();
  for (int s = tid; s < n_seg; s += blockDim.x)
    if (kn(s) > kBinCap) bl.flag = 1;
  __syncthreads();
  if (bl.flag != 0 || n_seg > kBinMaxSeg || q_len <= 0) {
    if (tid == 0) bins[0] = 0;
    return;
  }
  for (int s = tid; s <= n_seg; s += blockDim.x) {
    int nx = n_seg;
    bool head = false;
    if (s < n_seg && kn(s) > 0) {
      nx = next_of(s);
      head = s == 0 || row(s - 1) != row(s);
    }
    bl.jmp[0][s] = nx;
    bl.reach[s] = head ? 1 : 0;
  }
  __syncthreads();
  int cur = 0;
  for (int r = 0; (1 << r) <= n_seg; ++r) {
    for (int s = tid; s <= n_seg; s += blockDim.x) {
      const int j = bl.jmp[cur][s];
      if (bl.reach[s]) bl.reach[j] = 1;  // reached nodes only grow: a racing read is still a reached node
      bl.jmp[cur ^ 1][s] = bl.jmp[cur][j];
    }
    __syncthreads();
    cur ^= 1;
  }
  // Bin starts: reached documents (padding and the sentinel are not bins).
  // Each thread takes a contiguous run of segments; a workgroup scan of the
  // runs' counts gives every start its bin index in table order.
  const int per = (n_seg + static_cast<int>(blockDim.x) - 1) / static_cast<int>(blockDim.x);
  const int s0 = min(n_seg, tid * per), s1 = min(n_seg, s0 + per);
  int mine = 0;
  for (int s = s0; s < s1; ++s) mine += bl.reach[s] && kn(s) > 0 ? 1 : 0;
  int inc = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int x = __shfl_up(inc, off, 64);
    if (lane >= off) inc += x;
  }
  if (lane == 63) bl.wsum[wv] = inc;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < static_cast<int>(blockDim.x) / 64; ++w) {
    before += w < wv ? bl.wsum[w] : 0;
    total += bl.wsum[w];
  }
  int64_t idx = before + inc - mine;
  for (int s = s0; s < s1; ++s) {
    if (!(bl.reach[s] && kn(s) > 0)) continue;
    if (idx < cap) {
      bins[1 + 3 * idx] = cu_q[s];
      bins[2 + 3 * idx] = cu_q[next_of(s)];
      bins[3 + 3 * idx] = kb[s];
    }
    ++idx;
  }
  if (tid == 0) bins[0] = total <= cap ? total : 0;
}

// One launch for both halves: threads [0, n_rows) write row bounds, the
// rest key bounds.  `block` is the workgroup's index among those doing this.
__device__ __forceinline__ void meta_one(const int32_t* table, int n_seg, int seq_len, int row_offset,
                                         int q_len, int64_t n_rows, int64_t n_keys, MetaView m,
                                         int64_t block) {
  const int64_t idx = block * blockDim.x + threadIdx.x;
  if (idx < n_rows) {
    row_bounds(table, n_seg, seq_len, row_offset, q_len, idx, const_cast<int32_t*>(m.row_lo) + idx,
               const_cast<int32_t*>(m.row_hi) + idx);
  } else if (idx < n_rows + n_keys) {
    const int64_t kidx = idx - n_rows;
    key_bounds(table, n_seg, seq_len, q_len, kidx, const_cast<int32_t*>(m.key_qlo) + kidx,
               const_cast<int32_t*>(m.key_qhi) + kidx);
  }
}

// Workgroup roles of the metadata kernels: with the query-tile order built
// (m.q_order non-null) workgroup 0 builds it; the next one builds the bins;
// the others write the bounds.

// Tables of up to this many segments are staged in LDS by every workgroup
// (the bounds' binary searches and the order and bin walks would otherwise
// wait on global memory at every step); larger ones are searched in global
// memory and get no sorted order and no bins.
constexpr int kOrderStageSeg = kBinMaxSeg;

__global__ void meta_kernel(const int32_t* __restrict__ table, int n_seg, int batch, int seq_len, int row_offset,
                            int q_len, int64_t n_rows, int64_t n_keys, MetaView m) {
  __shared__ union {
    OrderLds ol;
    BinLds bl;
  } u;
  __shared__ int32_t stage[3 * kOrderStageSeg + 2];
  const int ord = m.q_order != nullptr ? 1 : 0;
  const int wg = static_cast<int>(blockIdx.x);
  const bool staged = n_seg <= kOrderStageSeg;
  if (staged) {
    for (int i = threadIdx.x; i < 3 * n_seg + 2; i += blockDim.x) stage[i] = table[i];
    __syncthreads();
  }
  if (wg < ord + 1) {
    if (wg == ord) {
      // (an empty chunk has no bin section; a table too long to stage gets no bins)
      if (n_rows > 0) {
        if (staged) {
          build_bins(stage, n_seg, q_len, max_bins(batch, q_len), const_cast<int32_t*>(m.bins), u.bl);
        } else if (threadIdx.x == 0) {
          const_cast<int32_t*>(m.bins)[0] = 0;
        }
      }
    } else if (staged) {
      build_q_order(stage, n_seg, batch, seq_len, row_offset, q_len, m, u.ol);
    } else if (threadIdx.x == 0) {
      // statistics that no kernel takes as a reason to follow the order
      int32_t* st = const_cast<int32_t*>(m.q_stats);
      st[0] = 0;
      st[1] = 0x7FFFFFFF;
    }
    return;
  }
  meta_one(staged ? stage : table, n_seg, seq_len, row_offset, q_len, n_rows, n_keys, m,
           static_cast<int64_t>(wg) - ord - 1);
}

// The table passed by value in the kernel arguments (small tables): no
// host-to-device copy before the launch.  Each block stages it in LDS.
struct InlineTable {
  int32_t v[kInlineTableInts];
};

__global__ void meta_inline_kernel(InlineTable tab, int n_seg, int batch, int seq_len, int row_offset, int q_len,
                                   int64_t n_rows, int64_t n_keys, MetaView m) {
  __shared__ int32_t sh[kInlineTableInts];
  __shared__ union {
    OrderLds ol;
    BinLds bl;
  } u;
  const int n_int = 3 * n_seg + 2;
  for (int i = threadIdx.x; i < n_int; i += blockDim.x) sh[i] = tab.v[i];
  __syncthreads();
  const int ord = m.q_order != nullptr ? 1 : 0;
  const int wg = static_cast<int>(blockIdx.x);
  if (wg < ord + 1) {
    if (wg == ord) {
      if (n_rows > 0) build_bins(sh, n_seg, q_len, max_bins(batch, q_len), const_cast<int32_t*>(m.bins), u.bl);
    } else {
      build_q_order(sh, n_seg, batch, seq_len, row_offset, q_len, m, u.ol);
    }
    return;
  }
  meta_one(sh, n_seg, seq_len, row_offset, q_len, n_rows, n_keys, m, static_cast<int64_t>(wg) - ord - 1);
}

}  // namespace

hipError_t launch_meta_build(const int32_t* table, bool host_table, int n_seg, int batch, int seq_len,
                             int row_offset, int q_len, int32_t* d_meta, hipStream_t stream) {
  MetaView m = meta_view(d_meta, batch, seq_len, q_len);
  const int64_t n_rows = static_cast<int64_t>(batch) * q_len;
  const int64_t n_keys = static_cast<int64_t>(batch) * seq_len;
  const int64_t n = n_rows + n_keys;
  if (n == 0) return hipSuccess;
  // one more workgroup (the first) builds the query-tile order, one the bins
  dim3 grid(static_cast<unsigned>((n + 255) / 256 + (m.q_order != nullptr ? 1 : 0) + 1));
  if (host_table) {
    InlineTable tab;
    const int n_int = 3 * n_seg + 2;
    for (int i = 0; i < kInlineTableInts; ++i) tab.v[i] = i < n_int ? table[i] : 0;
    meta_inline_kernel<<<grid, 256, 0, stream>>>(tab, n_seg, batch, seq_len, row_offset, q_len, n_rows, n_keys,
                                                 m);
  } else {
    meta_kernel<<<grid, 256, 0, stream>>>(table, n_seg, batch, seq_len, row_offset, q_len, n_rows, n_keys, m);
  }
  return hipGetLastError();
}

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

size_t meta_tail_ints(int batch, int seq_len, int q_len) {
  (void)seq_len;
  // the order, then its two statistics, when an order is built; then the bins
  return (order_built(batch, q_len) ? static_cast<size_t>(order_q_tiles(batch, q_len)) + 2 : 0) +
         static_cast<size_t>(meta_bin_ints(batch, q_len));
}

}  // namespace bd
