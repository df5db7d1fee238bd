// C ABI of the block-diagonal packed attention library: argument checks,
// workspace sizing and dispatch to the gfx950 kernels.  Every check runs on
// the host before anything is enqueued (Automodel page "feat(distributed):
// block-diagonal varlen CP for packed sequences", key property 4: kernel
// inputs are validated on the host so a bad offset raises instead of
// faulting asynchronously).
#include <hip/hip_runtime_api.h>
#include <math.h>

#include "blockdiag.h"
#include "internal.h"
#include "launch.h"

using bd::fail;

namespace {

constexpr int64_t kMaxElems = (int64_t{1} << 31) - 1;
// Start alignment of a K/V window: the largest key tile of any kernel.
constexpr int32_t kKvAlign = 64;

bd_status check_common(bd_dtype dtype, int32_t batch, int32_t seq_len, int32_t row_offset,
                       int32_t q_len, int32_t kv_begin, int32_t kv_len, int32_t h_q, int32_t h_kv,
                       int32_t head_dim, float scale) {
  if (dtype != BD_F32 && dtype != BD_BF16) return fail(BD_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
  if (batch < 0 || seq_len < 0 || row_offset < 0 || q_len < 0)
    return fail(BD_ERR_INVALID_ARG, "negative size");
  if (static_cast<int64_t>(row_offset) + q_len > seq_len)
    return fail(BD_ERR_INVALID_ARG, "row_offset + q_len > seq_len");
  if (h_q <= 0 || h_kv <= 0 || h_q % h_kv != 0)
    return fail(BD_ERR_INVALID_ARG, "h_q (%d) must be a positive multiple of h_kv (%d)", h_q, h_kv);
  if (head_dim <= 0 || head_dim > 256 || head_dim % 8 != 0)
    return fail(BD_ERR_UNSUPPORTED, "head_dim %d: supported are multiples of 8 up to 256", head_dim);
  if (!isfinite(scale)) return fail(BD_ERR_INVALID_ARG, "scale must be finite");
  // K/V window [kv_begin, kv_begin + kv_len): tile-aligned start (so no key
  // tile starts before the buffer), inside the row, reaching the chunk's end.
  if (kv_begin < 0 || kv_len < 0 || static_cast<int64_t>(kv_begin) + kv_len > seq_len)
    return fail(BD_ERR_INVALID_ARG, "K/V window [%d, %d + %d) outside the row of %d keys", kv_begin, kv_begin,
                kv_len, seq_len);
  if (kv_begin % kKvAlign != 0)
    return fail(BD_ERR_INVALID_ARG, "K/V window start %d is not a multiple of %d", kv_begin, kKvAlign);
  if (kv_begin > row_offset || static_cast<int64_t>(kv_begin) + kv_len < static_cast<int64_t>(row_offset) + q_len)
    return fail(BD_ERR_INVALID_ARG, "K/V window [%d, %d) does not cover the chunk [%d, %d)", kv_begin,
                kv_begin + kv_len, row_offset, row_offset + q_len);
  const int64_t nq = static_cast<int64_t>(batch) * q_len * h_q * head_dim;
  const int64_t nk = static_cast<int64_t>(batch) * kv_len * h_kv * head_dim;
  if (nq > kMaxElems || nk > kMaxElems || static_cast<int64_t>(batch) * seq_len > kMaxElems)
    return fail(BD_ERR_INVALID_ARG, "tensor too large for 32-bit element counts");
  return BD_OK;
}

bool use_mfma_fwd(bd_dtype dtype, int32_t kv_len, int32_t head_dim, int32_t h_q, int32_t h_kv, float scale) {
  return bd::mfma_supported(static_cast<int>(dtype), head_dim, h_q, h_kv) && scale > 0.f &&
         bd::fwd_mfma_fits(kv_len, h_kv, head_dim);
}

bool use_mfma_bwd(bd_dtype dtype, int32_t q_len, int32_t head_dim, int32_t h_q, int32_t h_kv, float scale) {
  return bd::mfma_supported(static_cast<int>(dtype), head_dim, h_q, h_kv) && scale > 0.f &&
         bd::bwd_mfma_fits(q_len, h_q, head_dim);
}

bool use_mfma_bwd_full(bd_dtype dtype, int32_t kv_len, int32_t q_len, int32_t head_dim, int32_t h_q,
                       int32_t h_kv, float scale) {
  return use_mfma_bwd(dtype, q_len, head_dim, h_q, h_kv, scale) && bd::bwd_dq_fits(kv_len, h_kv, head_dim);
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Dropout as the kernels take it: the 8-bit threshold round(256 p) (at most
// 255) and the scale of kept weights 256 / (256 - thr); thr = 0 is none.
bd_status drop_args(const bd_dropout* d, bd::DropArgs* out) {
  *out = bd::DropArgs{0, 1.f, 0, 0};
  if (d == nullptr) return BD_OK;
  if (!(d->p >= 0.f && d->p < 1.f)) return fail(BD_ERR_INVALID_ARG, "dropout p must be in [0, 1)");
  const int thr = static_cast<int>(floor(static_cast<double>(d->p) * 256.0 + 0.5));
  out->thr = static_cast<uint32_t>(thr < 255 ? thr : 255);
  out->scale = static_cast<float>(256.0 / (256.0 - out->thr));
  out->seed = d->seed;
  out->offset = d->offset;
  return BD_OK;
}

// O(1) host check that a metadata descriptor was built for this call's sizes
// (the kernels index the buffer with the call's batch, seq_len and q_len).
bd_status check_meta(const bd_meta* m, int32_t batch, int32_t seq_len, int32_t row_offset, int32_t q_len,
                     int32_t kv_begin, int32_t kv_len) {
  if (m == nullptr) return fail(BD_ERR_INVALID_ARG, "null metadata descriptor");
  if (m->magic != BD_META_MAGIC) return fail(BD_ERR_INVALID_ARG, "metadata descriptor was not built");
  if (m->batch != batch || m->seq_len != seq_len || m->row_offset != row_offset || m->q_len != q_len)
    return fail(BD_ERR_INVALID_ARG,
                "metadata built for batch %d seq_len %d row_offset %d q_len %d, called with %d %d %d %d",
                m->batch, m->seq_len, m->row_offset, m->q_len, batch, seq_len, row_offset, q_len);
  const size_t need = blockdiag_meta_ints(batch, seq_len, q_len);
  if (m->n_ints < need)
    return fail(BD_ERR_INVALID_ARG, "metadata holds %llu ints, %zu needed",
                static_cast<unsigned long long>(m->n_ints), need);
  if (need > 0 && m->data == nullptr) return fail(BD_ERR_INVALID_ARG, "null metadata buffer");
  if (kv_begin > m->kv_lo || static_cast<int64_t>(kv_begin) + kv_len < m->kv_hi)
    return fail(BD_ERR_INVALID_ARG, "K/V window [%d, %d) misses keys the chunk attends: [%d, %d)", kv_begin,
                kv_begin + kv_len, m->kv_lo, m->kv_hi);
  return BD_OK;
}

// Shared argument checks of the two metadata builders; clears *desc first.
bd_status check_meta_build(const int32_t* table, int32_t n_seg, int32_t batch, int32_t seq_len,
                           int32_t row_offset, int32_t q_len, int32_t* d_meta, size_t capacity,
                           bd_meta* desc) {
  if (desc == nullptr) return fail(BD_ERR_INVALID_ARG, "null descriptor");
  desc->magic = 0;
  if (batch < 0 || seq_len < 0 || row_offset < 0 || q_len < 0 || n_seg < 0)
    return fail(BD_ERR_INVALID_ARG, "negative size");
  if (static_cast<int64_t>(row_offset) + q_len > seq_len)
    return fail(BD_ERR_INVALID_ARG, "row_offset + q_len > seq_len");
  if (static_cast<int64_t>(batch) * seq_len > kMaxElems) return fail(BD_ERR_INVALID_ARG, "too large");
  const size_t need = blockdiag_meta_ints(batch, seq_len, q_len);
  if (need > 0) {
    if (table == nullptr || d_meta == nullptr) return fail(BD_ERR_INVALID_ARG, "null pointer");
    if (capacity < need) return fail(BD_ERR_CAPACITY, "metadata buffer holds %zu ints, %zu needed", capacity, need);
    if (n_seg == 0 && static_cast<int64_t>(batch) * q_len > 0)
      return fail(BD_ERR_BAD_METADATA, "empty segment table for a non-empty chunk");
  }
  return BD_OK;
}

// Keys the chunk attends over all batch rows, [*lo, *hi), from a host copy
// of the segment table: the union of the non-padding segments' key ranges
// (row coordinates); [row_offset, row_offset) when no row attends a key.
// Without the table: [0, row_offset + q_len), which admits only windows that
// start at key 0.
void table_window(const int32_t* h_table, int32_t n_seg, int32_t seq_len, int32_t row_offset, int32_t q_len,
                  int32_t* lo, int32_t* hi) {
  if (h_table == nullptr) {
    *lo = 0;
    *hi = row_offset + q_len;
    return;
  }
  const int32_t* cu_q = h_table;
  const int32_t* cu_k = h_table + n_seg + 1;
  const int32_t* kb = h_table + 2 * (n_seg + 1);
  int64_t wlo = row_offset, whi = row_offset;
  bool any = false;
  for (int32_t s = 0; s < n_seg; ++s) {
    const int64_t kn = static_cast<int64_t>(cu_k[s + 1]) - cu_k[s];
    if (kn <= 0 || q_len <= 0 || seq_len <= 0) continue;
    const int64_t b = cu_q[s] / q_len;
    const int64_t a = static_cast<int64_t>(kb[s]) - b * seq_len;
    wlo = any ? (a < wlo ? a : wlo) : a;
    whi = any ? (a + kn > whi ? a + kn : whi) : a + kn;
    any = true;
  }
  *lo = static_cast<int32_t>(wlo);
  *hi = static_cast<int32_t>(whi);
}

// Most keys of one segment of a host table (-1 without the table).
int32_t table_max_seg_k(const int32_t* h_table, int32_t n_seg) {
  if (h_table == nullptr) return -1;
  const int32_t* cu_k = h_table + n_seg + 1;
  int32_t mx = 0;
  for (int32_t s = 0; s < n_seg; ++s) mx = cu_k[s + 1] - cu_k[s] > mx ? cu_k[s + 1] - cu_k[s] : mx;
  return mx;
}

void fill_desc(bd_meta* desc, int32_t n_seg, int32_t batch, int32_t seq_len, int32_t row_offset, int32_t q_len,
               const int32_t* d_meta, const int32_t* h_table) {
  table_window(h_table, n_seg, seq_len, row_offset, q_len, &desc->kv_lo, &desc->kv_hi);
  desc->max_seg_k = table_max_seg_k(h_table, n_seg);
  desc->batch = batch;
  desc->seq_len = seq_len;
  desc->row_offset = row_offset;
  desc->q_len = q_len;
  desc->n_seg = n_seg;
  desc->n_ints = blockdiag_meta_ints(batch, seq_len, q_len);
  desc->data = d_meta;
  desc->magic = BD_META_MAGIC;
}

thread_local hipEvent_t g_mark_start = nullptr;
thread_local hipEvent_t g_mark_stop = nullptr;

// Takes the pending profiling marks (they apply to one call only).
void take_marks(hipEvent_t* start, hipEvent_t* stop) {
  *start = g_mark_start;
  *stop = g_mark_stop;
  g_mark_start = g_mark_stop = nullptr;
}

}  // namespace

extern "C" bd_status blockdiag_mark_main_kernel(void* start_event, void* stop_event) {
  bd::clear_error();
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(BD_ERR_INVALID_ARG, "both events or neither");
  g_mark_start = static_cast<hipEvent_t>(start_event);
  g_mark_stop = static_cast<hipEvent_t>(stop_event);
  return BD_OK;
}

extern "C" size_t blockdiag_meta_ints(int32_t batch, int32_t seq_len, int32_t q_len) {
  if (batch < 0 || seq_len < 0 || q_len < 0) return 0;
  // row bounds, key bounds, then the query-tile order and the short-document bins
  return 2 * static_cast<size_t>(batch) * q_len + 2 * static_cast<size_t>(batch) * seq_len +
         bd::meta_tail_ints(batch, seq_len, q_len);
}

extern "C" bd_status blockdiag_meta_build(const int32_t* d_table, const int32_t* h_table, int32_t n_seg,
                                          int32_t batch, int32_t seq_len, int32_t row_offset, int32_t q_len,
                                          int32_t* d_meta, size_t meta_capacity, bd_meta* desc,
                                          void* stream) {
  bd::clear_error();
  bd_status st = check_meta_build(d_table, n_seg, batch, seq_len, row_offset, q_len, d_meta, meta_capacity, desc);
  if (st != BD_OK) return st;
  if (blockdiag_meta_ints(batch, seq_len, q_len) > 0) {
    hipError_t e = bd::launch_meta_build(d_table, false, n_seg, batch, seq_len, row_offset, q_len, d_meta,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(BD_ERR_HIP, "meta_build launch: %s", hipGetErrorString(e));
  }
  fill_desc(desc, n_seg, batch, seq_len, row_offset, q_len, d_meta, h_table);
  return BD_OK;
}

extern "C" int32_t blockdiag_meta_inline_max_seg(void) { return bd::kInlineSeg; }

extern "C" bd_status blockdiag_meta_build_host(const int32_t* h_table, int32_t n_seg, int32_t batch,
                                               int32_t seq_len, int32_t row_offset, int32_t q_len,
                                               int32_t* d_meta, size_t meta_capacity, bd_meta* desc,
                                               void* stream) {
  bd::clear_error();
  bd_status st = check_meta_build(h_table, n_seg, batch, seq_len, row_offset, q_len, d_meta, meta_capacity, desc);
  if (st != BD_OK) return st;
  if (n_seg > bd::kInlineSeg)
    return fail(BD_ERR_CAPACITY, "%d segments: at most %d pass by value (use blockdiag_meta_build)", n_seg,
                bd::kInlineSeg);
  if (blockdiag_meta_ints(batch, seq_len, q_len) > 0) {
    hipError_t e = bd::launch_meta_build(h_table, true, n_seg, batch, seq_len, row_offset, q_len, d_meta,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(BD_ERR_HIP, "meta_build launch: %s", hipGetErrorString(e));
  }
  fill_desc(desc, n_seg, batch, seq_len, row_offset, q_len, d_meta, h_table);
  return BD_OK;
}

extern "C" size_t blockdiag_workspace_bytes(int is_bwd, bd_dtype dtype, int32_t batch, int32_t seq_len,
                                            int32_t q_len, int32_t h_q, int32_t h_kv, int32_t head_dim) {
  (void)dtype; (void)seq_len; (void)h_kv;
  if (!is_bwd || batch <= 0 || q_len <= 0 || h_q <= 0 || head_dim <= 0) return 0;
  const size_t rows = static_cast<size_t>(batch) * q_len * h_q;
  return align256(rows * 2 * sizeof(float));  // rowstat pairs
}

extern "C" bd_status blockdiag_attn_fwd(bd_dtype dtype, int32_t batch, int32_t seq_len, int32_t row_offset,
                                        int32_t q_len, int32_t kv_begin, int32_t kv_len, int32_t h_q,
                                        int32_t h_kv, int32_t head_dim,
                                        float scale, const bd_dropout* dropout, const void* q, const void* k,
                                        const void* v, const bd_meta* meta, void* o, float* lse, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  bd::clear_error();
  (void)workspace;
  bd_status st = check_common(dtype, batch, seq_len, row_offset, q_len, kv_begin, kv_len, h_q, h_kv, head_dim, scale);
  if (st != BD_OK) return st;
  if (batch == 0 || q_len == 0) return BD_OK;
  if (!q || !k || !v || !o || !lse) return fail(BD_ERR_INVALID_ARG, "null tensor pointer");
  st = check_meta(meta, batch, seq_len, row_offset, q_len, kv_begin, kv_len);
  if (st != BD_OK) return st;
  const size_t need = blockdiag_workspace_bytes(0, dtype, batch, seq_len, q_len, h_q, h_kv, head_dim);
  if (workspace_bytes < need) return fail(BD_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  bd::DropArgs dr;
  st = drop_args(dropout, &dr);
  if (st != BD_OK) return st;
  bd::FwdArgs a{static_cast<int>(dtype), batch, seq_len, row_offset, q_len, kv_begin, kv_len, h_q, h_kv, head_dim,
                scale, dr, q, k, v, meta->data, o, lse, nullptr, nullptr};
  take_marks(&a.mark_start, &a.mark_stop);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = use_mfma_fwd(dtype, kv_len, head_dim, h_q, h_kv, scale) ? bd::launch_fwd_mfma(a, s)
                                                                          : bd::launch_fwd_generic(a, s);
  if (e != hipSuccess) return fail(BD_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return BD_OK;
}

extern "C" bd_status blockdiag_attn_bwd(bd_dtype dtype, int32_t batch, int32_t seq_len, int32_t row_offset,
                                        int32_t q_len, int32_t kv_begin, int32_t kv_len, int32_t h_q,
                                        int32_t h_kv, int32_t head_dim,
                                        float scale, const bd_dropout* dropout, const void* q, const void* k,
                                        const void* v, const void* o, const float* lse, const void* d_o,
                                        const bd_meta* meta, void* dq, void* dk, void* dv,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  bd::clear_error();
  bd_status st = check_common(dtype, batch, seq_len, row_offset, q_len, kv_begin, kv_len, h_q, h_kv, head_dim, scale);
  if (st != BD_OK) return st;
  if (batch == 0) return BD_OK;
  if (!k || !v || !dk || !dv) return fail(BD_ERR_INVALID_ARG, "null tensor pointer");
  if (q_len > 0 && (!q || !o || !lse || !d_o || !dq)) return fail(BD_ERR_INVALID_ARG, "null tensor pointer");
  const size_t need = blockdiag_workspace_bytes(1, dtype, batch, seq_len, q_len, h_q, h_kv, head_dim);
  if (workspace_bytes < need) return fail(BD_ERR_WORKSPACE, "workspace %zu < %zu bytes", workspace_bytes, need);
  if (need > 0 && workspace == nullptr) return fail(BD_ERR_WORKSPACE, "null workspace");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (q_len == 0) {
    // No local rows: the chunk's partial dK/dV are zero.
    const int64_t words = static_cast<int64_t>(batch) * kv_len * h_kv * head_dim * (dtype == BD_F32 ? 2 : 1);
    hipError_t e = bd::launch_zero_u16(dk, words, s);
    if (e == hipSuccess) e = bd::launch_zero_u16(dv, words, s);
    if (e != hipSuccess) return fail(BD_ERR_HIP, "zero-fill: %s", hipGetErrorString(e));
    return BD_OK;
  }
  st = check_meta(meta, batch, seq_len, row_offset, q_len, kv_begin, kv_len);
  if (st != BD_OK) return st;
  bd::DropArgs dr;
  st = drop_args(dropout, &dr);
  if (st != BD_OK) return st;
  const bool mf = use_mfma_bwd_full(dtype, kv_len, q_len, head_dim, h_q, h_kv, scale);
  bd::BwdArgs a{static_cast<int>(dtype), batch, seq_len, row_offset, q_len, kv_begin, kv_len, h_q, h_kv, head_dim, scale,
                dr, q, k, v, o, lse, d_o, meta->data, dq, dk, dv, static_cast<float*>(workspace), nullptr, nullptr};
  a.n_seg = meta->n_seg;
  a.max_seg_k = meta->max_seg_k;
  a.live_lo = meta->kv_lo;
  a.live_hi = meta->kv_hi;
  take_marks(&a.mark_start, &a.mark_stop);
  hipError_t e = mf ? bd::launch_bwd_mfma(a, s) : bd::launch_bwd_generic(a, s);
  if (e != hipSuccess) return fail(BD_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return BD_OK;
}
