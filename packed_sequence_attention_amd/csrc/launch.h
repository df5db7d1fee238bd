// Host-side launch functions of the gfx950 kernels, called by the C ABI
// layer (api.cpp) after every argument has been checked.  Each returns the
// hipError_t of its launch(es).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace bd {

// Attention dropout as the kernels take it (thr = 0: none); see DropParams.
struct DropArgs {
  uint32_t thr;
  float scale;
  uint64_t seed;
  uint32_t offset;
};

struct FwdArgs {
  int dtype;  // 0 = f32, 1 = bf16
  int batch, seq_len, row_offset, q_len;
  int kv_begin, kv_len;  // k, v hold keys [kv_begin, kv_begin + kv_len) of every row
  int h_q, h_kv, head_dim;
  float scale;
  DropArgs drop;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* meta;
  void* o;
  float* lse;
  hipEvent_t mark_start;  // recorded around the main kernel when non-null
  hipEvent_t mark_stop;
};

struct BwdArgs {
  int dtype;
  int batch, seq_len, row_offset, q_len;
  int kv_begin, kv_len;  // k, v, dk, dv hold keys [kv_begin, kv_begin + kv_len) of every row
  int h_q, h_kv, head_dim;
  float scale;
  DropArgs drop;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* d_o;
  const int32_t* meta;
  void* dq;
  void* dk;
  void* dv;
  float* rowstat;  // workspace: [batch][h_q][q_len] pairs (lse * log2(e), delta)
  hipEvent_t mark_start;  // recorded around the main kernel when non-null
  hipEvent_t mark_stop;
  int n_seg = 0;        // segments of the table the metadata was built from
  int max_seg_k = -1;   // most keys of one segment (-1: unknown)
  // Key positions any local row of any batch row attends lie in [live_lo,
  // live_hi) (the metadata descriptor's window); other keys' dK/dV are zero.
  int live_lo = 0, live_hi = 0x7fffffff;
};

// Metadata expansion (segment table -> per-row / per-key bounds).  With
// host_table the table is host memory of at most kInlineSeg segments and is
// passed to the kernel by value; otherwise it is a device copy.
constexpr int kInlineSeg = 126;
constexpr int kInlineTableInts = 3 * kInlineSeg + 2;
hipError_t launch_meta_build(const int32_t* table, bool host_table, int n_seg, int batch, int seq_len,
                             int row_offset, int q_len, int32_t* d_meta, hipStream_t stream);
// int32 entries that follow the bounds in the metadata buffer: the
// query-tile order and its statistics (when built), then the bins.
size_t meta_tail_ints(int batch, int seq_len, int q_len);
// Compute units of the current device (cached per device).
int device_cu_count();

// Generic kernels: any head_dim <= 256 that is a multiple of 8, f32 or bf16.
hipError_t launch_fwd_generic(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_generic(const BwdArgs& a, hipStream_t stream);

// bf16 matrix-core kernels: head_dim in {64, 128, 256}, any GQA ratio.
bool mfma_supported(int dtype, int head_dim, int h_q, int h_kv);
// The matrix-core forward addresses a (batch row, K/V head)'s keys (the K/V
// window) with 31-bit buffer offsets; larger rows take the generic kernel.
bool fwd_mfma_fits(int64_t kv_len, int64_t h_kv, int64_t head_dim);
hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t stream);
// The matrix-core backward addresses one (batch row, head)'s Q / dO rows and
// one (batch row, K/V head)'s keys with 32-bit buffer offsets.
bool bwd_mfma_fits(int64_t q_len, int64_t h_q, int64_t head_dim);
bool bwd_dq_fits(int64_t kv_len, int64_t h_kv, int64_t head_dim);
// dQ of the matrix-core backward (query-stationary); also writes rowstat.
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);
// dK / dV of the matrix-core backward at head_dim 256 (bwd_dkdv256.hip) and
// 64 (bwd_dkdv64.hip); read rowstat.
hipError_t launch_bwd_dkdv256(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_dkdv64(const BwdArgs& a, hipStream_t stream);

// The short-document backward (bwd_short.hip): bf16, head_dim 64 or 128,
// every segment at most kBinCap keys; dQ, dK and dV in one kernel over the
// metadata's bins (no row statistics pass).
bool bwd_short_applies(const BwdArgs& a);
hipError_t launch_bwd_short(const BwdArgs& a, hipStream_t stream);

// Fill n 16-bit words with zeros (a kernel, so it is safe under graph capture).
hipError_t launch_zero_u16(void* p, int64_t n, hipStream_t stream);

// Records a profiling mark on the stream when the event is non-null.
inline hipError_t mark(hipEvent_t ev, hipStream_t stream) {
  return ev != nullptr ? hipEventRecord(ev, stream) : hipSuccess;
}

}  // namespace bd
