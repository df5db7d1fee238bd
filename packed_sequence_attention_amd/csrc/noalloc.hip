// blockdiag_attn_bwd_noalloc: the backward with its scratch buffer (the
// float32 row statistics, 8 bytes per local row and query head) in a
// file-scope device array instead of a caller-supplied workspace, for
// callers that cannot allocate device memory.  The kernels are those of
// blockdiag_attn_bwd; only where the statistics live differs.
#include <hip/hip_runtime.h>

#include <mutex>

#include "blockdiag.h"
#include "internal.h"

namespace {

constexpr size_t kScratchBytes = size_t{16} << 20;  // BLOCKDIAG_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;

// One copy per GPU the library runs on, held until the process ends.  Its
// name is a host-side stand-in: host code uses only the device address that
// hipGetSymbolAddress returns for the current device.
__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of this device's scratch array, looked up once per device
// with that device current (the caller's current device).
bd_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return bd::fail(BD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return bd::fail(BD_ERR_UNSUPPORTED, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return bd::fail(BD_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return BD_OK;
}

}  // namespace

extern "C" size_t blockdiag_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" bd_status blockdiag_attn_bwd_noalloc(bd_dtype dtype, int32_t batch, int32_t seq_len,
                                                int32_t row_offset, int32_t q_len, int32_t kv_begin,
                                                int32_t kv_len, int32_t h_q, int32_t h_kv,
                                                int32_t head_dim, float scale, const bd_dropout* dropout,
                                                const void* q, const void* k,
                                                const void* v, const void* o, const float* lse, const void* d_o,
                                                const bd_meta* meta, void* dq, void* dk, void* dv, void* stream) {
  bd::clear_error();
  // Size check before the device is touched: the statistics of every local
  // row and query head must fit the array.
  if (batch > 0 && q_len > 0 && h_q > 0 && head_dim > 0) {
    const size_t need = blockdiag_workspace_bytes(1, dtype, batch, seq_len, q_len, h_q, h_kv, head_dim);
    if (need > kScratchBytes)
      return bd::fail(BD_ERR_WORKSPACE,
                      "batch * q_len * h_q = %lld rows need %zu bytes of row statistics; the static scratch "
                      "holds %zu (use blockdiag_attn_bwd with a workspace)",
                      static_cast<long long>(batch) * q_len * h_q, need, kScratchBytes);
  }
  void* ws = nullptr;
  size_t ws_bytes = 0;
  if (batch > 0 && q_len > 0) {
    const bd_status st = scratch_ptr(&ws);
    if (st != BD_OK) return st;
    ws_bytes = kScratchBytes;
  }
  return blockdiag_attn_bwd(dtype, batch, seq_len, row_offset, q_len, kv_begin, kv_len, h_q, h_kv, head_dim, scale,
                            dropout, q, k, v, o, lse, d_o, meta, dq, dk, dv, ws, ws_bytes, stream);
}
