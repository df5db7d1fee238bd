// Device-side helpers shared by the gfx950 kernels of the block-diagonal
// packed attention library: vector types for the bf16 matrix-core
// instructions, bf16 <-> f32 conversion, wave reductions and the launch
// parameter blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Raw bf16 bits <-> float.  bf16 -> f32 is exact; f32 -> bf16 rounds to
// nearest even in hardware (v_cvt_pk_bf16_f32).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// Element loads/stores for the generic kernels (float or raw bf16 bits).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float x) { *p = f32_to_bf16_bits(x); }
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
// Lane l and lane l ^ 32 combined (all 64 lanes active): v_permlane32_swap
// exchanges the upper half of one register with the lower half of the other,
// so after swapping x with itself every lane holds both values of its pair.
// A VALU exchange, without the LDS round trip of a bpermute.
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide min / max (all 64 lanes active).  Every lane holds the result
// after the butterfly; reading it from the first lane marks it uniform, so
// it can feed scalar registers (buffer resources, loop bounds).
__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  return __builtin_amdgcn_readfirstlane(x);
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return __builtin_amdgcn_readfirstlane(x);
}

// Launch parameters.  Sizes are int32 (checked on the host); element
// offsets are computed in 64-bit.
struct AttnShape {
  int batch, seq_len, row_offset, q_len, h_q, h_kv, head_dim, group;
  float scale;
  // K/V (and dK/dV) hold keys [kv_begin, kv_begin + kv_len) of every row,
  // kv_begin a multiple of 64 (the whole row: 0 and seq_len).  Positions in
  // the metadata and the masks stay those of the row.
  int kv_begin, kv_len;
};

// Query-tile order: the metadata build also writes, for the 32-row query
// tiles of every batch row (the forward and dQ kernels' tiles), a
// permutation of the tile codes b * n_qt + qt sorted by the number of key
// tiles of 32 each visits, most first (ties keep ascending code order), and
// two statistics: the largest visit count and their sum.  A kernel follows
// the order when its longest tile is long against the load of a workgroup
// slot (order_pays), since then the launch order sets the tail; otherwise
// it keeps its fixed order, whose neighbouring tiles share K/V tiles in L2.
// Built only for at most kOrderCap query tiles over the batch.
constexpr int kOrderQB = 32;
constexpr int kOrderCap = 8192;

__host__ __device__ inline int64_t order_q_tiles(int batch, int q_len) {
  return static_cast<int64_t>(batch) * ((q_len + kOrderQB - 1) / kOrderQB);
}
__host__ __device__ inline bool order_built(int batch, int q_len) {
  const int64_t nq = order_q_tiles(batch, q_len);
  return nq > 0 && nq <= kOrderCap;
}
// The order pays when the longest tile's visits are at least half a slot's
// share of all visits: tiles * head groups spread over `slots` workgroups
// resident at once.
__host__ __device__ inline bool order_pays(int max_visits, int total_visits, int head_groups, int slots) {
  return 2 * static_cast<int64_t>(max_visits) * slots >= static_cast<int64_t>(total_visits) * head_groups;
}

struct MetaView {
  const int32_t* row_lo;   // [batch][q_len]
  const int32_t* row_hi;   // [batch][q_len]
  const int32_t* key_qlo;  // [batch][seq_len]
  const int32_t* key_qhi;  // [batch][seq_len]
  const int32_t* q_order;  // [batch * n_qt] tile codes, most visits first (null: not built)
  const int32_t* q_stats;  // [2] largest and total visits (null: not built)
};

__host__ __device__ inline MetaView meta_view(const int32_t* meta, int batch, int seq_len, int q_len) {
  const int64_t nr = static_cast<int64_t>(batch) * q_len;
  const int64_t nk = static_cast<int64_t>(batch) * seq_len;
  MetaView m;
  m.row_lo = meta;
  m.row_hi = meta + nr;
  m.key_qlo = meta + 2 * nr;
  m.key_qhi = meta + 2 * nr + nk;
  const bool ord = order_built(batch, q_len);
  m.q_order = ord ? meta + 2 * nr + 2 * nk : nullptr;
  m.q_stats = ord ? m.q_order + order_q_tiles(batch, q_len) : nullptr;
  return m;
}

}  // namespace bd
