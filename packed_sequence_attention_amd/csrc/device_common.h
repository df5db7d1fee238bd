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

// Partner exchanges on the vector ALU (all 64 lanes active), without the
// LDS round trip of a bpermute: lane_swap<O> returns (own value, partner's
// value) in either order, the partner being l ^ 32 and l ^ 16 (the permlane
// swaps), l ^ 15 (row mirror), l ^ 7 (half-row mirror), l ^ 2 and l ^ 1
// (quad permutes).  Those six masks span all six lane bits, so combining
// over them in turn reaches every lane once: a wave-wide reduction whose
// result is the same bits in every lane (each pair computes a + b and b + a).
template <int O>
__device__ __forceinline__ uint2 lane_swap_u(uint32_t x) {
  if constexpr (O >= 16) {
    const auto r = O == 32 ? __builtin_amdgcn_permlane32_swap(x, x, false, false)
                           : __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return make_uint2(r[0], r[1]);
  } else {
    constexpr int ctrl = O == 8 ? 0x140 : O == 4 ? 0x141 : O == 2 ? 0x4E : 0xB1;
    return make_uint2(x, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(x), ctrl, 0xF, 0xF, false)));
  }
}
template <int O>
__device__ __forceinline__ float2 lane_swap(float x) {
  const uint2 r = lane_swap_u<O>(__float_as_uint(x));
  return make_float2(__uint_as_float(r.x), __uint_as_float(r.y));
}
__device__ __forceinline__ float wave_max(float x) {
  float2 r;
  r = lane_swap<32>(x); x = fmaxf(r.x, r.y);
  r = lane_swap<16>(x); x = fmaxf(r.x, r.y);
  r = lane_swap<8>(x); x = fmaxf(r.x, r.y);
  r = lane_swap<4>(x); x = fmaxf(r.x, r.y);
  r = lane_swap<2>(x); x = fmaxf(r.x, r.y);
  r = lane_swap<1>(x); x = fmaxf(r.x, r.y);
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  float2 r;
  r = lane_swap<32>(x); x = r.x + r.y;
  r = lane_swap<16>(x); x = r.x + r.y;
  r = lane_swap<8>(x); x = r.x + r.y;
  r = lane_swap<4>(x); x = r.x + r.y;
  r = lane_swap<2>(x); x = r.x + r.y;
  r = lane_swap<1>(x); x = r.x + r.y;
  return x;
}
// Lane l and lane l ^ 32 combined (all 64 lanes active): v_permlane32_swap
// exchanges the upper half of one register with the lower half of the other,
// so after swapping x with itself every lane holds both values of its pair.
// A VALU exchange, without the LDS round trip of a bpermute.
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide min / max (all 64 lanes active).  Every lane holds the result
// after the butterfly; reading it from the first lane marks it uniform, so
// it can feed scalar registers (buffer resources, loop bounds).
// (The exchanges are those of wave_max above.)
template <bool MIN, int O = 32>
__device__ __forceinline__ int wave_minmax_i(int x) {
  const uint2 r = lane_swap_u<O>(static_cast<uint32_t>(x));
  const int a = static_cast<int>(r.x), b = static_cast<int>(r.y);
  x = MIN ? min(a, b) : max(a, b);
  if constexpr (O > 1) return wave_minmax_i<MIN, O / 2>(x);
  else return x;
}
__device__ __forceinline__ int wave_min_i(int x) { return __builtin_amdgcn_readfirstlane(wave_minmax_i<true>(x)); }
__device__ __forceinline__ int wave_max_i(int x) { return __builtin_amdgcn_readfirstlane(wave_minmax_i<false>(x)); }

// Attention dropout.  Keep decisions come from Philox4x32-10, the
// counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11): ten rounds, each multiplying words 0
// and 2 of the counter by two fixed 32-bit constants and mixing the high and
// low product halves with words 1 and 3 and the round key, the key advanced
// by two Weyl constants between rounds.  The pair (query position i, key
// position j) of batch row b and query head h -- positions in the packed
// row, so masks do not depend on chunking or on the K/V window -- reads
// counter (j / 4, i / 4, b * h_q + h, offset) under key (seed_lo, seed_hi):
// byte j % 4 of output word i % 4 is kept iff >= thr, and kept weights are
// multiplied by scale = 256 / (256 - thr).  thr = 0 keeps everything.
struct DropParams {
  uint32_t thr;
  float scale;
  uint32_t seed_lo, seed_hi, offset;
};

inline DropParams drop_params(uint32_t thr, float scale, uint64_t seed, uint32_t offset) {
  DropParams d;
  d.thr = thr;
  d.scale = scale;
  d.seed_lo = static_cast<uint32_t>(seed);
  d.seed_hi = static_cast<uint32_t>(seed >> 32);
  d.offset = offset;
  return d;
}

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Word w (0..3) of the generator's output for the 4 x 4 block of rows
// [4 * i4, 4 * i4 + 4) and keys [4 * j4, 4 * j4 + 4) of (b, h); byte e of
// word w is the draw of (row 4 * i4 + w, key 4 * j4 + e).
__device__ __forceinline__ uint4 drop_block(const DropParams& dp, uint32_t j4, uint32_t i4, uint32_t bh) {
  return philox4x32_10(make_uint4(j4, i4, bh, dp.offset), dp.seed_lo, dp.seed_hi);
}
__device__ __forceinline__ uint32_t pick_word(uint4 w, int i) {
  const int s = i & 3;
  return s == 0 ? w.x : s == 1 ? w.y : s == 2 ? w.z : w.w;
}
// The factor a weight is multiplied by: scale if byte e of word is kept, else 0.
__device__ __forceinline__ float keep_factor(const DropParams& dp, uint32_t word, int e) {
  return ((word >> (8 * e)) & 0xFFu) >= dp.thr ? dp.scale : 0.f;
}

// Keep factors of one query position i against the four keys j0 .. j0 + 3
// (j0 a multiple of 4) of (b, h) -- the layout of a lane that owns a row.
__device__ __forceinline__ void keep_factors_row(const DropParams& dp, uint32_t i, uint32_t j0, uint32_t bh,
                                                 float f[4]) {
  const uint32_t word = pick_word(drop_block(dp, j0 >> 2, i >> 2, bh), static_cast<int>(i));
#pragma unroll
  for (int e = 0; e < 4; ++e) f[e] = keep_factor(dp, word, e);
}
// Keep factors of the four query positions i0 .. i0 + 3 (any alignment: they
// may fall in two blocks) against one key position j of (b, h) -- the
// layout of a lane that owns a key.  i0 % 4 must be the same on every lane
// (then the second block's draw is a uniform branch).
__device__ __forceinline__ void keep_factors_col(const DropParams& dp, uint32_t i0, uint32_t j, uint32_t bh,
                                                 float f[4]) {
  const uint4 wa = drop_block(dp, j >> 2, i0 >> 2, bh);
  uint4 wb = wa;
  if ((i0 & 3u) != 0) wb = drop_block(dp, j >> 2, (i0 >> 2) + 1, bh);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t i = i0 + e;
    f[e] = keep_factor(dp, pick_word((i >> 2) == (i0 >> 2) ? wa : wb, static_cast<int>(i)), static_cast<int>(j & 3));
  }
}

// Keep factor of one (query position i, key position j) pair of (b, h).
__device__ __forceinline__ float keep_one(const DropParams& dp, uint32_t i, uint32_t j, uint32_t bh) {
  return keep_factor(dp, pick_word(drop_block(dp, j >> 2, i >> 2, bh), static_cast<int>(i)), static_cast<int>(j & 3));
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
  DropParams drop;  // thr = 0: no dropout
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

// Query heads a matrix-core workgroup takes from one K/V head of a GQA group
// of `group` heads: 4 when the group holds a multiple of 4 heads, else 2 when
// it holds a multiple of 2, else 1; its four waves then take 4 / that many
// consecutive query tiles (forward, dQ) or query-tile phases (dK/dV).
__host__ __device__ inline int heads_per_workgroup(int group) {
  return group % 4 == 0 ? 4 : (group % 2 == 0 ? 2 : 1);
}

// Short-document bins: consecutive documents (non-padding segments) of one
// batch row grouped greedily, in table order, so that each group's keys span
// at most kBinCap positions.  Built only when every segment has at most
// kBinCap keys and the table at most kBinMaxSeg segments; then every local row of a document and every key it attends
// belong to exactly one bin, and the short-document backward takes a bin
// per workgroup.  A bin is (first row, end row) of the flattened
// [batch * q_len] rows and the flattened key index (b * seq_len + position)
// of its first key; its keys end one past its last row's position.  Per
// batch row, two consecutive bins hold more than kBinCap keys together (the
// second one's first document did not fit the first) and the row's bins
// hold at most q_len + kBinCap - 1 keys (only the chunk's first document
// has keys before the chunk, fewer than kBinCap), which bounds the count.
constexpr int kBinCap = 128;
// Bins are built for tables of at most this many segments (the builder
// stages the table in LDS); longer tables get none.
constexpr int kBinMaxSeg = 2047;
__host__ __device__ inline int64_t max_bins(int batch, int q_len) {
  return static_cast<int64_t>(batch) * (2 * ((static_cast<int64_t>(q_len) + 2 * kBinCap - 2) / kBinCap) + 1);
}
// int32 entries of the bin section: the count, then 3 per bin (none for an
// empty chunk).
__host__ __device__ inline int64_t meta_bin_ints(int batch, int q_len) {
  return static_cast<int64_t>(batch) * q_len > 0 ? 1 + 3 * max_bins(batch, q_len) : 0;
}

struct MetaView {
  const int32_t* row_lo;   // [batch][q_len]
  const int32_t* row_hi;   // [batch][q_len]
  const int32_t* key_qlo;  // [batch][seq_len]
  const int32_t* key_qhi;  // [batch][seq_len]
  const int32_t* q_order;  // [batch * n_qt] tile codes, most visits first (null: not built)
  const int32_t* q_stats;  // [2] largest and total visits (null: not built)
  const int32_t* bins;     // [0]: bin count (0: not built), then (row begin, row end, first key) per bin
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
  m.bins = meta + 2 * nr + 2 * nk + (ord ? order_q_tiles(batch, q_len) + 2 : 0);
  return m;
}

}  // namespace bd
