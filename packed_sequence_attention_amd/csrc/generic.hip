// Generic (vector-ALU) kernels of block-diagonal packed attention: float32
// or bfloat16 tensors, any head_dim up to 256 that is a multiple of 8, any
// grouped-query ratio.  They serve the float32 path and the shapes the
// matrix-core kernels do not cover.  All arithmetic is float32.
//
// Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences": Summary/Motivation (block-causal attention per document, the
// same function as a dense masked SDPA) and the Proof section (forward and
// input gradients).  Each local row visits exactly the keys of its own
// document up to itself ([row_lo, row_hi) from the per-step metadata); each
// key visits exactly the local rows attending it ([key_qlo, key_qhi)), so no
// fully masked work is done and no atomics are needed.
//
// Backward uses the row statistic delta_i = sum_d dO_i O_i (equal to
// sum_j P_ij dP_ij), computed once by the preparation kernel.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace bd {
namespace {

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Load 8 consecutive elements as float.
__device__ __forceinline__ void load8(const float* p, float out[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, float out[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Work layout.  A wave owns one query row (forward, dQ) or one key (dK/dV)
// and sweeps its partners (the row's keys, the key's rows) in blocks of 64,
// one partner per lane, anchored at the row's document start (the key's
// first attending row), so a row's arithmetic does not depend on the chunk
// or on the K/V window.  Each lane loads its partner's rows once per block
// -- every load of the block goes out together, one memory round trip --
// and uses them twice: for its dot products (score, dP) and for the
// weighted sums over the block's partners (P V, dS K, P dO, dS Q), which
// are lane transposes: lane_sum64 adds the 64 lanes' vectors so that lane l
// ends with column l.

// Columns [c0, c0 + 64) of a row of D elements (D a multiple of 8); groups
// at or past D re-read the row's last group (their values are not used).
template <typename T>
__device__ __forceinline__ void load_cols64(const T* row, int c0, int D, float x[64]) {
#pragma unroll
  for (int g = 0; g < 8; ++g) load8(row + min(c0 + 8 * g, D - 8), x + 8 * g);
}

// acc + sum over d in [c0, min(c0 + 64, D)) of x_lds[d] * x[d - c0], in
// column order.
__device__ __forceinline__ float dot_cols64(const float* x_lds, const float x[64], int c0, int D, float acc) {
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if (c0 + 8 * g >= D) break;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(x_lds[c0 + 8 * g + e], x[8 * g + e], acc);
  }
  return acc;
}

// Sum over the wave's 64 lanes of the vectors x[0..64) (one per lane): lane
// l returns the total of element l.  Recursive halving: at offset O each
// lane holds 2 O partial sums, keeps the half its lane bit O selects, and
// adds its partner's copy of that half (the partner differs from l in bit O
// and agrees above it: l ^ 32, l ^ 16, l ^ 15, l ^ 7, l ^ 2, l ^ 1); after
// the six steps lane l holds element l.  x is used as scratch.  (The steps are templates
// so that every index is a constant and x stays in registers.)  The
// exchanges are vector-ALU lane permutes, without the LDS round trip of a
// bpermute.
template <int O>
__device__ __forceinline__ void lane_sum_step(float x[64], int lane) {
  if constexpr (O >= 16) {
    // v_permlane32_swap / v_permlane16_swap of (x[i], x[O + i]) hands every
    // lane its own kept value and its partner's copy of it.
#pragma unroll
    for (int i = 0; i < O; ++i) {
      const uint32_t a = __float_as_uint(x[i]), b = __float_as_uint(x[O + i]);
      const auto r = O == 32 ? __builtin_amdgcn_permlane32_swap(a, b, false, false)
                             : __builtin_amdgcn_permlane16_swap(a, b, false, false);
      x[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  } else {
    // partners by DPP: row mirror (l ^ 15) for bit 3, half-row mirror
    // (l ^ 7) for bit 2, quad permutes for bits 1 and 0; each partner
    // differs in the selecting bit and shares the higher ones.
    constexpr int ctrl = O == 8 ? 0x140 : O == 4 ? 0x141 : O == 2 ? 0x4E : 0xB1;
    const bool up = (lane & O) != 0;
#pragma unroll
    for (int i = 0; i < O; ++i) {
      const float send = up ? x[i] : x[O + i];
      const float keep = up ? x[O + i] : x[i];
      const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), ctrl, 0xF, 0xF, false));
      x[i] = keep + recv;
    }
  }
  if constexpr (O > 1) lane_sum_step<O / 2>(x, lane);
}
__device__ __forceinline__ float lane_sum64(float x[64], int lane) {
  lane_sum_step<32>(x, lane);
  return x[0];
}

constexpr int kWaves = 4;
constexpr int kMaxD = 256;

// One wave per (b, query head, local row); lane l accumulates output columns
// l + 64 r.
template <typename T, int NR>
__global__ __launch_bounds__(256) void fwd_generic_kernel(AttnShape s, const T* __restrict__ q,
                                                          const T* __restrict__ k,
                                                          const T* __restrict__ v, MetaView m,
                                                          T* __restrict__ o, float* __restrict__ lse) {
  __shared__ float sq[kWaves][kMaxD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const int64_t total = static_cast<int64_t>(s.batch) * s.q_len * s.h_q;
  if (w >= total) return;  // no block-wide barrier below: waves are independent
  const int D = s.head_dim;
  const int h = static_cast<int>(w % s.h_q);
  const int64_t bt = w / s.h_q;
  const int t = static_cast<int>(bt % s.q_len);
  const int b = static_cast<int>(bt / s.q_len);
  const int g = h / s.group;
  const T* qrow = q + (bt * s.h_q + h) * D;
  for (int d = lane; d < D; d += 64) sq[wave][d] = Elem<T>::load(qrow + d);
  wave_sync();
  // keys of the K/V window only (the host checks that it holds every key
  // the rows attend; the clamp keeps a mismatched table in bounds)
  const int lo = max(m.row_lo[bt], s.kv_begin), hi = min(m.row_hi[bt], s.kv_begin + s.kv_len);
  const int64_t kv_base = static_cast<int64_t>(b) * s.kv_len - s.kv_begin;  // row position j -> window row
  float mrun = -INFINITY, lrun = 0.f, acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;
  for (int j0 = lo; j0 < hi; j0 += 64) {
    const int j = j0 + lane;
    const bool in = j < hi;
    const int64_t jr = ((kv_base + min(j, hi - 1)) * s.h_kv + g) * D;  // lanes past hi re-read the last key
    // Score, with V columns 0-63 loaded beside K (one round trip at
    // head_dim <= 64; wider rows load V by 64 columns after the softmax).
    float vx[64];
    float sc = 0.f;
#pragma unroll
    for (int c = 0; c < NR; ++c) {
      float kx[64];
      load_cols64(k + jr, 64 * c, D, kx);
      if (c == 0) load_cols64(v + jr, 0, D, vx);
      sc = dot_cols64(sq[wave], kx, 64 * c, D, sc);
    }
    sc = in ? s.scale * sc : -INFINITY;
    const float mnew = fmaxf(mrun, wave_max(sc));  // finite: lane 0 is in range
    const float p = in ? expf(sc - mnew) : 0.f;
    const float alpha = expf(mrun - mnew);
    lrun = lrun * alpha + wave_sum(p);
    // dropout acts on the weights that multiply V, not on the row sum
    const float pw = (s.drop.thr != 0 && in)
                         ? p * keep_one(s.drop, static_cast<uint32_t>(s.row_offset + t), static_cast<uint32_t>(j),
                                        static_cast<uint32_t>(b * s.h_q + h))
                         : p;
#pragma unroll
    for (int c = 0; c < NR; ++c) {
      if (c > 0) load_cols64(v + jr, 64 * c, D, vx);
      float x[64];
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] = pw * vx[i];
      acc[c] = acc[c] * alpha + lane_sum64(x, lane);
    }
    mrun = mnew;
  }
  const bool any = hi > lo;
  const float inv = any ? 1.f / lrun : 0.f;
  T* orow = o + (bt * s.h_q + h) * D;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int d = lane + 64 * r;
    if (d < D) Elem<T>::store(orow + d, acc[r] * inv);
  }
  if (lane == 0)
    lse[(static_cast<int64_t>(b) * s.h_q + h) * s.q_len + t] = any ? mrun + logf(lrun) : -INFINITY;
}

// One wave per (b, query head, local row): dQ_i = scale * sum_j dS_ij k_j;
// lane l accumulates columns l + 64 r.
template <typename T, int NR>
__global__ __launch_bounds__(256) void dq_generic_kernel(AttnShape s, const T* __restrict__ q,
                                                         const T* __restrict__ k,
                                                         const T* __restrict__ v,
                                                         const T* __restrict__ d_o,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ rowstat, MetaView m,
                                                         T* __restrict__ dq) {
  __shared__ float sq[kWaves][kMaxD];
  __shared__ float sdo[kWaves][kMaxD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const int64_t total = static_cast<int64_t>(s.batch) * s.q_len * s.h_q;
  if (w >= total) return;
  const int D = s.head_dim;
  const int h = static_cast<int>(w % s.h_q);
  const int64_t bt = w / s.h_q;
  const int t = static_cast<int>(bt % s.q_len);
  const int b = static_cast<int>(bt / s.q_len);
  const int g = h / s.group;
  const int64_t row = (bt * s.h_q + h) * D;
  for (int d = lane; d < D; d += 64) {
    sq[wave][d] = Elem<T>::load(q + row + d);
    sdo[wave][d] = Elem<T>::load(d_o + row + d);
  }
  wave_sync();
  const int lo = max(m.row_lo[bt], s.kv_begin), hi = min(m.row_hi[bt], s.kv_begin + s.kv_len);
  const int64_t st = (static_cast<int64_t>(b) * s.h_q + h) * s.q_len + t;
  const float lse_t = hi > lo ? lse[st] : 0.f;
  const float delta_t = rowstat[2 * st + 1];
  const int64_t kv_base = static_cast<int64_t>(b) * s.kv_len - s.kv_begin;  // row position j -> window row
  float acc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = 0.f;
  for (int j0 = lo; j0 < hi; j0 += 64) {
    const int j = j0 + lane;
    const bool in = j < hi;
    const int64_t kr = ((kv_base + min(j, hi - 1)) * s.h_kv + g) * D;
    // K and V of the lane's key: the score and dP dots; K columns 0-63 stay
    // for the dS K sum (wider rows reload K by 64 columns).
    float kx[64];
    float sdot = 0.f, dp = 0.f;
#pragma unroll
    for (int c = 0; c < NR; ++c) {
      float vx[64];
      load_cols64(k + kr, 64 * c, D, kx);
      load_cols64(v + kr, 64 * c, D, vx);
      sdot = dot_cols64(sq[wave], kx, 64 * c, D, sdot);
      dp = dot_cols64(sdo[wave], vx, 64 * c, D, dp);
    }
    float ds = 0.f;
    if (in) {
      const float p = expf(s.scale * sdot - lse_t);
      if (s.drop.thr != 0)  // the gradient reaching P is (dO . v_j) * Z * c
        dp *= keep_one(s.drop, static_cast<uint32_t>(s.row_offset + t), static_cast<uint32_t>(j),
                       static_cast<uint32_t>(b * s.h_q + h));
      ds = p * (dp - delta_t);
    }
#pragma unroll
    for (int c = 0; c < NR; ++c) {
      if (NR > 1) load_cols64(k + kr, 64 * c, D, kx);
      float x[64];
#pragma unroll
      for (int i = 0; i < 64; ++i) x[i] = ds * kx[i];
      acc[c] += lane_sum64(x, lane);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int d = lane + 64 * r;
    if (d < D) Elem<T>::store(dq + row + d, acc[r] * s.scale);
  }
}

// One wave per (b, K/V head, key position): dV_j = sum_i P_ij dO_i and
// dK_j = scale * sum_i dS_ij q_i over the group's query heads and the local
// rows attending j; lane l accumulates columns l + 64 r.  Keys no row
// attends get zeros.
template <typename T, int NR>
__global__ __launch_bounds__(256) void dkv_generic_kernel(AttnShape s, const T* __restrict__ q,
                                                          const T* __restrict__ k,
                                                          const T* __restrict__ v,
                                                          const T* __restrict__ d_o,
                                                          const float* __restrict__ lse,
                                                          const float* __restrict__ rowstat, MetaView m,
                                                          T* __restrict__ dk, T* __restrict__ dv) {
  __shared__ float sk[kWaves][kMaxD];
  __shared__ float sv[kWaves][kMaxD];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  const int64_t total = static_cast<int64_t>(s.batch) * s.kv_len * s.h_kv;  // the window's keys
  if (w >= total) return;
  const int D = s.head_dim;
  const int g = static_cast<int>(w % s.h_kv);
  const int64_t bw = w / s.h_kv;  // b * kv_len + window row
  const int b = static_cast<int>(bw / s.kv_len);
  const int64_t bj = static_cast<int64_t>(b) * s.seq_len + s.kv_begin + bw % s.kv_len;  // metadata index
  const int64_t krow = (bw * s.h_kv + g) * D;
  for (int d = lane; d < D; d += 64) {
    sk[wave][d] = Elem<T>::load(k + krow + d);
    sv[wave][d] = Elem<T>::load(v + krow + d);
  }
  wave_sync();
  const int qlo = m.key_qlo[bj], qhi = m.key_qhi[bj];
  const uint32_t jpos = static_cast<uint32_t>(bj - static_cast<int64_t>(b) * s.seq_len);
  float adk[NR], adv[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) adk[r] = adv[r] = 0.f;
  for (int hh = 0; hh < s.group; ++hh) {
    const int h = g * s.group + hh;
    for (int t0 = qlo; t0 < qhi; t0 += 64) {
      const int t = t0 + lane;
      const bool in = t < qhi;
      const int tc = min(t, qhi - 1);  // lanes past qhi re-read the last row
      const int64_t row = ((static_cast<int64_t>(b) * s.q_len + tc) * s.h_q + h) * D;
      const int64_t st = (static_cast<int64_t>(b) * s.h_q + h) * s.q_len + tc;
      const float lse_r = lse[st], delta_r = rowstat[2 * st + 1];
      // Q and dO of the lane's row: the score and dP dots; columns 0-63
      // stay for the dS Q and P dO sums (wider rows reload them).
      float qx[64], ox[64];
      float sdot = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < NR; ++c) {
        load_cols64(q + row, 64 * c, D, qx);
        load_cols64(d_o + row, 64 * c, D, ox);
        sdot = dot_cols64(sk[wave], qx, 64 * c, D, sdot);
        dp = dot_cols64(sv[wave], ox, 64 * c, D, dp);
      }
      float p = 0.f, ds = 0.f;
      if (in) {
        p = expf(s.scale * sdot - lse_r);
        if (s.drop.thr != 0) {  // P * Z * c multiplies dO; the gradient reaching P is dP * Z * c
          const float z = keep_one(s.drop, static_cast<uint32_t>(s.row_offset + t), jpos,
                                   static_cast<uint32_t>(b * s.h_q + h));
          ds = p * (dp * z - delta_r);
          p *= z;
        } else {
          ds = p * (dp - delta_r);
        }
      }
#pragma unroll
      for (int c = 0; c < NR; ++c) {
        if (NR > 1) {
          load_cols64(q + row, 64 * c, D, qx);
          load_cols64(d_o + row, 64 * c, D, ox);
        }
        float x[64];
#pragma unroll
        for (int i = 0; i < 64; ++i) x[i] = p * ox[i];
        adv[c] += lane_sum64(x, lane);
#pragma unroll
        for (int i = 0; i < 64; ++i) x[i] = ds * qx[i];
        adk[c] += lane_sum64(x, lane);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int d = lane + 64 * r;
    if (d < D) {
      Elem<T>::store(dk + krow + d, adk[r] * s.scale);
      Elem<T>::store(dv + krow + d, adv[r]);
    }
  }
}

// Row statistics of the backward for every (b, local row, query head):
// delta = sum_d dO * O in float32, stored beside lse * log2(e) (the form the
// matrix-core kernels exponentiate with) as one 8-byte pair.  A group of lpr
// lanes (a power of two >= head_dim / 8) handles one row with 16-byte
// accesses, so consecutive lanes touch consecutive memory.
template <typename T>
__global__ __launch_bounds__(256) void bwd_prep_kernel(AttnShape s, const T* __restrict__ o,
                                                       const T* __restrict__ d_o,
                                                       const float* __restrict__ lse,
                                                       float* __restrict__ rowstat, int lpr) {
  const int64_t gtid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t idx = gtid / lpr;  // row (b, t, h), h fastest
  const int sub = static_cast<int>(gtid % lpr);
  const int64_t total = static_cast<int64_t>(s.batch) * s.q_len * s.h_q;
  const int D = s.head_dim;
  const bool in = idx < total && sub * 8 < D;
  float acc = 0.f;
  if (in) {
    float x[8], y[8];
    load8(o + idx * D + sub * 8, x);
    load8(d_o + idx * D + sub * 8, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(x[e], y[e], acc);
  }
  for (int off = lpr >> 1; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (sub == 0 && idx < total) {
    const int h = static_cast<int>(idx % s.h_q);
    const int64_t bt = idx / s.h_q;
    const int t = static_cast<int>(bt % s.q_len);
    const int b = static_cast<int>(bt / s.q_len);
    const int64_t st = (static_cast<int64_t>(b) * s.h_q + h) * s.q_len + t;
    *reinterpret_cast<float2*>(rowstat + 2 * st) = make_float2(lse[st] * kLog2e, acc);
  }
}

int lanes_per_row(int head_dim) {
  int l = 1;
  while (l < head_dim / 8) l <<= 1;
  return l;
}

AttnShape make_shape(int batch, int seq_len, int row_offset, int q_len, int kv_begin, int kv_len, int h_q,
                     int h_kv, int head_dim, float scale) {
  AttnShape s;
  s.batch = batch; s.seq_len = seq_len; s.row_offset = row_offset; s.q_len = q_len;
  s.h_q = h_q; s.h_kv = h_kv; s.head_dim = head_dim; s.group = h_q / h_kv; s.scale = scale;
  s.kv_begin = kv_begin; s.kv_len = kv_len;
  s.drop = drop_params(0, 1.f, 0, 0);
  return s;
}

unsigned blocks_for(int64_t waves) { return static_cast<unsigned>((waves + kWaves - 1) / kWaves); }

template <typename T, int NR>
hipError_t fwd_generic_t(const FwdArgs& a, hipStream_t st) {
  AttnShape s = make_shape(a.batch, a.seq_len, a.row_offset, a.q_len, a.kv_begin, a.kv_len, a.h_q, a.h_kv, a.head_dim,
                           a.scale);
  s.drop = drop_params(a.drop.thr, a.drop.scale, a.drop.seed, a.drop.offset);
  MetaView m = meta_view(a.meta, a.batch, a.seq_len, a.q_len);
  const int64_t waves = static_cast<int64_t>(a.batch) * a.q_len * a.h_q;
  hipError_t e = mark(a.mark_start, st);
  if (e != hipSuccess) return e;
  fwd_generic_kernel<T, NR><<<blocks_for(waves), 256, 0, st>>>(
      s, static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v), m,
      static_cast<T*>(a.o), a.lse);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return mark(a.mark_stop, st);
}

template <typename T, int NR>
hipError_t bwd_generic_t(const BwdArgs& a, hipStream_t st) {
  AttnShape s = make_shape(a.batch, a.seq_len, a.row_offset, a.q_len, a.kv_begin, a.kv_len, a.h_q, a.h_kv, a.head_dim,
                           a.scale);
  s.drop = drop_params(a.drop.thr, a.drop.scale, a.drop.seed, a.drop.offset);
  MetaView m = meta_view(a.meta, a.batch, a.seq_len, a.q_len);
  const int64_t rows = static_cast<int64_t>(a.batch) * a.q_len * a.h_q;
  const int lpr = lanes_per_row(a.head_dim);
  bwd_prep_kernel<T><<<static_cast<unsigned>((rows * lpr + 255) / 256), 256, 0, st>>>(
      s, static_cast<const T*>(a.o), static_cast<const T*>(a.d_o), a.lse, a.rowstat, lpr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dq_generic_kernel<T, NR><<<blocks_for(rows), 256, 0, st>>>(
      s, static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
      static_cast<const T*>(a.d_o), a.lse, a.rowstat, m, static_cast<T*>(a.dq));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t keys = static_cast<int64_t>(a.batch) * a.kv_len * a.h_kv;
  e = mark(a.mark_start, st);
  if (e != hipSuccess) return e;
  dkv_generic_kernel<T, NR><<<blocks_for(keys), 256, 0, st>>>(
      s, static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
      static_cast<const T*>(a.d_o), a.lse, a.rowstat, m, static_cast<T*>(a.dk),
      static_cast<T*>(a.dv));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return mark(a.mark_stop, st);
}

template <typename T>
hipError_t fwd_generic_d(const FwdArgs& a, hipStream_t st) {
  if (a.head_dim <= 64) return fwd_generic_t<T, 1>(a, st);
  if (a.head_dim <= 128) return fwd_generic_t<T, 2>(a, st);
  return fwd_generic_t<T, 4>(a, st);
}
template <typename T>
hipError_t bwd_generic_d(const BwdArgs& a, hipStream_t st) {
  if (a.head_dim <= 64) return bwd_generic_t<T, 1>(a, st);
  if (a.head_dim <= 128) return bwd_generic_t<T, 2>(a, st);
  return bwd_generic_t<T, 4>(a, st);
}

}  // namespace

hipError_t launch_fwd_generic(const FwdArgs& a, hipStream_t st) {
  return a.dtype == 0 ? fwd_generic_d<float>(a, st) : fwd_generic_d<uint16_t>(a, st);
}

hipError_t launch_bwd_generic(const BwdArgs& a, hipStream_t st) {
  return a.dtype == 0 ? bwd_generic_d<float>(a, st) : bwd_generic_d<uint16_t>(a, st);
}

__global__ __launch_bounds__(256) void zero_u16_kernel(uint16_t* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_u16(void* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  zero_u16_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), 256, 0, st>>>(static_cast<uint16_t*>(p), n);
  return hipGetLastError();
}

}  // namespace bd
