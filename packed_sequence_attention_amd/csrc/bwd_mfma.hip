// bf16 matrix-core backward of block-diagonal packed attention for gfx950.
//
// Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences", Proof section (forward/backward parity, input gradients) and
// Design overview, exchange.py (the chunk's K/V gradients are partial sums
// over its rows, summed over ranks).  The gradients of softmax attention:
//   P_ij  = exp(scale q_i.k_j - LSE_i)          (LSE saved by the forward)
//   dP_ij = dO_i . v_j,   delta_i = dO_i . O_i  (= sum_j P_ij dP_ij)
//   dS_ij = P_ij (dP_ij - delta_i)
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i,  dQ_i = scale sum_j dS_ij k_j
//
// Work decomposition: a workgroup owns 128 keys (4 waves x 32) of one K/V
// head of one batch row and sweeps the group's query heads and the 32-row
// query tiles that attend any of its keys ([min key_qlo, max key_qhi) from
// the per-step metadata).  Per query tile each wave computes, for its 32
// keys (v_mfma_f32_32x32x16_bf16, lane l: key l % 32):
//   S = Q K^T and dP = dO V^T   (A = Q / dO rows from LDS, B = K / V in registers)
//   dV^T += dO^T P, dK^T += Q^T dS  (A = dO^T / Q^T via the LDS transpose
//                                    load, B = P / dS from the accumulators)
// dS^T is written to LDS; then the tile's dQ (32 rows x head_dim) is computed
// over all 128 keys (A = dS via transpose load, B = K via transpose load) and
// added to a float32 accumulator with float32 atomics; a final kernel scales
// and rounds it.  dK and dV stay in registers until the end and are written
// once (deterministic).  Elements outside the block-causal mask are zeroed
// only on tiles that are not entirely allowed; waves whose keys no row of
// the tile attends skip the tile.
#include <limits.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace bd {
namespace {

constexpr int kKB = 128;  // keys per workgroup
constexpr int kQB = 32;   // query rows per tile

template <int D>
struct BwdLds {
  static constexpr int KP = D * 2 + 64;  // K tile, read by transpose loads
  static constexpr int QP = D * 2 + 32;  // Q / dO tiles, read both ways
  static constexpr int SP = kQB * 2;     // dS^T rows (keys) of 32 bf16
  static constexpr int off_q = kKB * KP;
  static constexpr int off_do = off_q + kQB * QP;
  static constexpr int off_ds = off_do + kQB * QP;
  static constexpr int off_stat = off_ds + kKB * SP;
  static constexpr int bytes = off_stat + 4 * kQB * 4 + 16 * 4;
};

__device__ __forceinline__ bf16x8 lds_tr_pair(const char* p0, int second_off) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + second_off));
  const auto ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

template <int D>
__global__ __launch_bounds__(256, 1) void bwd_mfma_kernel(
    AttnShape s, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o, const float* __restrict__ lse,
    const float* __restrict__ delta, MetaView m, float* __restrict__ dq_acc,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int n_kt) {
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int CH = D / 8;
  using L = BwdLds<D>;
  __shared__ __attribute__((aligned(16))) char smem[L::bytes];
  char* sK = smem;
  char* sQ = smem + L::off_q;
  char* sdO = smem + L::off_do;
  char* sdS = smem + L::off_ds;
  float* sLse = reinterpret_cast<float*>(smem + L::off_stat);
  float* sDel = sLse + kQB;
  int* sLo = reinterpret_cast<int*>(sDel + kQB);
  int* sHi = sLo + kQB;
  int* sRed = sHi + kQB;  // 16 ints of reduction scratch

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, kg = lane >> 5;

  const int kt = static_cast<int>(blockIdx.x) % n_kt;
  const int bg = static_cast<int>(blockIdx.x) / n_kt;
  const int b = bg / s.h_kv, g = bg % s.h_kv;
  const int k0 = kt * kKB;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + n;  // this lane's key (columns of S)
  const bool key_ok = key < s.seq_len;
  const int64_t kv_row = (static_cast<int64_t>(b) * s.seq_len + key) * s.h_kv + g;

  // K / V fragments of this wave's keys (B operands of S and dP).
  bf16x8 kf[KK], vf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    if (key_ok) {
      kf[kk] = *reinterpret_cast<const bf16x8*>(k + kv_row * D + kk * 16 + kg * 8);
      vf[kk] = *reinterpret_cast<const bf16x8*>(v + kv_row * D + kk * 16 + kg * 8);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) kf[kk][i] = vf[kk][i] = static_cast<__bf16>(0.f);
    }
  }
  // Stage the whole K tile for the dQ product.
  for (int ci = tid; ci < kKB * CH; ci += 256) {
    const int r = ci / CH, col = ci % CH;
    const int j = k0 + r;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (j < s.seq_len)
      x = *reinterpret_cast<const uint4*>(
          k + ((static_cast<int64_t>(b) * s.seq_len + j) * s.h_kv + g) * D + col * 8);
    *reinterpret_cast<uint4*>(sK + r * L::KP + col * 16) = x;
  }
  // Query rows attending this wave's keys and the workgroup's keys.
  int qlo_k = INT_MAX, qhi_k = 0;
  if (key_ok) {
    const int64_t kidx = static_cast<int64_t>(b) * s.seq_len + key;
    const int a0 = m.key_qlo[kidx], a1 = m.key_qhi[kidx];
    if (a1 > a0) {
      qlo_k = a0;
      qhi_k = a1;
    }
  }
  const int wqlo = wave_min_i(qlo_k), wqhi = wave_max_i(qhi_k);
  if (lane == 0) {
    sRed[wave] = wqlo;
    sRed[4 + wave] = wqhi;
  }
  __syncthreads();
  const int gqlo = min(min(sRed[0], sRed[1]), min(sRed[2], sRed[3]));
  const int gqhi = max(max(sRed[4], sRed[5]), max(sRed[6], sRed[7]));

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) dkacc[db][j] = dvacc[db][j] = 0.f;

  const float c = s.scale * kLog2e;
  // Per-lane LDS offsets.
  const int nat_rd = n * L::QP + kg * 16;                       // natural 16-byte row reads
  const int tr_row = 4 * kg + ((lane & 15) >> 2);               // transpose-load row within 8
  const int tr_col = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;  // byte column
  // dQ split: wave -> (d block, key part).
  constexpr int DQ_PARTS = 4 / DB;            // key parts per d block
  constexpr int DQ_KEYS = kKB / DQ_PARTS;     // keys per wave in the dQ product
  const int dq_db = wave % DB;
  const int dq_k0 = (wave / DB) * DQ_KEYS;

  if (gqhi > gqlo) {
    const int qt0 = gqlo / kQB, qt1 = (gqhi - 1) / kQB;
    for (int hh = 0; hh < s.group; ++hh) {
      const int h = g * s.group + hh;
      for (int qt = qt0; qt <= qt1; ++qt) {
        const int t0 = qt * kQB;
        __syncthreads();
        // Stage Q, dO rows and their statistics.
        for (int ci = tid; ci < kQB * CH; ci += 256) {
          const int r = ci / CH, col = ci % CH;
          const int t = t0 + r;
          uint4 xq = make_uint4(0, 0, 0, 0), xo = make_uint4(0, 0, 0, 0);
          if (t < s.q_len) {
            const int64_t off = ((static_cast<int64_t>(b) * s.q_len + t) * s.h_q + h) * D + col * 8;
            xq = *reinterpret_cast<const uint4*>(q + off);
            xo = *reinterpret_cast<const uint4*>(d_o + off);
          }
          *reinterpret_cast<uint4*>(sQ + r * L::QP + col * 16) = xq;
          *reinterpret_cast<uint4*>(sdO + r * L::QP + col * 16) = xo;
        }
        if (tid < kQB) {
          const int t = t0 + tid;
          float ls = 0.f, de = 0.f;
          int lo = 0, hi = 0;
          if (t < s.q_len) {
            const int64_t bt = static_cast<int64_t>(b) * s.q_len + t;
            lo = m.row_lo[bt];
            hi = m.row_hi[bt];
            const int64_t st = (static_cast<int64_t>(b) * s.h_q + h) * s.q_len + t;
            if (hi > lo) {
              ls = lse[st] * kLog2e;
              de = delta[st];
            }
          }
          sLse[tid] = ls;
          sDel[tid] = de;
          sLo[tid] = lo;
          sHi[tid] = hi;
        }
        __syncthreads();
        const bool active = wqlo < t0 + kQB && wqhi > t0;
        char* dsrow = sdS + (wave * 32 + n) * L::SP + kg * 8;
        if (active) {
          // Is every (row, key) pair of this 32x32 block allowed?
          const int rlo = sLo[n], rhi = sHi[n];
          const bool rreal = rhi > rlo;
          const bool full = wave_min_i(rreal ? 1 : 0) == 1 && wave_max_i(rlo) <= kw0 &&
                            kw0 + 31 <= s.row_offset + t0;
          f32x16 sacc, pacc;
#pragma unroll
          for (int j = 0; j < 16; ++j) sacc[j] = pacc[j] = 0.f;
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQ + nat_rd + kk * 32);
            const bf16x8 ao = *reinterpret_cast<const bf16x8*>(sdO + nat_rd + kk * 32);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[kk], sacc, 0, 0, 0);
            pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vf[kk], pacc, 0, 0, 0);
          }
          // sacc[j] = S[row (j/4)*8 + kg*4 + j%4][key n]
          float pv[16], dsv[16];
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const int r0 = jq * 8 + kg * 4;
            const float4 ls4 = *reinterpret_cast<const float4*>(sLse + r0);
            const float4 de4 = *reinterpret_cast<const float4*>(sDel + r0);
            const float lsv[4] = {ls4.x, ls4.y, ls4.z, ls4.w};
            const float dev[4] = {de4.x, de4.y, de4.z, de4.w};
            int4 lo4 = make_int4(0, 0, 0, 0), hi4 = make_int4(0, 0, 0, 0);
            if (!full) {
              lo4 = *reinterpret_cast<const int4*>(sLo + r0);
              hi4 = *reinterpret_cast<const int4*>(sHi + r0);
            }
            const int lov[4] = {lo4.x, lo4.y, lo4.z, lo4.w};
            const int hiv[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int j = jq * 4 + e;
              float p = __builtin_amdgcn_exp2f(fmaf(sacc[j], c, -lsv[e]));
              if (!full && (key < lov[e] || key >= hiv[e])) p = 0.f;
              pv[j] = p;
              dsv[j] = p * (pacc[j] - dev[e]);
            }
          }
          bf16x8 pb[2], dsb[2];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            pb[0][i] = static_cast<__bf16>(pv[i]);
            pb[1][i] = static_cast<__bf16>(pv[8 + i]);
            dsb[0][i] = static_cast<__bf16>(dsv[i]);
            dsb[1][i] = static_cast<__bf16>(dsv[8 + i]);
          }
          // dV^T += dO^T P, dK^T += Q^T dS (k = query rows, accumulator order).
#pragma unroll
          for (int kk2 = 0; kk2 < 2; ++kk2) {
            const int rowb = (16 * kk2 + tr_row) * L::QP + tr_col;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const bf16x8 a_do = lds_tr_pair(sdO + rowb + db * 64, 8 * L::QP);
              const bf16x8 a_q = lds_tr_pair(sQ + rowb + db * 64, 8 * L::QP);
              dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_do, pb[kk2], dvacc[db], 0, 0, 0);
              dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_q, dsb[kk2], dkacc[db], 0, 0, 0);
            }
          }
          // dS^T rows (this lane's key), 4 consecutive query rows per store.
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            uint2 pk;
            pk.x = pack_bf16x2(dsv[4 * jq], dsv[4 * jq + 1]);
            pk.y = pack_bf16x2(dsv[4 * jq + 2], dsv[4 * jq + 3]);
            *reinterpret_cast<uint2*>(dsrow + jq * 16) = pk;
          }
        } else {
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) *reinterpret_cast<uint2*>(dsrow + jq * 16) = make_uint2(0, 0);
        }
        __syncthreads();
        // dQ tile part: rows t0..t0+31, d block dq_db, keys dq_k0 .. +DQ_KEYS.
        {
          f32x16 qacc;
#pragma unroll
          for (int j = 0; j < 16; ++j) qacc[j] = 0.f;
#pragma unroll
          for (int ks = 0; ks < DQ_KEYS / 16; ++ks) {
            const int krow = dq_k0 + ks * 16 + tr_row;
            const bf16x8 a_ds = lds_tr_pair(sdS + krow * L::SP + tr_col, 8 * L::SP);
            const bf16x8 b_k = lds_tr_pair(sK + krow * L::KP + tr_col + dq_db * 64, 8 * L::KP);
            qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_ds, b_k, qacc, 0, 0, 0);
          }
          // qacc[j] = dQ[row (j/4)*8 + kg*4 + j%4][d = 32*dq_db + n]
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int t = t0 + (j >> 2) * 8 + kg * 4 + (j & 3);
            if (t < s.q_len) {
              float* dst = dq_acc + ((static_cast<int64_t>(b) * s.q_len + t) * s.h_q + h) * D +
                           dq_db * 32 + n;
              __hip_atomic_fetch_add(dst, qacc[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    }
  }
  // dK, dV of this lane's key: dvacc[db][j] = dV^T[d = 32db + (j/4)*8 + kg*4 + j%4][key n]
  if (key_ok) {
    uint16_t* dkr = dk + kv_row * D + kg * 4;
    uint16_t* dvr = dv + kv_row * D + kg * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        uint2 a, bb;
        a.x = pack_bf16x2(dkacc[db][4 * jq] * s.scale, dkacc[db][4 * jq + 1] * s.scale);
        a.y = pack_bf16x2(dkacc[db][4 * jq + 2] * s.scale, dkacc[db][4 * jq + 3] * s.scale);
        bb.x = pack_bf16x2(dvacc[db][4 * jq], dvacc[db][4 * jq + 1]);
        bb.y = pack_bf16x2(dvacc[db][4 * jq + 2], dvacc[db][4 * jq + 3]);
        *reinterpret_cast<uint2*>(dkr + db * 32 + jq * 8) = a;
        *reinterpret_cast<uint2*>(dvr + db * 32 + jq * 8) = bb;
      }
  }
}

// dQ = bf16(scale * dq_acc), 8 elements per thread.
__global__ __launch_bounds__(256) void dq_finalize_kernel(const float* __restrict__ acc,
                                                          uint16_t* __restrict__ dq, int64_t n8,
                                                          float scale) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(acc)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(acc)[2 * i + 1];
  uint4 r;
  r.x = pack_bf16x2(a.x * scale, a.y * scale);
  r.y = pack_bf16x2(a.z * scale, a.w * scale);
  r.z = pack_bf16x2(b.x * scale, b.y * scale);
  r.w = pack_bf16x2(b.z * scale, b.w * scale);
  reinterpret_cast<uint4*>(dq)[i] = r;
}

template <int D>
hipError_t bwd_mfma_t(const BwdArgs& a, hipStream_t st) {
  AttnShape s;
  s.batch = a.batch; s.seq_len = a.seq_len; s.row_offset = a.row_offset; s.q_len = a.q_len;
  s.h_q = a.h_q; s.h_kv = a.h_kv; s.head_dim = D; s.group = a.h_q / a.h_kv; s.scale = a.scale;
  MetaView m = meta_view(a.meta, a.batch, a.seq_len, a.q_len);
  hipError_t e = launch_bwd_prep(a, st);
  if (e != hipSuccess) return e;
  const int n_kt = (a.seq_len + kKB - 1) / kKB;
  const int64_t grid = static_cast<int64_t>(n_kt) * a.batch * a.h_kv;
  if (grid > 0) {
    e = mark(a.mark_start, st);
    if (e != hipSuccess) return e;
    bwd_mfma_kernel<D><<<dim3(static_cast<unsigned>(grid)), 256, 0, st>>>(
        s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
        static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.d_o), a.lse, a.delta, m,
        a.dq_acc, static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), n_kt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = mark(a.mark_stop, st);
    if (e != hipSuccess) return e;
  }
  const int64_t n8 = static_cast<int64_t>(a.batch) * a.q_len * a.h_q * D / 8;
  if (n8 > 0) {
    dq_finalize_kernel<<<dim3(static_cast<unsigned>((n8 + 255) / 256)), 256, 0, st>>>(
        a.dq_acc, static_cast<uint16_t*>(a.dq), n8, a.scale);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t st) {
  return a.head_dim == 64 ? bwd_mfma_t<64>(a, st) : bwd_mfma_t<128>(a, st);
}

}  // namespace bd
