// bf16 matrix-core dK/dV kernel of the block-diagonal packed attention
// backward for head_dim 256 on gfx950 (key-stationary).
//
// Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences", Proof section (forward/backward parity, input gradients).  The
// same products as the head_dim 64 / 128 kernel (bwd_dkdv.h):
//   P_ij = exp(scale q_i.k_j - LSE_i), dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - delta_i),
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i.
//
// At 256 columns the dK^T and dV^T accumulators of one wave's 32 keys would
// take 256 registers and the Q / dO tiles of four heads 128 KB per stage, so
// the work is split differently from the narrower kernel: a workgroup owns
// 128 keys of one K/V head and one half of the columns of their dK and dV
// (two workgroups per key block, each computing S and dP in full), runs four
// waves of 32 keys, one wave per SIMD, and visits the heads of the GQA group
// one after another, so each wave's dK and dV columns are complete in its
// registers (no cross-head sum).  K of a wave's keys
// stays in registers (B operand of S = Q K^T), V of the workgroup's keys in
// LDS (B operand of dP = dO V^T).  One head's 32-row Q / dO tile and its row
// statistics are double-buffered in LDS (two stages of 32.25 KB) and loaded
// by direct global -> LDS loads one tile ahead, split over the four waves;
// the query tiles visited are those attending any of the workgroup's keys
// ([min key_qlo, max key_qhi) from the per-step metadata).  LDS tiles are
// unpadded rows with the 16-byte chunk c of row r at c ^ f(r) (the swizzle
// of the narrower kernels: a bank depends on the chunk index mod 16 only, for
// a 512-byte pitch as for 256).  Deterministic: every dK / dV row is written
// once by the wave that owns its key.
#include <limits.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace bd {
namespace {

constexpr int kD = 256;
constexpr int kKW = 32;              // keys per wave
constexpr int kWaves = 4;
constexpr int kKB = kKW * kWaves;    // keys per workgroup
constexpr int kQB = 32;              // query rows per tile
constexpr int kQP = kD * 2;          // row pitch (bytes)
constexpr int kTile = kQB * kQP;     // one Q or dO tile
constexpr int kStat = 2 * kQB * 4;   // (lse * log2(e), delta) per row
constexpr int kStage = 2 * kTile + kStat;
constexpr int kVt = kKB * kQP;       // V rows of the workgroup's keys
constexpr int kCH = 128;             // dK / dV columns per workgroup

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

template <int B>
struct Stage {
  static constexpr int value = B;
};

__device__ __forceinline__ bf16x8 lds_tr_pair(const char* p0, const char* p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p1));
  const auto ab = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, ab);
}

template <bool DROP>
__global__ __launch_bounds__(kWaves * 64, 1) void bwd_dkdv256_kernel(
    AttnShape s, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ rowstat, MetaView m, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int n_kt, int n_bg, int live_lo, int live_hi) {
  constexpr int KK = kD / 16;
  constexpr int DB = kCH / 32;  // 32-column blocks of this workgroup's dK / dV
  __shared__ __attribute__((aligned(16))) char stage0[kStage];
  __shared__ __attribute__((aligned(16))) char stage1[kStage];
  __shared__ __attribute__((aligned(16))) char vt[kVt];
  __shared__ int sRed[2 * kWaves];
  typedef __attribute__((address_space(3))) void lds_void;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, kg = lane >> 5;

  // Every key tile of one (batch row, K/V head) on one XCD (workgroups are
  // dispatched to the 8 XCDs round-robin by index), so their reads of the
  // same Q / dO tiles can hit that XCD's L2.
  const int xcd = static_cast<int>(blockIdx.x) & 7, slot2 = static_cast<int>(blockIdx.x) >> 3;
  const int ch = slot2 & 1, slot = slot2 >> 1;  // column half, key block
  const int bg = xcd + 8 * (slot / n_kt);
  const int kt = slot % n_kt;
  if (bg >= n_bg) return;  // whole workgroup: no barrier has been reached
  const int b = bg / s.h_kv, g = bg % s.h_kv;
  const int key0 = s.kv_begin + kt * kKB;  // the workgroup's first key (row position)
  const int key = key0 + wave * kKW + n;  // this lane's key
  // key is a position in the row; K/V/dK/dV hold keys [kv_begin, kv_begin +
  // kv_len) of every row (key tiles are counted from kv_begin).
  const bool key_ok = key < s.kv_begin + s.kv_len;
  const int64_t kv_row = (static_cast<int64_t>(b) * s.kv_len + (key - s.kv_begin)) * s.h_kv + g;
  // Keys outside [live_lo, live_hi) (the positions any local row attends,
  // known on the host) are attended by no row: their columns of dK and dV
  // are zero, written before any load (the same bits as the products' sums
  // of nothing; uniform over the workgroup, no barrier reached yet).
  if (key0 + kKB <= live_lo || key0 >= live_hi) {
    if (key_ok) {
      const uint2 z = make_uint2(0u, 0u);
      uint16_t* dkr = dk + kv_row * kD + ch * kCH + kg * 4;
      uint16_t* dvr = dv + kv_row * kD + ch * kCH + kg * 4;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          *reinterpret_cast<uint2*>(dkr + db * 32 + jq * 8) = z;
          *reinterpret_cast<uint2*>(dvr + db * 32 + jq * 8) = z;
        }
    }
    return;
  }

  int a0 = 0, a1 = 0;  // local rows attending this lane's key: [a0, a1) when a1 > a0
  if (key_ok) {
    const int64_t kidx = static_cast<int64_t>(b) * s.seq_len + key;
    a0 = m.key_qlo[kidx];
    a1 = m.key_qhi[kidx];
  }
  const int row_stride = s.h_q * kD;  // elements between consecutive rows

  // Direct loads of tile (head h, rows t0 .. t0+31) into stage buf.  Q and
  // dO are 16 loads of 64 lanes x 16 bytes each; wave w issues loads 4w ..
  // 4w+3 of both (tile rows 8w .. 8w+7), wave 0 also the 32 statistics
  // pairs.  Lane l of load J writes LDS chunk 64 J + l, i.e. position l % 32
  // of row 2 J + l / 32, so it fetches the global chunk that the swizzle puts
  // there.  Rows past the chunk read as zero (buffer bounds).
  auto issue_tile = [&](int h, int t0, int buf) {
    const int64_t tile0 = ((static_cast<int64_t>(b) * s.q_len + t0) * s.h_q + h) * kD;
    const int nbytes = ((s.q_len - t0) * row_stride - h * kD) * 2;
    char* hb = buf == 0 ? stage0 : stage1;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int r0 = 8 * wave + ln / 32;
    const int pos = ln % 32;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>((t == 0 ? q : d_o) + tile0), 0, nbytes, 0x00020000);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = r0 + 2 * j;
        const int voff = (r * row_stride + (pos ^ swz(r)) * 8) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(hb + t * kTile + (4 * wave + j) * 64 * 16), 16,
                                                 voff, 0, 0, 0);
      }
    }
    if (wave == 0) {
      const int64_t st0 = (static_cast<int64_t>(b) * s.h_q + h) * s.q_len + t0;
      const __amdgpu_buffer_rsrc_t rst = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(rowstat + 2 * st0), 0, (s.q_len - t0) * 8, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rst, (lds_void*)(hb + 2 * kTile), 4, lane * 4, 0, 0, 0);
    }
  };

  // The first tile (first head, first query tile attending the workgroup's
  // first key) is known before the metadata arrives; its loads go out with
  // the K / V / metadata loads and are reissued only if the metadata
  // disagrees.
  const int qt0e = max(key0 - s.row_offset, 0) / kQB;
  const bool early = qt0e * kQB < s.q_len;
  if (early) issue_tile(g * s.group, qt0e * kQB, 0);

  // K fragments of this wave's keys in registers, V rows in LDS; loads
  // without branches (keys past the row read the row's last key and are
  // zeroed where used).
  const int64_t kv_row_c = key_ok ? kv_row : (static_cast<int64_t>(b) * s.kv_len + s.kv_len - 1) * s.h_kv + g;
  bf16x8 kf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(k + kv_row_c * kD + kk * 16 + kg * 8);
  char* sV = vt + wave * kKW * kQP;
  {
    bf16x8 x[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) x[kk] = *reinterpret_cast<const bf16x8*>(v + kv_row_c * kD + kk * 16 + kg * 8);
    bf16x8 zero;
#pragma unroll
    for (int i = 0; i < 8; ++i) zero[i] = static_cast<__bf16>(0.f);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      *reinterpret_cast<bf16x8*>(sV + n * kQP + (((2 * kk + kg) ^ swz(n)) << 4)) = key_ok ? x[kk] : zero;
  }
  // Rows attending this lane's key [qlo_k, qhi_k); the wave's and the
  // workgroup's unions; rows inside every key's interval of this wave.
  const int qlo_k = a1 > a0 ? a0 : INT_MAX, qhi_k = a1 > a0 ? a1 : INT_MIN;
  const int wqlo = wave_min_i(qlo_k), wqhi = wave_max_i(qhi_k);
  const int kq_lo_max = wave_max_i(qlo_k), kq_hi_min = wave_min_i(qhi_k);
  int kq_lo_v = kq_lo_max, kq_hi_v = kq_hi_min;
  asm volatile("" : "+v"(kq_lo_v), "+v"(kq_hi_v));
  // Element mask: row t is allowed iff (unsigned)(t - mask_lo) < mask_span.
  const int mask_lo = qhi_k > qlo_k ? qlo_k : 0;
  const unsigned mask_span = qhi_k > qlo_k ? static_cast<unsigned>(qhi_k - qlo_k) : 0u;
  if (lane == 0) {
    sRed[wave] = wqlo;
    sRed[kWaves + wave] = wqhi;
  }
  __builtin_amdgcn_s_waitcnt(0);  // the early tile's loads and the V stores
  __syncthreads();
  int gqlo = INT_MAX, gqhi = INT_MIN;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    gqlo = min(gqlo, sRed[w]);
    gqhi = max(gqhi, sRed[kWaves + w]);
  }
  if (!key_ok) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i) kf[kk][i] = static_cast<__bf16>(0.f);
  }
  const int n_q = gqhi > gqlo ? (gqhi - 1) / kQB - gqlo / kQB + 1 : 0;
  const int qt0 = n_q > 0 ? gqlo / kQB : 0;
  const int n_it = n_q * s.group;  // iteration it: head g*group + it / n_q, tile qt0 + it % n_q
  auto issue_loads = [&](int it, int buf) {
    issue_tile(g * s.group + it / n_q, (qt0 + it % n_q) * kQB, buf);
  };

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) dkacc[db][j] = dvacc[db][j] = 0.f;

  const float c = s.scale * kLog2e;
  const int tr_row = 4 * kg + ((lane & 15) >> 2);  // transpose-load row within a group of 8
  const int tr_g = (lane >> 4) & 1;                // 16-column half of a transpose load
  const int tr_s = lane & 3;                       // 4-column quarter
  if (n_it > 0 && (!early || qt0 != qt0e)) {
    issue_loads(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // One barrier per iteration: the loads of tile it+1 go into the other
  // stage, which every wave last read before the previous barrier.  The loop
  // is unrolled by two so that the stage is a compile-time constant.
  auto step = [&](int it, auto stage) {
    constexpr int buf = decltype(stage)::value;
    const int t0 = (qt0 + it % n_q) * kQB;
    const char* sQ = buf == 0 ? stage0 : stage1;
    const char* sdO = sQ + kTile;
    const float* sStat = reinterpret_cast<const float*>(sQ + 2 * kTile);  // (lse2, delta) pairs
    // (An empty asm on the K fragments before the loads: the compiler's wait
    // bookkeeping otherwise keeps them pending from their global loads.)
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(kf[kk]));
    if (it + 1 < n_it) issue_loads(it + 1, buf ^ 1);

    // S = Q K^T and dP = dO V^T; sacc[j] = S[row t0 + (j/4)*8 + kg*4 + j%4][key n].
    f32x16 sacc, pacc;
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[j] = pacc[j] = 0.f;
    {
      // Row reads two k-steps ahead of their products; the scheduling
      // barriers keep the compiler from hoisting all of them (which would
      // need 192 registers).
      const int nat_row = n * kQP;
      const int nat_swz = swz(n);
      constexpr int PF = 2;
      bf16x8 aq[KK], ao[KK], bv[KK];
      auto rd = [&](int kk) {
        const int pos = nat_row + (((2 * kk + kg) ^ nat_swz) << 4);
        aq[kk] = *reinterpret_cast<const bf16x8*>(sQ + pos);
        ao[kk] = *reinterpret_cast<const bf16x8*>(sdO + pos);
        bv[kk] = *reinterpret_cast<const bf16x8*>(sV + pos);
      };
#pragma unroll
      for (int kk = 0; kk < PF; ++kk) rd(kk);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + PF < KK) rd(kk + PF);
        __builtin_amdgcn_sched_barrier(0);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[kk], kf[kk], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao[kk], bv[kk], pacc, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // P (zero outside the mask, which also covers padding rows, rows past
    // the chunk and keys no row of this tile attends), dS, then dV^T += dO^T P
    // and dK^T += Q^T dS; tiles inside every key's row interval skip the mask.
    auto finish = [&](auto masked) {
      float pv[16], dsv[16];
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int r0 = jq * 8 + kg * 4;
        const f32x4 st01 = *reinterpret_cast<const f32x4*>(sStat + 2 * r0);
        const f32x4 st23 = *reinterpret_cast<const f32x4*>(sStat + 2 * r0 + 4);
        const float lsv[4] = {st01[0], st01[2], st23[0], st23[2]};
        const float dev[4] = {st01[1], st01[3], st23[1], st23[3]};
        // With dropout: the weights that multiply dO are P * Z * c, and the
        // gradient reaching P is dP = (dO V^T) * Z * c.
        float zf[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (DROP)
          keep_factors_col(s.drop, static_cast<uint32_t>(s.row_offset + t0 + r0), static_cast<uint32_t>(key),
                           static_cast<uint32_t>(b * s.h_q + g * s.group + it / n_q), zf);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jq * 4 + e;
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[j], c, -lsv[e]));
          if constexpr (decltype(masked)::value) {
            const unsigned rel = static_cast<unsigned>(t0 + r0 + e - mask_lo);
            p = rel < mask_span ? p : 0.f;  // a select: also clears inf on padding rows
          }
          pv[j] = DROP ? p * zf[e] : p;
          dsv[j] = DROP ? p * (pacc[j] * zf[e] - dev[e]) : p * (pacc[j] - dev[e]);
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
      // Transpose reads one (k-step, column block) ahead of their products.
      constexpr int NT = 2 * DB, PFT = 1;
      auto tread = [&](int st_, const char* base) {
        const int kk2 = st_ / DB, db = ch * DB + st_ % DB;  // column block of Q^T / dO^T
        const int r_a = 16 * kk2 + tr_row, r_b = r_a + 8;
        const int chunk = 4 * db + 2 * tr_g + (tr_s >> 1);
        const int half = (tr_s & 1) * 8;
        const int pa = r_a * kQP + ((chunk ^ swz(r_a)) << 4) + half;
        const int pb_ = r_b * kQP + ((chunk ^ swz(r_b)) << 4) + half;
        return lds_tr_pair(base + pa, base + pb_);
      };
      bf16x8 tdo[NT], tq[NT];
#pragma unroll
      for (int st_ = 0; st_ < PFT; ++st_) {
        tdo[st_] = tread(st_, sdO);
        tq[st_] = tread(st_, sQ);
      }
#pragma unroll
      for (int st_ = 0; st_ < NT; ++st_) {
        if (st_ + PFT < NT) {
          tdo[st_ + PFT] = tread(st_ + PFT, sdO);
          tq[st_ + PFT] = tread(st_ + PFT, sQ);
        }
        __builtin_amdgcn_sched_barrier(0);
        dvacc[st_ % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tdo[st_], pb[st_ / DB], dvacc[st_ % DB], 0, 0, 0);
        dkacc[st_ % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[st_], dsb[st_ / DB], dkacc[st_ % DB], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (t0 >= kq_lo_v && t0 + kQB <= kq_hi_v)
      finish(Stage<0>{});
    else
      finish(Stage<1>{});
    __builtin_amdgcn_s_waitcnt(0);  // direct loads of tile it+1 have landed in LDS
    __syncthreads();                // next stage ready; this one free
  };
  for (int it = 0; it < n_it; it += 2) {
    step(it, Stage<0>{});
    if (it + 1 < n_it) step(it + 1, Stage<1>{});
  }

  // dkacc[db][j] = dK^T[d = ch*128 + 32db + (j/4)*8 + kg*4 + j%4][key n] (unscaled)
  if (key_ok) {
    uint16_t* dkr = dk + kv_row * kD + ch * kCH + kg * 4;
    uint16_t* dvr = dv + kv_row * kD + ch * kCH + kg * 4;
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

}  // namespace

template <bool DROP>
hipError_t dkdv256_t(const BwdArgs& a, hipStream_t st) {
  AttnShape s;
  s.batch = a.batch; s.seq_len = a.seq_len; s.row_offset = a.row_offset; s.q_len = a.q_len;
  s.h_q = a.h_q; s.h_kv = a.h_kv; s.head_dim = kD; s.group = a.h_q / a.h_kv; s.scale = a.scale;
  s.kv_begin = a.kv_begin; s.kv_len = a.kv_len;
  s.drop = drop_params(a.drop.thr, a.drop.scale, a.drop.seed, a.drop.offset);
  MetaView m = meta_view(a.meta, a.batch, a.seq_len, a.q_len);
  const int n_kt = (a.kv_len + kKB - 1) / kKB;
  const int n_bg = a.batch * a.h_kv;
  const int64_t grid = 8 * static_cast<int64_t>((n_bg + 7) / 8) * n_kt * (kD / kCH);
  if (n_kt == 0) return hipSuccess;
  hipError_t e = mark(a.mark_start, st);
  if (e != hipSuccess) return e;
  bwd_dkdv256_kernel<DROP><<<dim3(static_cast<unsigned>(grid)), kWaves * 64, 0, st>>>(
      s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
      static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.d_o), a.rowstat, m,
      static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), n_kt, n_bg, a.live_lo, a.live_hi);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return mark(a.mark_stop, st);
}

hipError_t launch_bwd_dkdv256(const BwdArgs& a, hipStream_t st) {
  return a.drop.thr != 0 ? dkdv256_t<true>(a, st) : dkdv256_t<false>(a, st);
}

}  // namespace bd
