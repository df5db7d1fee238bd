// bf16 matrix-core dQ kernel of the block-diagonal packed attention backward
// for gfx950 (query-stationary).
//
// Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences", Proof section (input gradients).  The kernel also produces the
// row statistics (lse * log2(e), delta_i = dO_i . O_i) that the dK/dV kernel
// reads.  For each local row i:
//   P_ij  = exp(scale q_i.k_j - LSE_i),  dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - delta_i),      dQ_i = scale sum_j dS_ij k_j
// over the keys j of row i's document up to i.
//
// Work decomposition mirrors the forward: a workgroup is (batch row, 4 query
// heads sharing one K/V head, 32 local rows); wave w owns head 4*hg + w for
// those rows and keeps its Q and dO rows (B operands), LSE, delta and the
// dQ^T accumulator in registers (at head_dim 256 these take 256 registers:
// one workgroup per CU, one wave per SIMD).  Key tiles of 64 (32 at head_dim
// 256) are streamed through an LDS double buffer with direct global -> LDS
// loads (buffer form: keys past the row read as zero); the tiles from the
// workgroup's last row down to doc_start(first row) are visited in
// descending order (the first one is known before the metadata arrives) and
// the mask is applied only on tiles not entirely allowed.  Per 32-key block (v_mfma_f32_32x32x16_bf16, lane l: query row l % 32):
//   S^T  = K Q^T    (A = K rows from LDS, B = Q in registers)
//   dP^T = V dO^T   (A = V rows from LDS, B = dO in registers)
//   dS^T = P^T (dP^T - delta) in the accumulator layout, rounded to bf16
//   dQ^T += K^T dS^T  (A = K^T with the LDS transpose load, B = dS^T)
// K / V tiles are stored without padding with the 16-byte chunk c of row r
// at chunk c ^ f(r); f makes both the row reads (16 rows, one chunk) and the
// transpose reads (4 rows x 4 chunks) free of bank conflicts.  No atomics:
// dQ is written once, deterministically.
#include <limits.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace bd {
namespace {

constexpr int kBM = 32;  // query rows per workgroup
static_assert(kBM == kOrderQB, "the metadata's query-tile order is built for this tile size");
// Keys per tile: 64, or 32 at head_dim 256 (two 32 KB stages).
template <int D>
constexpr int kBNd = D == 256 ? 32 : 64;
constexpr int kBNmax = 64;
// Workgroups per CU: two, or one at head_dim 256 (its dQ^T accumulators, Q
// and dO fragments alone take 256 registers; one wave per SIMD may use 512).
template <int D>
constexpr int kDqOcc = D == 256 ? 1 : 2;

template <int D>
struct DqLds {
  static constexpr int RP = D * 2;                  // row pitch (bytes), swizzled chunks
  static constexpr int tile = 2 * kBNd<D> * RP;     // K tile then V tile (one stage)
  static constexpr int NCH = kBNd<D> * (D / 8) / 256;  // direct loads per thread per tensor
};

template <int D>
__device__ __forceinline__ int rswz(int r) {
  if constexpr (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

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

template <int D, bool DROP>
__global__ __launch_bounds__(256, kDqOcc<D>) void bwd_dq_kernel(
    AttnShape s, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o, const uint16_t* __restrict__ o,
    const float* __restrict__ lse, float* __restrict__ rowstat, MetaView m, uint16_t* __restrict__ dq,
    int n_qtg, int n_hg, int slots, int hpw) {
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int kBN = kBNd<D>;
  constexpr int CH = D / 8;
  using L = DqLds<D>;
  constexpr int RP = L::RP;
  // The two stages are separate LDS objects: the compiler then knows that
  // the direct loads into one stage do not alias reads of the other, and
  // does not make those reads wait for the loads in flight.
  __shared__ __attribute__((aligned(16))) char stage0[L::tile];
  __shared__ __attribute__((aligned(16))) char stage1[L::tile];
  typedef __attribute__((address_space(3))) void lds_void;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, kg = lane >> 5;

  // Work of the workgroup: hpw query heads of one K/V head times
  // tpw = 4 / hpw consecutive 32-row query tiles (hpw = 4 when the GQA group
  // has a multiple of 4 heads, 2 for a multiple of 2, else 1): wave w takes
  // head hg * hpw + w % hpw and tile qtg * tpw + w / hpw.  The four share
  // every K/V tile staged in LDS and visit the union of their key ranges (a
  // tile outside a wave's own range is fully masked for it and adds exact
  // zeros, so a row's result does not depend on its neighbours).
  // Launch order: the last query tiles of the chunk first (neighbouring
  // workgroups share K/V tiles); when the metadata's statistics say the
  // longest tile is long against a slot's share of the work (order_pays),
  // the tiles with the most key tiles to visit first instead (the order the
  // metadata build sorted; built for single 32-row tiles, so only used when
  // tpw = 1).  All n_hg head groups of a tile group are adjacent.
  const int tpw = 4 / hpw;
  int qtg, b;
  const int hg = static_cast<int>(blockIdx.x) % n_hg;
  bool sorted = false;
  int code = 0;
  if (m.q_order != nullptr) {
    code = __builtin_amdgcn_readfirstlane(m.q_order[static_cast<int>(blockIdx.x) / n_hg]);
    sorted = order_pays(__builtin_amdgcn_readfirstlane(m.q_stats[0]), __builtin_amdgcn_readfirstlane(m.q_stats[1]),
                        n_hg, slots);
  }
  if (sorted) {
    if (code < 0 || code >= s.batch * n_qtg) return;  // whole workgroup: no barrier has been reached
    b = code / n_qtg;
    qtg = code % n_qtg;
  } else {
    const int per_qt = s.batch * n_hg;
    qtg = n_qtg - 1 - static_cast<int>(blockIdx.x) / per_qt;
    b = (static_cast<int>(blockIdx.x) % per_qt) / n_hg;
  }
  const int qt = qtg * tpw + wave / hpw;
  const int h = hg * hpw + wave % hpw;
  const int g = (hg * hpw) / s.group;

  const int t = qt * kBM + n;
  const bool valid = t < s.q_len;
  const int64_t bt = static_cast<int64_t>(b) * s.q_len + t;
  const int64_t st = (static_cast<int64_t>(b) * s.h_q + h) * s.q_len + t;
  // Every prologue load is issued before any of them is used, without
  // branches (rows past the chunk read the chunk's last row and are zeroed
  // below), so they share one memory round trip.
  const int tc = valid ? t : s.q_len - 1;
  const int64_t btc = static_cast<int64_t>(b) * s.q_len + tc;
  const int64_t stc = (static_cast<int64_t>(b) * s.h_q + h) * s.q_len + tc;
  const int lo_l = m.row_lo[btc], hi_l = m.row_hi[btc];
  const float lse_l = lse[stc];
  bf16x8 qf[KK], of[KK], ov[KK];
  {
    const int64_t row = (btc * s.h_q + h) * D + kg * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      qf[kk] = *reinterpret_cast<const bf16x8*>(q + row + kk * 16);
      of[kk] = *reinterpret_cast<const bf16x8*>(d_o + row + kk * 16);
      ov[kk] = *reinterpret_cast<const bf16x8*>(o + row + kk * 16);
    }
  }
  // The K/V buffer holds keys [kv_begin, kv_begin + kv_len) of every row;
  // kv0 is its first key of (b, g).  Visited tiles start at or after
  // kv_begin (a multiple of 64), so a tile's offset from there is >= 0.
  const int64_t kv0 = (static_cast<int64_t>(b) * s.kv_len * s.h_kv + g) * D;
  const int kv_stride = s.h_kv * D;
  const int kv_bytes = (s.kv_len * kv_stride - g * D) * 2;
  // Direct load c (of 2 NCH: K and V chunks alternately) of key tile kt into
  // stage buf.  The loads of the next tile are spread over the first S/dP
  // block (one per step): issued together, a workgroup's loads queue up at
  // the address unit and stall the waves.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  // With live == false the load reads nothing (zero-sized resource) and
  // writes zeros into the free stage: the loop issues it unconditionally, as
  // a branch around it would split the S/dP block and stop the scheduler
  // from overlapping its LDS reads with the products.
  // Per-lane part of the offsets of load i (K and V tiles share it); the
  // tile's row offset goes into the resource base.
  int dma_off[L::NCH];
#pragma unroll
  for (int i = 0; i < L::NCH; ++i) {
    const int lc = i * 256 + wave_u * 64 + lane;  // LDS chunk written by this lane
    const int r = lc / CH, pc = lc % CH;
    dma_off[i] = (r * kv_stride + (pc ^ rswz<D>(r)) * 8) * 2;
  }
  auto issue_chunk = [&](int kt, int buf, int c, bool live) {
    char* sK = buf == 0 ? stage0 : stage1;
    char* dst = (c & 1) ? sK + kBN * RP : sK;
    const int i = c >> 1;
    const int tile_off = (kt * kBN - s.kv_begin) * kv_stride;  // elements from key kv_begin
    const int vo = dma_off[i];
    const int nbytes = live ? max(kv_bytes - tile_off * 2, 0) : 0;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(((c & 1) ? v : k) + kv0 + tile_off), 0, nbytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (i * 256 + wave_u * 64) * 16), 16,
                                             vo, 0, 0, 0);
  };
  constexpr int LSTEP = KK / (2 * L::NCH);
  static_assert(LSTEP * 2 * L::NCH == KK, "direct loads spread evenly over the first S/dP block");

  // Key tiles are visited from the last one (the tile's diagonal, known from
  // its position) down to the first document start, so the first tile's
  // loads go out with the prologue loads; a row's dQ depends only on the
  // tiles that are not fully masked for it, summed in descending order
  // whatever the chunk (fully masked tiles add exact zeros).
  const int kt1 = (s.row_offset + min((qtg + 1) * tpw * kBM - 1, s.q_len - 1)) / kBN;  // the workgroup's last row
#pragma unroll
  for (int c = 0; c < 2 * L::NCH; ++c) issue_chunk(kt1, 0, c, true);
  // Keep the metadata reductions below these loads, and the Q loads above
  // them (the compiler would otherwise move each load next to its use).
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qf[kk]));

  const int lo = valid ? lo_l : 0, hi = valid ? hi_l : 0;
  const float lse2 = valid ? lse_l * kLog2e : 0.f;  // -inf on padding rows
  const bool real = hi > lo;
  const int kmin = wave_min_i(real ? lo : INT_MAX);
  const int kmax = wave_max_i(real ? hi : 0);
  const int lomax = wave_max_i(real ? lo : 0);
  const bool all_real = wave_min_i(real ? 1 : 0) == 1;
  const int pfirst = s.row_offset + qt * kBM;
  // The key range the workgroup visits: the union over its waves (they
  // differ only when the waves take different query tiles).
  int kmin_g = kmin, kmax_g = kmax;
  if (tpw > 1) {
    __shared__ int s_rng[2][4];
    if (lane == 0) {
      s_rng[0][wave] = kmin;
      s_rng[1][wave] = kmax;
    }
    __syncthreads();
    kmin_g = __builtin_amdgcn_readfirstlane(min(min(s_rng[0][0], s_rng[0][1]), min(s_rng[0][2], s_rng[0][3])));
    kmax_g = __builtin_amdgcn_readfirstlane(max(max(s_rng[1][0], s_rng[1][1]), max(s_rng[1][2], s_rng[1][3])));
  }

  // Row statistic delta = dO . O (float32): this lane's half of the row, then
  // the partner lane's.  The (lse * log2(e), delta) pair is also written for
  // the dK/dV kernel, which runs after this one.
  float dlt = 0.f;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
#pragma unroll
    for (int i = 0; i < 8; ++i) dlt = fmaf(static_cast<float>(of[kk][i]), static_cast<float>(ov[kk][i]), dlt);
  if (!valid) {
    dlt = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i) qf[kk][i] = of[kk][i] = static_cast<__bf16>(0.f);
  }
  dlt = pair32_sum(dlt);
  if (valid && kg == 0) *reinterpret_cast<float2*>(rowstat + 2 * st) = make_float2(lse2, dlt);

  f32x16 dqacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) dqacc[db][j] = 0.f;
  const float c = s.scale * kLog2e;
  // Rows with no allowed key (padding, past the chunk) take +inf, so every
  // P of theirs is exp2(-inf) = 0 (with -inf from the rows' own LSE the
  // masked -inf - (-inf) would be NaN).
  const float lse2m = real ? lse2 : INFINITY;

  const int nat_swz = rswz<D>(n);
  const int tr_row = 4 * kg + ((lane & 15) >> 2);
  const int tr_g = (lane >> 4) & 1, tr_s = lane & 3;
  // Per-lane LDS offsets, one integer per read (the compiler keeps these live
  // across the loop; at head_dim 256 one per read pushed the Q / dO fragments
  // out of the vector registers).  The swizzle only permutes the low four
  // bits of the chunk index and depends on the row index mod 16, so
  //   K / V row reads: chunk 2 kk + kg of row sb*32 + n; for kk >= 8 (chunks
  //   16..31, head_dim 256) the offset of kk - 8 plus 256 bytes;
  //   K^T transpose reads: rows 16 kk2 + tr_row (+ 8) of block sb, column
  //   block db; blocks 4..7 at the offsets of blocks 0..3 plus 256 bytes,
  //   and the row block sb*32 + 16 kk2 adds a multiple of 16 rows.
  constexpr int KKR = KK < 8 ? KK : 8;
  constexpr int DBT = DB < 4 ? DB : 4;
  int rro[KKR];
#pragma unroll
  for (int kk = 0; kk < KKR; ++kk) rro[kk] = n * RP + (((2 * kk + kg) ^ nat_swz) << 4);
  int tro[DBT][2];
#pragma unroll
  for (int db = 0; db < DBT; ++db) {
    const int chunk = 4 * db + 2 * tr_g + (tr_s >> 1);
    const int half = (tr_s & 1) * 8;
    tro[db][0] = tr_row * RP + ((chunk ^ rswz<D>(tr_row)) << 4) + half;
    tro[db][1] = (tr_row + 8) * RP + ((chunk ^ rswz<D>(tr_row + 8)) << 4) + half;
  }

  if (kmax_g > kmin_g) {
    // kt1 >= (kmax - 1) / kBN: extra tiles are fully masked; none before the
    // K/V buffer's first key (clamped as in the forward).
    const int kt0 = max(kmin_g, s.kv_begin) / kBN;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Unrolled by two so that the stage is a compile-time constant.
    auto step = [&](int kt, auto stage) {
      constexpr int buf = decltype(stage)::value;
      const bool pre = kt > kt0;  // tile kt-1 goes to the other stage, last read before the last barrier
      const char* sK = buf == 0 ? stage0 : stage1;
      const char* sV = sK + kBN * RP;
      const int k0 = kt * kBN;
      const bool full = all_real && lomax <= k0 && k0 + kBN - 1 <= pfirst;
#pragma unroll
      for (int sb = 0; sb < kBN / 32; ++sb) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[j] = pacc[j] = 0.f;
        // K / V row reads two k-steps ahead of their products (the
        // compiler, left alone, keeps one pair in flight and each pair of
        // products waits for its reads).
        constexpr int PF = D == 256 ? 1 : 2;
        auto rpos = [&](int kk) { return rro[kk & 7] + (kk >> 3) * 256 + sb * 32 * RP; };
        bf16x8 ak[KK], av[KK];
#pragma unroll
        for (int kk = 0; kk < PF; ++kk) {
          ak[kk] = *reinterpret_cast<const bf16x8*>(sK + rpos(kk));
          av[kk] = *reinterpret_cast<const bf16x8*>(sV + rpos(kk));
        }
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (kk + PF < KK) {
            ak[kk + PF] = *reinterpret_cast<const bf16x8*>(sK + rpos(kk + PF));
            av[kk + PF] = *reinterpret_cast<const bf16x8*>(sV + rpos(kk + PF));
          }
          if (sb == 0 && kk % LSTEP == 0) issue_chunk(pre ? kt - 1 : kt, buf ^ 1, kk / LSTEP, pre);
          __builtin_amdgcn_sched_barrier(0);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[kk], qf[kk], sacc, 0, 0, 0);
          pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[kk], of[kk], pacc, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // sacc[j] = S[key k0 + sb*32 + (j/4)*8 + kg*4 + j%4][row n]
        // The mask is one block over the whole accumulator (S = -inf, so
        // P = 0): a test inside the exp loop would be split into one branch
        // per element and keep the exps from overlapping the products.
        if (!full) {
          // The row's allowed keys [lo, hi) as bits of key - kb (bit pos of
          // element j: (j/4)*8 + j%4); element j keeps its score where its
          // bit is set and becomes -inf elsewhere (two instructions each).
          const int kb = k0 + sb * 32 + kg * 4;
          const int a = min(max(lo - kb, 0), 32), e = min(max(hi - kb, 0), 32);
          const uint32_t allow = (a >= 32 ? 0u : ~0u << a) & (e >= 32 ? ~0u : (1u << e) - 1u);
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const uint32_t keep = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(allow), (j >> 2) * 8 + (j & 3), 1));
            sacc[j] = __uint_as_float((__float_as_uint(sacc[j]) & keep) | (0xff800000u & ~keep));
          }
        }
        // K^T transpose reads of the dQ^T products, flattened over (k-step,
        // column block) and issued two ahead of their products, the first
        // two before the exponentials.
        constexpr int NT = 2 * DB, PFT = D == 256 ? 1 : 2;
        auto kread = [&](int st_) {
          const int kk2 = st_ / DB, db = st_ % DB;
          const int r1 = (sb * 32 + 16 * kk2) * RP + (db >> 2) * 256;
          return lds_tr_pair(sK + (tro[db & 3][0] + r1), sK + (tro[db & 3][1] + r1));
        };
        bf16x8 kq[NT];
#pragma unroll
        for (int st_ = 0; st_ < PFT; ++st_) kq[st_] = kread(st_);
        __builtin_amdgcn_sched_barrier(0);
        // With dropout, the gradient reaching P is dP = (dO V^T) * Z * c.
        float zf[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) zf[j] = 1.f;
        if constexpr (DROP) {
          const uint32_t ip = static_cast<uint32_t>(s.row_offset + qt * kBM + n);
          const uint32_t bh = static_cast<uint32_t>(b * s.h_q + h);
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4)
            keep_factors_row(s.drop, ip, static_cast<uint32_t>(k0 + sb * 32 + g4 * 8 + kg * 4), bh, zf + 4 * g4);
        }
        float dsv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[j], c, -lse2m));
          dsv[j] = DROP ? p * (pacc[j] * zf[j] - dlt) : p * (pacc[j] - dlt);
        }
        bf16x8 dsb[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dsb[0][i] = static_cast<__bf16>(dsv[i]);
          dsb[1][i] = static_cast<__bf16>(dsv[8 + i]);
        }
        // dQ^T += K^T dS^T: A = K^T (rows = keys in accumulator order).
#pragma unroll
        for (int st_ = 0; st_ < NT; ++st_) {
          if (st_ + PFT < NT) kq[st_ + PFT] = kread(st_ + PFT);
          __builtin_amdgcn_sched_barrier(0);
          dqacc[st_ % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kq[st_], dsb[st_ / DB], dqacc[st_ % DB], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);  // the next tile's direct loads have landed
      __syncthreads();
    };
    for (int kt = kt1; kt >= kt0; kt -= 2) {
      step(kt, Stage<0>{});
      if (kt - 1 >= kt0) step(kt - 1, Stage<1>{});
    }
  } else {
    __builtin_amdgcn_s_waitcnt(0);  // the first tile's loads land before the workgroup's LDS is released
  }

  // dqacc[db][j] = dQ^T[d = 32db + (j/4)*8 + kg*4 + j%4][row n]
  if (valid) {
    uint16_t* drow = dq + (bt * s.h_q + h) * D + kg * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        uint2 pk;
        pk.x = pack_bf16x2(dqacc[db][4 * jq] * s.scale, dqacc[db][4 * jq + 1] * s.scale);
        pk.y = pack_bf16x2(dqacc[db][4 * jq + 2] * s.scale, dqacc[db][4 * jq + 3] * s.scale);
        *reinterpret_cast<uint2*>(drow + db * 32 + jq * 8) = pk;
      }
  }
}

template <int D, bool DROP>
hipError_t bwd_dq_t(const BwdArgs& a, hipStream_t st) {
  AttnShape s;
  s.batch = a.batch; s.seq_len = a.seq_len; s.row_offset = a.row_offset; s.q_len = a.q_len;
  s.h_q = a.h_q; s.h_kv = a.h_kv; s.head_dim = D; s.group = a.h_q / a.h_kv; s.scale = a.scale;
  s.kv_begin = a.kv_begin; s.kv_len = a.kv_len;
  s.drop = drop_params(a.drop.thr, a.drop.scale, a.drop.seed, a.drop.offset);
  MetaView m = meta_view(a.meta, a.batch, a.seq_len, a.q_len);
  const int hpw = heads_per_workgroup(a.h_q / a.h_kv);
  if (hpw < 4) m.q_order = m.q_stats = nullptr;  // the order is built for single query tiles
  const int n_qtg = ((a.q_len + kBM - 1) / kBM + 4 / hpw - 1) / (4 / hpw);
  const int n_hg = a.h_q / hpw;
  const int64_t grid = static_cast<int64_t>(n_qtg) * a.batch * n_hg;
  bwd_dq_kernel<D, DROP><<<dim3(static_cast<unsigned>(grid)), 256, 0, st>>>(
      s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
      static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.d_o),
      static_cast<const uint16_t*>(a.o), a.lse, a.rowstat, m, static_cast<uint16_t*>(a.dq), n_qtg, n_hg,
      device_cu_count() * kDqOcc<D>, hpw);
  return hipGetLastError();
}

}  // namespace

bool bwd_dq_fits(int64_t kv_len, int64_t h_kv, int64_t head_dim) {
  // a (batch row, K/V head)'s keys, including the last tile's keys past the
  // window, must be addressable with 31-bit buffer offsets
  return (kv_len + kBNmax) * h_kv * head_dim * 2 < (int64_t{1} << 31);
}

hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t st) {
  const bool drop = a.drop.thr != 0;
  switch (a.head_dim) {
    case 64: return drop ? bwd_dq_t<64, true>(a, st) : bwd_dq_t<64, false>(a, st);
    case 128: return drop ? bwd_dq_t<128, true>(a, st) : bwd_dq_t<128, false>(a, st);
    case 256: return drop ? bwd_dq_t<256, true>(a, st) : bwd_dq_t<256, false>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bd
