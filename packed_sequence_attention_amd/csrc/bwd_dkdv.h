// bf16 matrix-core dK/dV kernel of the block-diagonal packed attention
// backward for gfx950 (key-stationary) and its launcher, as templates over
// head_dim: bwd_mfma.hip instantiates head_dim 128 and the backward's launch
// sequence, bwd_dkdv64.hip head_dim 64 (a translation unit of its own, so it
// can be built with another instruction scheduler).
//
// Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences", Proof section (forward/backward parity, input gradients) and
// Design overview, exchange.py (the chunk's K/V gradients are partial sums
// over its rows, summed over ranks).  The gradients of softmax attention:
//   P_ij  = exp(scale q_i.k_j - LSE_i)          (LSE saved by the forward)
//   dP_ij = dO_i . v_j,   delta_i = dO_i . O_i  (= sum_j P_ij dP_ij)
//   dS_ij = P_ij (dP_ij - delta_i)
//   dV_j = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i
// (dQ is computed by the query-stationary kernel in bwd_dq.hip.)
//
// Work decomposition: a workgroup owns 64 keys of one K/V head of one batch
// row and runs 8 waves: two key groups of 32 times four query heads of the
// GQA group, so the heads are processed concurrently rather than one after
// another (the key tiles at the start of a long document attend many query
// tiles; splitting their work by head shortens the longest workgroup 4x).
// Each wave sweeps the 32-row query tiles that attend any of the
// workgroup's keys ([min key_qlo, max key_qhi) from the per-step metadata),
// once per group of four heads (for GQA groups of 1 or 2 heads, or not a
// multiple of 4, the four wave pairs split a head's query tiles instead),
// and computes for its 32 keys
// (v_mfma_f32_32x32x16_bf16, lane l: key l % 32):
//   S = Q K^T and dP = dO V^T   (A = Q / dO rows from LDS, B = K / V in registers)
//   dV^T += dO^T P, dK^T += Q^T dS  (A = dO^T / Q^T via the LDS transpose
//                                    load, B = P / dS from the accumulators)
// dK and dV stay in registers until the end; the four heads' partial sums
// of each key are then added through LDS in a fixed order ((h0 + h2) +
// (h1 + h3)) and written once (deterministic); for head_dim 128 each wave of
// a key group sums and writes a quarter of the columns.  The element mask uses the
// per-key row interval [key_qlo, key_qhi); it also zeroes padding rows and
// rows past the chunk.
//
// LDS layout (64 banks of 4 bytes; 16-byte reads serve 16 lanes per cycle,
// 8-byte reads and transpose loads 32 lanes): Q / dO tiles are rows of
// head_dim bf16 without padding; the 16-byte chunk c of row r is stored at
// chunk c ^ f(r), with f chosen so that 16 rows of a row read and 4 rows x 4
// chunks of a transpose read all land on distinct banks.  Q / dO / LSE /
// delta of the next query tile of each head are loaded straight into the
// other half of an LDS double buffer (LDS-DMA), one load per k-step of the
// current tile's S / dP products; two barriers per iteration (the ping-pong
// of the loop below).
#pragma once

#include <limits.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace bd {
namespace {

constexpr int kKW = 32;        // keys per wave
constexpr int kKB = 2 * kKW;   // keys per workgroup
constexpr int kQB = 32;        // query rows per tile
constexpr int kHW = 4;         // query heads processed concurrently

template <int D>
struct BwdLds {
  static constexpr int QP = D * 2;                  // Q / dO tile row pitch (xor-swizzled chunks)
  static constexpr int stat = 2 * kQB * 4;          // (lse * log2(e), delta) per row
  static constexpr int head = 2 * kQB * QP + stat;  // one head's Q, dO, statistics
  static constexpr int stage = kHW * head;          // one stage of the double buffer
  static constexpr int vtile = kKB * QP;            // the workgroup's V rows
  static constexpr int NCH = kQB * (D / 8) / 64;    // 16-byte direct loads per wave per tensor
  static constexpr int part = kKW * D * 2 * 4;      // one wave's dK and dV partials (float32)
  static_assert(2 * part <= stage, "head reduction must fit in the tile buffers");
};

// Chunk swizzle of row r of a Q / dO tile (see the file comment).
template <int D>
__device__ __forceinline__ int qswz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
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
__global__ __launch_bounds__(512) void bwd_dkdv_kernel(
    AttnShape s, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ rowstat, MetaView m, uint16_t* __restrict__ dk,
    uint16_t* __restrict__ dv, int n_kt, int n_bg, int live_lo, int live_hi) {
  constexpr int KK = D / 16;
  constexpr int DB = D / 32;
  constexpr int CH = D / 8;
  using L = BwdLds<D>;
  constexpr int NCH = L::NCH;
  // The two stages are separate LDS objects: the compiler then knows that
  // the direct loads into one stage do not alias reads of the other, and
  // does not make those reads wait for the loads in flight.
  __shared__ __attribute__((aligned(16))) char stage0[L::stage];
  __shared__ __attribute__((aligned(16))) char stage1[L::stage];
  __shared__ __attribute__((aligned(16))) char vt[L::vtile];
  __shared__ int sRed[16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kgrp = wave & 1, hsub = wave >> 1;  // key group, head within the four
  const int n = lane & 31, kg = lane >> 5;

  // Workgroups are dispatched to the 8 XCDs round-robin by index; keep every
  // key tile of one (batch row, K/V head) on one XCD so their reads of the
  // same Q / dO tiles can hit that XCD's L2.
  const int xcd = static_cast<int>(blockIdx.x) & 7, slot = static_cast<int>(blockIdx.x) >> 3;
  const int bg = xcd + 8 * (slot / n_kt);
  const int kt = slot % n_kt;
  if (bg >= n_bg) return;  // whole workgroup: no barrier has been reached
  const int b = bg / s.h_kv, g = bg % s.h_kv;
  const int key0 = s.kv_begin + kt * kKB;  // the workgroup's first key (row position)
  const int key = key0 + kgrp * kKW + n;  // this lane's key (columns of S)
  // key is a position in the row; K/V/dK/dV hold keys [kv_begin, kv_begin +
  // kv_len) of every row (key tiles are counted from kv_begin).
  const bool key_ok = key < s.kv_begin + s.kv_len;
  const int64_t kv_row = (static_cast<int64_t>(b) * s.kv_len + (key - s.kv_begin)) * s.h_kv + g;

  // Zero dK and dV rows of this lane's key: wave (key group, hsub) writes
  // the 32-column blocks db with db % 4 == hsub (the same bits as summing
  // four zero partials).
  auto write_zero_rows = [&]() {
    if (!key_ok) return;
    const uint2 z = make_uint2(0u, 0u);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if (db % kHW != hsub) continue;
      uint16_t* rk = dk + kv_row * D + kg * 4 + db * 32;
      uint16_t* rv = dv + kv_row * D + kg * 4 + db * 32;
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        *reinterpret_cast<uint2*>(rk + jq * 8) = z;
        *reinterpret_cast<uint2*>(rv + jq * 8) = z;
      }
    }
  };
  // Keys outside [live_lo, live_hi) (the positions any local row of any
  // batch row attends, known on the host) are attended by no row: zero at
  // once, before any load.  (Uniform over the workgroup: no barrier yet.)
  if (key0 + kKB <= live_lo || key0 >= live_hi) {
    write_zero_rows();
    return;
  }

  // Local rows attending this lane's key: [a0, a1) when a1 > a0 (loaded
  // here, used after the other prologue loads have been issued).
  int a0 = 0, a1 = 0;
  if (key_ok) {
    const int64_t kidx = static_cast<int64_t>(b) * s.seq_len + key;
    a0 = m.key_qlo[kidx];
    a1 = m.key_qhi[kidx];
  }
  const int row_stride = s.h_q * D;  // elements between consecutive rows

  // Q / dO / statistics staging: direct global -> LDS loads (buffer form,
  // so rows past the chunk read as zero) into an LDS double buffer, issued
  // one iteration ahead.  Iteration it covers, for the wave pair hsub, the
  // query tile qt0 + it_tile(it) of head it_head(it) (below); of that
  // pair, key group 0 loads Q, key group 1 loads dO and the row statistics.
  // Q / dO land in the swizzled layout: lane l of a load writes LDS chunk
  // (base + l), so each lane fetches the global chunk that belongs there.
  typedef __attribute__((address_space(3))) void lds_void;
  // Per-lane part of the direct-load offsets: load i of a wave covers RPL
  // tile rows (64 lanes x 16 bytes = 4 rows of 16 chunks for head_dim 128,
  // 8 rows of 8 for 64); the row part common to the wave goes into the
  // resource base.
  constexpr int RPL = 64 / CH;  // rows per direct load
  // With live == false (a padding iteration) the loads read nothing and
  // write zeros; tiles starting past the chunk read zeros as well.
  // (The prologue's loads; the loop issues its own, spread over the S / dP
  // products.  Keeping the buffer resources in a struct or returning them
  // from a lambda made the host pass drop a kernel's launch stub, so the
  // loop's copy of this code uses plain locals.)
  auto issue_tile = [&](int h, int t0, int buf, bool live) {
    // row t0 of (b, h); bytes from there to the end of the tensor's rows for this head
    const int64_t tile0 = ((static_cast<int64_t>(b) * s.q_len + t0) * s.h_q + h) * D;
    const int nbytes = live ? max(((s.q_len - t0) * row_stride - h * D) * 2, 0) : 0;
    const uint16_t* src = kgrp == 0 ? q : d_o;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src + tile0), 0, nbytes, 0x00020000);
    char* hb = (buf == 0 ? stage0 : stage1) + hsub * L::head;
    char* dst = hb + kgrp * (kQB * L::QP);
    // Recomputed here rather than kept live across the loop: the opaque copy
    // of the lane index stops the compiler from hoisting (and then spilling)
    // this offset, whose reload would wait on the direct loads in flight.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // Load i covers tile rows i * RPL + ln / CH.  The swizzle splits over
    // the two parts of the row index, qswz(i * RPL + x) = qswz(i * RPL) ^
    // qswz(x) (x < RPL), and the row pitch in bytes is a multiple of 16
    // chunks, so load i's offset is the lane's offset for load 0 with the
    // chunk bits xor-ed by qswz(i * RPL), plus i * RPL rows: one xor-add.
    const int row_bytes = row_stride * 2;
    const int off0 = (ln / CH) * row_bytes + (((ln % CH) ^ qswz<D>(ln / CH)) << 4);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int voff = (off0 ^ (qswz<D>((i * RPL) & 15) << 4)) + i * RPL * row_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + i * 64 * 16), 16, voff, 0, 0, 0);
    }
    if (kgrp == 1) {  // the tile's (lse * log2(e), delta) pairs: 64 x 4 bytes
      const int64_t st0 = (static_cast<int64_t>(b) * s.h_q + h) * s.q_len + t0;
      const __amdgpu_buffer_rsrc_t rst = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(rowstat + 2 * st0), 0, live ? max((s.q_len - t0) * 8, 0) : 0, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rst, (lds_void*)(hb + 2 * kQB * L::QP), 4, lane * 4, 0, 0, 0);
    }
  };

  // The first query tile is known before the metadata arrives: no row
  // attends a key after it, so the first local row attending the
  // workgroup's keys is max(first key - row_offset, 0) whenever any row
  // attends them.  Its loads go out with the K / V / metadata loads (one
  // memory round trip for the prologue instead of two); the metadata only
  // confirms the tile below.
  // Slot hsub of the four wave pairs: the iteration's heads are hpw heads of
  // the GQA group (hpw = 4 when the group holds a multiple of 4 heads, 2 for
  // a multiple of 2, else 1); slot hsub takes head offset hs = hsub % hpw
  // and query-tile phase ph = hsub / hpw, so with hpw < 4 the slots of one
  // head split its query tiles tpw = 4 / hpw ways.  Their partial dK / dV
  // are summed below like those of four heads.
  const int hpw = heads_per_workgroup(s.group), tpw = kHW / hpw;
  const int hs = hsub % hpw, ph = hsub / hpw;
  const int qt0e = max(key0 - s.row_offset, 0) / kQB;
  const bool early = qt0e * kQB < s.q_len;
  if (early) issue_tile(g * s.group + hs, (qt0e + ph) * kQB, 0, true);

  // K fragments of this wave's keys (B operand of S) in registers; the
  // workgroup's V tile (B operand of dP) in LDS, swizzled like Q / dO.
  // Loads without branches (keys past the row read the row's last key and
  // are zeroed where the values are used), so that no load waits for the
  // ones issued before it.
  const int64_t kv_row_c = key_ok ? kv_row : (static_cast<int64_t>(b) * s.kv_len + s.kv_len - 1) * s.h_kv + g;
  bf16x8 kf[KK];
  char* sV = vt + kgrp * kKW * L::QP;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) kf[kk] = *reinterpret_cast<const bf16x8*>(k + kv_row_c * D + kk * 16 + kg * 8);
  if (hsub == 0) {
    // All of the row's loads first, then the LDS stores (one round trip).
    bf16x8 x[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) x[kk] = *reinterpret_cast<const bf16x8*>(v + kv_row_c * D + kk * 16 + kg * 8);
    bf16x8 zero;
#pragma unroll
    for (int i = 0; i < 8; ++i) zero[i] = static_cast<__bf16>(0.f);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      *reinterpret_cast<bf16x8*>(sV + n * L::QP + (((2 * kk + kg) ^ qswz<D>(n)) << 4)) = key_ok ? x[kk] : zero;
  }
  // Local rows attending this lane's key: [qlo_k, qhi_k) (empty: qlo_k >= qhi_k).
  const int qlo_k = a1 > a0 ? a0 : INT_MAX, qhi_k = a1 > a0 ? a1 : INT_MIN;
  const int wqlo = wave_min_i(qlo_k), wqhi = wave_max_i(qhi_k);
  // Rows inside every key's interval of this wave: [kq_lo_max, kq_hi_min).
  const int kq_lo_max = wave_max_i(qlo_k), kq_hi_min = wave_min_i(qhi_k);
  // (Tested per tile as a per-lane compare: a uniform branch there makes the
  // compiler restructure the loop and run out of registers.)
  int kq_lo_v = kq_lo_max, kq_hi_v = kq_hi_min;
  asm volatile("" : "+v"(kq_lo_v), "+v"(kq_hi_v));
  // Element mask: row t is allowed iff (unsigned)(t - mask_lo) < mask_span.
  const int mask_lo = qhi_k > qlo_k ? qlo_k : 0;
  const unsigned mask_span = qhi_k > qlo_k ? static_cast<unsigned>(qhi_k - qlo_k) : 0u;
  if (lane == 0 && hsub == 0) {
    sRed[kgrp] = wqlo;
    sRed[2 + kgrp] = wqhi;
  }
  // The early tile is written into LDS by direct loads that another wave
  // reads: wait for every load of this wave (the early tile's, and the V
  // loads behind the LDS stores above) before the barrier publishes them.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int gqlo = min(sRed[0], sRed[1]);
  const int gqhi = max(sRed[2], sRed[3]);
  if (!key_ok) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < 8; ++i) kf[kk][i] = static_cast<__bf16>(0.f);
  }
  const int qt0 = gqlo / kQB;
  const int n_q = gqhi > gqlo ? (gqhi - 1) / kQB - qt0 + 1 : 0;
  // Iteration it covers heads g * group + (it / n_qp) * hpw + [0, hpw) and,
  // for slot hsub, query tile qt0 + it_tile(it); a tile index >= n_q pads
  // the last iteration (its rows lie past every key's row interval, so the
  // mask zeroes them; the loads write zeros).
  const int n_qp = (n_q + tpw - 1) / tpw;
  const int n_it = n_qp * (s.group / hpw);
  auto it_tile = [&](int it) { return (it % n_qp) * tpw + ph; };
  auto it_head = [&](int it) { return g * s.group + (it / n_qp) * hpw + hs; };
  auto issue_loads = [&](int it, int buf) {
    const int ti = it_tile(it);
    issue_tile(it_head(it), (qt0 + ti) * kQB, buf, ti < n_q);
  };

  // No local row attends any of the workgroup's keys: their dK and dV are
  // zero, written at once instead of summing four zero partials.  (n_q is
  // the workgroup's, read from LDS after the barrier: every wave takes this
  // branch or none.)
  if (n_q == 0) {
    write_zero_rows();
    return;
  }

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) dkacc[db][j] = dvacc[db][j] = 0.f;

  const float c = s.scale * kLog2e;
  // Per-lane LDS addressing.
  const int tr_row = 4 * kg + ((lane & 15) >> 2);   // transpose-load row within a group of 8
  const int tr_g = (lane >> 4) & 1;                 // 16-column half of a transpose load
  const int tr_s = lane & 3;                        // 4-column quarter
  // Two barriers per iteration, and the two wave groups run half an
  // iteration apart ("ping-pong"): group A (heads 0, 1 of the four) and
  // group B (heads 2, 3) each put one wave on every SIMD, and while one
  // group runs the softmax (vector ALU) the other keeps the matrix cores
  // busy with S and dP.  Per wave, iteration it is
  //   H1: S and dP products, with the direct loads of tile it+1 into the
  //   other stage between them (barrier: scheduling only, no memory ordering)
  //   H2: softmax, dV/dK products of tile it; wait for the direct loads;
  //   barrier.
  // Group B enters the loop one barrier later and group A leaves it one
  // barrier later, so every wave executes the same number of barriers.  The
  // two groups share no tile buffers, so only the full barrier at the end of
  // a wave's own H2 orders its group's loads and reads.
  const bool late = hsub >= 2;
  if (n_it > 0) {
    // The early tile landed before the barrier above (the explicit wait
    // before it); it is reloaded only if the metadata disagrees.
    if (!early || qt0 != qt0e) {
      issue_loads(0, 0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (late) __builtin_amdgcn_s_barrier();
  }
  // The loop is unrolled by two so that the stage is a compile-time
  // constant and every LDS address is a per-lane base plus an immediate.
  auto step = [&](int it, auto stage) {
    constexpr int buf = decltype(stage)::value;
    const int t0 = (qt0 + it_tile(it)) * kQB;
    const char* sQ = (buf == 0 ? stage0 : stage1) + hsub * L::head;
    const char* sdO = sQ + kQB * L::QP;
    const float* sStat = reinterpret_cast<const float*>(sdO + kQB * L::QP);  // (lse2, delta) pairs
    // The K fragments pass through an empty asm here, before the loads of
    // tile it+1: without it, the compiler's wait bookkeeping still counted
    // them as pending from their global loads and made every S product of
    // the first unrolled step wait for one more of the new tile loads.
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) asm volatile("" : "+v"(kf[kk]));
    // The direct loads of iteration it+1 (into the other stage, last read
    // before the last barrier) go out one per k-step of the S / dP products
    // below: issued at once, the workgroup's 72 loads queue at the address
    // unit and stall each wave's issue for hundreds of cycles.  Resources
    // and the lane offset are plain locals (see issue_tile).
    const bool more = it + 1 < n_it;
    const int ti1 = it_tile(it + 1);
    const int h1 = it_head(it + 1), t1 = (qt0 + ti1) * kQB;
    const bool live1 = more && ti1 < n_q;
    const int64_t tile1 = ((static_cast<int64_t>(b) * s.q_len + t1) * s.h_q + h1) * D;
    const int nb1 = live1 ? max(((s.q_len - t1) * row_stride - h1 * D) * 2, 0) : 0;
    const __amdgpu_buffer_rsrc_t rs1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>((kgrp == 0 ? q : d_o) + tile1), 0, nb1, 0x00020000);
    const int64_t st1 = (static_cast<int64_t>(b) * s.h_q + h1) * s.q_len + t1;
    const __amdgpu_buffer_rsrc_t rst1 = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(rowstat + 2 * st1), 0, live1 ? max((s.q_len - t1) * 8, 0) : 0, 0x00020000);
    char* hb1 = (buf == 1 ? stage0 : stage1) + hsub * L::head;
    char* dst1 = hb1 + kgrp * (kQB * L::QP);
    int ln1 = lane;
    asm volatile("" : "+v"(ln1));
    const int rbytes = row_stride * 2;
    const int off01 = (ln1 / CH) * rbytes + (((ln1 % CH) ^ qswz<D>(ln1 / CH)) << 4);
    static_assert(NCH <= KK, "at most one direct load per k-step");

    f32x16 sacc, pacc;
#pragma unroll
    for (int j = 0; j < 16; ++j) sacc[j] = pacc[j] = 0.f;
    {
      const int nat_row = n * L::QP;
      const int nat_swz = qswz<D>(n);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int pos = nat_row + (((2 * kk + kg) ^ nat_swz) << 4);
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQ + pos);
        const bf16x8 ao = *reinterpret_cast<const bf16x8*>(sdO + pos);
        const bf16x8 bv = *reinterpret_cast<const bf16x8*>(sV + pos);
        if (more && kk < NCH) {
          const int voff = (off01 ^ (qswz<D>((kk * RPL) & 15) << 4)) + kk * RPL * rbytes;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs1, (lds_void*)(dst1 + kk * 64 * 16), 16, voff, 0, 0, 0);
          if (kk == 0 && kgrp == 1)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rst1, (lds_void*)(hb1 + 2 * kQB * L::QP), 4, lane * 4, 0, 0, 0);
        }
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[kk], sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, bv, pacc, 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_barrier();  // H1 / H2 boundary (see above)
    // sacc[j] = S[row t0 + (j/4)*8 + kg*4 + j%4][key n].  P is zero outside
    // the mask, which also covers padding rows, rows past the chunk and
    // waves whose keys no row of this tile attends.  Tiles inside every
    // key's row interval skip the mask.
    // The softmax and the dV/dK products, with or without the mask (one
    // copy each so that nothing but the accumulators is live across the
    // branch).
    auto finish = [&](auto masked) {
      float pv[16], dsv[16];
      // The key's allowed rows [mask_lo, mask_lo + mask_span) as bits of
      // row - (t0 + kg*4), clamped to the 32 bits.
      uint32_t allow = 0;
      if constexpr (decltype(masked)::value) {
        const int rb = t0 + kg * 4;
        const int a = min(max(mask_lo - rb, 0), 32);
        const int e = min(max(mask_lo + static_cast<int>(mask_span) - rb, 0), 32);
        allow = (a >= 32 ? 0u : ~0u << a) & (e >= 32 ? ~0u : (1u << e) - 1u);
      }
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
                           static_cast<uint32_t>(b * s.h_q + it_head(it)), zf);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = jq * 4 + e;
          float x = fmaf(sacc[j], c, -lsv[e]);
          if constexpr (decltype(masked)::value) {
            // bit (j/4)*8 + j%4 of allow: row t0 + kg*4 + that is allowed;
            // elsewhere the exponent becomes -inf, so P = 0 (also on padding
            // rows, whose exponent may be +inf)
            const uint32_t keep = static_cast<uint32_t>(__builtin_amdgcn_sbfe(static_cast<int>(allow), jq * 8 + e, 1));
            x = __uint_as_float((__float_as_uint(x) & keep) | (0xff800000u & ~keep));
          }
          const float p = __builtin_amdgcn_exp2f(x);
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
      // dV^T += dO^T P, dK^T += Q^T dS (k = query rows, accumulator order).
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        const int r_a = 16 * kk2 + tr_row, r_b = r_a + 8;
        const int sw_a = qswz<D>(r_a), sw_b = qswz<D>(r_b);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int chunk = 4 * db + 2 * tr_g + (tr_s >> 1);
          const int half = (tr_s & 1) * 8;
          const int pa = r_a * L::QP + ((chunk ^ sw_a) << 4) + half;
          const int pb_ = r_b * L::QP + ((chunk ^ sw_b) << 4) + half;
          const bf16x8 a_do = lds_tr_pair(sdO + pa, sdO + pb_);
          const bf16x8 a_q = lds_tr_pair(sQ + pa, sQ + pb_);
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_do, pb[kk2], dvacc[db], 0, 0, 0);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_q, dsb[kk2], dkacc[db], 0, 0, 0);
        }
      }
    };
    if (t0 >= kq_lo_v && t0 + kQB <= kq_hi_v)
      finish(Stage<0>{});
    else
      finish(Stage<1>{});
    __builtin_amdgcn_s_waitcnt(0);  // direct loads of tile it+1 have landed in LDS
    __syncthreads();                // next Q/dO buffer ready
  };
  for (int it = 0; it < n_it; it += 2) {
    step(it, Stage<0>{});
    if (it + 1 < n_it) step(it + 1, Stage<1>{});
  }
  if (n_it > 0 && !late) __builtin_amdgcn_s_barrier();

  // Sum the four heads' partials in a fixed order, (h0 + h2) + (h1 + h3),
  // through LDS (the tile buffers are free once every wave has left the
  // loop), and write dK and dV once.
  __syncthreads();
  if constexpr (DB == kHW) {
    // head_dim 128: reduce-scatter.  Wave hsub owns d-block hsub (32 of the
    // 128 columns) of its key group's dK, then of its dV: it stores its other
    // three blocks for their owners, and sums the owners' copies of its own
    // block with its registers.  All eight waves work in each phase; a block
    // is stored lane-major, one float4 per lane per step (contiguous).
    // Slot (key group, block, writer) is 4 KB: 16 slots per stage.
    constexpr int SLOT4 = 16 * 64 / 4;  // float4 per slot
    static_assert(16 * SLOT4 * 16 <= L::stage, "16 reduction slots per stage");
    auto slot_ptr = [&](int kg_, int db_, int w_) {
      const int sl = kg_ * 16 + db_ * 4 + w_;
      return reinterpret_cast<float4*>(sl < 16 ? stage0 : stage1) + (sl & 15) * SLOT4;
    };
    auto reduce = [&](f32x16 (&acc)[DB], uint16_t* out, float mul) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if (db == hsub) continue;
        float4* p = slot_ptr(kgrp, db, hsub);
#pragma unroll
        for (int jq = 0; jq < 4; ++jq)
          p[jq * 64 + lane] = make_float4(acc[db][4 * jq], acc[db][4 * jq + 1], acc[db][4 * jq + 2], acc[db][4 * jq + 3]);
      }
      __syncthreads();
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if (db != hsub) continue;
        f32x16 part[kHW];
#pragma unroll
        for (int w = 0; w < kHW; ++w) {
          if (w == db) {
            part[w] = acc[db];
          } else {
            const float4* p = slot_ptr(kgrp, db, w);
#pragma unroll
            for (int jq = 0; jq < 4; ++jq) {
              const float4 x = p[jq * 64 + lane];
              part[w][4 * jq] = x.x; part[w][4 * jq + 1] = x.y;
              part[w][4 * jq + 2] = x.z; part[w][4 * jq + 3] = x.w;
            }
          }
        }
        const f32x16 r = (part[0] + part[2]) + (part[1] + part[3]);
        // acc[db][j] = X^T[d = 32db + (j/4)*8 + kg*4 + j%4][key n]
        if (key_ok) {
          uint16_t* row = out + kv_row * D + kg * 4 + db * 32;
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            uint2 pk;
            pk.x = pack_bf16x2(r[4 * jq] * mul, r[4 * jq + 1] * mul);
            pk.y = pack_bf16x2(r[4 * jq + 2] * mul, r[4 * jq + 3] * mul);
            *reinterpret_cast<uint2*>(row + jq * 8) = pk;
          }
        }
      }
    };
    reduce(dkacc, dk, s.scale);
    __syncthreads();  // every wave has read its dK blocks before the dV blocks overwrite them
    reduce(dvacc, dv, 1.f);
  } else {
    // head_dim 64: the partials of two waves at a time fit the buffers;
    // two levels, h0 += h2 and h1 += h3, then h0 += h1.
    constexpr int P4 = L::part / 16;  // float4 per wave partial
    auto slot_ptr = [&](int slot_) {  // slots 0, 1 in stage 0; 2, 3 in stage 1
      return reinterpret_cast<float4*>(slot_ < 2 ? stage0 : stage1) + (slot_ & 1) * P4;
    };
    auto put = [&](int slot_) {
      float4* p = slot_ptr(slot_);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const int f = (db * 4 + jq) * 2;
          p[f * 64 + lane] = make_float4(dkacc[db][4 * jq], dkacc[db][4 * jq + 1], dkacc[db][4 * jq + 2],
                                         dkacc[db][4 * jq + 3]);
          p[(f + 1) * 64 + lane] = make_float4(dvacc[db][4 * jq], dvacc[db][4 * jq + 1],
                                               dvacc[db][4 * jq + 2], dvacc[db][4 * jq + 3]);
        }
    };
    auto add = [&](int slot_) {
      const float4* p = slot_ptr(slot_);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const int f = (db * 4 + jq) * 2;
          const float4 x = p[f * 64 + lane], y = p[(f + 1) * 64 + lane];
          dkacc[db][4 * jq] += x.x; dkacc[db][4 * jq + 1] += x.y;
          dkacc[db][4 * jq + 2] += x.z; dkacc[db][4 * jq + 3] += x.w;
          dvacc[db][4 * jq] += y.x; dvacc[db][4 * jq + 1] += y.y;
          dvacc[db][4 * jq + 2] += y.z; dvacc[db][4 * jq + 3] += y.w;
        }
    };
    if (hsub >= 2) put((hsub - 2) * 2 + kgrp);
    __syncthreads();
    if (hsub < 2) add(hsub * 2 + kgrp);
    __syncthreads();
    if (hsub == 1) put(kgrp);
    __syncthreads();
    if (hsub != 0) return;
    add(kgrp);

    // dvacc[db][j] = dV^T[d = 32db + (j/4)*8 + kg*4 + j%4][key n]
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
}

// Launches the dK/dV kernel (the row statistics must already be in
// a.rowstat: the dQ kernel writes them), bracketed by the profiling marks.
template <int D, bool DROP>
hipError_t launch_dkdv_t(const BwdArgs& a, hipStream_t st) {
  AttnShape s;
  s.batch = a.batch; s.seq_len = a.seq_len; s.row_offset = a.row_offset; s.q_len = a.q_len;
  s.h_q = a.h_q; s.h_kv = a.h_kv; s.head_dim = D; s.group = a.h_q / a.h_kv; s.scale = a.scale;
  s.kv_begin = a.kv_begin; s.kv_len = a.kv_len;
  s.drop = drop_params(a.drop.thr, a.drop.scale, a.drop.seed, a.drop.offset);
  MetaView m = meta_view(a.meta, a.batch, a.seq_len, a.q_len);
  const int n_kt = (a.kv_len + kKB - 1) / kKB;
  const int n_bg = a.batch * a.h_kv;
  const int64_t grid = 8 * static_cast<int64_t>((n_bg + 7) / 8) * n_kt;
  if (n_kt == 0) return hipSuccess;
  hipError_t e = mark(a.mark_start, st);
  if (e != hipSuccess) return e;
  bwd_dkdv_kernel<D, DROP><<<dim3(static_cast<unsigned>(grid)), 512, 0, st>>>(
      s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
      static_cast<const uint16_t*>(a.v), static_cast<const uint16_t*>(a.d_o), a.rowstat, m,
      static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), n_kt, n_bg, a.live_lo, a.live_hi);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return mark(a.mark_stop, st);
}

// Rows of one (batch row, head) of Q / dO, including the last tile's rows
// past the chunk, in 31-bit buffer offsets.
constexpr bool dkdv_rows_fit(int64_t q_len, int64_t h_q, int64_t head_dim) {
  return (q_len + kQB) * h_q * head_dim * 2 < (int64_t{1} << 31);
}

}  // namespace
}  // namespace bd
