// bf16 matrix-core backward of the block-diagonal packed attention for
// packings of short documents (no segment of more than kBinCap = 128 keys)
// on gfx950: dQ, dK and dV in one kernel, one workgroup per (bin, K/V head).
//
// Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences", Proof section (forward/backward parity, input gradients); the
// gradients are those of the tile kernels (bwd_dq.hip, bwd_dkdv.h):
//   P_ij  = exp(scale q_i.k_j - LSE_i),  dP_ij = dO_i . v_j,
//   delta_i = dO_i . O_i,                dS_ij = P_ij (dP_ij - delta_i),
//   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i,
//   dV_j = sum_i P_ij dO_i.
// A bin of the metadata holds whole documents: its rows attend only its
// keys and its keys are attended only by its rows.  So one workgroup
// computes all three gradients of a bin, each (row, key) pair once: no
// atomics, no recomputation of S and dP, and Q, dO, O, K and V read once.
// With short documents the backward is bound by HBM bytes, and the tile
// kernels (a dQ pass and a dK/dV pass, each recomputing S and dP and
// reading Q and dO) move about 1.6 times the bytes.
//
// Work decomposition: four waves, two workgroups per CU.  The bin's
// iterations are its 32-row blocks times the GQA group's query heads (rows
// outer, heads inner: the heads of a row are adjacent in memory).  Wave w
// owns key block w of the bin (keys 32w .. 32w + 31 from the bin's first
// key: K rows in LDS, V fragments in registers, dK and dV accumulated in
// registers over the whole bin) and, in the dQ products, columns 32w ..
// 32w + 31 of head_dim.
// Per iteration (row block, head), v_mfma_f32_32x32x16_bf16 throughout:
//   stats  delta of the block's rows from O (registers) and dO (LDS),
//          with lse * log2(e), into LDS;
//   keys   wave w, if a row of the block attends a key of its block:
//          S = Q K^T, dP = dO V^T (A = Q / dO rows from LDS, B = K rows
//          from LDS / V in registers),
//          P and dS in the accumulator layout (lane: key), then
//          dV^T += dO^T P and dK^T += Q^T dS (A = dO^T / Q^T with the LDS
//          transpose load); dS in bf16 goes to LDS, key-major;
//   dQ     wave w: dQ^T[32w .. 32w + 31] = sum over the live key blocks of
//          K^T dS^T (A = K^T, B = dS^T, both with the transpose load),
//          written once for the block's rows that are the bin's.
// Q / dO blocks come in by direct global -> LDS loads into a double
// buffer, one block ahead; O rows for delta likewise, in registers.
// Rows and keys past the bin inside a 32-row or 32-key block are another
// bin's: a key's row interval from the metadata masks them, and nothing of
// theirs is written.  Rows of padding and keys no row attends lie in no
// bin: extra workgroups of the same launch write their zeros.
#include <limits.h>
#include <math.h>

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace bd {
namespace {

constexpr int kSB = 32;  // rows / keys of a block
constexpr int kSW = 4;   // waves = key blocks of a bin
static_assert(kSB * kSW == kBinCap, "the waves' key blocks cover a bin");
constexpr int kZT = 64;          // rows / keys of a zero-fill tile
constexpr int kThreads = 256;  // four waves; two workgroups per CU (LDS and registers)

template <int D>
struct ShortLds {
  static constexpr int RP = D * 2;                // row pitch (bytes), swizzled 16-byte chunks
  static constexpr int CH = D / 8;                // 16-byte chunks per row
  static constexpr int ktile = kBinCap * RP;      // the bin's K (or V) rows
  static constexpr int qtile = kSB * RP;          // one 32-row block of Q or dO
  static constexpr int stage = 2 * qtile;         // Q then dO
  static constexpr int PER_T = kSB * CH / kThreads;  // direct loads per thread per tensor
  static constexpr int DSP = kSB * 2 + 8;         // dS tile pitch: a key's 32 rows + 8 bytes
  static constexpr int dstile = kSB * DSP;        // one key block's dS (key-major)
  static_assert(PER_T * kThreads == kSB * CH, "whole tensors per load round");
};

// Chunk swizzle of row r: 16 rows of a row read, and 4 rows x 4 chunks of a
// transpose read, land on distinct banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
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

// A lane's value moved by a DPP pattern (quad permutation 0x00-0xFF, 0x141
// mirror within each group of 8 lanes); all lanes take part.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Workgroup barrier for LDS data written by the waves: waits for this
// wave's LDS operations only, not for direct global -> LDS loads in flight
// (a fence on the workgroup would wait for those too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Zero-fill tile z: local rows of padding (their dQ over all query heads)
// or, after the n_zr row tiles, window keys no local row attends (their dK
// and dV over all K/V heads).
template <int D>
__device__ void zero_tile(const AttnShape& s, const MetaView& m, uint16_t* dq, uint16_t* dk, uint16_t* dv, int z,
                          int n_zr) {
  constexpr int NW = kThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  // Lane l of every wave reads the bounds of tile row / key l (one load for
  // the tile); a ballot then names the rows / keys to clear, and the waves
  // take them in turn.
  if (z < n_zr) {
    const int nrt = (s.q_len + kZT - 1) / kZT;
    const int b = z / nrt, t0 = (z % nrt) * kZT;
    const int t = t0 + lane;
    bool pad = false;
    if (t < s.q_len) {
      const int64_t bt = static_cast<int64_t>(b) * s.q_len + t;
      pad = m.row_hi[bt] <= m.row_lo[bt];  // no key: padding (a real row's bin writes it)
    }
    uint64_t todo = __ballot(pad);
    const int words = s.h_q * D / 8;  // 16-byte stores per row
    for (int r = 0; todo != 0; ++r) {
      const int l = __ffsll(static_cast<unsigned long long>(todo)) - 1;
      todo &= todo - 1;
      if (r % NW != wave) continue;
      uint4* row = reinterpret_cast<uint4*>(dq + (static_cast<int64_t>(b) * s.q_len + t0 + l) * s.h_q * D);
      for (int i = lane; i < words; i += 64) row[i] = zero;
    }
  } else {
    z -= n_zr;
    const int nkt = (s.kv_len + kZT - 1) / kZT;
    const int b = z / nkt, w0 = (z % nkt) * kZT;
    const int kw = w0 + lane;  // key index in the window
    bool dead = false;
    if (kw < s.kv_len) {
      const int64_t kidx = static_cast<int64_t>(b) * s.seq_len + s.kv_begin + kw;
      dead = m.key_qhi[kidx] <= m.key_qlo[kidx];  // no row attends it (else its bin writes it)
    }
    uint64_t todo = __ballot(dead);
    const int words = s.h_kv * D / 8;
    for (int r = 0; todo != 0; ++r) {
      const int l = __ffsll(static_cast<unsigned long long>(todo)) - 1;
      todo &= todo - 1;
      if (r % NW != wave) continue;
      const int64_t kr = (static_cast<int64_t>(b) * s.kv_len + w0 + l) * s.h_kv * D;
      uint4* rk = reinterpret_cast<uint4*>(dk + kr);
      uint4* rv = reinterpret_cast<uint4*>(dv + kr);
      for (int i = lane; i < words; i += 64) {
        rk[i] = zero;
        rv[i] = zero;
      }
    }
  }
}

template <int D, bool DROP>
__global__ __launch_bounds__(kThreads, 2) void bwd_short_kernel(
    AttnShape s, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ d_o, const uint16_t* __restrict__ o, const float* __restrict__ lse, MetaView m,
    uint16_t* __restrict__ dq, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int n_bin_wg, int n_zr) {
  constexpr int KK = D / 16;  // k-steps over head_dim
  constexpr int DB = D / 32;  // 32-column blocks of head_dim
  constexpr int OE = D / 64;  // 16-byte chunks of O per lane in the delta step
  using L = ShortLds<D>;
  constexpr int RP = L::RP;
  // The two stages are separate LDS objects, so the compiler knows that
  // direct loads into one do not alias reads of the other.
  __shared__ __attribute__((aligned(16))) char st0[L::stage];
  __shared__ __attribute__((aligned(16))) char st1[L::stage];
  __shared__ __attribute__((aligned(16))) char sK[L::ktile];
  __shared__ __attribute__((aligned(16))) char sdS[kSW * L::dstile];
  __shared__ __attribute__((aligned(16))) float2 sStat[kSB];  // (lse * log2(e), delta) per block row
  __shared__ int sRng[2][kSW];                                   // local rows attending each key block
  typedef __attribute__((address_space(3))) void lds_void;

  const int wg = static_cast<int>(blockIdx.x);
  if (wg >= n_bin_wg * s.h_kv) {
    zero_tile<D>(s, m, dq, dk, dv, wg - n_bin_wg * s.h_kv, n_zr);
    return;
  }
  const int bi = wg / s.h_kv, g = wg % s.h_kv;
  const int n_bins = __builtin_amdgcn_readfirstlane(m.bins[0]);
  if (bi >= n_bins) return;  // whole workgroup: no barrier has been reached
  const int q0 = __builtin_amdgcn_readfirstlane(m.bins[1 + 3 * bi]);
  const int q1 = __builtin_amdgcn_readfirstlane(m.bins[2 + 3 * bi]);
  const int k0f = __builtin_amdgcn_readfirstlane(m.bins[3 + 3 * bi]);
  const int b = q0 / s.q_len;
  const int t0 = q0 - b * s.q_len;                     // first local row
  const int nrows = q1 - q0;
  const int pos0 = k0f - b * s.seq_len;                // first key (row position)
  const int nkeys = s.row_offset + t0 + nrows - pos0;  // keys end one past the last row
  // Bins come from the metadata build; anything outside these limits is
  // skipped rather than read out of bounds.
  if (nrows <= 0 || nkeys < nrows || nkeys > kBinCap || t0 + nrows > s.q_len || pos0 < s.kv_begin ||
      pos0 + nkeys > s.kv_begin + s.kv_len)
    return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wk = wave;  // key block (and dQ column block)
  const int G = s.group;
  const int row_stride = s.h_q * D;

  // This lane's key: index in the bin, row position, K/V row.
  const int kb0 = wk * kSB + (lane & 31);
  const bool kok = kb0 < nkeys;
  const int kpos = pos0 + kb0;
  const int64_t kv_row_c =
      (static_cast<int64_t>(b) * s.kv_len + ((kok ? kpos : pos0) - s.kv_begin)) * s.h_kv + g;

  // Iteration it of the bin: row block it / G, head g * G + it % G.
  const int n_rb = (nrows + kSB - 1) / kSB;
  const int n_it = n_rb * G;

  // Direct loads of the Q / dO block of iteration it into stage buf: chunk
  // ci = i * 256 + tid of each tensor lands at LDS chunk ci, so each lane
  // fetches the global chunk that belongs there under the swizzle.  Rows
  // past the chunk read as zero.  Loads p0 .. p1-1 of the wave's 2 * PER_T
  // (tensor-major), so that the loop can spread them over its products.
  auto issue_tile = [&](int it, int buf, int p0, int p1) __attribute__((always_inline)) {
    char* dst = buf == 0 ? st0 : st1;
    const int ib = it / G, h = g * G + it % G;
    const int trow0 = t0 + ib * kSB;
    const int64_t tile0 = ((static_cast<int64_t>(b) * s.q_len + trow0) * s.h_q + h) * D;
    const int nbytes = max(((s.q_len - trow0) * row_stride - h * D) * 2, 0);
    // (The tensor is a compile-time index: a select between the sources
    // would keep the closure, and what it refers to, in scratch memory.)
#pragma unroll
    for (int tensor = 0; tensor < 2; ++tensor) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>((tensor == 0 ? q : d_o) + tile0), 0, nbytes, 0x00020000);
#pragma unroll
      for (int i = 0; i < L::PER_T; ++i) {
        if (tensor * L::PER_T + i < p0 || tensor * L::PER_T + i >= p1) continue;
        const int cw = i * kThreads + wk * 64;  // the wave's first chunk of the tensor (uniform)
        const int lc = cw + lane;
        const int r = lc / L::CH, pc = (lc % L::CH) ^ swz<D>(r);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + tensor * L::qtile + cw * 16), 16,
                                                 (r * row_stride + pc * 8) * 2, 0, 0, 0);
      }
    }
  };
  // O rows and lse of iteration it for the delta step: lane l takes row
  // 8 * wk + l / 8 of the block, 16-byte chunks (l % 8) * OE + e.
  bf16x8 ov[OE];
  float lsev = 0.f;
  auto load_o = [&](int it) __attribute__((always_inline)) {
    const int ib = it / G, h = g * G + it % G;
    const int drow = 8 * wk + (lane >> 3), dc = lane & 7;
    const int t = min(t0 + ib * kSB + drow, s.q_len - 1);
    const bf16x8* src =
        reinterpret_cast<const bf16x8*>(o + ((static_cast<int64_t>(b) * s.q_len + t) * s.h_q + h) * D) + dc * OE;
#pragma unroll
    for (int e = 0; e < OE; ++e) ov[e] = src[e];
    lsev = lse[(static_cast<int64_t>(b) * s.h_q + h) * s.q_len + t];
  };

  issue_tile(0, 0, 0, 2 * L::PER_T);  // (n_it >= 1: a bin has a row)
  load_o(0);
  // K rows of this wave's key block into LDS (swizzled) and V fragments
  // (B operand of dP) in registers; keys past the bin are zero.
  bf16x8 vf[KK];
  {
    const int kg = lane >> 5;
    bf16x8 x[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      x[kk] = *reinterpret_cast<const bf16x8*>(k + kv_row_c * D + kg * 8 + kk * 16);
      vf[kk] = *reinterpret_cast<const bf16x8*>(v + kv_row_c * D + kg * 8 + kk * 16);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (!kok) {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[kk][i] = vf[kk][i] = static_cast<__bf16>(0.f);
      }
      *reinterpret_cast<bf16x8*>(sK + kb0 * RP + (((2 * kk + kg) ^ swz<D>(kb0)) << 4)) = x[kk];
    }
  }
  int a0 = 0, a1 = 0;
  if (kok) {
    const int64_t kidx = static_cast<int64_t>(b) * s.seq_len + kpos;
    a0 = m.key_qlo[kidx];
    a1 = m.key_qhi[kidx];
  }
  // Local rows attending this lane's key: row t is allowed iff
  // (unsigned)(t - mask_lo) < mask_span (empty past the bin's keys).
  const bool att = kok && a1 > a0;
  const int mask_lo = att ? a0 : 0;
  const unsigned mask_span = att ? static_cast<unsigned>(a1 - a0) : 0u;
  const int wqlo = wave_min_i(att ? a0 : INT_MAX), wqhi = wave_max_i(att ? a1 : INT_MIN);
  if (lane == 0) {
    sRng[0][wk] = wqlo;
    sRng[1][wk] = wqhi;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();  // K rows, the key blocks' row ranges and the first block in LDS
  int rlo[kSW], rhi[kSW];
#pragma unroll
  for (int j = 0; j < kSW; ++j) {
    rlo[j] = __builtin_amdgcn_readfirstlane(sRng[0][j]);
    rhi[j] = __builtin_amdgcn_readfirstlane(sRng[1][j]);
  }

  f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) dkacc[db][j] = dvacc[db][j] = 0.f;

  const float c = s.scale * kLog2e;
  char* sdSg = sdS;
  float2* sSt = sStat;

  // A block's dQ rows are stored at the start of the next iteration (or
  // after the last one), not before the wait at the end of their own: vmcnt
  // counts stores too, and that wait is for the next block's loads only.
  uint2 pend[4];
  uint16_t* pend_out = nullptr;
  auto store_pending = [&]() __attribute__((always_inline)) {
    if (pend_out != nullptr) {
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) *reinterpret_cast<uint2*>(pend_out + jq * 8) = pend[jq];
    }
    pend_out = nullptr;
  };

  auto step = [&](int it, auto stage) __attribute__((always_inline)) {
    constexpr int buf = decltype(stage)::value;
    const int ib = it / G, h = g * G + it % G;
    const int trow0 = t0 + ib * kSB;  // the block's first local row
    const char* sQ = buf == 0 ? st0 : st1;
    const char* sdO = sQ + L::qtile;
    // The next block goes to the other stage (last read before the last
    // barrier), one load per k-step of the key phase's S / dP products
    // (all at once on a wave whose key block no row of this block attends).
    const bool more = it + 1 < n_it;
    static_assert(2 * L::PER_T <= KK, "one direct load per k-step covers the block");
    store_pending();
    // Per-lane LDS offsets from an opaque copy of the lane index: hoisted
    // out of the loop, they would hold registers that the dK / dV
    // accumulators need.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int n = ln & 31, kg = ln >> 5;
    const int tr_row = 4 * kg + ((ln & 15) >> 2);  // transpose-load row within a group of 8
    const int tr_g = (ln >> 4) & 1, tr_s = ln & 3;
    const int drow = 8 * wk + (ln >> 3), dc = ln & 7;
    const int kb = wk * kSB + n;
    const int nat_swz = swz<D>(n);

    // Row statistics of the block: delta = dO . O (float32) over 8 lanes
    // per row, and lse in base 2.  Rows past the chunk take zeros.
    {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < OE; ++e) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(sdO + drow * RP + (((dc * OE + e) ^ swz<D>(drow)) << 4));
#pragma unroll
        for (int i = 0; i < 8; ++i) part = fmaf(static_cast<float>(x[i]), static_cast<float>(ov[e][i]), part);
      }
      // sum over the row's 8 lanes with DPP moves (lane ^ 1, lane ^ 2 in
      // a quad, then lane 7 - i in a group of 8): no LDS round trips
      part += dpp_move<0xB1>(part);
      part += dpp_move<0x4E>(part);
      part += dpp_move<0x141>(part);
      const bool in_chunk = trow0 + drow < s.q_len;
      if (dc == 0) sSt[drow] = in_chunk ? make_float2(lsev * kLog2e, part) : make_float2(0.f, 0.f);
    }
    if (it + 1 < n_it) load_o(it + 1);
    lds_barrier();  // statistics of the block

    // Key phase: S, dP, softmax and dS for this wave's key block; dV, dK.
    const bool live = wqlo < trow0 + kSB && wqhi > trow0;
    if (!live && more) issue_tile(it + 1, buf ^ 1, 0, 2 * L::PER_T);
    if (live) {
      f32x16 sacc, pacc;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) sacc[jj] = pacc[jj] = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int pos = n * RP + (((2 * kk + kg) ^ nat_swz) << 4);
        const int kpos_l = kb * RP + (((2 * kk + kg) ^ nat_swz) << 4);
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQ + pos);
        const bf16x8 ao = *reinterpret_cast<const bf16x8*>(sdO + pos);
        const bf16x8 bk = *reinterpret_cast<const bf16x8*>(sK + kpos_l);
        if (more && kk < 2 * L::PER_T) issue_tile(it + 1, buf ^ 1, kk, kk + 1);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, sacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vf[kk], pacc, 0, 0, 0);
        // LDS reads at most two k-steps ahead of their products
        if (kk % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
      // sacc[jj] = S[row trow0 + (jj/4)*8 + kg*4 + jj%4][key kb]
      float pv[16], dsv[16];
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int r0 = jq * 8 + kg * 4;
        float zf[4] = {1.f, 1.f, 1.f, 1.f};
        // With dropout: the weights that multiply dO are P * Z * c, and
        // the gradient reaching P is dP = (dO V^T) * Z * c.
        if constexpr (DROP)
          keep_factors_col(s.drop, static_cast<uint32_t>(s.row_offset + trow0 + r0), static_cast<uint32_t>(pos0 + kb),
                           static_cast<uint32_t>(b * s.h_q + h), zf);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int jj = jq * 4 + e;
          const float2 st = sSt[r0 + e];
          float p = __builtin_amdgcn_exp2f(fmaf(sacc[jj], c, -st.x));
          const unsigned rel = static_cast<unsigned>(trow0 + r0 + e - mask_lo);
          p = rel < mask_span ? p : 0.f;  // a select: also clears inf
          pv[jj] = DROP ? p * zf[e] : p;
          dsv[jj] = DROP ? p * (pacc[jj] * zf[e] - st.y) : p * (pacc[jj] - st.y);
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
      // dS, key-major: this lane's key row, rows (jj/4)*8 + kg*4 + [0, 4).
      char* dsr = sdSg + wk * L::dstile + n * L::DSP + kg * 8;
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        bf16x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = dsb[jq >> 1][(jq & 1) * 4 + e];
        *reinterpret_cast<bf16x4*>(dsr + jq * 16) = x;
      }
      // dV^T += dO^T P, dK^T += Q^T dS (k = block rows, accumulator order).
#pragma unroll
      for (int kk2 = 0; kk2 < 2; ++kk2) {
        const int r_a = 16 * kk2 + tr_row, r_b = r_a + 8;
        const int sw_a = swz<D>(r_a), sw_b = swz<D>(r_b);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int chunk = 4 * db + 2 * tr_g + (tr_s >> 1);
          const int half = (tr_s & 1) * 8;
          const int pa = r_a * RP + ((chunk ^ sw_a) << 4) + half;
          const int pb_ = r_b * RP + ((chunk ^ sw_b) << 4) + half;
          const bf16x8 a_do = lds_tr_pair(sdO + pa, sdO + pb_);
          const bf16x8 a_q = lds_tr_pair(sQ + pa, sQ + pb_);
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_do, pb[kk2], dvacc[db], 0, 0, 0);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_q, dsb[kk2], dkacc[db], 0, 0, 0);
          if (db % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    lds_barrier();  // dS of every live key block

    // dQ phase: wave wk < DB owns columns 32 wk .. 32 wk + 31.
    if (wk < DB) {
      f32x16 qacc;
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) qacc[jj] = 0.f;
#pragma unroll
      for (int jb = 0; jb < kSW; ++jb) {
        if (!(rlo[jb] < trow0 + kSB && rhi[jb] > trow0)) continue;  // uniform
        const char* sdj = sdSg + jb * L::dstile;
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
          const int ra = jb * kSB + 16 * kk2 + tr_row, rb = ra + 8;
          const int chunk = 4 * wk + 2 * tr_g + (tr_s >> 1);
          const int half = (tr_s & 1) * 8;
          const bf16x8 a_k = lds_tr_pair(sK + ra * RP + ((chunk ^ swz<D>(ra)) << 4) + half,
                                         sK + rb * RP + ((chunk ^ swz<D>(rb)) << 4) + half);
          const int da = 16 * kk2 + tr_row, dbr = da + 8;
          const int col = (2 * tr_g + (tr_s >> 1)) * 16 + half;
          const bf16x8 b_ds = lds_tr_pair(sdj + da * L::DSP + col, sdj + dbr * L::DSP + col);
          qacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_k, b_ds, qacc, 0, 0, 0);
        }
      }
      // qacc[jj] = dQ^T[d = 32 wk + (jj/4)*8 + kg*4 + jj%4][row trow0 + n];
      // stored at the start of the next iteration
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        pend[jq].x = pack_bf16x2(qacc[4 * jq] * s.scale, qacc[4 * jq + 1] * s.scale);
        pend[jq].y = pack_bf16x2(qacc[4 * jq + 2] * s.scale, qacc[4 * jq + 3] * s.scale);
      }
      pend_out = trow0 + n < t0 + nrows
                     ? dq + ((static_cast<int64_t>(b) * s.q_len + trow0 + n) * s.h_q + h) * D + wk * 32 + kg * 4
                     : nullptr;
    }
    __builtin_amdgcn_s_waitcnt(0);  // the next blocks' direct loads and O rows have landed
    __syncthreads();                // next stages ready; dS and statistics free
  };
  for (int it = 0; it < n_it; it += 2) {
    step(it, Stage<0>{});
    if (it + 1 < n_it) step(it + 1, Stage<1>{});
  }
  store_pending();

  // dkacc[db][jj] = dK^T[d = 32db + (jj/4)*8 + kg*4 + jj%4][key kb0]
  if (kok) {
    const int64_t kv_row = (static_cast<int64_t>(b) * s.kv_len + (kpos - s.kv_begin)) * s.h_kv + g;
    uint16_t* dkr = dk + kv_row * D + (lane >> 5) * 4;
    uint16_t* dvr = dv + kv_row * D + (lane >> 5) * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        uint2 a2, bb;
        a2.x = pack_bf16x2(dkacc[db][4 * jq] * s.scale, dkacc[db][4 * jq + 1] * s.scale);
        a2.y = pack_bf16x2(dkacc[db][4 * jq + 2] * s.scale, dkacc[db][4 * jq + 3] * s.scale);
        bb.x = pack_bf16x2(dvacc[db][4 * jq], dvacc[db][4 * jq + 1]);
        bb.y = pack_bf16x2(dvacc[db][4 * jq + 2], dvacc[db][4 * jq + 3]);
        *reinterpret_cast<uint2*>(dkr + db * 32 + jq * 8) = a2;
        *reinterpret_cast<uint2*>(dvr + db * 32 + jq * 8) = bb;
      }
  }
}

template <int D, bool DROP>
hipError_t bwd_short_t(const BwdArgs& a, hipStream_t st) {
  AttnShape s;
  s.batch = a.batch; s.seq_len = a.seq_len; s.row_offset = a.row_offset; s.q_len = a.q_len;
  s.h_q = a.h_q; s.h_kv = a.h_kv; s.head_dim = D; s.group = a.h_q / a.h_kv; s.scale = a.scale;
  s.kv_begin = a.kv_begin; s.kv_len = a.kv_len;
  s.drop = drop_params(a.drop.thr, a.drop.scale, a.drop.seed, a.drop.offset);
  MetaView m = meta_view(a.meta, a.batch, a.seq_len, a.q_len);
  // Bins: at most one per non-padding segment, and at most the layout's bound.
  const int64_t nb = std::min<int64_t>(max_bins(a.batch, a.q_len), std::max(a.n_seg, 0));
  const int64_t n_zr = static_cast<int64_t>(a.batch) * ((a.q_len + kZT - 1) / kZT);
  const int64_t n_zk = static_cast<int64_t>(a.batch) * ((a.kv_len + kZT - 1) / kZT);
  const int64_t grid = nb * a.h_kv + n_zr + n_zk;
  if (grid == 0) return hipSuccess;
  hipError_t e = mark(a.mark_start, st);
  if (e != hipSuccess) return e;
  bwd_short_kernel<D, DROP><<<dim3(static_cast<unsigned>(grid)), kThreads, 0, st>>>(
      s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), static_cast<const uint16_t*>(a.v),
      static_cast<const uint16_t*>(a.d_o), static_cast<const uint16_t*>(a.o), a.lse, m,
      static_cast<uint16_t*>(a.dq), static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv),
      static_cast<int>(nb), static_cast<int>(n_zr));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return mark(a.mark_stop, st);
}

}  // namespace

bool bwd_short_applies(const BwdArgs& a) {
  return a.dtype == 1 && (a.head_dim == 64 || a.head_dim == 128) && a.max_seg_k >= 0 && a.max_seg_k <= kBinCap &&
         a.n_seg <= kBinMaxSeg && static_cast<int64_t>(a.batch) * a.q_len > 0;
}

hipError_t launch_bwd_short(const BwdArgs& a, hipStream_t st) {
  const bool drop = a.drop.thr != 0;
  switch (a.head_dim) {
    case 64: return drop ? bwd_short_t<64, true>(a, st) : bwd_short_t<64, false>(a, st);
    case 128: return drop ? bwd_short_t<128, true>(a, st) : bwd_short_t<128, false>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bd
