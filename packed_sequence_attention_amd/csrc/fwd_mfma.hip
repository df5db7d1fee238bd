// bf16 matrix-core forward of block-diagonal packed attention for gfx950.
//
// Automodel page "feat(distributed): block-diagonal varlen CP for packed
// sequences": Summary (varlen attention over packed documents, block-causal
// per document) and Design overview (one GPU's contiguous query chunk against
// the whole row's K/V).  The online softmax (running max, running sum,
// rescaled accumulator) is the standard streaming form of softmax attention.
//
// Work decomposition (one workgroup = 4 waves):
//   workgroup = (batch row b, 4 query heads sharing one K/V head, 32 local
//   query rows); wave w owns query head 4*hg + w for those 32 rows, so all
//   four waves share every K/V tile staged in LDS (grouped-query reuse) and
//   have the same live key range.
//   Key tiles are 32 keys anchored at multiples of 32 in the row; the tiles
//   from the one holding the workgroup's last row down to the one holding
//   doc_start(first real row) are visited, in descending order (the first
//   one is known before the metadata arrives), and the element mask is
//   applied only on tiles that are not entirely allowed.
// Matrix-core layout (v_mfma_f32_32x32x16_bf16, lane l, n = l % 32,
// kg = l / 32):
//   S^T = K Q^T per 32-key block: A = K rows from LDS, B = the wave's Q rows
//   held in registers; accumulator element j is key (j/4)*8 + kg*4 + j%4,
//   query n, so each lane owns one query row and its softmax statistics stay
//   in the lane (the two lanes of a row exchange one value per block).
//   O^T += V^T P^T: B = P straight from the accumulator (bf16), A = V^T read
//   with the LDS transpose load (ds_read_b64_tr_b16) from row-major V, with
//   the key order of the accumulator; O^T accumulates in registers.
// K / V tiles reach LDS by direct global -> LDS loads (buffer form: keys past
// the row read as zero) into a two-stage buffer; the loads of the next tile
// are spread over the tile's S products.  32-key tiles keep a workgroup's
// LDS at 32 KB, so three workgroups (three waves per SIMD) fit on a CU
// (head_dim 256: 64 KB and two).
// Rows are stored without padding, the 16-byte chunk c of row r at chunk
// c ^ f(r), which keeps both the row reads (16 rows, one chunk) and the
// transpose reads (4 rows x 4 chunks) free of bank conflicts.
// Softmax in base 2 with scale*log2(e) folded in; the running max is only
// raised when it grows by more than 8 (a factor 256), which keeps every
// exponent <= 2^8 and skips most accumulator rescales; the result is the
// same function since numerator and denominator share the reference.
#include <limits.h>
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace bd {
namespace {

constexpr int kBN = 32;  // keys per tile
constexpr int kBM = 32;  // query rows per workgroup (one per lane pair)
static_assert(kBM == kOrderQB, "the metadata's query-tile order is built for this tile size");

template <int D>
struct FwdLds {
  static constexpr int RP = D * 2;                 // row pitch (bytes), swizzled chunks
  static constexpr int tile = 2 * kBN * RP;        // K tile then V tile (one stage)
  static constexpr int NCH = kBN * (D / 8) / 256;  // direct loads per thread per tensor
};

// Chunk swizzle of row r of a K / V tile.  A bank depends on the chunk index
// mod 16 only for row pitches of 256 and 512 bytes, so head_dim 256 uses
// the swizzle of 128 (it permutes the low four bits of the chunk index).
template <int D>
__device__ __forceinline__ int rswz(int r) {
  if constexpr (D >= 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Workgroups per CU: three at head_dim 64 / 128 (32 KB of LDS each), two at
// 256 (64 KB; the O^T accumulators and Q fragments take 192 registers).
template <int D>
constexpr int kFwdOcc = D == 256 ? 2 : 3;

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
__global__ __launch_bounds__(256, kFwdOcc<D>) void fwd_mfma_kernel(AttnShape s, const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k,
                                                          const uint16_t* __restrict__ v, MetaView m,
                                                          uint16_t* __restrict__ o,
                                                          float* __restrict__ lse, int n_qtg, int n_hg,
                                                          int slots, int hpw) {
  constexpr int KK = D / 16;  // k-steps of Q K^T
  constexpr int DB = D / 32;  // 32-wide blocks of O^T
  constexpr int CH = D / 8;   // 16-byte chunks per K/V row
  using L = FwdLds<D>;
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
  // The metadata and Q loads go out together, without branches (rows past
  // the chunk read the chunk's last row and are zeroed below).
  const int64_t btc = static_cast<int64_t>(b) * s.q_len + (valid ? t : s.q_len - 1);
  const int lo_l = m.row_lo[btc], hi_l = m.row_hi[btc];
  bf16x8 qf[KK];
  {
    const uint16_t* qrow = q + (btc * s.h_q + h) * D + kg * 8;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qrow + kk * 16);
  }
  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const float c = s.scale * kLog2e;

  // Direct load c (of 2 NCH: K and V chunks alternately) of key tile kt into
  // stage buf.  With live == false the load reads nothing (zero-sized
  // resource) and writes zeros into the free stage: it is issued without a
  // branch, which would split the S block and stop the scheduler from
  // overlapping its LDS reads with the products.
  // The K/V buffer holds keys [kv_begin, kv_begin + kv_len) of every row;
  // kv0 is its first key of (b, g).  Visited tiles start at or after
  // kv_begin (a multiple of 64), so a tile's offset from there is >= 0.
  const int64_t kv0 = (static_cast<int64_t>(b) * s.kv_len * s.h_kv + g) * D;
  const int kv_stride = s.h_kv * D;
  const int kv_bytes = (s.kv_len * kv_stride - g * D) * 2;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
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
  static_assert(2 * L::NCH <= KK, "at most one direct load per step of the first S block");

  // Key tiles are visited from the last one (the tile's diagonal, known from
  // its position) down to the first document start, so the first tile's
  // loads go out with the metadata and Q loads; a row's result depends only
  // on the tiles that are not fully masked for it, visited in descending
  // order whatever the chunk (fully masked tiles change nothing).
  const int kt1 = (s.row_offset + min((qtg + 1) * tpw * kBM - 1, s.q_len - 1)) / kBN;  // the workgroup's last row
#pragma unroll
  for (int cc = 0; cc < 2 * L::NCH; ++cc) issue_chunk(kt1, 0, cc, true);
  // Keep the metadata reductions below these loads, and the Q loads above
  // them (the compiler would otherwise move each load next to its use).
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) asm volatile("" ::"v"(qf[kk]));

  const int lo = valid ? lo_l : 0, hi = valid ? hi_l : 0;
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

  const int nat_swz = rswz<D>(n);
  const int tr_row = 4 * kg + ((lane & 15) >> 2);
  const int tr_g = (lane >> 4) & 1, tr_s = lane & 3;
  // Byte offsets in a V tile of this lane's two transpose reads for block db
  // (rows tr_row and tr_row + 8 of each 16-row group; the swizzle repeats
  // every 16 rows, so other groups add a multiple of 16 rows).  Each read's
  // address is the stage's base plus one integer: the compiler tags an LDS
  // access with its LDS object only through a few address steps, and an
  // untagged read is made to wait for every direct load in flight (here the
  // next tile's, into the other stage) in the middle of the products.
  // Blocks 4..7 (head_dim 256) read 256 bytes further along the same rows:
  // the swizzle only permutes the low four bits of the chunk index.
  constexpr int DBT = DB < 4 ? DB : 4;
  int tro[DBT][2];
#pragma unroll
  for (int db = 0; db < DBT; ++db) {
    const int chunk = 4 * db + 2 * tr_g + (tr_s >> 1);
    const int half = (tr_s & 1) * 8;
    tro[db][0] = tr_row * RP + ((chunk ^ rswz<D>(tr_row)) << 4) + half;
    tro[db][1] = (tr_row + 8) * RP + ((chunk ^ rswz<D>(tr_row + 8)) << 4) + half;
  }

  if (kmax_g > kmin_g) {
    // kt1 >= (kmax - 1) / kBN: extra tiles are fully masked.  No tile before
    // the K/V buffer's first key is visited (the host checks that the rows'
    // keys lie in the buffer; the clamp keeps a mismatched table in bounds).
    const int kt0 = max(kmin_g, s.kv_begin) / kBN;
    if (!valid) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) qf[kk][i] = static_cast<__bf16>(0.f);
    }
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
        f32x16 sacc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sacc[j] = 0.f;
        const int rown = sb * 32 + n;
        auto kread = [&](int kk) {
          return *reinterpret_cast<const bf16x8*>(sK + rown * RP + (((2 * kk + kg) ^ nat_swz) << 4));
        };
        if constexpr (D <= 128) {
          // K row reads two k-steps ahead of their products (left alone, the
          // compiler issues each read after the previous product and every
          // product waits for its read).  Not at head_dim 256, whose
          // registers are not free for it.
          constexpr int KPF = 2;
          bf16x8 ak[KK];
#pragma unroll
          for (int kk = 0; kk < KPF; ++kk) ak[kk] = kread(kk);
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            if (kk + KPF < KK) ak[kk + KPF] = kread(kk + KPF);
            if (sb == 0 && kk < 2 * L::NCH) issue_chunk(pre ? kt - 1 : kt, buf ^ 1, kk, pre);
            __builtin_amdgcn_sched_barrier(0);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[kk], qf[kk], sacc, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) {
            const bf16x8 a = kread(kk);
            if (sb == 0 && kk < 2 * L::NCH) issue_chunk(pre ? kt - 1 : kt, buf ^ 1, kk, pre);
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc, 0, 0, 0);
          }
        }
        // sacc[j] = S[key k0 + sb*32 + (j/4)*8 + kg*4 + j%4][row n]
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
        // V^T transpose reads of the O^T products, flattened over (k-step,
        // column block) and issued two ahead of their products, the first two
        // before the softmax (head_dim 64 / 128; at 256 the registers for
        // them are not free, and each read directly precedes its product).
        constexpr int NV = 2 * DB;
        constexpr int PFV = D <= 128 ? 2 : 0;
        auto vread = [&](int st_) {
          const int r1 = (sb * 32 + 16 * (st_ / DB)) * RP + ((st_ % DB) >> 2) * 256;
          return lds_tr_pair(sV + (tro[(st_ % DB) & 3][0] + r1), sV + (tro[(st_ % DB) & 3][1] + r1));
        };
        bf16x8 vq[NV];
        if constexpr (PFV > 0) {
#pragma unroll
          for (int st_ = 0; st_ < PFV; ++st_) vq[st_] = vread(st_);
          __builtin_amdgcn_sched_barrier(0);
        }
        // (maximum: no NaN quieting of the operands, three per instruction)
        float mx = sacc[0];
#pragma unroll
        for (int j = 1; j < 16; ++j) mx = __builtin_elementwise_maximum(mx, sacc[j]);
        mx = pair32_max(mx);
        const float mnew = __builtin_elementwise_maximum(mrun, mx * c);
        const bool need = mnew > mrun + 8.f;
        // A row whose reference is still -inf has accumulated nothing (every
        // weight so far was exp2(-inf) = 0): it takes the new reference
        // without a rescale, so the first live tile of a row costs none.
        const bool resc = need && mrun != -INFINITY;
        if (__any(resc)) {
          const float alpha = resc ? __builtin_amdgcn_exp2f(mrun - mnew) : 1.f;
          lrun *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[db][j] *= alpha;
        }
        if (need) mrun = mnew;
        const float mu = (mrun == -INFINITY) ? 0.f : mrun;
        float p[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(sacc[j], c, -mu));
        // The row sum in float32 (of the undropped weights), as a tree.
        float ps[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) ps[j] = p[j] + p[8 + j];
#pragma unroll
        for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
          for (int j = 0; j < w; ++j) ps[j] += ps[j + w];
        lrun += ps[0];
        if constexpr (DROP) {
          // dropout of the weights that multiply V (the row sum above is the
          // undropped one): this lane's row, keys in groups of 4
          const uint32_t ip = static_cast<uint32_t>(s.row_offset + qt * kBM + n);
          const uint32_t bh = static_cast<uint32_t>(b * s.h_q + h);
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            float f[4];
            keep_factors_row(s.drop, ip, static_cast<uint32_t>(k0 + sb * 32 + g4 * 8 + kg * 4), bh, f);
#pragma unroll
            for (int e = 0; e < 4; ++e) p[g4 * 4 + e] *= f[e];
          }
        }
        bf16x8 pb[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pb[0][i] = static_cast<__bf16>(p[i]);
          pb[1][i] = static_cast<__bf16>(p[8 + i]);
        }
        // O^T += V^T P^T: A = V^T (rows = keys in accumulator order).
#pragma unroll
        for (int st_ = 0; st_ < NV; ++st_) {
          if constexpr (PFV > 0) {
            if (st_ + PFV < NV) vq[st_ + PFV] = vread(st_ + PFV);
            __builtin_amdgcn_sched_barrier(0);
          } else {
            vq[st_] = vread(st_);
          }
          oacc[st_ % DB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[st_], pb[st_ / DB], oacc[st_ % DB], 0, 0, 0);
          if constexpr (PFV > 0) __builtin_amdgcn_sched_barrier(0);
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

  const float ltot = pair32_sum(lrun);
  if (valid) {
    const bool any = ltot > 0.f;
    const float inv = any ? 1.f / ltot : 0.f;
    uint16_t* orow = o + (bt * s.h_q + h) * D + kg * 4;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        uint2 pk;
        pk.x = pack_bf16x2(oacc[db][4 * jq] * inv, oacc[db][4 * jq + 1] * inv);
        pk.y = pack_bf16x2(oacc[db][4 * jq + 2] * inv, oacc[db][4 * jq + 3] * inv);
        *reinterpret_cast<uint2*>(orow + db * 32 + jq * 8) = pk;
      }
    if (kg == 0)
      lse[(static_cast<int64_t>(b) * s.h_q + h) * s.q_len + t] =
          any ? fmaf(mrun, kLn2, logf(ltot)) : -INFINITY;
  }
}

template <int D, bool DROP>
hipError_t fwd_mfma_t(const FwdArgs& a, hipStream_t st) {
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
  hipError_t e = mark(a.mark_start, st);
  if (e != hipSuccess) return e;
  fwd_mfma_kernel<D, DROP><<<dim3(static_cast<unsigned>(grid)), 256, 0, st>>>(
      s, static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
      static_cast<const uint16_t*>(a.v), m, static_cast<uint16_t*>(a.o), a.lse, n_qtg, n_hg,
      device_cu_count() * kFwdOcc<D>, hpw);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return mark(a.mark_stop, st);
}

}  // namespace

bool mfma_supported(int dtype, int head_dim, int h_q, int h_kv) {
  return dtype == 1 && (head_dim == 64 || head_dim == 128 || head_dim == 256) && h_kv > 0 && h_q % h_kv == 0;
}

bool fwd_mfma_fits(int64_t kv_len, int64_t h_kv, int64_t head_dim) {
  // a (batch row, K/V head)'s keys, including the last tile's keys past the
  // window, must be addressable with 31-bit buffer offsets
  return (kv_len + kBN) * h_kv * head_dim * 2 < (int64_t{1} << 31);
}

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t st) {
  const bool drop = a.drop.thr != 0;
  switch (a.head_dim) {
    case 64: return drop ? fwd_mfma_t<64, true>(a, st) : fwd_mfma_t<64, false>(a, st);
    case 128: return drop ? fwd_mfma_t<128, true>(a, st) : fwd_mfma_t<128, false>(a, st);
    case 256: return drop ? fwd_mfma_t<256, true>(a, st) : fwd_mfma_t<256, false>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bd
