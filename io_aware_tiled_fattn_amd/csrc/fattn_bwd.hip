// Backward kernels: gradients of exact attention by recomputation.
//
// Method (page "从零实现 FlashAttention-2：分块在线 Softmax", backward section; page "mianstack
// q-0277", backward section; page "FlashAttention为什么更快更省显存", recompute section): the
// probability tiles are rebuilt from Q, K and the per-row statistic saved by the forward
// (LSE = m + ln l, so P = exp(S - LSE)) instead of being stored. With the causal mask fused into
// the tile loop, only tiles on or below the diagonal are visited. The chain rule through
// O = P V and the row softmax gives, per (batch, head):
//     dV = P^T dO,  dP = dO V^T,  D_i = sum_t dO[i,t] O[i,t],  dS = P * (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels (fattn_bwd runs 3 then 2: the dQ kernel also computes D and writes it for 2):
//  1. bwd_pre:   D = rowsum(dO * O) (float32 workspace), one pass over O and dO.
//  2. bwd_dkdv_pair: one work-group per (b*h, 128-key tile); waves p and p + 4 share 32 keys:
//               the first keeps K in registers and accumulates dV (S, P, dV += P^T dO), the
//               second keeps V and accumulates dK (dP, dS, dK += dS^T Q), taking P from the first
//               through LDS, one query tile behind it. Q, dO tiles of 64 queries stream
//               memory -> LDS, three stages deep. Scores are formed as S = Q K^T so that every
//               lane owns ONE key: P and dS then serve directly as the MFMA A operand of the
//               second product, whose B operand (dO or Q with the query index as reduction
//               index) comes from the same LDS tiles through ds_read_b64_tr_b16.
//  3. bwd_dq:    one work-group per (b*h, 256-query tile; 128 in block-sparse runs), the
//               forward's layout: S^T = K Q^T and dP^T = V dO^T give each lane ONE query (its LSE
//               and D are per-lane scalars); dQ^T += K^T dS^T takes K^T from the row-major K tile
//               via the transposed read.
// Every kernel writes its outputs once; there are no atomics, so results are deterministic.
#include <type_traits>

#include "fattn_device.hpp"
#include "fattn_launch.hpp"

#include "../../include/fattn.h"

namespace fattn {
namespace {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dO;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dvec;  // D = rowsum(dO * O): read, or written by the dQ kernel that computes it
  int N;
  int ntiles;   // tiles per head along the grid's sequence axis
  int bh_total; // B * H
  int hgroup;   // causal grid order: heads of an XCD taken this many at a time
  float c;      // scale * log2(e) (signed)
  float scale;  // signed softmax scale
  DropParams drop;  // dropout on P (DROP instances only)
  const uint8_t* bmask;  // block mask [B*H][nb][nb] over 128 x 128 (query, key) blocks (SPARSE)
  int nb;                // ceil(N / 128)
};

template <typename TR>
__device__ inline float to_f32(uint16_t x);
template <>
__device__ inline float to_f32<Bf16>(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
template <>
__device__ inline float to_f32<F16>(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

// ---------------------------------------------------------------------------------------------
// 1. D = rowsum(dO * O): D/8 threads per row, 16-byte loads.

// Sum of the 8 products of one 16-byte chunk of O and dO, in a fixed order (the dQ kernel's own
// computation of D must match this kernel bit for bit).
template <typename TR>
__device__ inline float chunk_dot(u32x4 a, u32x4 b) {
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sum = fmaf(to_f32<TR>((uint16_t)(a[i] & 0xffff)), to_f32<TR>((uint16_t)(b[i] & 0xffff)), sum);
    sum = fmaf(to_f32<TR>((uint16_t)(a[i] >> 16)), to_f32<TR>((uint16_t)(b[i] >> 16)), sum);
  }
  return sum;
}

template <typename TR, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ dvec, long long rows) {
  constexpr int TPR = D / 8;
  const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float sum = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)(o + row * D + part * 8);
    const u32x4 b = *(const u32x4*)(dO + row * D + part * 8);
    sum = chunk_dot<TR>(a, b);
  }
  // the tree the dQ kernel reproduces when it computes D itself: partner chunks p ^ TPR/2, ...
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, TPR);
  if (row < rows && part == 0) dvec[row] = sum;
}

// ---------------------------------------------------------------------------------------------
// Shared by the two matmul kernels.

// Block id -> (head, tile along the grid's sequence axis). Each of the 8 XCDs (block x runs on
// XCD x % 8) takes a contiguous range of heads. With the causal mask the tiles with the most work
// run first across all heads of an XCD: for dK/dV that is the first key tile (it sees every query
// tile), for dQ the last query tile.
__device__ inline void bwd_block_coords(int bid, int nblocks, int ntiles, int bh_total, bool causal,
                                        bool long_is_low, int hgroup, int* bh, int* t) {
  if ((bh_total & 7) == 0) {
    const int hpx = bh_total >> 3;
    const int xcd = bid & 7, local = bid >> 3;
    if (causal) {
      int hh, r;
      causal_xcd_order(local, hpx, ntiles, hgroup, &hh, &r);
      *bh = xcd * hpx + hh;
      *t = long_is_low ? r : ntiles - 1 - r;
    } else {
      const int hh = local / ntiles;
      *bh = xcd * hpx + hh;
      *t = local - hh * ntiles;
    }
    return;
  }
  const int logical = xcd_remap(bid, nblocks);
  *bh = logical / ntiles;
  *t = logical - *bh * ntiles;
  if (causal && !long_is_low) *t = ntiles - 1 - *t;
}

// Byte address, inside a tile swizzled with swz_dual, of the 8 bytes this lane contributes to a
// ds_read_b64_tr_b16: row R, 16-bit element column E (a multiple of 4).
template <int D>
__device__ inline int tr_read_addr(int R, int E) {
  return R * (D * 2) + (((E >> 3) ^ swz_dual<D>(R)) << 4) + ((E & 7) << 1);
}
// Byte address of the 16-byte chunk c of row R in a tile swizzled with swz_dual.
template <int D>
__device__ inline int row_read_addr(int R, int c) {
  return R * (D * 2) + ((c ^ swz_dual<D>(R)) << 4);
}

// ---------------------------------------------------------------------------------------------
// 2. dK, dV in one pass, by wave pairs.
//
// One work-group per (b*h, 128-key tile) of 8 waves; waves p and p + 4 (which share a SIMD) own
// the same 32 keys. Wave p ("A") keeps K in registers and accumulates dV: S = Q K^T,
// P = exp(S - LSE), dV += P^T dO. Wave p + 4 ("B") keeps V and accumulates dK: dP = dO V^T,
// dS = P (dP - D), dK += dS^T Q, taking P from A through LDS (16-bit, as rounded for the dV
// product; with dropout, a set sign bit marks a dropped element, so only A draws the keep mask).
// B works one query tile behind A, so the two never wait for each other inside a tile: while A runs tile i, B runs tile i - 1; the tiles i - 1, i and the one being fetched
// (i + 1) sit in three LDS stages, and P goes through two exchange buffers. S is computed once
// per (query, key) pair, and each wave holds one accumulator and one operand set, so two waves
// share every SIMD and one wave's VALU work overlaps the other's MFMAs.

template <int D>
struct PairCfg {
  static constexpr int BKV = 128;               // keys per work-group (32 per wave pair)
  static constexpr int BQ = 64;                 // queries per tile
  static constexpr int NT = 512;                // 8 waves
  static constexpr int CPR = D / 8;
  static constexpr int LPT = BQ * CPR / NT;     // 16-byte loads per thread per tile per tensor
  static constexpr int TILE_B = BQ * D * 2;     // bytes of one Q (or dO) tile
  static constexpr int ROWS_B = 2 * BQ * 4;     // LSE (log2 domain) then D, float32
  static constexpr int STAGE_B = 2 * TILE_B + ROWS_B;
  static constexpr int NSTG = 3;
  static constexpr int XBUF_B = 4 * (BQ / 32) * 2 * 64 * 16;  // P of one tile: pairs x blocks x halves x lanes x 16 B
  static constexpr int LDS_B = NSTG * STAGE_B + 2 * XBUF_B;
  static_assert(BQ * CPR % NT == 0 && LPT >= 1, "tile split");
  static_assert(LDS_B <= 160 * 1024, "LDS");
};

template <typename TR>
__device__ inline void unpack2(uint32_t u, float& x, float& y);
template <>
__device__ inline void unpack2<Bf16>(uint32_t u, float& x, float& y) {
  x = __uint_as_float(u << 16);
  y = __uint_as_float(u & 0xffff0000u);
}
template <>
__device__ inline void unpack2<F16>(uint32_t u, float& x, float& y) {
  const f32x2v f = __builtin_convertvector(__builtin_bit_cast(f16x2v, u), f32x2v);
  x = f[0];
  y = f[1];
}

// SPARSE: block-sparse attention over 128 x 128 (query, key) blocks; the work-group's 128 keys are
// one mask column, and only the query tiles whose mask block is set are loaded and computed.
template <typename TR, int D, bool CAUSAL, bool BIG, bool DROP, bool SPARSE>
__global__ __launch_bounds__(PairCfg<D>::NT) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dkdv_pair_kernel(BwdArgs a) {
  using Cfg = PairCfg<D>;
  using vec8 = typename TR::vec8;
  constexpr int BKV = Cfg::BKV, BQ = Cfg::BQ, NT = Cfg::NT, CPR = Cfg::CPR, LPT = Cfg::LPT;
  constexpr int TILE_B = Cfg::TILE_B, NSTG = Cfg::NSTG;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS_B];
  uint8_t* const xbuf = smem + NSTG * Cfg::STAGE_B;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const bool role_a = w < 4;
  const int pair = w & 3;
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int N = a.N;

  int bh, jt;
  bwd_block_coords(blockIdx.x, gridDim.x, a.ntiles, a.bh_total, CAUSAL, true, a.hgroup, &bh, &jt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const size_t rowbase = (size_t)bh * (size_t)N;
  const uint16_t* __restrict__ Qh = a.q + head;
  const uint16_t* __restrict__ dOh = a.dO + head;

  const int key0 = jt * BKV + 32 * pair;  // first key of this wave pair
  const int key = key0 + lr;              // this lane's key
  const bool wave_active = key0 < N;

  f32x16 acc[D / 32];  // dV (A) or dK (B)
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;

  const int n_qt = (N + BQ - 1) / BQ;
  const int i_begin = CAUSAL ? (jt * BKV) / BQ : 0;

  // The swizzle repeats every 16 rows: when one load instruction spans a multiple of 16 rows,
  // load t lies exactly t*NT*16 bytes after load 0, and only load 0's offset is kept.
  constexpr bool kPeriodic = NT % CPR == 0 && (NT / CPR) % 16 == 0;
  uint32_t off[kPeriodic ? 1 : LPT];
#pragma unroll
  for (int i = 0; i < (kPeriodic ? 1 : LPT); ++i) {
    const int chunk = i * NT + tid;
    const int row = chunk / CPR, pos = chunk % CPR;
    off[i] = (uint32_t)(row * D * 2 + (pos ^ swz_dual<D>(row)) * 16);
  }
  auto off_t = [&](int t) { return kPeriodic ? off[0] + (uint32_t)(t * NT * 16) : off[t]; };
  const uint32_t head_bytes = BIG ? 0u : (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Qh, head_bytes);
  const __amdgpu_buffer_rsrc_t rdO = make_rsrc(dOh, head_bytes);
  // tiles are numbered by their position in the sequence the work-group visits (consecutive
  // tiles, or the allowed ones of a block-sparse run): position p sits in stage p % 3 and its P in
  // exchange buffer p % 2
  auto stage = [&](int p) { return smem + (p % NSTG) * Cfg::STAGE_B; };
  auto issue = [&](int i, int p) {
    uint8_t* st = stage(p) + w * 64 * 16;
    const uint32_t soff = (uint32_t)(i * BQ) * (D * 2);
    if (!BIG && (i + 1) * BQ <= N) {
#pragma unroll
      for (int t = 0; t < LPT; ++t) {
        const uint32_t add = kPeriodic ? (uint32_t)(t * NT * 16) : 0u;
        buffer_lds16(rQ, st + t * NT * 16, kPeriodic ? off[0] : off[t], soff + add);
        buffer_lds16(rdO, st + TILE_B + t * NT * 16, kPeriodic ? off[0] : off[t], soff + add);
      }
    } else if (!BIG) {
      // ragged last tile: the whole offset goes in the lane's offset register, which the
      // buffer's range check covers, so rows past the end read as zeros; A masks them (P = 0),
      // so B's dS is 0 there as well
#pragma unroll
      for (int t = 0; t < LPT; ++t) {
        buffer_lds16(rQ, st + t * NT * 16, off_t(t) + soff, 0u);
        buffer_lds16(rdO, st + TILE_B + t * NT * 16, off_t(t) + soff, 0u);
      }
    } else {
      // a head of 2 GiB or more: 64-bit addresses, rows past the end repeat row N - 1
#pragma unroll
      for (int t = 0; t < LPT; ++t) {
        const size_t src_row = (size_t)min(i * BQ + (t * NT + tid) / CPR, N - 1) * (D * 2);
        const uint32_t in_row = off_t(t) - (uint32_t)((t * NT + tid) / CPR * D * 2);
        global_lds16((const uint8_t*)Qh + src_row + in_row, st + t * NT * 16);
        global_lds16((const uint8_t*)dOh + src_row + in_row, st + TILE_B + t * NT * 16);
      }
    }
  };
  float lr2 = 0.f, dvr = 0.f;
  auto load_rows = [&](int i) {
    if (tid < BQ) {
      const int q = min(i * BQ + tid, N - 1);
      lr2 = a.lse[rowbase + q];  // scaled to log2 units when stored, so the load need not land first
      dvr = a.dvec[rowbase + q];
    }
  };
  auto store_rows = [&](int p) {
    if (tid < BQ) {
      float* rows = (float*)(stage(p) + 2 * TILE_B);
      rows[tid] = lr2 * kLog2e;
      rows[BQ + tid] = dvr;
    }
  };

  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // query tile i's mask block: row (i BQ) / 128, column jt (BKV = 128); the column's allowed rows
  // are scanned 64 at a time (MaskLine)
  static_assert(BKV == 128 && 128 % BQ == 0, "a dK/dV work-group is one mask column");
  constexpr int TPR = 128 / BQ;  // query tiles per mask row
  MaskLine mcol = mask_line(SPARSE ? a.bmask + (size_t)bh * a.nb * a.nb + jt : nullptr, a.nb, SPARSE ? a.nb : 0);
  // the visited tile after i: the next tile of i's mask row, else the first of the next allowed row
  auto next = [&](int i) {
    const int ii = i + 1;
    if (!SPARSE) return ii;
    if (ii >= n_qt) return n_qt;
    if (ii % TPR != 0) return ii;
    const int r = mask_next(mcol, ii / TPR, lane);
    return r >= (n_qt + TPR - 1) / TPR ? n_qt : r * TPR;
  };
  // A dense run visits the tiles i_begin, i_begin + 1, ...; a block-sparse run only the allowed
  // ones. Either way the visited tiles take positions 0, 1, ...
  int cur = SPARSE ? next(i_begin - 1) : i_begin;  // A's tile
  int prev = -1;                                   // B's tile (A's previous one)
  if (cur < n_qt) {
    load_rows(cur);
    issue(cur, 0);
  }
  // MFMA B operand of the first product: K for A (S = Q K^T), V for B (dP = dO V^T);
  // lane holds X[key][16s + 8h .. +7] (zeros past the last key; the loads themselves read key
  // N - 1, so they need no branch). The first query tile's loads are already in flight.
  vec8 xf[D / 16];
  {
    const uint16_t* src = (role_a ? a.k : a.v) + head + (size_t)min(key, N - 1) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      u32x4 r = *(const u32x4*)(src + 16 * s + 8 * h);
      if (key >= N) r = u32x4{0u, 0u, 0u, 0u};
      xf[s] = bitcast<vec8>(r);
    }
  }
  if (cur < n_qt) store_rows(0);
  // iteration p: A runs the tile at position p, B the one at p - 1; the last iteration is B's.
  // A dense run counts p over the tile indices i_begin .. n_qt.
  for (int p = 0; cur < n_qt || prev >= 0; ++p) {
    wait_vmcnt<0>();
    barrier_lds();
    const int nxt = cur < n_qt ? next(cur) : n_qt;
    if (nxt < n_qt) {
      load_rows(nxt);
      issue(nxt, p + 1);
    }
    const int i = role_a ? cur : prev;
    const int pos = role_a ? p : p - 1;
    const int q_base = i * BQ;
    const bool mine = role_a ? cur < n_qt : prev >= 0;
    if (mine && wave_active && !(CAUSAL && q_base + BQ - 1 < key0)) {
      const uint8_t* Qs = stage(pos);
      const uint8_t* dOs = Qs + TILE_B;
      const float* lse2s = (const float*)(Qs + 2 * TILE_B);
      const float* dvs = lse2s + BQ;
      const uint8_t* X1 = role_a ? Qs : dOs;  // A operand of the first product (row reads)
      const uint8_t* X2 = role_a ? dOs : Qs;  // B operand of the second (transposed reads)
      uint8_t* xb = xbuf + ((pos & 1) * 4 + pair) * (Cfg::XBUF_B / 4);
      const bool need_mask = (CAUSAL && key0 + 31 > q_base) || (q_base + BQ > N);
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        f32x16 s;
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          const vec8 xa = *(const vec8*)(X1 + row_read_addr<D>(qb * 32 + lr, 2 * st + h));
          s = TR::mma(xa, xf[st], s);
        }
        // all fragment reads first, so their latency hides behind the MFMA chain
        __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, D / 16, 0);
        // element 4j + r: query q_base + qb*32 + 8j + 4h + r, this lane's key
        u32x4* xq = (u32x4*)(xb + qb * 2048 + lane * 16);
        vec8 pk[2];
        if (role_a) {
          float p[16];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 l4 = *(const f32x4*)(lse2s + qb * 32 + 8 * j + 4 * h);
#pragma unroll
            for (int r = 0; r < 4; ++r) p[4 * j + r] = fmaf(s[4 * j + r], a.c, -l4[r]);
          }
          if (need_mask) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              const int qq = q_base + qb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
              p[e] = ((CAUSAL && key > qq) || qq >= N) ? -__builtin_inff() : p[e];
            }
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(p[e]);
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4 pu;
            if (!DROP) {
#pragma unroll
              for (int e2 = 0; e2 < 4; ++e2) pu[e2] = TR::pack2(p[8 * half + 2 * e2], p[8 * half + 2 * e2 + 1]);
              xq[half * 64] = pu;  // P for B
            } else {
              // B gets P with the sign bit marking a dropped element (P >= 0, so the sign is
              // free): it then needs no generator of its own; dV takes P M / (1 - p)
              // bit e: this lane's key for query q_base + 32 qb + 8 (2 half + e / 4) + 4h + e % 4
              const uint32_t bits = col_keep_bits((uint32_t)key >> 3, (uint32_t)(q_base + qb * 32 + 16 * half + 4 * h),
                                                  (uint32_t)bh, a.drop, lane);
              u32x4 ps;
#pragma unroll
              for (int e2 = 0; e2 < 4; ++e2) {
                const int e = 2 * e2;
                const bool k0 = (bits >> e) & 1u, k1 = (bits >> (e + 1)) & 1u;
                const float p0 = p[8 * half + e], p1 = p[8 * half + e + 1];
                ps[e2] = TR::pack2(k0 ? p0 : -p0, k1 ? p1 : -p1);
                pu[e2] = TR::pack2(k0 ? p0 * a.drop.inv_keep : 0.f, k1 ? p1 * a.drop.inv_keep : 0.f);
              }
              xq[half * 64] = ps;
            }
            pk[half] = bitcast<vec8>(pu);
          }
        } else {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const u32x4 pu = xq[half * 64];
            u32x4 du;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              const f32x4 d4 = *(const f32x4*)(dvs + qb * 32 + 8 * (2 * half + jj) + 4 * h);
#pragma unroll
              for (int r2 = 0; r2 < 2; ++r2) {
                const int e = 8 * half + 4 * jj + 2 * r2;  // element index in s
                float p0, p1;
                unpack2<TR>(pu[2 * jj + r2], p0, p1);
                const float dp0 = s[e], dp1 = s[e + 1];
                if (DROP) {
                  // kept: dS = P (dP / (1 - p) - D); dropped (sign bit set, value -P):
                  // dS = P (0 - D), which is the signed value times D
                  const bool k0 = !(__float_as_uint(p0) >> 31), k1 = !(__float_as_uint(p1) >> 31);
                  du[2 * jj + r2] = TR::pack2(k0 ? p0 * (dp0 * a.drop.inv_keep - d4[2 * r2]) : p0 * d4[2 * r2],
                                              k1 ? p1 * (dp1 * a.drop.inv_keep - d4[2 * r2 + 1]) : p1 * d4[2 * r2 + 1]);
                } else {
                  du[2 * jj + r2] = TR::pack2(p0 * (dp0 - d4[2 * r2]), p1 * (dp1 - d4[2 * r2 + 1]));
                }
              }
            }
            pk[half] = bitcast<vec8>(du);
          }
        }
        // dV += P^T dO (A) or dK += dS^T Q (B) over this block's two 16-query chunks
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int c = 2 * qb + half;
#pragma unroll
          for (int b = 0; b < D / 32; ++b) {
            const i16x4 x0 = lds_read_tr16(X2 + tr_read_addr<D>(16 * c + tr_row, 32 * b + tr_col));
            const i16x4 x1 = lds_read_tr16(X2 + tr_read_addr<D>(16 * c + tr_row + 8, 32 * b + tr_col));
            const i16x8 xx = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
            acc[b] = TR::mma(pk[half], bitcast<vec8>(xx), acc[b]);
          }
        }
        // likewise: the transposed reads of both chunks, then their MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * 2 * (D / 32), 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * (D / 32), 0);
      }
    }
    if (nxt < n_qt) store_rows(p + 1);
    prev = cur < n_qt ? cur : -1;
    cur = nxt;
  }

  if (!wave_active) return;
  uint16_t* out = role_a ? a.dv : a.dk;
  const float osc = role_a ? 1.f : a.scale;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = key0 + 8 * j + 4 * h + r;
      if (kk < N) {
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
          out[head + (size_t)kk * D + 32 * b + lr] = __builtin_bit_cast(uint16_t, TR::from_f32(acc[b][4 * j + r] * osc));
      }
    }
}

// ---------------------------------------------------------------------------------------------
// 3. dQ.
//
// One work-group per (b*h, 256-query tile; 128 queries in block-sparse runs), the forward's layout: S^T = K Q^T and dP^T = V dO^T
// give each lane ONE query (its LSE and D are per-lane scalars); dQ^T += K^T dS^T takes K^T from
// the K tile through the transposed read. K and V tiles of 64 keys stream memory -> LDS, two
// stages deep.

template <int D, int BQ_ = 256>
struct DqCfg {
  static constexpr int BQ = BQ_;              // queries per work-group (32 per wave)
  static constexpr int BK = 64;               // keys per step
  static constexpr int NT = BQ / 32 * 64;
  static constexpr int CPR = D / 8;
  static constexpr int LPT = BK * CPR / NT;
  static constexpr int TILE_B = BK * D * 2;
  static constexpr int STAGE_B = 2 * TILE_B;  // K then V
  static_assert(BK * CPR % NT == 0, "tile split");
};

// DROP: dS = P (dO V^T M / (1 - p) - D).
// SPARSE: block-sparse attention over 128 x 128 (query, key) blocks: a work-group of 128 queries
// (4 waves) is one mask row and loads and computes only the key tiles that row allows.
// WITH_D: compute D = rowsum(dO * O) of the wave's rows here (from the dO fragments already in
// registers and the O rows) instead of reading it, and write it for the dK/dV kernel; the result
// is the preprocess kernel's bit for bit (same chunk sums, same pairing tree).
template <typename TR, int D, bool CAUSAL, bool BIG, bool DROP, bool SPARSE, bool WITH_D>
__global__ __launch_bounds__((DqCfg<D, SPARSE ? 128 : 256>::NT)) __attribute__((amdgpu_waves_per_eu(2))) void bwd_dq_kernel(BwdArgs a) {
  using Cfg = DqCfg<D, SPARSE ? 128 : 256>;
  using vec8 = typename TR::vec8;
  constexpr int BQ = Cfg::BQ, BK = Cfg::BK, NT = Cfg::NT, CPR = Cfg::CPR, LPT = Cfg::LPT;
  constexpr int TILE_B = Cfg::TILE_B;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * Cfg::STAGE_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int N = a.N;

  int bh, qt;
  bwd_block_coords(blockIdx.x, gridDim.x, a.ntiles, a.bh_total, CAUSAL, false, a.hgroup, &bh, &qt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Kh = a.k + head;
  const uint16_t* __restrict__ Vh = a.v + head;

  const int q_base = qt * BQ;
  const int q0 = q_base + 32 * w;
  const int qrow = q0 + lr;
  const bool wave_active = q0 < N;
  const int wave_kv_end = CAUSAL ? min(q0 + 31, N - 1) + 1 : N;

  f32x16 acc[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;

  const int kv_end = CAUSAL ? min(N, q_base + BQ) : N;
  const int n_kv = (kv_end + BK - 1) / BK;

  // K tiles are read both row-wise and transposed (swz_dual); V tiles only row-wise.
  // Both swizzles repeat every 16 rows: when one load instruction spans a multiple of 16 rows,
  // load i lies exactly i*NT*16 bytes after load 0, and only load 0's offsets are kept.
  constexpr bool kPeriodic = NT % CPR == 0 && (NT / CPR) % 16 == 0;
  constexpr int NOFF = kPeriodic ? 1 : LPT;
  uint32_t offK[NOFF], offV[NOFF];
#pragma unroll
  for (int i = 0; i < NOFF; ++i) {
    const int chunk = i * NT + tid;
    const int row = chunk / CPR, pos = chunk % CPR;
    offK[i] = (uint32_t)(row * D * 2 + (pos ^ swz_dual<D>(row)) * 16);
    offV[i] = (uint32_t)(row * D * 2 + (pos ^ swz_rowread<D>(row)) * 16);
  }
  auto off_k = [&](int i) { return kPeriodic ? offK[0] + (uint32_t)(i * NT * 16) : offK[i]; };
  auto off_v = [&](int i) { return kPeriodic ? offV[0] + (uint32_t)(i * NT * 16) : offV[i]; };
  const uint32_t head_bytes = BIG ? 0u : (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(Kh, head_bytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(Vh, head_bytes);
  // key tile j into stage t & 1 (t = j except for block-sparse runs, which skip tiles)
  auto issue = [&](int j, int t) {
    uint8_t* st = smem + (t & 1) * Cfg::STAGE_B + w * 64 * 16;
    const uint32_t soff = (uint32_t)(j * BK) * (D * 2);
    if (!BIG && (j + 1) * BK <= N) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const uint32_t add = kPeriodic ? (uint32_t)(i * NT * 16) : 0u;
        buffer_lds16(rK, st + i * NT * 16, kPeriodic ? offK[0] : offK[i], soff + add);
        buffer_lds16(rV, st + TILE_B + i * NT * 16, kPeriodic ? offV[0] : offV[i], soff + add);
      }
    } else if (!BIG) {
      // ragged last tile: the whole offset goes in the lane's offset register, which the
      // buffer's range check covers, so rows past the end read as zeros (masked below)
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        buffer_lds16(rK, st + i * NT * 16, off_k(i) + soff, 0u);
        buffer_lds16(rV, st + TILE_B + i * NT * 16, off_v(i) + soff, 0u);
      }
    } else {
      // a head of 2 GiB or more: 64-bit addresses, rows past the end repeat row N - 1
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const size_t src_row = (size_t)min(j * BK + (i * NT + tid) / CPR, N - 1) * (D * 2);
        const uint32_t in_row = (uint32_t)((i * NT + tid) / CPR * D * 2);
        global_lds16((const uint8_t*)Kh + src_row + (off_k(i) - in_row), st + i * NT * 16);
        global_lds16((const uint8_t*)Vh + src_row + (off_v(i) - in_row), st + TILE_B + i * NT * 16);
      }
    }
  };

  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // Key tile j lies in mask column j / TPC. A block-sparse work-group holds 128 queries, one mask
  // row, and visits only the key tiles that row allows; the row is scanned 64 columns at a time
  // (MaskLine), only right after the vmcnt wait that empties the prefetch queue.
  static_assert(!SPARSE || (BQ == 128 && 128 % BK == 0), "a block-sparse dQ work-group is one mask row");
  constexpr int TPC = 128 / BK;  // key tiles per mask column
  MaskLine mrow = mask_line(SPARSE ? a.bmask + ((size_t)bh * a.nb + (q_base >> 7)) * a.nb : nullptr, 1,
                            SPARSE ? a.nb : 0);
  auto next = [&](int j) {
    const int jj = j + 1;
    if (!SPARSE) return jj;
    if (jj >= n_kv) return n_kv;
    if (jj % TPC != 0) return jj;  // the same mask column
    const int c = mask_next(mrow, jj / TPC, lane);
    return c >= (n_kv + TPC - 1) / TPC ? n_kv : c * TPC;
  };
  int j = next(-1);
  if (j < n_kv) issue(j, 0);

  // The first key tile's loads are in flight while the wave reads its Q, dO (and O) rows.
  // Q^T and dO^T fragments as MFMA B operands: lane holds X[qrow][16s + 8h .. +7].
  // (zeros past the last row; the loads themselves read row N - 1, so they need no branch)
  const int qsrc = min(qrow, N - 1);
  u32x4 qr[D / 16], dr[D / 16], orw[WITH_D ? D / 16 : 1];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qr[s] = *(const u32x4*)(a.q + head + (size_t)qsrc * D + 16 * s + 8 * h);
    dr[s] = *(const u32x4*)(a.dO + head + (size_t)qsrc * D + 16 * s + 8 * h);
    if constexpr (WITH_D) orw[s] = *(const u32x4*)(a.o + head + (size_t)qsrc * D + 16 * s + 8 * h);
  }
  const float lse_row = a.lse[(size_t)bh * N + qsrc];
  const float d_row = WITH_D ? 0.f : a.dvec[(size_t)bh * N + qsrc];
  // every row load is issued before the first one is used, so their latencies overlap
  __builtin_amdgcn_sched_barrier(0);
  vec8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (qrow >= N) qr[s] = dr[s] = u32x4{0u, 0u, 0u, 0u};
    qf[s] = bitcast<vec8>(qr[s]);
    df[s] = bitcast<vec8>(dr[s]);
  }
  const float lse2 = qrow < N ? lse_row * kLog2e : __builtin_inff();
  float dval = qrow < N ? d_row : 0.f;
  if constexpr (WITH_D) {
    // lane (h, lr) holds chunks p = 2s + h of its row; the preprocess tree pairs chunk p with
    // p ^ D/16, then p ^ D/32, ..., within the lane, and finally p ^ 1 across the two halves
    float ps[D / 16];
#pragma unroll
    for (int s2 = 0; s2 < D / 16; ++s2) ps[s2] = chunk_dot<TR>(orw[s2], bitcast<u32x4>(df[s2]));
#pragma unroll
    for (int off = D / 32; off >= 1; off >>= 1)
#pragma unroll
      for (int s2 = 0; s2 < off; ++s2) ps[s2] = ps[s2] + ps[s2 + off];
    dval = qrow < N ? sum_halves(ps[0]) : 0.f;
    if (qrow < N && h == 0) a.dvec[(size_t)bh * N + qrow] = dval;
  }

  for (int t = 0; j < n_kv; ++t) {
    wait_vmcnt<0>();
    barrier_lds();
    const int jn = next(j);
    if (jn < n_kv) issue(jn, t + 1);
    const int k0 = j * BK;
    j = jn;
    if (!(wave_active && k0 < wave_kv_end)) continue;
    const uint8_t* Ks = smem + (t & 1) * Cfg::STAGE_B;
    const uint8_t* Vs = Ks + TILE_B;
    const bool need_mask = (k0 + BK > N) || (CAUSAL && k0 + BK - 1 > q0);
#pragma unroll
    for (int kb = 0; kb < BK / 32; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = 0.f;
        dp[e] = 0.f;
      }
      const int row = kb * 32 + lr;
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {  // two independent chains
        const vec8 ka = *(const vec8*)(Ks + row_read_addr<D>(row, 2 * st + h));
        const vec8 va = *(const vec8*)(Vs + row * (D * 2) + (((2 * st + h) ^ swz_rowread<D>(row)) << 4));
        s = TR::mma(ka, qf[st], s);
        dp = TR::mma(va, df[st], dp);
      }
      // element e is key k0 + kb*32 + 8(e>>2) + 4h + (e&3), query qrow; the exponent (in place
      // in s) is the log2-domain logit minus the row's log2 LSE, -inf where masked (P = 0 there)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = fmaf(s[e], a.c, -lse2);
      if (need_mask) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kk = k0 + kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
          s[e] = (kk >= N || (CAUSAL && kk > qrow)) ? -__builtin_inff() : s[e];
        }
      }
      vec8 dsp[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // element 8 half + t holds key 4h + (t % 4) of 8-key group k0 / 8 + 4 kb + 2 half + t / 4
        uint32_t kf[8];
        if (DROP) row_keep_fields((uint32_t)(k0 / 8 + 4 * kb + 2 * half), (uint32_t)qrow, (uint32_t)bh, a.drop, h, kf);
        u32x4 packed;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e = 8 * half + 2 * e2;
          float dp0 = dp[e], dp1 = dp[e + 1];
          if (DROP) {
            dp0 = kf[2 * e2] >= (a.drop.thr << 16) ? dp0 * a.drop.inv_keep : 0.f;
            dp1 = kf[2 * e2 + 1] >= (a.drop.thr << 16) ? dp1 * a.drop.inv_keep : 0.f;
          }
          const float ds0 = __builtin_amdgcn_exp2f(s[e]) * (dp0 - dval);
          const float ds1 = __builtin_amdgcn_exp2f(s[e + 1]) * (dp1 - dval);
          packed[e2] = TR::pack2(ds0, ds1);
        }
        dsp[half] = bitcast<vec8>(packed);
      }
      // dQ^T += K^T dS^T over this block's two 16-key chunks
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int c = 2 * kb + half;
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
          const i16x4 lo = lds_read_tr16(Ks + tr_read_addr<D>(16 * c + tr_row, 32 * b + tr_col));
          const i16x4 hi = lds_read_tr16(Ks + tr_read_addr<D>(16 * c + tr_row + 8, 32 * b + tr_col));
          const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[b] = TR::mma(bitcast<vec8>(both), dsp[half], acc[b]);
        }
      }
    }
  }

  if (!wave_active || qrow >= N) return;
  uint16_t* row = a.dq + head + (size_t)qrow * D;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      u32x2 v2;
      v2[0] = TR::pack2(acc[b][4 * jj] * a.scale, acc[b][4 * jj + 1] * a.scale);
      v2[1] = TR::pack2(acc[b][4 * jj + 2] * a.scale, acc[b][4 * jj + 3] * a.scale);
      *(u32x2*)(row + 32 * b + 8 * jj + 4 * h) = v2;
    }
}

// ---------------------------------------------------------------------------------------------

template <typename TR, int D, bool DROP, bool SPARSE>
hipError_t launch_all(const BwdReq& r, hipStream_t st, int stage) {
  BwdArgs a;
  a.q = (const uint16_t*)r.q;
  a.k = (const uint16_t*)r.k;
  a.v = (const uint16_t*)r.v;
  a.o = (const uint16_t*)r.o;
  a.dO = (const uint16_t*)r.dO;
  a.lse = r.lse;
  a.dq = (uint16_t*)r.dq;
  a.dk = (uint16_t*)r.dk;
  a.dv = (uint16_t*)r.dv;
  a.dvec = r.dvec;
  a.N = r.N;
  a.c = r.scale * kLog2e;
  a.scale = r.scale;
  a.drop = r.drop;
  a.bmask = r.bmask;
  a.nb = (r.N + 127) / 128;
  const long long BH = (long long)r.B * r.H;
  const long long rows = BH * r.N;

  const bool big = (size_t)r.N * D * 2 >= ((size_t)1 << 31);
  a.bh_total = (int)BH;
  auto dkdv = [&]() {
    a.ntiles = (r.N + PairCfg<D>::BKV - 1) / PairCfg<D>::BKV;
    a.hgroup = head_group(a.bh_total, (size_t)2 * r.N * D * 2);
    dim3 gp((unsigned)(BH * a.ntiles));
    auto gop = [&](auto kern) { hipLaunchKernelGGL(kern, gp, dim3(PairCfg<D>::NT), 0, st, a); };
    if (r.causal)
      big ? gop(bwd_dkdv_pair_kernel<TR, D, true, true, DROP, SPARSE>) : gop(bwd_dkdv_pair_kernel<TR, D, true, false, DROP, SPARSE>);
    else
      big ? gop(bwd_dkdv_pair_kernel<TR, D, false, true, DROP, SPARSE>) : gop(bwd_dkdv_pair_kernel<TR, D, false, false, DROP, SPARSE>);
    return hipGetLastError();
  };
  auto dq = [&](auto with_d) {
    constexpr bool WD = decltype(with_d)::value;
    using DC = DqCfg<D, SPARSE ? 128 : 256>;
    a.ntiles = (r.N + DC::BQ - 1) / DC::BQ;
    a.hgroup = head_group(a.bh_total, (size_t)2 * r.N * D * 2);
    dim3 g2((unsigned)(BH * a.ntiles));
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, g2, dim3(DC::NT), 0, st, a); };
    if (r.causal)
      big ? go(bwd_dq_kernel<TR, D, true, true, DROP, SPARSE, WD>) : go(bwd_dq_kernel<TR, D, true, false, DROP, SPARSE, WD>);
    else
      big ? go(bwd_dq_kernel<TR, D, false, true, DROP, SPARSE, WD>) : go(bwd_dq_kernel<TR, D, false, false, DROP, SPARSE, WD>);
    return hipGetLastError();
  };
  if (stage < 0) {
    // the whole backward: dQ first, computing D on the way, then dK/dV (which reads D)
    hipError_t e = dq(std::true_type{});
    return e != hipSuccess ? e : dkdv();
  }
  if (stage == 0) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<TR, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                       a.o, a.dO, r.dvec, rows);
    return hipGetLastError();
  }
  if (stage == 1) return dkdv();
  return dq(std::false_type{});
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  const size_t dvec = (size_t)B * H * N * sizeof(float);
  return (dvec + 255) & ~(size_t)255;
}

template <bool DROP, bool SPARSE>
hipError_t launch_bwd_t(const BwdReq& r, hipStream_t st, int stage) {
  if (r.dtype == FATTN_BF16)
    return r.d == 64 ? launch_all<Bf16, 64, DROP, SPARSE>(r, st, stage) : launch_all<Bf16, 128, DROP, SPARSE>(r, st, stage);
  if (r.dtype == FATTN_F16)
    return r.d == 64 ? launch_all<F16, 64, DROP, SPARSE>(r, st, stage) : launch_all<F16, 128, DROP, SPARSE>(r, st, stage);
  return hipErrorInvalidValue;
}

// Dropout and block-sparse runs are separate instances; the two together are not built.
hipError_t launch_bwd(const BwdReq& r, hipStream_t st, int stage) {
  if (r.bmask) return r.dropout ? hipErrorInvalidValue : launch_bwd_t<false, true>(r, st, stage);
  return r.dropout ? launch_bwd_t<true, false>(r, st, stage) : launch_bwd_t<false, false>(r, st, stage);
}

}  // namespace fattn
