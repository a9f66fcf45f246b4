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
// Three kernels, all in stream order:
//  1. bwd_pre:   D = rowsum(dO * O) (float32 workspace), one pass over O and dO.
//  2. bwd_dkdv:  one work-group per (b*h, 128-key tile); each of its 4 waves keeps 32 keys of K
//               and V in registers and the float32 dK, dV accumulators, while Q, dO tiles of 64
//               queries stream through double-buffered LDS. Scores are formed as S = Q K^T so
//               that every lane owns ONE key: P and dS then serve directly as the MFMA A
//               operand of dV += P^T dO and dK += dS^T Q, whose B operands (dO and Q with the
//               query index as reduction index) come from the row-major LDS tiles through
//               ds_read_b64_tr_b16.
//  3. bwd_dq:    one work-group per (b*h, 128-query tile), the forward's layout: S^T = K Q^T and
//               dP^T = V dO^T give each lane ONE query (its LSE and D are per-lane scalars);
//               dQ^T += K^T dS^T takes K^T from the row-major K tile via the transposed read.
// Every kernel writes its outputs once; there are no atomics, so results are deterministic.
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
  const float* dvec;
  int N;
  int ntiles;   // tiles per head along the grid's sequence axis
  float c;      // scale * log2(e) (signed)
  float scale;  // signed softmax scale
};

template <typename TR>
__device__ inline float to_f32(uint16_t x);
template <>
__device__ inline float to_f32<Bf16>(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
template <>
__device__ inline float to_f32<F16>(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

// ---------------------------------------------------------------------------------------------
// 1. D = rowsum(dO * O): D/8 threads per row, 16-byte loads.

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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sum += to_f32<TR>((uint16_t)(a[i] & 0xffff)) * to_f32<TR>((uint16_t)(b[i] & 0xffff));
      sum += to_f32<TR>((uint16_t)(a[i] >> 16)) * to_f32<TR>((uint16_t)(b[i] >> 16));
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, TPR);
  if (row < rows && part == 0) dvec[row] = sum;
}

// ---------------------------------------------------------------------------------------------
// 2. dK, dV.

template <int D>
struct DkdvCfg {
  static constexpr int BKV = 128;            // keys per work-group (32 per wave)
  static constexpr int BQ = 64;              // queries per step
  static constexpr int NT = 256;
  static constexpr int STR = D + 8;          // LDS row pitch of the Q and dO tiles (elements)
  static constexpr int CPR = D / 8;
  static constexpr int CH = BQ * CPR / NT;   // 16-byte chunks per thread per tensor per step
  static constexpr int TILE = BQ * STR;      // elements of one Q (or dO) tile
  static constexpr int STAGE_E = 2 * TILE;   // Q + dO
  static_assert(BQ * CPR % NT == 0, "tile split");
};

template <typename TR, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  using Cfg = DkdvCfg<D>;
  using vec8 = typename TR::vec8;
  constexpr int BKV = Cfg::BKV, BQ = Cfg::BQ;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Cfg::STAGE_E];
  __shared__ __attribute__((aligned(16))) float srow[2][2][BQ];  // [stage][lse2 | D][query]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int N = a.N;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.ntiles;
  const int jt = logical - bh * a.ntiles;  // causal: low tiles see the most queries, so go first
  const size_t head = (size_t)bh * (size_t)N * D;
  const size_t rowbase = (size_t)bh * (size_t)N;
  const uint16_t* __restrict__ Qh = a.q + head;
  const uint16_t* __restrict__ dOh = a.dO + head;

  const int key0 = jt * BKV + 32 * w;  // first key of this wave
  const int key = key0 + lr;           // this lane's key
  const bool wave_active = key0 < N;

  // K and V fragments as MFMA B operands: lane holds X[key][16s + 8h .. +7].
  vec8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 kr = {0u, 0u, 0u, 0u}, vr = {0u, 0u, 0u, 0u};
    if (key < N) {
      kr = *(const u32x4*)(a.k + head + (size_t)key * D + 16 * s + 8 * h);
      vr = *(const u32x4*)(a.v + head + (size_t)key * D + 16 * s + 8 * h);
    }
    kf[s] = bitcast<vec8>(kr);
    vf[s] = bitcast<vec8>(vr);
  }

  f32x16 adk[D / 32], adv[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      adk[b][e] = 0.f;
      adv[b][e] = 0.f;
    }

  const int n_qt = (N + BQ - 1) / BQ;
  const int i_begin = CAUSAL ? (jt * BKV) / BQ : 0;

  u32x4 qr[Cfg::CH], dr[Cfg::CH];
  float lr2 = 0.f, dvr = 0.f;
  auto load_tile = [&](int i) {
#pragma unroll
    for (int t = 0; t < Cfg::CH; ++t) {
      const int c = tid + t * Cfg::NT;
      const int row = c / Cfg::CPR;
      const int col = c % Cfg::CPR;
      const int q = i * BQ + row;
      if (q < N) {
        qr[t] = *(const u32x4*)(Qh + (size_t)q * D + col * 8);
        dr[t] = *(const u32x4*)(dOh + (size_t)q * D + col * 8);
      } else {
        qr[t] = u32x4{0u, 0u, 0u, 0u};
        dr[t] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < BQ) {
      const int q = i * BQ + tid;
      // rows past the end get LSE = +inf, so their P is exactly 0
      lr2 = q < N ? a.lse[rowbase + q] * kLog2e : __builtin_inff();
      dvr = q < N ? a.dvec[rowbase + q] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* Qs = smem + buf * Cfg::STAGE_E;
    uint16_t* dOs = Qs + Cfg::TILE;
#pragma unroll
    for (int t = 0; t < Cfg::CH; ++t) {
      const int c = tid + t * Cfg::NT;
      const int row = c / Cfg::CPR;
      const int col = c % Cfg::CPR;
      *(u32x4*)(Qs + row * Cfg::STR + col * 8) = qr[t];
      *(u32x4*)(dOs + row * Cfg::STR + col * 8) = dr[t];
    }
    if (tid < BQ) {
      srow[buf][0][tid] = lr2;
      srow[buf][1][tid] = dvr;
    }
  };

  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  if (i_begin < n_qt) {
    load_tile(i_begin);
    store_tile(0);
  }
  for (int i = i_begin; i < n_qt; ++i) {
    const int buf = (i - i_begin) & 1;
    if (i + 1 < n_qt) load_tile(i + 1);
    __syncthreads();
    const int q_base = i * BQ;
    // causal: the whole tile lies above this wave's keys -> P = 0, nothing to add
    if (wave_active && !(CAUSAL && q_base + BQ - 1 < key0)) {
      const uint16_t* Qs = smem + buf * Cfg::STAGE_E;
      const uint16_t* dOs = Qs + Cfg::TILE;
      const float* lse2s = srow[buf][0];
      const float* dvs = srow[buf][1];

      vec8 pp[BQ / 16], dsp[BQ / 16];
      const bool need_mask = CAUSAL && key0 + 31 > q_base;
#pragma unroll
      for (int qb = 0; qb < BQ / 32; ++qb) {
        f32x16 s, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[e] = 0.f;
          dp[e] = 0.f;
        }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {  // two independent chains, interleaved
          const vec8 qa = *(const vec8*)(Qs + (qb * 32 + lr) * Cfg::STR + 16 * st + 8 * h);
          const vec8 da = *(const vec8*)(dOs + (qb * 32 + lr) * Cfg::STR + 16 * st + 8 * h);
          s = TR::mma(qa, kf[st], s);
          dp = TR::mma(da, vf[st], dp);
        }
        // element 4j + r is query qb*32 + 8j + 4h + r of the tile, key = this lane's key
        float p[16], ds[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 l4 = *(const f32x4*)(lse2s + qb * 32 + 8 * j + 4 * h);
          const f32x4 d4 = *(const f32x4*)(dvs + qb * 32 + 8 * j + 4 * h);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = 4 * j + r;
            float pv = __builtin_amdgcn_exp2f(fmaf(s[e], a.c, -l4[r]));
            if (need_mask) pv = (key > q_base + qb * 32 + 8 * j + 4 * h + r) ? 0.f : pv;
            p[e] = pv;
            ds[e] = pv * (dp[e] - d4[r]);
          }
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 pu, du;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            pu[e2] = TR::pack2(p[8 * half + 2 * e2], p[8 * half + 2 * e2 + 1]);
            du[e2] = TR::pack2(ds[8 * half + 2 * e2], ds[8 * half + 2 * e2 + 1]);
          }
          pp[2 * qb + half] = bitcast<vec8>(pu);
          dsp[2 * qb + half] = bitcast<vec8>(du);
        }
      }
      // dV += P^T dO and dK += dS^T Q; B operands via the transposed LDS read.
#pragma unroll
      for (int c = 0; c < BQ / 16; ++c) {
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
          const int off = (16 * c + tr_row) * Cfg::STR + 32 * b + tr_col;
          const i16x4 d0 = lds_read_tr16(dOs + off);
          const i16x4 d1 = lds_read_tr16(dOs + off + 8 * Cfg::STR);
          const i16x8 dd = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
          adv[b] = TR::mma(pp[c], bitcast<vec8>(dd), adv[b]);
          const i16x4 q0 = lds_read_tr16(Qs + off);
          const i16x4 q1 = lds_read_tr16(Qs + off + 8 * Cfg::STR);
          const i16x8 qq = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
          adk[b] = TR::mma(dsp[c], bitcast<vec8>(qq), adk[b]);
        }
      }
    }
    if (i + 1 < n_qt) store_tile(buf ^ 1);
  }

  if (!wave_active) return;
  // Output element 4j + r of block b is key key0 + 8j + 4h + r, column 32b + lr.
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = key0 + 8 * j + 4 * h + r;
      if (kk < N) {
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
          const size_t idx = head + (size_t)kk * D + 32 * b + lr;
          a.dk[idx] = __builtin_bit_cast(uint16_t, TR::from_f32(adk[b][4 * j + r] * a.scale));
          a.dv[idx] = __builtin_bit_cast(uint16_t, TR::from_f32(adv[b][4 * j + r]));
        }
      }
    }
}

// ---------------------------------------------------------------------------------------------
// 3. dQ.

template <int D>
struct DqCfg {
  static constexpr int BQ = 128;           // queries per work-group (32 per wave)
  static constexpr int BK = 64;            // keys per step
  static constexpr int NT = 256;
  static constexpr int KSTR = D + 8;
  static constexpr int VSTR = D + 8;
  static constexpr int CPR = D / 8;
  static constexpr int CH = BK * CPR / NT;
  static constexpr int KBUF = BK * KSTR;
  static constexpr int STAGE = KBUF + BK * VSTR;
  static_assert(BK * CPR % NT == 0, "tile split");
};

template <typename TR, int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  using Cfg = DqCfg<D>;
  using vec8 = typename TR::vec8;
  constexpr int BQ = Cfg::BQ, BK = Cfg::BK;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Cfg::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int N = a.N;

  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.ntiles;
  int qt = logical - bh * a.ntiles;
  if (CAUSAL) qt = a.ntiles - 1 - qt;
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Kh = a.k + head;
  const uint16_t* __restrict__ Vh = a.v + head;

  const int q_base = qt * BQ;
  const int q0 = q_base + 32 * w;
  const int qrow = q0 + lr;
  const bool wave_active = q0 < N;
  const int wave_kv_end = CAUSAL ? min(q0 + 31, N - 1) + 1 : N;

  // Q^T and dO^T fragments as MFMA B operands: lane holds X[qrow][16s + 8h .. +7].
  vec8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 qr = {0u, 0u, 0u, 0u}, dr = {0u, 0u, 0u, 0u};
    if (qrow < N) {
      qr = *(const u32x4*)(a.q + head + (size_t)qrow * D + 16 * s + 8 * h);
      dr = *(const u32x4*)(a.dO + head + (size_t)qrow * D + 16 * s + 8 * h);
    }
    qf[s] = bitcast<vec8>(qr);
    df[s] = bitcast<vec8>(dr);
  }
  const float lse2 = qrow < N ? a.lse[(size_t)bh * N + qrow] * kLog2e : __builtin_inff();
  const float dval = qrow < N ? a.dvec[(size_t)bh * N + qrow] : 0.f;

  f32x16 acc[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;

  const int kv_end = CAUSAL ? min(N, q_base + BQ) : N;
  const int n_kv = (kv_end + BK - 1) / BK;

  u32x4 kr[Cfg::CH], vr[Cfg::CH];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < Cfg::CH; ++i) {
      const int c = tid + i * Cfg::NT;
      const int row = c / Cfg::CPR;
      const int col = c % Cfg::CPR;
      const int kk = j * BK + row;
      if (kk < N) {
        kr[i] = *(const u32x4*)(Kh + (size_t)kk * D + col * 8);
        vr[i] = *(const u32x4*)(Vh + (size_t)kk * D + col * 8);
      } else {
        kr[i] = u32x4{0u, 0u, 0u, 0u};
        vr[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* Ks = smem + buf * Cfg::STAGE;
    uint16_t* Vs = Ks + Cfg::KBUF;
#pragma unroll
    for (int i = 0; i < Cfg::CH; ++i) {
      const int c = tid + i * Cfg::NT;
      const int row = c / Cfg::CPR;
      const int col = c % Cfg::CPR;
      *(u32x4*)(Ks + row * Cfg::KSTR + col * 8) = kr[i];
      *(u32x4*)(Vs + row * Cfg::VSTR + col * 8) = vr[i];
    }
  };

  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  load_tile(0);
  store_tile(0);
  for (int j = 0; j < n_kv; ++j) {
    if (j + 1 < n_kv) load_tile(j + 1);
    __syncthreads();
    const int k0 = j * BK;
    if (wave_active && k0 < wave_kv_end) {
      const uint16_t* Ks = smem + (j & 1) * Cfg::STAGE;
      const uint16_t* Vs = Ks + Cfg::KBUF;
      const bool need_mask = (k0 + BK > N) || (CAUSAL && k0 + BK - 1 > q0);
      vec8 dsp[BK / 16];
#pragma unroll
      for (int kb = 0; kb < BK / 32; ++kb) {
        f32x16 s, dp;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s[e] = 0.f;
          dp[e] = 0.f;
        }
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {  // two independent chains, interleaved
          const vec8 ka = *(const vec8*)(Ks + (kb * 32 + lr) * Cfg::KSTR + 16 * st + 8 * h);
          const vec8 va = *(const vec8*)(Vs + (kb * 32 + lr) * Cfg::VSTR + 16 * st + 8 * h);
          s = TR::mma(ka, qf[st], s);
          dp = TR::mma(va, df[st], dp);
        }
        // element e is key k0 + kb*32 + 8(e>>2) + 4h + (e&3), query qrow
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 packed;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            float ds2[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int e = 8 * half + 2 * e2 + u;
              float pv = __builtin_amdgcn_exp2f(fmaf(s[e], a.c, -lse2));
              if (need_mask) {
                const int kk = k0 + kb * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                pv = (kk >= N || (CAUSAL && kk > qrow)) ? 0.f : pv;
              }
              ds2[u] = pv * (dp[e] - dval);
            }
            packed[e2] = TR::pack2(ds2[0], ds2[1]);
          }
          dsp[2 * kb + half] = bitcast<vec8>(packed);
        }
      }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int c = 0; c < BK / 16; ++c) {
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
          const uint16_t* p0 = Ks + (16 * c + tr_row) * Cfg::KSTR + 32 * b + tr_col;
          const i16x4 lo = lds_read_tr16(p0);
          const i16x4 hi = lds_read_tr16(p0 + 8 * Cfg::KSTR);
          const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          acc[b] = TR::mma(bitcast<vec8>(both), dsp[c], acc[b]);
        }
      }
    }
    if (j + 1 < n_kv) store_tile((j + 1) & 1);
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

template <typename TR, int D>
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
  const long long BH = (long long)r.B * r.H;
  const long long rows = BH * r.N;

  hipError_t e = hipSuccess;
  if (stage < 0 || stage == 0) {
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_pre_kernel<TR, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st,
                       a.o, a.dO, r.dvec, rows);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage < 0 || stage == 1) {
    a.ntiles = (r.N + DkdvCfg<D>::BKV - 1) / DkdvCfg<D>::BKV;
    dim3 g1((unsigned)(BH * a.ntiles));
    if (r.causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<TR, D, true>), g1, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<TR, D, false>), g1, dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stage < 0 || stage == 2) {
    a.ntiles = (r.N + DqCfg<D>::BQ - 1) / DqCfg<D>::BQ;
    dim3 g2((unsigned)(BH * a.ntiles));
    if (r.causal)
      hipLaunchKernelGGL((bwd_dq_kernel<TR, D, true>), g2, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<TR, D, false>), g2, dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

size_t bwd_workspace_bytes(int B, int H, int N, int d) {
  (void)d;
  const size_t dvec = (size_t)B * H * N * sizeof(float);
  return (dvec + 255) & ~(size_t)255;
}

hipError_t launch_bwd(const BwdReq& r, hipStream_t st, int stage) {
  if (r.dtype == FATTN_BF16)
    return r.d == 64 ? launch_all<Bf16, 64>(r, st, stage) : launch_all<Bf16, 128>(r, st, stage);
  if (r.dtype == FATTN_F16)
    return r.d == 64 ? launch_all<F16, 64>(r, st, stage) : launch_all<F16, 128>(r, st, stage);
  return hipErrorInvalidValue;
}

}  // namespace fattn
