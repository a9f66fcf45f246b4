// K-outer forward: the same tiled attention in the other loop order, as a measured ablation.
//
// Page "从零实现 FlashAttention-2：分块在线 Softmax", FA-1 to FA-2 section: with the key/value
// blocks as the outer loop, every key block has to bring each query block back in, together with
// its running statistics, instead of keeping a query tile on chip while the key/value tiles stream
// past it. This kernel does exactly that so the cost can be measured on the same hardware:
// launch j handles key/value block j for every query tile at once (grid = heads x query tiles);
// each work-group loads K_j and V_j into LDS, reads its query tile and its float32 running state
// (u, m, l) from HBM, merges the block with page 3's rule (m_new = max, rescale the old state by
// exp(m - m_new)), and writes the state back, or O = u / l and LSE at the tile's last block.
// The per-row merge sequence is the Q-outer one, so the result is the same attention.
//
// Per visit the MFMA work (S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16, lane = query
// row, V^T by transposed LDS reads) is the same as in the Q-outer kernel; what differs is the
// HBM traffic: Q and (d + 2) floats of state per row move on every visit.
#include "fattn_device.hpp"
#include "fattn_launch.hpp"

#include "../../include/fattn.h"

namespace fattn {
namespace {

struct KoArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* st_u;  // [B*H][N][D]  unnormalised output relative to m
  float* st_m;  // [B*H][N]     running max, log2 domain (scaled logits * log2 e)
  float* st_l;  // [B*H][N]     exp-sum relative to m
  int N;
  int n_qtiles;
  int n_kblocks;
  int j;        // key/value block of this launch
  float c;      // |scale| * log2(e)
  uint32_t neg_mask;
  uint32_t keep_mask;
};

template <typename TR, int D, int BR, int BC, bool CAUSAL>
__global__ __launch_bounds__(BR / 32 * 64) void ko_kernel(KoArgs a) {
  using vec8 = typename TR::vec8;
  constexpr int NT = BR / 32 * 64;
  constexpr int CPR = D / 8;
  constexpr int LPT = BC * CPR / NT;
  constexpr int TILE_B = BC * D * 2;
  static_assert(BC * CPR % NT == 0, "tile load split");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * TILE_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int N = a.N;
  const int bh = blockIdx.x / a.n_qtiles;
  const int qt = blockIdx.x - bh * a.n_qtiles;
  const int q_base = qt * BR;
  const int k0 = a.j * BC;
  const int tile_last_row = min(q_base + BR, N) - 1;
  if (CAUSAL && k0 > tile_last_row) return;  // block above the diagonal for the whole tile

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Kh = a.k + head;
  const uint16_t* __restrict__ Vh = a.v + head;

  // K_j and V_j into LDS (rows past N repeat row N - 1 and are masked below)
  uint8_t* Ks = smem;
  uint8_t* Vs = smem + TILE_B;
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int chunk = i * NT + tid;
    const int row = chunk / CPR, pos = chunk % CPR;
    const size_t src = (size_t)min(k0 + row, N - 1) * (D * 2);
    // lane l of wave w lands at chunk i * NT + 64 w + l: the LDS base is per wave
    global_lds16((const uint8_t*)Kh + src + (pos ^ swz_rowread<D>(row)) * 16, Ks + (i * NT + 64 * w) * 16);
    global_lds16((const uint8_t*)Vh + src + (pos ^ swz_trread<D>(row)) * 16, Vs + (i * NT + 64 * w) * 16);
  }
  wait_vmcnt<0>();
  barrier_lds();

  const int q0 = q_base + 32 * w;
  if (q0 >= N) return;
  const int wave_last_row = min(q0 + 31, N - 1);
  if (CAUSAL && k0 > wave_last_row) return;  // this wave's rows all precede the block
  const int last_j = CAUSAL ? min(a.n_kblocks - 1, wave_last_row / BC) : a.n_kblocks - 1;
  const bool first = a.j == 0, last = a.j == last_j;
  const int qrow = q0 + lr;
  const bool row_ok = qrow < N;

  vec8 qf[D / 16];
  const uint16_t* Qh = a.q + head;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (row_ok) raw = *(const u32x4*)(Qh + (size_t)qrow * D + 16 * s + 8 * h);
    raw = (raw ^ a.neg_mask) & a.keep_mask;
    qf[s] = bitcast<vec8>(raw);
  }

  // running state of this lane's row: u in the accumulator layout (element 4jj + r of block b is
  // column 32b + 8jj + 4h + r), m per row, l split over the two half-waves (held by half 0)
  const size_t srow = (size_t)bh * N + (row_ok ? qrow : 0);
  f32x16 acc[D / 32];
  float m_ref = -__builtin_inff();
  float l_part = 0.f;
  if (!first) {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f32x4 u4 = *(const f32x4*)(a.st_u + srow * D + 32 * b + 8 * jj + 4 * h);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[b][4 * jj + r] = u4[r];
      }
    m_ref = a.st_m[srow];
    l_part = h == 0 ? a.st_l[srow] : 0.f;
  } else {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
  }

  // scores of this block, masked on the diagonal and past N
  f32x16 s[BC / 32];
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) s[kb][e] = 0.f;
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      const int row = kb * 32 + lr;
      const vec8 kf = *(const vec8*)(Ks + row * (D * 2) + (((2 * st + h) ^ swz_rowread<D>(row)) * 16));
      s[kb] = TR::mma(kf, qf[st], s[kb]);
    }
  if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0)) {
    int lim = N - 1 - k0;
    if (CAUSAL) lim = min(lim, qrow - k0);
    lim -= 4 * h;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        s[kb][e] = (kb * 32 + 8 * (e >> 2) + (e & 3) > lim) ? -__builtin_inff() : s[kb][e];
  }
  float mx = -__builtin_inff();
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
  mx = max_halves(mx) * a.c;
  // merge rule: the row's first visit sees key 0 (mx finite), so m_new is always finite
  const float m_new = fmaxf(m_ref, mx);
  const float alpha = first ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
  m_ref = m_new;
  l_part *= alpha;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;

  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_colb = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  vec8 pf[BC / 16];
  float ls = 0.f;
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      u32x4 packed;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * half + 2 * e2], a.c, -m_ref));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * half + 2 * e2 + 1], a.c, -m_ref));
        ls += p0 + p1;
        packed[e2] = TR::pack2(p0, p1);
      }
      pf[2 * kb + half] = bitcast<vec8>(packed);
    }
  l_part += ls;
#pragma unroll
  for (int c = 0; c < BC / 16; ++c)
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
      const int r0 = 16 * c + tr_row, r1 = r0 + 8;
      const i16x4 lo = lds_read_tr16(Vs + r0 * (D * 2) + (((4 * b) ^ swz_trread<D>(r0)) * 16) + tr_colb);
      const i16x4 hi = lds_read_tr16(Vs + r1 * (D * 2) + (((4 * b) ^ swz_trread<D>(r1)) * 16) + tr_colb);
      const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[b] = TR::mma(bitcast<vec8>(both), pf[c], acc[b]);
    }

  const float l_tot = sum_halves(l_part);
  if (!row_ok) return;
  if (last) {
    const float inv = 1.0f / l_tot;
    uint16_t* Orow = a.o + head + (size_t)qrow * D;
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 v2;
        v2[0] = TR::pack2(acc[b][4 * jj] * inv, acc[b][4 * jj + 1] * inv);
        v2[1] = TR::pack2(acc[b][4 * jj + 2] * inv, acc[b][4 * jj + 3] * inv);
        *(u32x2*)(Orow + 32 * b + 8 * jj + 4 * h) = v2;
      }
    if (h == 0) a.lse[srow] = (m_ref + __log2f(l_tot)) * kLn2;
  } else {
#pragma unroll
    for (int b = 0; b < D / 32; ++b)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 u4;
#pragma unroll
        for (int r = 0; r < 4; ++r) u4[r] = acc[b][4 * jj + r];
        *(f32x4*)(a.st_u + srow * D + 32 * b + 8 * jj + 4 * h) = u4;
      }
    if (h == 0) {
      a.st_m[srow] = m_ref;
      a.st_l[srow] = l_tot;
    }
  }
}

template <typename TR, int D, int BR, int BC>
hipError_t launch_ko_t(const KoReq& r, hipStream_t st) {
  KoArgs a;
  a.q = (const uint16_t*)r.q;
  a.k = (const uint16_t*)r.k;
  a.v = (const uint16_t*)r.v;
  a.o = (uint16_t*)r.o;
  a.lse = r.lse;
  const size_t rows = (size_t)r.B * r.H * r.N;
  a.st_u = r.workspace;
  a.st_m = r.workspace + rows * D;
  a.st_l = a.st_m + rows;
  a.N = r.N;
  a.n_qtiles = (r.N + BR - 1) / BR;
  a.n_kblocks = (r.N + BC - 1) / BC;
  a.c = r.scale == 0.f ? 1.f : fabsf(r.scale) * kLog2e;
  a.neg_mask = r.scale < 0.f ? 0x80008000u : 0u;
  a.keep_mask = r.scale == 0.f ? 0u : 0xffffffffu;
  const dim3 grid((unsigned)((long long)r.B * r.H * a.n_qtiles)), block(BR / 32 * 64);
  for (int j = 0; j < a.n_kblocks; ++j) {
    a.j = j;
    if (r.causal) hipLaunchKernelGGL((ko_kernel<TR, D, BR, BC, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((ko_kernel<TR, D, BR, BC, false>), grid, block, 0, st, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

size_t kouter_workspace_bytes(int B, int H, int N, int d) {
  const size_t rows = (size_t)B * H * N;
  return (rows * (size_t)(d + 2) * sizeof(float) + 255) & ~(size_t)255;
}

// Same tile shapes as the Q-outer forward's defaults: 256 x 128 at d = 128, 128 x 64 at d = 64.
hipError_t launch_kouter(const KoReq& r, hipStream_t st) {
  if (r.dtype == FATTN_BF16)
    return r.d == 64 ? launch_ko_t<Bf16, 64, 128, 64>(r, st) : launch_ko_t<Bf16, 128, 256, 128>(r, st);
  return r.d == 64 ? launch_ko_t<F16, 64, 128, 64>(r, st) : launch_ko_t<F16, 128, 256, 128>(r, st);
}

}  // namespace fattn
