// A layout ablation of the forward kernel, built on request as a measurement library
// (libfwd_one_wave.so): one wave per SIMD instead of two, so each wave can hold 512 registers.
//
// Method: the same exact forward as the library's fwd_kernel (page "从零实现 FlashAttention-2：分块
// 在线 Softmax", FA-1 to FA-2 section): query tile on chip, key/value tiles streamed through LDS,
// running max and exp-sum per row, lazy rescale with a 2^8 slack.
//
// Layout: a work-group of 4 waves (one per SIMD) owns 256 query rows; wave w owns rows
// [q_base + 64w, +64) as two 32-row blocks, so every K and V^T fragment read from LDS feeds two
// MFMAs (half the LDS reads per MFMA of the two-wave kernel). Key tiles are 64 keys, NS stages
// deep. With one wave per SIMD there is no second wave to overlap with, so the work of one wave is
// skewed across tiles instead: step j runs the score MFMAs of tile j beside the exponentials of
// tile j-1, then the PV MFMAs of tile j-1 beside the row max and s*c - m of tile j. The compiler
// places every MFMA result in AGPRs (the accumulators no longer fit next to everything else in
// 256 VGPRs), so the scores come back to VGPRs with one v_accvgpr_read each.
//
// SCHED 0 leaves the order inside a step to the compiler; SCHED 1 fixes it in 16 + 16 slots
// (two MFMAs each) separated by scheduling barriers: phase 1 slot f holds K fragment f's two
// MFMAs, the read of fragment f + 2 and 4 of the 64 exponentials; phase 2 slot s holds V^T
// fragment s's two MFMAs, the reads of fragment s + 2 and a part of the statistics.
//
// Tile loads are issued from inline asm (M0 = LDS base, then buffer_load_dwordx4 ... lds): after
// the compiler's own LDS-DMA builtin, each ds_read_b64_tr_b16 gets a vmcnt(0) wait, which here
// would wait for the next tile's prefetch in the middle of the step. The kernel orders its stages
// itself (vmcnt wait and barrier before a stage is read). Heads of 2 GiB or more and 16-bit types
// other than bf16 are not built.
#include "../csrc/fattn_device.hpp"

namespace fattn {
namespace {

constexpr float kSlack = 8.0f;

typedef int i32x4v __attribute__((ext_vector_type(4)));
struct AsmRsrc {
  i32x4v w;  // raw buffer descriptor: base (48 bits), stride 0, num_records = bytes, flags
};
__device__ inline AsmRsrc make_asm_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  return AsmRsrc{i32x4v{(int)(uint32_t)p, (int)((uint32_t)(p >> 32) & 0xffffu), (int)bytes, 0x00020000}};
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from the buffer into LDS at (lds + 16 * lane); 5 wait states after the M0
// write cover an SALU write of M0 and a VALU write of an SGPR operand.
__device__ inline void asm_lds16(const AsmRsrc& r, void* lds, uint32_t voff, uint32_t soff) {
  const uint32_t base = (uint32_t)(uintptr_t)(lds_void*)lds;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 4\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(base), "v"(voff), "s"(r.w), "s"(soff)
      : "memory", "m0");
}
#pragma clang diagnostic pop

struct OwArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int N;
  int n_qtiles;
  int bh_total;
  int hgroup;
  float c;             // |scale| * log2(e)
  uint32_t neg_mask;   // flips the sign of Q (scale < 0)
  uint32_t keep_mask;  // 0 zeroes Q (scale == 0)
};

// Block id -> (head, query tile), the library forward's order: contiguous head ranges per XCD,
// causal heads a few at a time with their longest tiles first.
__device__ inline void ow_block_coords(int bid, int nblocks, int n_qtiles, int bh_total, bool causal, int hgroup,
                                       int* bh, int* qt) {
  if ((bh_total & 7) == 0) {
    const int hpx = bh_total >> 3;
    const int xcd = bid & 7, local = bid >> 3;
    if (causal) {
      int hh, r;
      causal_xcd_order(local, hpx, n_qtiles, hgroup, &hh, &r);
      *bh = xcd * hpx + hh;
      *qt = n_qtiles - 1 - r;
    } else {
      const int hh = local / n_qtiles;
      *bh = xcd * hpx + hh;
      *qt = local - hh * n_qtiles;
    }
    return;
  }
  const int logical = xcd_remap(bid, nblocks);
  *bh = logical / n_qtiles;
  *qt = logical - *bh * n_qtiles;
  if (causal) *qt = n_qtiles - 1 - *qt;
}

constexpr int D = 128, BR = 256, BC = 64, NT = 256, CPR = D / 8;
constexpr int LPT = BC * CPR / NT;  // 16-byte loads per thread per tile per tensor
constexpr int LPI = 2 * LPT;        // load instructions per thread per tile
constexpr int TILE_B = BC * D * 2;  // one K (or V) tile: 16 KiB
constexpr int STAGE_B = 2 * TILE_B;

template <typename TR, int NS, bool CAUSAL, int SCHED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_one_wave_kernel(OwArgs a) {
  using vec8 = typename TR::vec8;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE_B];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int N = a.N;

  int bh, qt;
  ow_block_coords(blockIdx.x, gridDim.x, a.n_qtiles, a.bh_total, CAUSAL, a.hgroup, &bh, &qt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qh = a.q + head;
  const uint16_t* __restrict__ Kh = a.k + head;
  const uint16_t* __restrict__ Vh = a.v + head;

  const int q_base = qt * BR;
  const int q0 = q_base + 64 * w;
  const bool wave_active = q0 < N;

  vec8 qf[2][D / 16];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const int qrow = q0 + 32 * b + lr;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qrow < N) raw = *(const u32x4*)(Qh + (size_t)qrow * D + 16 * s + 8 * h);
      raw = (raw ^ a.neg_mask) & a.keep_mask;
      qf[b][s] = bitcast<vec8>(raw);
    }

  const int kv_end = CAUSAL ? min(N, q_base + BR) : N;
  const int n_kv = (kv_end + BC - 1) / BC;
  const int jlast = !wave_active ? -1 : (CAUSAL ? min(n_kv - 1, q0 / BC) : n_kv - 1);

  uint32_t offK, offV;
  {
    const int row = tid / CPR, pos = tid % CPR;
    offK = (uint32_t)(row * D * 2 + (pos ^ swz_rowread<D>(row)) * 16);
    offV = (uint32_t)(row * D * 2 + (pos ^ swz_trread<D>(row)) * 16);
  }
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const AsmRsrc rK = make_asm_rsrc(Kh, head_bytes);
  const AsmRsrc rV = make_asm_rsrc(Vh, head_bytes);
  auto issue = [&](int j) {
    uint8_t* st = smem + (j % NS) * STAGE_B + w * 64 * 16;
    const uint32_t soff = (uint32_t)(j * BC) * (D * 2);
    if ((j + 1) * BC <= N) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const uint32_t add = (uint32_t)(i * NT * 16);
        asm_lds16(rK, st + i * NT * 16, offK, soff + add);
        asm_lds16(rV, st + TILE_B + i * NT * 16, offV, soff + add);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const uint32_t add = (uint32_t)(i * NT * 16);
        asm_lds16(rK, st + i * NT * 16, offK + soff + add, 0u);
        asm_lds16(rV, st + TILE_B + i * NT * 16, offV + soff + add, 0u);
      }
    }
  };
  auto tile_wait = [&](int j) {
    if (NS > 3 && j + NS - 3 < n_kv) wait_vmcnt<(NS > 3 ? (NS - 3) * LPI : 0)>();
    else wait_vmcnt<0>();
    barrier_lds();
  };

  f32x16 o[2][D / 32];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[b][d][e] = 0.f;
  float m_ref[2] = {0.f, 0.f}, m_use[2] = {0.f, 0.f}, l_part[2] = {0.f, 0.f};
  f32x16 sp[2][2];  // scores of the tile waiting for its exponentials (as s*c - m_use)
  vec8 pf[2][BC / 16];

  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_colb = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  // S(j) for both row blocks: each K fragment feeds two MFMAs.
  auto scores = [&](int j, f32x16 (&sa)[2][2]) {
    const uint8_t* Ks = smem + (j % NS) * STAGE_B;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sa[b][kb][e] = 0.f;
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int row = kb * 32 + lr;
        const vec8 kf = *(const vec8*)(Ks + row * (D * 2) + (((2 * st + h) ^ swz_rowread<D>(row)) * 16));
        sa[0][kb] = TR::mma(kf, qf[0][st], sa[0][kb]);
        sa[1][kb] = TR::mma(kf, qf[1][st], sa[1][kb]);
      }
  };
  // exponentials of sp -> P fragments and row sums
  auto expo = [&]() {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4 packed;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float p0 = __builtin_amdgcn_exp2f(sp[b][kb][8 * half + 2 * e2]);
            const float p1 = __builtin_amdgcn_exp2f(sp[b][kb][8 * half + 2 * e2 + 1]);
            ls += p0 + p1;
            packed[e2] = TR::pack2(p0, p1);
          }
          pf[b][2 * kb + half] = bitcast<vec8>(packed);
        }
      l_part[b] += ls;
    }
  };
  // O += V^T P for the tile in stage j
  auto pv = [&](int j) {
    const uint8_t* Vs = smem + (j % NS) * STAGE_B + TILE_B;
#pragma unroll
    for (int c = 0; c < BC / 16; ++c)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int r0 = 16 * c + tr_row, r1 = r0 + 8;
        const uint8_t* p0 = Vs + r0 * (D * 2) + (((4 * db) ^ swz_trread<D>(r0)) * 16) + tr_colb;
        const uint8_t* p1 = Vs + r1 * (D * 2) + (((4 * db) ^ swz_trread<D>(r1)) * 16) + tr_colb;
        const i16x4 lo = lds_read_tr16(p0);
        const i16x4 hi = lds_read_tr16(p1);
        const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[0][db] = TR::mma(bitcast<vec8>(both), pf[0][c], o[0][db]);
        o[1][db] = TR::mma(bitcast<vec8>(both), pf[1][c], o[1][db]);
      }
  };
  // sp <- sa, masked; row max; new reference; sp <- sp*c - m_use
  auto stats = [&](int j, const f32x16 (&sa)[2][2], bool masked, bool first) {
    const int k0 = j * BC;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sp[b][kb] = sa[b][kb];
      if (masked) {
        int lim = N - 1 - k0;
        if (CAUSAL) lim = min(lim, q0 + 32 * b + lr - k0);
        lim -= 4 * h;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            sp[b][kb][e] = (kb * 32 + 8 * (e >> 2) + (e & 3) > lim) ? -__builtin_inff() : sp[b][kb][e];
      }
      float mk0 = -__builtin_inff(), mk1 = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        mk0 = fmaxf(mk0, sp[b][0][e]);
        mk1 = fmaxf(mk1, sp[b][1][e]);
      }
      const float mx = max_halves(fmaxf(mk0, mk1)) * a.c;
      if (first) {
        m_ref[b] = mx;
        m_use[b] = mx;
      } else {
        const float mn = fmaxf(m_ref[b], mx);
        m_use[b] = mn > m_ref[b] + kSlack ? mn : m_ref[b];
      }
      const float neg_m = -m_use[b];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sp[b][kb][e] = fmaf(sp[b][kb][e], a.c, neg_m);
    }
  };
  auto rescale = [&]() {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float alpha = __builtin_amdgcn_exp2f(m_ref[b] - m_use[b]);
      m_ref[b] = m_use[b];
      l_part[b] *= alpha;
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[b][d][e] *= alpha;
    }
  };
  // one skewed step: S(j) beside exp(j-1), then PV(j-1) beside the statistics of j
  auto step = [&](int j, bool masked) {
    f32x16 sa[2][2];
    if (SCHED == 0) {
      scores(j, sa);
      expo();
      pv(j - 1);
      stats(j, sa, masked, false);
      return;
    }
    // ---- phase 1: 16 slots; slot f: K fragment f's two MFMAs, the read of fragment f + 2, and
    // the exponentials of 4 of the 64 scores of tile j - 1
    const uint8_t* Ks = smem + (j % NS) * STAGE_B;
    auto kread = [&](int f) {
      const int st = f >> 1, kb = f & 1;
      const int row = kb * 32 + lr;
      return *(const vec8*)(Ks + row * (D * 2) + (((2 * st + h) ^ swz_rowread<D>(row)) * 16));
    };
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sa[b][kb][e] = 0.f;
    vec8 kf[16];
    kf[0] = kread(0);
    kf[1] = kread(1);
    float ls[2] = {0.f, 0.f};
    u32x4 packed;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < 16; ++f) {
      if (f + 2 < 16) kf[f + 2] = kread(f + 2);
      const int st = f >> 1, kb = f & 1;
      sa[0][kb] = TR::mma(kf[f], qf[0][st], sa[0][kb]);
      sa[1][kb] = TR::mma(kf[f], qf[1][st], sa[1][kb]);
      // exponentials: part f = (block, kb, half, pair group)
      const int b = f >> 3, ekb = (f >> 2) & 1, half = (f >> 1) & 1, g = f & 1;
#pragma unroll
      for (int e2 = 2 * g; e2 < 2 * g + 2; ++e2) {
        const float p0 = __builtin_amdgcn_exp2f(sp[b][ekb][8 * half + 2 * e2]);
        const float p1 = __builtin_amdgcn_exp2f(sp[b][ekb][8 * half + 2 * e2 + 1]);
        ls[b] += p0 + p1;
        packed[e2] = TR::pack2(p0, p1);
      }
      if (g == 1) pf[b][2 * ekb + half] = bitcast<vec8>(packed);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_part[0] += ls[0];
    l_part[1] += ls[1];
    // ---- phase 2: 16 slots; slot s: V^T fragment s's two MFMAs, the reads of fragment s + 2,
    // and a part of the statistics of tile j (copy, mask, max, then s*c - m)
    const uint8_t* Vs = smem + ((j - 1) % NS) * STAGE_B + TILE_B;
    auto vread = [&](int s) {
      const int c = s >> 2, db = s & 3;
      const int r0 = 16 * c + tr_row, r1 = r0 + 8;
      const uint8_t* p0 = Vs + r0 * (D * 2) + (((4 * db) ^ swz_trread<D>(r0)) * 16) + tr_colb;
      const uint8_t* p1 = Vs + r1 * (D * 2) + (((4 * db) ^ swz_trread<D>(r1)) * 16) + tr_colb;
      const i16x4 lo = lds_read_tr16(p0);
      const i16x4 hi = lds_read_tr16(p1);
      const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      return bitcast<vec8>(both);
    };
    vec8 vf[16];
    vf[0] = vread(0);
    vf[1] = vread(1);
    const int k0 = j * BC;
    float mk[2] = {-__builtin_inff(), -__builtin_inff()};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s + 2 < 16) vf[s + 2] = vread(s + 2);
      const int c = s >> 2, db = s & 3;
      o[0][db] = TR::mma(vf[s], pf[0][c], o[0][db]);
      o[1][db] = TR::mma(vf[s], pf[1][c], o[1][db]);
      const int b = s >> 3, p = s & 7;
      if (p < 4) {
        const int kb = p >> 1, e0 = 8 * (p & 1);
        int lim = N - 1 - k0;
        if (CAUSAL) lim = min(lim, q0 + 32 * b + lr - k0);
        lim -= 4 * h;
#pragma unroll
        for (int e = e0; e < e0 + 8; ++e) {
          float x = sa[b][kb][e];
          if (masked) x = (kb * 32 + 8 * (e >> 2) + (e & 3) > lim) ? -__builtin_inff() : x;
          sp[b][kb][e] = x;
          mk[b] = fmaxf(mk[b], x);
        }
      } else if (p == 4) {
        const float mx = max_halves(mk[b]) * a.c;
        const float mn = fmaxf(m_ref[b], mx);
        m_use[b] = mn > m_ref[b] + kSlack ? mn : m_ref[b];
      } else {
        const float neg_m = -m_use[b];
        const int i0 = (p - 5) * 11, i1 = p == 7 ? 32 : i0 + 11;
#pragma unroll
        for (int i = i0; i < i1; ++i) sp[b][i >> 4][i & 15] = fmaf(sp[b][i >> 4][i & 15], a.c, neg_m);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int t = 0; t < NS - 2 && t < n_kv; ++t) issue(t);
  tile_wait(0);
  if (NS - 2 < n_kv) issue(NS - 2);
  if (jlast >= 0) {
    f32x16 sa[2][2];
    scores(0, sa);
    stats(0, sa, true, true);
  }
  const bool mask_last = CAUSAL || (jlast + 1) * BC > N;
  const int jend = mask_last ? jlast : jlast + 1;  // unmasked steps run j = 1 .. jend - 1
  int j = 1;
  while (j < jend) {
    bool grew = false;
    for (; j < jend; ++j) {
      tile_wait(j);
      if (j + NS - 2 < n_kv) issue(j + NS - 2);
      step(j, false);
      if (wave_any(m_use[0] != m_ref[0] || m_use[1] != m_ref[1])) {
        grew = true;
        ++j;
        break;
      }
    }
    if (!grew) break;
    rescale();
  }
  if (mask_last && jlast >= 1) {
    tile_wait(jlast);
    if (jlast + NS - 2 < n_kv) issue(jlast + NS - 2);
    step(jlast, true);
    if (wave_any(m_use[0] != m_ref[0] || m_use[1] != m_ref[1])) rescale();
  }
  if (jlast >= 0) {
    expo();
    pv(jlast);
  }
  for (int jj = jlast + 1 > 1 ? jlast + 1 : 1; jj < n_kv; ++jj) {
    tile_wait(jj);
    if (jj + NS - 2 < n_kv) issue(jj + NS - 2);
  }

  if (!wave_active) return;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const float l_tot = sum_halves(l_part[b]);
    const int qrow = q0 + 32 * b + lr;
    if (qrow < N) {
      const float inv = 1.0f / l_tot;
      uint16_t* Orow = a.o + head + (size_t)qrow * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          u32x2 v2;
          v2[0] = TR::pack2(o[b][db][4 * jj] * inv, o[b][db][4 * jj + 1] * inv);
          v2[1] = TR::pack2(o[b][db][4 * jj + 2] * inv, o[b][db][4 * jj + 3] * inv);
          *(u32x2*)(Orow + 32 * db + 8 * jj + 4 * h) = v2;
        }
      if (h == 0) a.lse[(size_t)bh * N + qrow] = (m_ref[b] + __log2f(l_tot)) * kLn2;
    }
  }
}

template <int NS, int SCHED>
int launch(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, float scale,
           int causal, hipStream_t st) {
  OwArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.lse = lse;
  a.N = N;
  a.n_qtiles = (N + BR - 1) / BR;
  a.bh_total = B * H;
  // the library forward's causal head grouping: 4 heads, fewer once their K and V pass 8 MiB
  const int hpx = a.bh_total / 8;
  int g = (int)(((size_t)8 << 20) / ((size_t)2 * N * D * 2));
  g = g < 1 ? 1 : (g > 4 ? 4 : g);
  a.hgroup = hpx <= 1 ? 1 : (g > hpx ? hpx : g);
  a.c = scale == 0.f ? 1.f : fabsf(scale) * kLog2e;
  a.neg_mask = scale < 0.f ? 0x80008000u : 0u;
  a.keep_mask = scale == 0.f ? 0u : 0xffffffffu;
  const dim3 grid((unsigned)((long long)B * H * a.n_qtiles)), block(NT);
  if (causal) hipLaunchKernelGGL((fwd_one_wave_kernel<Bf16, NS, true, SCHED>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((fwd_one_wave_kernel<Bf16, NS, false, SCHED>), grid, block, 0, st, a);
  return (int)hipGetLastError();
}

}  // namespace
}  // namespace fattn

// bf16 q, k, v, o: [B, H, N, 128] contiguous device buffers; lse: float32 [B, H, N]. ns: K/V
// stages (3 or 4); sched: 0 = compiler order inside a step, 1 = fixed slots. Returns 0, a HIP
// error code, -1 for a head of 2 GiB or more, -2 for an unbuilt (ns, sched).
extern "C" int fwd_one_wave(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                            float scale, int causal, int ns, int sched, void* stream) {
  using namespace fattn;
  if (B < 1 || H < 1 || N < 1) return -3;
  if ((size_t)N * D * 2 >= ((size_t)1 << 31)) return -1;
  hipStream_t st = (hipStream_t)stream;
  if (ns == 3 && sched == 0) return launch<3, 0>(q, k, v, o, lse, B, H, N, scale, causal, st);
  if (ns == 3 && sched == 1) return launch<3, 1>(q, k, v, o, lse, B, H, N, scale, causal, st);
  if (ns == 4 && sched == 1) return launch<4, 1>(q, k, v, o, lse, B, H, N, scale, causal, st);
  return -2;
}
