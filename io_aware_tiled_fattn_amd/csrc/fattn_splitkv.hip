// Split-KV forward: partial attention over key ranges, and the merge of the partials.
//
// Method: the keys of every row are cut into consecutive ranges (splits). A work-group computes,
// for up to 32 query rows of one head, the attention over ONE split exactly as the tiled forward
// does over the whole row (page "从零实现 FlashAttention-2：分块在线 Softmax", hands-on section:
// the query tile stays on chip while key/value tiles stream past; page "mianstack q-0277", merge
// rule for the running max m, exp-sum l and unnormalised output u), and writes the split's
// normalised partial output O_s = u / l and LSE_s = m + ln l in float32. The combine kernel then
// applies the same two-state merge rule across the splits, taking each partial as the state
// (m, l, u) = (LSE_s, 1, O_s), which is the split's own state divided through by its exp-sum.
//
// This is the shape of decoding against a key/value cache (page 3, backward section, which
// names the cache): few query rows, many keys. The whole-row kernel would give each head one
// work-group and leave most of the chip idle; splitting the keys gives splits x heads
// work-groups that all stream K/V at once, so the kernel runs at the memory bound.
//
// gfx950 mapping: one wave per work-group, its 32 query rows on the lanes exactly as in the
// whole-row kernel (S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16, Q^T in registers, K read
// from LDS with ds_read_b128, V with ds_read_b64_tr_b16). K/V tiles of BC keys go from memory
// straight into LDS (buffer_load ... lds), NS stages deep: each tile's loads go out NS - 1 tiles
// ahead of its use, and those still in flight are drained before a tile's V^T reads. With one
// wave per work-group the LDS budget, not the register file, sets how far ahead a CU loads; the kernel is bound by HBM bandwidth, and the MFMA
// work (32 query rows per tile even for one real query) stays far below its own bound.
//
// Causal with Nq queries and Nk keys: query i is position i + Nk - Nq of the sequence and sees
// keys j <= i + Nk - Nq (with Nq == Nk, the ordinary causal mask).
//
// Rows that see no key of their split (a split past a causal row's last key, or an empty split)
// get O_s = 0 and LSE_s = -inf, the empty state that the merge ignores.
#include "fattn_device.hpp"
#include "fattn_launch.hpp"

#include "../../include/fattn.h"

#include <float.h>

namespace fattn {
namespace {

constexpr float kSlack = 8.0f;  // lazy rescale slack in log2 units, as in the whole-row kernel

struct SplitArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o_part;    // [S][B*H][Nq][D]
  float* lse_part;  // [S][B*H][Nq]
  int Nq, Nk;
  int n_qtiles;     // ceil(Nq / 32)
  int num_splits;
  int split_len;    // keys per split, a multiple of kSplitAlign
  int bh_total;
  int causal_off;   // Nk - Nq
  float c;          // |scale| * log2(e), > 0
  uint32_t neg_mask;
  uint32_t keep_mask;
};

template <int D, int BC, int NS>
struct SplitCfg {
  static constexpr int CPR = D / 8;          // 16-byte chunks per row
  static constexpr int LPT = BC * CPR / 64;  // 16-byte loads per lane per tile per tensor
  static constexpr int TILE_B = BC * D * 2;
  static constexpr int STAGE_B = 2 * TILE_B;
  static constexpr int LDS_B = NS * STAGE_B;
  static constexpr int LPI = 2 * LPT;        // load instructions per tile (K and V)
  static_assert(BC % 32 == 0 && D % 32 == 0 && BC * CPR % 64 == 0, "tile shape");
  static_assert(NS >= 2 && (NS - 2) * LPI < 64, "vmcnt range");
};

template <typename TR, int D, int BC, int NS, bool CAUSAL, bool BIG>
__global__ __launch_bounds__(64) void splitkv_kernel(SplitArgs a) {
  using Cfg = SplitCfg<D, BC, NS>;
  using vec8 = typename TR::vec8;
  constexpr int CPR = Cfg::CPR, LPT = Cfg::LPT, TILE_B = Cfg::TILE_B;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS_B];

  const int lane = threadIdx.x;
  const int h = lane >> 5;
  const int lr = lane & 31;

  // block -> (split, query tile, head); splits of one head are adjacent
  const int bid = blockIdx.x;
  const int sp = bid % a.num_splits;
  const int rest = bid / a.num_splits;
  const int qt = rest % a.n_qtiles;
  const int bh = rest / a.n_qtiles;

  const int Nq = a.Nq, Nk = a.Nk;
  const int q0 = qt * 32;
  const int qrow = q0 + lr;
  const int k_begin = sp * a.split_len;
  const int k_end = min(Nk, k_begin + a.split_len);
  // last key any row of this wave sees, plus one
  int vis_end = k_end;
  if (CAUSAL) vis_end = min(vis_end, min(q0 + 31, Nq - 1) + a.causal_off + 1);
  const int n_kv = vis_end > k_begin ? (vis_end - k_begin + BC - 1) / BC : 0;

  const size_t part_row = ((size_t)sp * a.bh_total + bh) * (size_t)Nq + qrow;
  float* __restrict__ Op = a.o_part + part_row * D;

  const size_t khead = (size_t)bh * (size_t)Nk * D;
  const uint16_t* __restrict__ Kh = a.k + khead;
  const uint16_t* __restrict__ Vh = a.v + khead;
  const uint16_t* __restrict__ Qh = a.q + (size_t)bh * (size_t)Nq * D;

  vec8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qrow < Nq) raw = *(const u32x4*)(Qh + (size_t)qrow * D + 16 * s + 8 * h);
    raw = (raw ^ a.neg_mask) & a.keep_mask;
    qf[s] = bitcast<vec8>(raw);
  }

  uint32_t offK[LPT], offV[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int chunk = i * 64 + lane;
    const int row = chunk / CPR, pos = chunk % CPR;
    offK[i] = (uint32_t)(row * D * 2 + (pos ^ swz_rowread<D>(row)) * 16);
    offV[i] = (uint32_t)(row * D * 2 + (pos ^ swz_trread<D>(row)) * 16);
  }
  const uint32_t head_bytes = BIG ? 0u : (uint32_t)Nk * D * 2;
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(Kh, head_bytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(Vh, head_bytes);
  auto issue = [&](int j) {
    uint8_t* st = smem + (j % NS) * Cfg::STAGE_B;
    const int k0 = k_begin + j * BC;
    if (!BIG && k0 + BC <= Nk) {
      const uint32_t soff = (uint32_t)k0 * (D * 2);
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        buffer_lds16(rK, st + i * 64 * 16, offK[i], soff);
        buffer_lds16(rV, st + TILE_B + i * 64 * 16, offV[i], soff);
      }
    } else {
      // last tile of the sequence (or a huge head): rows past the end repeat row Nk - 1, so
      // every LDS row holds finite data; those keys are masked below
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int row = (i * 64 + lane) / CPR;
        const size_t src_row = (size_t)min(k0 + row, Nk - 1) * (D * 2);
        const uint32_t in_row = (uint32_t)(row * D * 2);
        global_lds16((const uint8_t*)Kh + src_row + (offK[i] - in_row), st + i * 64 * 16);
        global_lds16((const uint8_t*)Vh + src_row + (offV[i] - in_row), st + TILE_B + i * 64 * 16);
      }
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
  // A finite start keeps exp2(s*c - m_ref) at 0 (not NaN) for rows whose keys are all masked so
  // far; the first real logit always outgrows it, and its rescale factor is then exactly 0.
  float m_ref = -FLT_MAX;
  float l_part = 0.f;

  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_colb = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  for (int j = 0; j < NS - 1 && j < n_kv; ++j) issue(j);
  for (int j = 0; j < n_kv; ++j) {
    if (j + NS - 2 < n_kv) wait_vmcnt<(NS - 2) * Cfg::LPI>();
    else wait_vmcnt<0>();
    barrier_lds();  // tile j is in LDS; this wave's reads of stage (j - 1) % NS are done
    if (j + NS - 1 < n_kv) issue(j + NS - 1);

    const int k0 = k_begin + j * BC;
    const uint8_t* Ks = smem + (j % NS) * Cfg::STAGE_B;
    const uint8_t* Vs = Ks + TILE_B;
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
    const bool need_mask = (k0 + BC > k_end) || (CAUSAL && k0 + BC - 1 > q0 + a.causal_off);
    if (need_mask) {
      int lim = k_end - 1 - k0;
      if (CAUSAL) lim = min(lim, qrow + a.causal_off - k0);
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
    const float m_new = fmaxf(m_ref, mx);
    const bool grow = m_new > m_ref + kSlack;
    if (wave_any(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      if (grow) m_ref = m_new;
      l_part *= alpha;
#pragma unroll
      for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;
    }
    const float neg_m = -m_ref;
    vec8 pf[BC / 16];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 packed;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * half + 2 * e2], a.c, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * half + 2 * e2 + 1], a.c, neg_m));
          ls += p0 + p1;
          packed[e2] = TR::pack2(p0, p1);
        }
        pf[2 * kb + half] = bitcast<vec8>(packed);
      }
    l_part += ls;
    // The tiles still in flight land before the V^T reads; the next iterations' waits then find
    // nothing outstanding, and each tile's loads overlap only the score phase that follows their
    // issue. Measured on the decode workload (B=8 H=32 Nk=16384): 2.4% faster than keeping up to
    // NS - 1 tiles in flight through the whole loop.
    wait_vmcnt<0>();
#pragma unroll
    for (int c = 0; c < BC / 16; ++c)
#pragma unroll
      for (int b = 0; b < D / 32; ++b) {
        const int r0 = 16 * c + tr_row, r1 = r0 + 8;
        const uint8_t* p0 = Vs + r0 * (D * 2) + (((4 * b) ^ swz_trread<D>(r0)) * 16) + tr_colb;
        const uint8_t* p1 = Vs + r1 * (D * 2) + (((4 * b) ^ swz_trread<D>(r1)) * 16) + tr_colb;
        const i16x4 lo = lds_read_tr16(p0);
        const i16x4 hi = lds_read_tr16(p1);
        const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        acc[b] = TR::mma(bitcast<vec8>(both), pf[c], acc[b]);
      }
  }

  const float l_tot = sum_halves(l_part);
  if (qrow >= Nq) return;
  const bool seen = l_tot > 0.f;
  const float inv = seen ? 1.0f / l_tot : 0.f;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4 v4;
#pragma unroll
      for (int r = 0; r < 4; ++r) v4[r] = acc[b][4 * jj + r] * inv;
      *(f32x4*)(Op + 32 * b + 8 * jj + 4 * h) = v4;
    }
  if (h == 0) a.lse_part[part_row] = seen ? (m_ref + __log2f(l_tot)) * kLn2 : -__builtin_inff();
}

// ---------------------------------------------------------------------------------------------
// Merge of S partials per row. TPR = D / 4 threads per row, each owning 4 consecutive columns;
// a 256-thread work-group covers 256 / TPR rows.

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  long long rows;  // B * H * Nq
  int num_splits;
};

template <int D, int OUT>  // OUT: fattn_dtype of o
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int t = threadIdx.x % TPR;
  if (row >= a.rows) return;
  const int S = a.num_splits;
  const size_t stride = (size_t)a.rows;
  float m = -__builtin_inff();
  for (int s = 0; s < S; ++s) m = fmaxf(m, a.lse_part[s * stride + row]);
  f32x4 u = {0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  if (m != -__builtin_inff()) {
    for (int s = 0; s < S; ++s) {
      const float ls = a.lse_part[s * stride + row];
      if (ls == -__builtin_inff()) continue;  // empty partial: contributes nothing
      const float w = __builtin_amdgcn_exp2f((ls - m) * kLog2e);
      const f32x4 os = *(const f32x4*)(a.o_part + (s * stride + row) * D + 4 * t);
#pragma unroll
      for (int r = 0; r < 4; ++r) u[r] = fmaf(w, os[r], u[r]);
      l += w;
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  if (OUT == FATTN_F32) {
    f32x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = u[r] * inv;
    *(f32x4*)((float*)a.o + row * D + 4 * t) = v;
  } else {
    using TR = typename std::conditional<OUT == FATTN_BF16, Bf16, F16>::type;
    u32x2 v;
    v[0] = TR::pack2(u[0] * inv, u[1] * inv);
    v[1] = TR::pack2(u[2] * inv, u[3] * inv);
    *(u32x2*)((uint16_t*)a.o + row * D + 4 * t) = v;
  }
  if (t == 0) a.lse[row] = l > 0.f ? m + __log2f(l) * kLn2 : -__builtin_inff();
}

// ---------------------------------------------------------------------------------------------
// Dispatch.

template <typename TR, int D, int BC, int NS>
hipError_t launch_split_t(const SplitReq& r, hipStream_t st) {
  SplitArgs a;
  a.q = (const uint16_t*)r.q;
  a.k = (const uint16_t*)r.k;
  a.v = (const uint16_t*)r.v;
  a.o_part = r.o_part;
  a.lse_part = r.lse_part;
  a.Nq = r.Nq;
  a.Nk = r.Nk;
  a.n_qtiles = (r.Nq + 31) / 32;
  a.num_splits = r.num_splits;
  a.split_len = splitkv_split_len(r.Nk, r.num_splits);
  a.bh_total = r.B * r.H;
  a.causal_off = r.Nk - r.Nq;
  a.c = r.scale == 0.f ? 1.f : fabsf(r.scale) * kLog2e;
  a.neg_mask = r.scale < 0.f ? 0x80008000u : 0u;
  a.keep_mask = r.scale == 0.f ? 0u : 0xffffffffu;
  const long long nblk = (long long)a.bh_total * a.n_qtiles * r.num_splits;
  const dim3 grid((unsigned)nblk), block(64);
  const bool big = (size_t)r.Nk * D * 2 >= ((size_t)1 << 31);
  if (r.causal) {
    if (big) hipLaunchKernelGGL((splitkv_kernel<TR, D, BC, NS, true, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((splitkv_kernel<TR, D, BC, NS, true, false>), grid, block, 0, st, a);
  } else {
    if (big) hipLaunchKernelGGL((splitkv_kernel<TR, D, BC, NS, false, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((splitkv_kernel<TR, D, BC, NS, false, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_combine_t(const CombineReq& r, hipStream_t st) {
  CombineArgs a;
  a.o_part = r.o_part;
  a.lse_part = r.lse_part;
  a.o = r.o;
  a.lse = r.lse;
  a.rows = (long long)r.B * r.H * r.Nq;
  a.num_splits = r.num_splits;
  constexpr int RPB = 256 / (D / 4);
  const dim3 grid((unsigned)((a.rows + RPB - 1) / RPB)), block(256);
  if (r.dtype == FATTN_BF16) hipLaunchKernelGGL((combine_kernel<D, FATTN_BF16>), grid, block, 0, st, a);
  else if (r.dtype == FATTN_F16) hipLaunchKernelGGL((combine_kernel<D, FATTN_F16>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((combine_kernel<D, FATTN_F32>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

int splitkv_split_len(int Nk, int num_splits) {
  const long long per = ((long long)Nk + (long long)kSplitAlign * num_splits - 1) /
                        ((long long)kSplitAlign * num_splits);
  return (int)((per < 1 ? 1 : per) * kSplitAlign);
}

hipError_t launch_splitkv_partial(const SplitReq& r, hipStream_t st) {
  // 32-key tiles, four stages: three tiles per wave in flight (64 KiB of LDS at d = 128, two
  // work-groups per CU). Measured against 32/64-key tiles with 2..5 stages on the decode shapes.
  if (r.dtype == FATTN_BF16)
    return r.d == 64 ? launch_split_t<Bf16, 64, 32, 4>(r, st) : launch_split_t<Bf16, 128, 32, 4>(r, st);
  return r.d == 64 ? launch_split_t<F16, 64, 32, 4>(r, st) : launch_split_t<F16, 128, 32, 4>(r, st);
}

hipError_t launch_combine(const CombineReq& r, hipStream_t st) {
  return r.d == 64 ? launch_combine_t<64>(r, st) : launch_combine_t<128>(r, st);
}

}  // namespace fattn
