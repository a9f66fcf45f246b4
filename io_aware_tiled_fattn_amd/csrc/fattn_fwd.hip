// Forward kernels: exact attention, one work-group per (batch*head, query tile).
//
// Method (page "从零实现 FlashAttention-2：分块在线 Softmax", FA-1 to FA-2 section and hands-on
// section; page "mianstack q-0277", merge rule): a query tile stays on chip (in registers) while
// the key/value tiles of its head stream through LDS. Each key tile updates, per query row, a
// running max m, an exp-sum l and an unnormalised output accumulator; when the max grows the old
// state is rescaled by exp(m_old - m_new). After the last tile O = acc / l and LSE = m + ln l.
// Causal masking happens inside the tile loop; tiles wholly above the diagonal are never
// visited (page 2, backward section and tips).
//
// gfx950 mapping (16-bit inputs):
//  * a work-group of Br/32 waves; wave w owns query rows [q_base + 32w, +32). Each SIMD runs two
//    waves whose MFMA and VALU phases can overlap: two of one 8-wave work-group for the 256-row
//    tiles (d = 128), one of each of two 4-wave work-groups for the 128-row tiles.
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: each lane then owns
//    ONE query row (l % 32) and 16 keys per 32-key block, so the row max and row sum are
//    in-register reductions plus one v_permlane32_swap between the two half-waves.
//  * Q^T is the MFMA B operand, loaded once from HBM into registers; K is the A operand, read
//    from the LDS tile with ds_read_b128.
//  * O^T = V^T P^T: P^T comes straight from the score accumulators (fp32 -> RNE 16-bit), V^T
//    fragments come from the row-major V tile with ds_read_b64_tr_b16, so V is never transposed
//    in memory. The MFMA reduction index is permuted consistently on both operands: slot s of
//    half-wave h stands for key 16c + 4h + (s & 3) + 8 (s >> 2) of 16-key chunk c.
//  * K/V tiles go from memory straight into LDS (buffer_load ... lds, no VGPR staging), two
//    stages deep: the next tile's loads are issued right after the barrier that frees its stage
//    and land while the current tile is computed. Tiles are stored unpadded with their 16-byte
//    chunks XOR-swizzled per row, which keeps both read patterns free of bank conflicts.
//  * The running max is kept in the log2 domain with scale*log2(e) folded into one multiply, and
//    is only moved when a row's max grows by more than kRescaleSlack (2^8): the factor is then
//    exactly 1 for almost every tile (page 2, tips), the exp2 arguments stay <= 8, and the result
//    is unchanged because O and l always share the same reference max.
//  * Work-group order: the 8 XCDs each take a contiguous range of heads; with the causal mask an
//    XCD takes its heads a few at a time (four, or fewer once their K/V pass 8 MiB) and runs
//    their query tiles longest first (the group's last tiles, then the ones before), which
//    balances the triangular work across CUs while only those heads' K/V compete for the XCD's
//    L2.
#include "fattn_device.hpp"
#include "fattn_launch.hpp"

#include "../../include/fattn.h"

namespace fattn {
namespace {

constexpr float kRescaleSlack = 8.0f;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int N;
  int n_qtiles;
  int bh_total;        // B * H
  int hgroup;          // causal grid order: heads of an XCD taken this many at a time
  float c;             // |scale| * log2(e), > 0
  uint32_t neg_mask;   // 0x80008000 flips the sign of two packed 16-bit Q elements (scale < 0)
  uint32_t keep_mask;  // 0 zeroes Q (scale == 0: every logit is 0), else all ones
  DropParams drop;     // dropout on P (used by the DROP instances only)
  const uint8_t* bmask;  // block mask [B*H][nb][nb] over 128 x 128 (query, key) blocks (SPARSE)
  int nb;                // ceil(N / 128)
};

// Block id -> (head, query tile). Hardware deals block ids round-robin over the 8 XCDs, so
// block x runs on XCD x % 8; each XCD is given a contiguous range of heads.
__device__ inline void fwd_block_coords(int bid, int nblocks, int n_qtiles, int bh_total, bool causal,
                                        int hgroup, int* bh, int* qt) {
  if ((bh_total & 7) == 0) {
    const int hpx = bh_total >> 3;
    const int xcd = bid & 7, local = bid >> 3;
    if (causal) {
      int hh, r;  // r: rank of the tile length, longest first
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

template <int D, int BR, int BC, int NS>
struct FwdCfg {
  static constexpr int NW = BR / 32;          // waves per work-group
  static constexpr int NT = NW * 64;          // threads per work-group
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int LPT = BC * CPR / NT;   // 16-byte loads per thread per tile per tensor
  static constexpr int TILE_B = BC * D * 2;   // bytes of one K (or V) tile
  static constexpr int STAGE_B = 2 * TILE_B;  // K then V
  static constexpr int LDS_B = NS * STAGE_B;  // NS stages: NS - 1 tiles in flight
  static constexpr int LPI = 2 * LPT;         // load instructions per thread per tile
  static_assert(BC * CPR % NT == 0, "tile load split");
  static_assert(BR % 32 == 0 && BC % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(NS >= 2 && (NS - 2) * LPI < 64, "vmcnt range");
};

// BIG: the head's K/V exceed the 32-bit range of buffer offsets, so tiles are fetched with
// per-lane 64-bit global addresses instead.
// DROP: dropout on P. The exp-sum l keeps every key (LSE is the undropped statistic); a dropped
// key's probability is zeroed before the PV product, and O is scaled by 1 / (1 - p) at the end.
// SPARSE: block-sparse attention. Key tiles whose 128 x 128 mask block is zero for every row of
// the work-group are neither loaded nor computed; a wave skips the tiles its own mask row zeroes.
// Rows with no allowed key give O = 0, LSE = -inf.
template <typename TR, int D, int BR, int BC, int NS, bool CAUSAL, bool BIG, bool DROP, bool SPARSE>
__global__ __launch_bounds__(BR / 32 * 64) void fwd_kernel(FwdArgs a) {
  using Cfg = FwdCfg<D, BR, BC, NS>;
  using vec8 = typename TR::vec8;
  constexpr int NT = Cfg::NT, CPR = Cfg::CPR, LPT = Cfg::LPT, TILE_B = Cfg::TILE_B;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[Cfg::LDS_B];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int N = a.N;

  int bh, qt;
  fwd_block_coords(blockIdx.x, gridDim.x, a.n_qtiles, a.bh_total, CAUSAL, a.hgroup, &bh, &qt);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qh = a.q + head;
  const uint16_t* __restrict__ Kh = a.k + head;
  const uint16_t* __restrict__ Vh = a.v + head;

  const int q_base = qt * BR;
  const int q0 = q_base + 32 * w;
  const int qrow = q0 + lr;
  const bool wave_active = q0 < N;
  const int wave_last = min(q0 + 31, N - 1);
  const int wave_kv_end = CAUSAL ? wave_last + 1 : N;

  const int kv_end = CAUSAL ? min(N, q_base + BR) : N;
  const int n_kv = (kv_end + BC - 1) / BC;

  // Load i of this thread fills LDS chunk i*NT + tid of a tile: row r = chunk / CPR holds, at
  // chunk position p = chunk % CPR, the source chunk p ^ swizzle(r). Both swizzles repeat every
  // 16 rows, so when one load instruction spans a multiple of 16 rows, load i lies exactly
  // i*NT*16 bytes after load 0 in memory and in LDS, and only load 0's offsets are kept.
  constexpr bool kPeriodic = NT % CPR == 0 && (NT / CPR) % 16 == 0;
  constexpr int NOFF = kPeriodic ? 1 : LPT;
  uint32_t offK[NOFF], offV[NOFF];  // byte offsets within a tile: row * 2D + source chunk * 16
#pragma unroll
  for (int i = 0; i < NOFF; ++i) {
    const int chunk = i * NT + tid;
    const int row = chunk / CPR, pos = chunk % CPR;
    offK[i] = (uint32_t)(row * D * 2 + (pos ^ swz_rowread<D>(row)) * 16);
    offV[i] = (uint32_t)(row * D * 2 + (pos ^ swz_trread<D>(row)) * 16);
  }
  auto off_k = [&](int i) { return kPeriodic ? offK[0] + (uint32_t)(i * NT * 16) : offK[i]; };
  auto off_v = [&](int i) { return kPeriodic ? offV[0] + (uint32_t)(i * NT * 16) : offV[i]; };
  const uint32_t head_bytes = BIG ? 0u : (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(Kh, head_bytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(Vh, head_bytes);
  // tile j into stage stg % NS (stg = j except for block-sparse runs, which skip tiles)
  auto issue = [&](int j, int stg) {
    uint8_t* st = smem + (stg % NS) * Cfg::STAGE_B + w * 64 * 16;
    const uint32_t soff = (uint32_t)(j * BC) * (D * 2);
    if (!BIG && (j + 1) * BC <= N) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const uint32_t add = kPeriodic ? (uint32_t)(i * NT * 16) : 0u;
        buffer_lds16(rK, st + i * NT * 16, kPeriodic ? offK[0] : offK[i], soff + add);
        buffer_lds16(rV, st + TILE_B + i * NT * 16, kPeriodic ? offV[0] : offV[i], soff + add);
      }
    } else if (!BIG) {
      // ragged last tile: the whole offset goes in the lane's offset register, which the
      // buffer's range check covers, so rows past the end of the head read as zeros (finite;
      // those keys are masked below)
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        buffer_lds16(rK, st + i * NT * 16, off_k(i) + soff, 0u);
        buffer_lds16(rV, st + TILE_B + i * NT * 16, off_v(i) + soff, 0u);
      }
    } else {
      // a head of 2 GiB or more: 64-bit addresses, rows past the end repeat row N - 1
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const size_t src_row = (size_t)min(j * BC + (i * NT + tid) / CPR, N - 1) * (D * 2);
        const uint32_t in_row = (uint32_t)((i * NT + tid) / CPR * D * 2);
        global_lds16((const uint8_t*)Kh + src_row + (off_k(i) - in_row), st + i * NT * 16);
        global_lds16((const uint8_t*)Vh + src_row + (off_v(i) - in_row), st + TILE_B + i * NT * 16);
      }
    }
  };
  // The first tiles' loads go out before the Q rows are read, so the two latencies overlap.
  if (!SPARSE)
    for (int t = 0; t < NS - 1 && t < n_kv; ++t) issue(t, t);

  // Q^T fragments: lane holds Q[qrow][16s + 8h .. +7] (zeros past the last row; the load itself
  // reads row N - 1, so it needs no branch).
  vec8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 raw = *(const u32x4*)(Qh + (size_t)min(qrow, N - 1) * D + 16 * s + 8 * h);
    if (qrow >= N) raw = u32x4{0u, 0u, 0u, 0u};
    raw = (raw ^ a.neg_mask) & a.keep_mask;
    qf[s] = bitcast<vec8>(raw);
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
  // A row of a block-sparse run can meet a tile whose keys it cannot see before its first real
  // one; a finite start keeps exp2(s*c - m_ref) at 0 there (not NaN), and the first real logit
  // always outgrows it with a rescale factor of exactly 0. Dense rows see key 0 in tile 0.
  float m_ref = SPARSE ? -3.402823466e38f : -__builtin_inff();
  float l_part = 0.f;

  const int tr_row = 4 * h + ((lane & 15) >> 2);
  const int tr_colb = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;  // byte offset in a 64-B group

  // S^T = K Q^T for tile j (BC/32 independent 32-key accumulator chains), masked on diagonal and
  // ragged tiles; returns the row max of the log2-domain logits.
  auto scores = [&](int j, int stg, f32x16 (&s)[BC / 32]) {
    const int k0 = j * BC;
    const uint8_t* Ks = smem + (stg % NS) * Cfg::STAGE_B;
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
    // keep the K fragment reads one step ahead of the MFMAs that consume them
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (BC / 32), 0);
#pragma unroll
    for (int st = 0; st < D / 16 - 2; ++st) {
      __builtin_amdgcn_sched_group_barrier(0x008, BC / 32, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, BC / 32, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * (BC / 32), 0);

    const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
    if (need_mask) {
      // element (kb, e) holds key k0 + kb*32 + 8(e>>2) + 4h + (e&3); it is masked when that
      // relative index exceeds lim
      int lim = N - 1 - k0;
      if (CAUSAL) lim = min(lim, qrow - k0);
      lim -= 4 * h;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          s[kb][e] = (kb * 32 + 8 * (e >> 2) + (e & 3) > lim) ? -__builtin_inff() : s[kb][e];
    }
    // one max chain per 32-key block, then across them: BC / 32 short dependent chains instead of
    // one of BC / 2 steps (both waves of a SIMD reach this point together, so its latency shows)
    float mk[BC / 32];
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      mk[kb] = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) mk[kb] = fmaxf(mk[kb], s[kb][e]);
    }
#pragma unroll
    for (int w2 = BC / 64; w2 >= 1; w2 >>= 1)
#pragma unroll
      for (int kb = 0; kb < w2; ++kb) mk[kb] = fmaxf(mk[kb], mk[kb + w2]);
    return max_halves(mk[0]) * a.c;  // c > 0, so this is the max of the log2-domain logits
  };
  // P^T = exp2(s*c - m_ref) (masked scores are -inf and give 0), packed to 16-bit MFMA B
  // fragments (8 keys per 16-key chunk), then O^T += V^T P^T with V^T fragments from the
  // transposed LDS read (rows 16c + tr_row and +8).
  auto softmax_pv = [&](int j, int stg, const f32x16 (&s)[BC / 32]) {
    const uint8_t* Vs = smem + (stg % NS) * Cfg::STAGE_B + TILE_B;
    const float neg_m = -m_ref;
    vec8 pf[BC / 16];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // element 8 half + t (t = 4g + r) holds key j BC + 32 kb + 8 (2 half + g) + 4h + r, i.e.
        // key 4h + r of 8-key group (j BC + 32 kb) / 8 + 2 half + g: keep bit t
        uint32_t kf[8];
        if (DROP)
          row_keep_fields((uint32_t)((j * BC) / 8 + 4 * kb + 2 * half), (uint32_t)qrow, (uint32_t)bh, a.drop, h, kf);
        u32x4 packed;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * half + 2 * e2], a.c, neg_m));
          float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * half + 2 * e2 + 1], a.c, neg_m));
          ls += p0 + p1;
          if (DROP) {
            p0 = kf[2 * e2] >= (a.drop.thr << 16) ? p0 : 0.f;
            p1 = kf[2 * e2 + 1] >= (a.drop.thr << 16) ? p1 : 0.f;
          }
          packed[e2] = TR::pack2(p0, p1);
        }
        pf[2 * kb + half] = bitcast<vec8>(packed);
      }
    l_part += ls;
#pragma unroll
    for (int c = 0; c < BC / 16; ++c) {
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
    // order: every exponential first, then the V^T reads of the first two MFMA chunks, then each
    // MFMA with the two reads of a later one (the reads lead by four MFMAs)
    __builtin_amdgcn_sched_group_barrier(0x002, 1000, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < BC / 16 * (D / 32) - 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  };

  // The tile loop leaves as soon as some row's max outgrows the slack; the rescale (rare) is
  // done outside it and the loop resumes. Keeping the conditional rescale out of the loop body
  // keeps the accumulator in one set of registers (a join inside the loop made the compiler copy
  // all of it on every tile).
  f32x16 s[BC / 32];
  float m_new = 0.f;
  int free_stage;  // an LDS stage that no wave reads or loads into once its loop has ended
  if constexpr (!SPARSE) {
    free_stage = n_kv % NS;  // the last tile, n_kv - 1, sits in the stage before it
    int j = 0;
    while (j < n_kv) {
      bool grew = false;
      for (; j < n_kv; ++j) {
        // this wave's loads of tile j have landed (tiles j+1 .. j+NS-2 may still be in flight)
        if (j + NS - 2 < n_kv) wait_vmcnt<(NS - 2) * Cfg::LPI>();
        else wait_vmcnt<0>();
        barrier_lds();  // ... and everyone's; stage (j - 1) % NS is no longer being read
        if (j + NS - 1 < n_kv) issue(j + NS - 1, j + NS - 1);
        if (!(wave_active && j * BC < wave_kv_end)) continue;
        const float mx = scores(j, j, s);
        m_new = fmaxf(m_ref, mx);
        if (wave_any(m_new > m_ref + kRescaleSlack)) {
          grew = true;
          break;
        }
        softmax_pv(j, j, s);
      }
      if (!grew) break;
      // Move the reference max of the rows that outgrew it, rescale their state, finish tile j.
      const bool grow = m_new > m_ref + kRescaleSlack;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      if (grow) m_ref = m_new;
      l_part *= alpha;
#pragma unroll
      for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;
      softmax_pv(j, j, s);
      ++j;
    }
  } else {
    // Block-sparse: the work-group's 128 query rows are one mask row; it visits the key tiles
    // whose mask column is set in that row, in order, two stages deep (stage = position in that
    // sequence). The row's allowed columns are scanned 64 at a time (MaskLine).
    static_assert(NS == 2, "block-sparse runs use two stages");
    static_assert(BR == 128 && 128 % BC == 0, "a block-sparse work-group is one mask row");
    constexpr int TPC = 128 / BC;  // key tiles per mask column
    MaskLine row = mask_line(a.bmask + ((size_t)bh * a.nb + qt) * a.nb, 1, a.nb);
    // the visited tile after j: the next tile of j's column, else the first of the next allowed one
    auto next = [&](int j) {
      const int jj = j + 1;
      if (jj >= n_kv) return n_kv;
      if (jj % TPC != 0) return jj;
      const int c = mask_next(row, jj / TPC, lane);
      return c >= (n_kv + TPC - 1) / TPC ? n_kv : c * TPC;
    };
    int j = next(-1), t = 0;
    if (j < n_kv) issue(j, 0);
    while (j < n_kv) {
      bool grew = false;
      int jn = j;
      for (; j < n_kv; j = jn, ++t) {
        wait_vmcnt<0>();
        barrier_lds();
        jn = next(j);
        if (jn < n_kv) issue(jn, t + 1);
        if (!(wave_active && j * BC < wave_kv_end)) continue;
        const float mx = scores(j, t, s);
        m_new = fmaxf(m_ref, mx);
        if (wave_any(m_new > m_ref + kRescaleSlack)) {
          grew = true;
          break;
        }
        softmax_pv(j, t, s);
      }
      if (!grew) break;
      const bool grow = m_new > m_ref + kRescaleSlack;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
      if (grow) m_ref = m_new;
      l_part *= alpha;
#pragma unroll
      for (int b = 0; b < D / 32; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;
      softmax_pv(j, t, s);
      j = jn;
      ++t;
    }
    free_stage = t % NS;  // positions 0 .. t - 1 were visited
  }

  if (!wave_active) return;
  const float l_tot = sum_halves(l_part);
  float inv = (DROP ? a.drop.inv_keep : 1.0f) / l_tot;
  if (SPARSE && !(l_tot > 0.f)) inv = 0.f;  // no allowed key: O = 0
  u32x2 ov[D / 8];
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      ov[4 * b + jj][0] = TR::pack2(acc[b][4 * jj] * inv, acc[b][4 * jj + 1] * inv);
      ov[4 * b + jj][1] = TR::pack2(acc[b][4 * jj + 2] * inv, acc[b][4 * jj + 3] * inv);
    }
  // O leaves through the free stage, each wave through its own slice of it
  constexpr int RP = Cfg::STAGE_B >= Cfg::NW * 32 * D * 2 ? 32 : 16;
  static_assert(Cfg::NW * RP * D * 2 <= Cfg::STAGE_B, "output staging");
  store_rows_via_lds<D, RP>(ov, smem + free_stage * Cfg::STAGE_B + w * (RP * D * 2), a.o + head + (size_t)q0 * D, N - q0);
  if (h == 0 && qrow < N)
    a.lse[(size_t)bh * N + qrow] = (SPARSE && !(l_tot > 0.f)) ? -__builtin_inff() : (m_ref + __log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------------------------
// float32 path: same algorithm on v_mfma_f32_32x32x2_f32 (full fp32 products), 32-key tiles.
// The A operand of S^T is K[key][d = 2s + h], the B operand Q[query][2s + h]; for O^T the
// reduction slot h of chunk (j, r) is key 8j + 4h + r, which is exactly where the score
// accumulator already holds it, so P^T needs no repacking.

template <int D, int BR>
struct FwdCfgF32 {
  static constexpr int BC = 32;
  static constexpr int NW = BR / 32;
  static constexpr int NT = NW * 64;
  static constexpr int KSTR = D + 2;
  static constexpr int VSTR = D + 4;
  static constexpr int CPR = D / 4;  // 16-byte chunks per row
  static constexpr int CH = BC * CPR / NT;
  static constexpr int KBUF = BC * KSTR;
  static constexpr int STAGE = KBUF + BC * VSTR;
  static_assert(BC * CPR % NT == 0, "tile load split");
};

struct FwdArgsF32 {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int N;
  int n_qtiles;
  float c;
  float qsign;
};

template <int D, int BR, bool CAUSAL>
__global__ __launch_bounds__(BR / 32 * 64) void fwd_kernel_f32(FwdArgsF32 a) {
  using Cfg = FwdCfgF32<D, BR>;
  constexpr int BC = Cfg::BC;
  __shared__ __attribute__((aligned(16))) float smem[2 * Cfg::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int N = a.N;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = logical / a.n_qtiles;
  int qt = logical - bh * a.n_qtiles;
  if (CAUSAL) qt = a.n_qtiles - 1 - qt;
  const size_t head = (size_t)bh * (size_t)N * D;
  const float* __restrict__ Qh = a.q + head;
  const float* __restrict__ Kh = a.k + head;
  const float* __restrict__ Vh = a.v + head;
  const int q_base = qt * BR;
  const int q0 = q_base + 32 * w;
  const int qrow = q0 + lr;
  const bool wave_active = q0 < N;
  const int wave_kv_end = CAUSAL ? min(q0 + 31, N - 1) + 1 : N;

  float qv[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qv[s] = (qrow < N) ? Qh[(size_t)qrow * D + 2 * s + h] * a.qsign : 0.f;

  const int kv_end = CAUSAL ? min(N, q_base + BR) : N;
  const int n_kv = (kv_end + BC - 1) / BC;

  f32x4 kr[Cfg::CH], vr[Cfg::CH];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < Cfg::CH; ++i) {
      const int c = tid + i * Cfg::NT;
      const int row = c / Cfg::CPR;
      const int col = c % Cfg::CPR;
      const int key = j * BC + row;
      if (key < N) {
        kr[i] = *(const f32x4*)(Kh + (size_t)key * D + col * 4);
        vr[i] = *(const f32x4*)(Vh + (size_t)key * D + col * 4);
      } else {
        kr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        vr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };
  auto store_tile = [&](int buf) {
    float* Ks = smem + buf * Cfg::STAGE;
    float* Vs = Ks + Cfg::KBUF;
#pragma unroll
    for (int i = 0; i < Cfg::CH; ++i) {
      const int c = tid + i * Cfg::NT;
      const int row = c / Cfg::CPR;
      const int col = c % Cfg::CPR;
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[row * Cfg::KSTR + col * 4 + e] = kr[i][e];
      *(f32x4*)(Vs + row * Cfg::VSTR + col * 4) = vr[i];
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[b][e] = 0.f;
  float m_ref = -__builtin_inff();
  float l_part = 0.f;

  load_tile(0);
  store_tile(0);
  for (int j = 0; j < n_kv; ++j) {
    if (j + 1 < n_kv) load_tile(j + 1);
    __syncthreads();
    const int k0 = j * BC;
    if (wave_active && k0 < wave_kv_end) {
      const float* Ks = smem + (j & 1) * Cfg::STAGE;
      const float* Vs = Ks + Cfg::KBUF;
      f32x16 s;
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int st = 0; st < D / 2; ++st)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[lr * Cfg::KSTR + 2 * st + h], qv[st], s, 0, 0, 0);

      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
      float mx = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float t = s[e] * a.c;
        if (need_mask) {
          const int key = k0 + 8 * (e >> 2) + 4 * h + (e & 3);
          t = (key >= N || (CAUSAL && key > qrow)) ? -__builtin_inff() : t;
        }
        s[e] = t;
        mx = fmaxf(mx, t);
      }
      mx = max_halves(mx);
      const float m_new = fmaxf(m_ref, mx);
      const bool grow = m_new > m_ref + kRescaleSlack;
      if (wave_any(grow)) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
        if (grow) m_ref = m_new;
        l_part *= alpha;
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[b][e] *= alpha;
      }
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = __builtin_amdgcn_exp2f(s[e] - m_ref);
        ls += s[e];
      }
      l_part += ls;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
        for (int b = 0; b < D / 32; ++b)
          acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * Cfg::VSTR + 32 * b + lr], s[e], acc[b], 0, 0, 0);
      }
    }
    if (j + 1 < n_kv) store_tile((j + 1) & 1);
  }

  if (!wave_active) return;
  const float l_tot = sum_halves(l_part);
  if (qrow >= N) return;
  const float inv = 1.0f / l_tot;
  float* Orow = a.o + head + (size_t)qrow * D;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      f32x4 v4;
#pragma unroll
      for (int r = 0; r < 4; ++r) v4[r] = acc[b][4 * jj + r] * inv;
      *(f32x4*)(Orow + 32 * b + 8 * jj + 4 * h) = v4;
    }
  if (h == 0) a.lse[(size_t)bh * N + qrow] = (m_ref + __log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------------------------
// Dispatch.

template <typename TR, int D, int BR, int BC, int NS, bool DROP = false, bool SPARSE = false>
hipError_t launch16(const FwdReq& r, hipStream_t st) {
  FwdArgs a;
  a.q = (const uint16_t*)r.q;
  a.k = (const uint16_t*)r.k;
  a.v = (const uint16_t*)r.v;
  a.o = (uint16_t*)r.o;
  a.lse = r.lse;
  a.N = r.N;
  a.n_qtiles = (r.N + BR - 1) / BR;
  a.bh_total = r.B * r.H;
  a.hgroup = head_group(a.bh_total, (size_t)2 * r.N * D * 2);
  a.c = r.scale == 0.f ? 1.f : fabsf(r.scale) * kLog2e;
  a.neg_mask = r.scale < 0.f ? 0x80008000u : 0u;
  a.keep_mask = r.scale == 0.f ? 0u : 0xffffffffu;
  a.drop = r.drop;
  a.bmask = r.bmask;
  a.nb = (r.N + 127) / 128;
  const long long nblk = (long long)r.B * r.H * a.n_qtiles;
  const dim3 grid((unsigned)nblk), block(BR / 32 * 64);
  // buffer offsets are 32-bit: heads of 2 GiB or more take the 64-bit address path
  const bool big = (size_t)r.N * D * 2 >= ((size_t)1 << 31);
  if (r.causal) {
    if (big) hipLaunchKernelGGL((fwd_kernel<TR, D, BR, BC, NS, true, true, DROP, SPARSE>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<TR, D, BR, BC, NS, true, false, DROP, SPARSE>), grid, block, 0, st, a);
  } else {
    if (big) hipLaunchKernelGGL((fwd_kernel<TR, D, BR, BC, NS, false, true, DROP, SPARSE>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((fwd_kernel<TR, D, BR, BC, NS, false, false, DROP, SPARSE>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <int D, int BR>
hipError_t launch32(const FwdReq& r, hipStream_t st) {
  FwdArgsF32 a;
  a.q = (const float*)r.q;
  a.k = (const float*)r.k;
  a.v = (const float*)r.v;
  a.o = (float*)r.o;
  a.lse = r.lse;
  a.N = r.N;
  a.n_qtiles = (r.N + BR - 1) / BR;
  a.c = fabsf(r.scale) * kLog2e;
  a.qsign = r.scale < 0.f ? -1.f : 1.f;
  const long long nblk = (long long)r.B * r.H * a.n_qtiles;
  const dim3 grid((unsigned)nblk), block(BR / 32 * 64);
  if (r.causal)
    hipLaunchKernelGGL((fwd_kernel_f32<D, BR, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((fwd_kernel_f32<D, BR, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <typename TR, int D>
hipError_t launch16_tile(const FwdReq& r, hipStream_t st) {
  // Block-sparse runs use 128 x 64 tiles: a work-group then covers one 128-row mask row, so its
  // waves never stream tiles allowed only for another mask row (measured 3-10% faster than
  // 256 x 128 at block densities 0.1-0.5). Dropout uses the default tile of each head dim.
  if (r.bmask) return launch16<TR, D, 128, 64, 2, false, true>(r, st);
  if (r.dropout) {
    if constexpr (D == 128) {
      if (r.Br != 256 || r.Bc != 128) return hipErrorInvalidValue;
      return launch16<TR, D, 256, 128, 2, true>(r, st);
    } else {
      if (r.Br != 128 || r.Bc != 64) return hipErrorInvalidValue;
      return launch16<TR, D, 128, 64, 2, true>(r, st);
    }
  }
  if (r.Br == 128 && r.Bc == 64) return launch16<TR, D, 128, 64, 2>(r, st);
  if (r.Br == 128 && r.Bc == 128) return launch16<TR, D, 128, 128, 2>(r, st);
  if (r.Br == 64 && r.Bc == 64) return launch16<TR, D, 64, 64, 2>(r, st);
  if (r.Br == 64 && r.Bc == 128) return launch16<TR, D, 64, 128, 2>(r, st);
  if (r.Br == 256 && r.Bc == 64) return launch16<TR, D, 256, 64, 2>(r, st);
  if (r.Br == 256 && r.Bc == 128) return launch16<TR, D, 256, 128, 2>(r, st);
  return hipErrorInvalidValue;
}

}  // namespace

bool fwd_tile_supported(int dtype, int d, int Br, int Bc) {
  if (d != 64 && d != 128) return false;
  if (dtype == FATTN_F32) return Bc == 32 && (Br == 64 || Br == 128);
  if (dtype == FATTN_F16 || dtype == FATTN_BF16)
    return (Br == 64 || Br == 128 || Br == 256) && (Bc == 64 || Bc == 128);
  return false;
}

bool fwd_default_tile(int dtype, int d, int causal, int* Br, int* Bc) {
  (void)causal;
  if (d != 64 && d != 128) return false;
  if (dtype == FATTN_F32) {
    *Br = 128;
    *Bc = 32;
    return true;
  }
  if (dtype == FATTN_F16 || dtype == FATTN_BF16) {
    // measured on MI355X: at d = 128, eight waves sharing 128-key tiles (128 KiB of LDS, one
    // work-group per CU) beat four waves on 64-key tiles by 4-10%; at d = 64 the smaller tile wins
    *Br = d == 128 ? 256 : 128;
    *Bc = d == 128 ? 128 : 64;
    return true;
  }
  return false;
}

hipError_t launch_fwd(const FwdReq& r, hipStream_t st) {
  if (r.dtype == FATTN_F32) {
    if (r.d == 64) return r.Br == 128 ? launch32<64, 128>(r, st) : launch32<64, 64>(r, st);
    return r.Br == 128 ? launch32<128, 128>(r, st) : launch32<128, 64>(r, st);
  }
  if (r.dtype == FATTN_BF16) return r.d == 64 ? launch16_tile<Bf16, 64>(r, st) : launch16_tile<Bf16, 128>(r, st);
  return r.d == 64 ? launch16_tile<F16, 64>(r, st) : launch16_tile<F16, 128>(r, st);
}

}  // namespace fattn
