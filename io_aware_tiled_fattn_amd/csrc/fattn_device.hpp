// Device primitives for the gfx950 (CDNA4) attention kernels: element traits, MFMA wrappers,
// the LDS transposed read, and the cross-half-wave reductions.
//
// Register layouts used throughout (v_mfma_f32_32x32x16_{bf16,f16}, wave64, lane l, h = l / 32):
//   A operand (M x K = 32 x 16): lane l holds A[l % 32][8h + i], i = 0..7
//   B operand (K x N = 16 x 32): lane l holds B[8h + i][l % 32]
//   C/D (32 x 32, 16 floats)    : lane l holds D[8j + 4h + r][l % 32] in element 4j + r
// The float32 path uses v_mfma_f32_32x32x2_f32: A[l % 32][h], B[h][l % 32], same C/D layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fattn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element traits for the 16-bit input types: MFMA on 8-element fragments, RNE conversions.
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));

struct Bf16 {
  using vec8 = bf16x8;
  using scalar = __bf16;
  static __device__ inline f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ inline scalar from_f32(float x) { return (__bf16)x; }
  // two floats -> two RNE bf16 in one dword (low half = x)
  static __device__ inline uint32_t pack2(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{x, y}, bf16x2v));
  }
};
struct F16 {
  using vec8 = f16x8;
  using scalar = _Float16;
  static __device__ inline f32x16 mma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ inline scalar from_f32(float x) { return (_Float16)x; }
  static __device__ inline uint32_t pack2(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{x, y}, f16x2v));
  }
};

template <typename V, typename U>
__device__ inline V bitcast(U u) {
  static_assert(sizeof(U) == sizeof(V), "bitcast size");
  return __builtin_bit_cast(V, u);
}

// Cross-half reductions: lanes l and l ^ 32 combine (v_permlane32_swap gives both halves).
__device__ inline float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives element j % 4 of the 8-byte
// chunks addressed by lanes 4e + j / 4 (e = 0..3), i.e. a 4 x 16 block of 16-bit elements whose
// four rows are addressed by lanes {0..3}, {4..7}, {8..11}, {12..15} (each lane one 4-element
// quarter of its row) comes back column by column.
// The pointer is declared restrict so that, once inlined, the read carries alias-scope
// information: the compiler then does not make it wait for every global->LDS load in flight
// (the kernels' own waits and barriers order those; a transposed read never touches a stage
// that is still being filled).
__device__ inline i16x4 lds_read_tr16(const void* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ inline bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }


// ---- direct global -> LDS loads (buffer_load_dwordx4 ... lds) --------------------------------
// One instruction moves 16 bytes per lane from memory straight into LDS, without VGPRs: lane i's
// 16 bytes land at LDS byte (lds + 16 * i), where lds is the same for the whole wave. The source
// is the buffer resource's base + voffset (per lane) + soffset (scalar). Completion is tracked by
// vmcnt; the caller waits with wait_vmcnt and then barriers before other waves read the data.
typedef __attribute__((address_space(3))) void lds_void;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer (stride 0), num_records in bytes; out-of-range lanes read zeros
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ inline void buffer_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}
__device__ inline void global_lds16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Work-group barrier without the memory fence of __syncthreads (which would also wait for every
// outstanding global->LDS prefetch). LDS reads of this wave are drained first, so no other wave
// can overwrite a buffer this wave is still reading; prefetches stay in flight.
__device__ inline void barrier_lds() {
  __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Store of a wave's 32 output rows of D 16-bit elements held the MFMA accumulator way (lane l owns
// row l % 32 and, in vals[4b + g], the 4 elements at columns 32b + 8g + 4(l / 32) .. + 3 as two
// packed pairs). Stored directly, each store instruction would write 8 bytes into each of 32 rows.
// The rows go through `stage` (RP * D * 2 bytes of LDS that no other wave uses meanwhile; 16-byte
// chunks XOR-swizzled per row, and the two 8-byte halves of a chunk swapped in every other group
// of D / 8 rows, so that the 8-byte writes of lanes l and l + D / 8 land in different banks), RP
// rows at a time, and leave as 16-byte stores that cover
// 64 / (D / 8) whole rows per instruction. Rows r >= nvalid are not stored. `out` is row 0,
// 16-byte aligned, rows D elements apart.
template <int D, int RP>
__device__ inline void store_rows_via_lds(const u32x2 (&vals)[D / 8], uint8_t* stage, uint16_t* out, int nvalid) {
  static_assert(RP == 16 || RP == 32, "rows per pass");
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;  // rows per read instruction
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, h = lane >> 5;
  const int cc = lane % CPR;
#pragma unroll
  for (int p = 0; p < 32 / RP; ++p) {
    const int sr = lr - p * RP;  // this lane's row within the pass
    if (sr >= 0 && sr < RP) {
#pragma unroll
      for (int c = 0; c < CPR; ++c)
        *(u32x2*)(stage + sr * (D * 2) + ((c ^ (sr & (CPR - 1))) << 4) + 8 * (h ^ ((sr / CPR) & 1))) = vals[c];
    }
    // the same wave reads what its other lanes wrote: LDS serves one wave's accesses in order,
    // and the wait and the compiler barriers keep the reads after the writes (and the next
    // pass's writes after these reads)
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < RP / RPI; ++i) {
      const int r = i * RPI + lane / CPR;
      u32x4 x = *(const u32x4*)(stage + r * (D * 2) + ((cc ^ (r & (CPR - 1))) << 4));
      if ((r / CPR) & 1) x = u32x4{x[2], x[3], x[0], x[1]};
      if (p * RP + r < nvalid) *(u32x4*)(out + (size_t)(p * RP + r) * D + cc * 8) = x;
    }
    asm volatile("" ::: "memory");
  }
}

// XOR swizzles of the 16-byte chunks of a row-major LDS tile (rows of D 16-bit elements), chosen
// so that the reads below hit distinct banks:
//  * K tiles are read with ds_read_b128, 32 consecutive rows at one chunk column per instruction;
//  * V tiles are read with ds_read_b64_tr_b16, 64-byte column groups of 4 rows at a time, so the
//    swizzle moves whole 4-chunk groups (it is a multiple of 4).
template <int D>
__device__ inline int swz_rowread(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ inline int swz_trread(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
// For tiles read both ways (row reads of 16 consecutive rows at one chunk, and transposed reads
// of 4-row x 4-chunk blocks): the low row bits pick the 4-chunk group, the next bits the chunk
// inside it, so both patterns touch distinct 16-byte bank slots. Individual chunks move, so a
// transposed read addresses each lane's chunk separately (tr_read_addr).
template <int D>
__device__ inline int swz_dual(int row) {
  return D == 128 ? 4 * (row & 3) + ((row >> 2) & 3) : 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// ---- dropout keep mask ---------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011): ten rounds of
//   (hi0, lo0) = M0 * c0, (hi1, lo1) = M1 * c2, c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0),
// the key bumped by the Weyl constants between rounds.
__device__ inline u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                      uint32_t k1) {
  // one v_mad_u64_u32 per 32 x 32 -> 64-bit product and one three-input v_bitop3_b32 (truth
  // table 0x96: a ^ b ^ c) per xor pair, half the instructions of separate mul_lo / mul_hi / xor
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    c0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    c1 = (uint32_t)p1;
    c2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// The keep decision of (head bh, query i, key j) is 16-bit field f = j % 8 of Philox4x32-10 at
// counter (j / 8, i, bh, 0) under the 64-bit seed (field f: the low half of word f for f < 4, the
// high half of word f - 4 otherwise), compared with floor(p 2^16). One generator call thus
// decides 8 keys of one query.
struct DropParams {
  uint32_t seed_lo, seed_hi;
  uint32_t thr;      // floor(p * 2^16)
  float inv_keep;    // 1 / (1 - p)
};

template <int T>
__device__ inline uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, T | (T << 2) | (T << 4) | (T << 6), 0xF, 0xF, false);
}

// Row layout (forward and dQ kernels: lanes l and l ^ 32 own the same query row, lane half h
// holds keys 4h .. 4h + 3 of every 8-key group). For the two 8-key groups g8 and g8 + 1, lane
// half h draws the generator once, for group g8 + h, and the two halves swap the 16-bit fields the
// other one needs. On return f[4g + r] holds, in its high 16 bits, the field of key
// 8 (g8 + g) + 4h + r of this lane's row (the low bits are not defined): the key is kept iff
// f[4g + r] >= dp.thr << 16. Both lanes of every pair must be active.
__device__ inline void row_keep_fields(uint32_t g8, uint32_t row, uint32_t bh, const DropParams& dp, int h,
                                       uint32_t (&f)[8]) {
  const u32x4 w = philox4x32_10(g8 + (uint32_t)h, row, bh, 0u, dp.seed_lo, dp.seed_hi);
  const uint32_t sh_own = 16u - 16u * (uint32_t)h, sh_send = 16u * (uint32_t)h;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t own = w[r] << sh_own;    // field 4h + r of the drawn group, moved to the top
    const uint32_t send = w[r] << sh_send;  // field 4(1 - h) + r: the partner's key
    // v_permlane32_swap of a value with itself leaves {low half's, high half's} value in the two
    // results; xor-ing both with the lane's own value leaves the partner's, whichever order
    const auto sw = __builtin_amdgcn_permlane32_swap(send, send, false, false);
    const uint32_t got = sw[0] ^ sw[1] ^ send;
    f[r] = h ? got : own;  // group g8 (drawn by the h = 0 lane)
    f[4 + r] = h ? own : got;
  }
}

// Column layout (dK/dV kernel: a lane owns one key, key % 8 = lane % 8, so the 8 lanes of an
// octet hold one 8-key group g8; lane half h owns queries 4h + r of each 8-query block). Octet
// lane t draws the generator once, for query q0 + 8 (t / 4) + (t % 4), and turns its 8 fields
// into an 8-bit mask (bit k = key k of the group); the octet then transposes the 8 x 8 bits over
// DPP (the other quad's masks arrive by a half-row mirror, then quad broadcasts). Bit u of the
// result is the keep bit of this lane's key for query q0 + 8 (u / 4) + (u % 4). Every lane of the
// octet must be active.
__device__ inline uint32_t col_keep_bits(uint32_t g8, uint32_t q0, uint32_t bh, const DropParams& dp, int lane) {
  const int t = lane & 7;
  const u32x4 w = philox4x32_10(g8, q0 + 8u * (uint32_t)(t >> 2) + (uint32_t)(t & 3), bh, 0u, dp.seed_lo, dp.seed_hi);
  uint32_t m = 0u;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    m |= ((w[r] & 0xffffu) >= dp.thr ? 1u : 0u) << r;
    m |= ((w[r] >> 16) >= dp.thr ? 1u : 0u) << (r + 4);
  }
  // row_half_mirror: octet lane i receives lane 7 - i's mask, so quad lane v of this quad holds
  // the other quad's lane 3 - v
  const uint32_t oth = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x141, 0xF, 0xF, false);
  uint32_t x = 0u, y = 0u;  // this quad's queries, the other quad's
  x |= ((quad_bcast<0>(m) >> t) & 1u) | (((quad_bcast<1>(m) >> t) & 1u) << 1) |
       (((quad_bcast<2>(m) >> t) & 1u) << 2) | (((quad_bcast<3>(m) >> t) & 1u) << 3);
  y |= ((quad_bcast<3>(oth) >> t) & 1u) | (((quad_bcast<2>(oth) >> t) & 1u) << 1) |
       (((quad_bcast<1>(oth) >> t) & 1u) << 2) | (((quad_bcast<0>(oth) >> t) & 1u) << 3);
  return t < 4 ? (x | (y << 4)) : (y | (x << 4));
}

// ---- block-mask scans ------------------------------------------------------------------------
// One line of a block mask (a mask row, or a mask column read with a stride), 64 entries at a
// time: lane l tests entry base + l, and a ballot turns the 64 tests into one wave-uniform bit
// set, so the next allowed entry is found by a scalar bit scan instead of one dependent memory
// load per entry. Windows are loaded only where no tile prefetch is in flight (right after a
// tile loop's vmcnt wait), so the load waits for nothing but itself.
struct MaskLine {
  const uint8_t* p;  // entry e at p[e * stride]
  long long stride;
  int n;             // entries in the line (0: an empty line)
  int base;          // first entry of the loaded window (negative before the first load)
  uint64_t bits;     // bit i: entry base + i is nonzero
};
__device__ inline MaskLine mask_line(const uint8_t* p, long long stride, int n) {
  return MaskLine{p, stride, n, -64, 0ull};
}
// Smallest allowed entry >= e, or 0x7fffffff if there is none.
__device__ inline int mask_next(MaskLine& m, int e, int lane) {
  if (e < 0) e = 0;
  while (e < m.n) {
    if (e < m.base || e >= m.base + 64) {
      const int base = e & ~63;
      const int x = base + lane;
      const bool on = x < m.n && m.p[(size_t)x * m.stride] != 0;
      m.bits = __builtin_amdgcn_ballot_w64(on);
      m.base = base;
    }
    const uint64_t rest = m.bits >> (e - m.base);
    if (rest) return e + (int)__builtin_ctzll(rest);
    e = m.base + 64;
  }
  return 0x7fffffff;
}

// Causal grid order within one XCD: its hpx heads are taken `group` at a time, and inside a group
// the tiles of all its heads run longest first (rank 0 = longest), so the triangular work stays
// balanced while at most `group` heads' K/V (or Q/dO) compete for the XCD's L2. `local` runs over
// hpx * ntiles values; every (head, rank) pair comes out exactly once.
__device__ inline void causal_xcd_order(int local, int hpx, int ntiles, int group, int* head, int* rank) {
  const int G = group < 1 ? 1 : (group > hpx ? hpx : group);
  const int g = local / (G * ntiles);
  const int rem = local - g * G * ntiles;
  const int Gg = min(G, hpx - g * G);  // the last group may hold fewer heads
  *rank = rem / Gg;
  *head = g * G + (rem - *rank * Gg);
}

// Block index remap so that consecutive logical blocks share an XCD: hardware dispatches block
// ids round-robin over the 8 XCDs, so physical id x runs on XCD x % 8. When the grid is a
// multiple of 8 the logical order visits, per XCD, one contiguous range of work.
__device__ inline int xcd_remap(int bid, int nblocks) {
  if ((nblocks & 7) != 0) return bid;
  return (bid & 7) * (nblocks >> 3) + (bid >> 3);
}

}  // namespace fattn
