// Issue-rate micro-benchmark for gfx950: how many SIMD cycles one wave64 instruction of each kind
// occupies (bf16 MFMA 32x32x16, v_exp_f32, v_fma_f32, v_mad_u64_u32, v_bitop3_b32, ds_read_b128,
// ds_read_b64_tr_b16, and a whole Philox4x32-10 call of the dropout kernels), and how
// well MFMA overlaps VALU work from the same wave and from another wave on the same SIMD. These
// are the ceilings the attention kernels work against: per score element the forward issues
// 2 x 2d / 32768 MFMAs, one v_exp_f32 and a handful of plain VALU instructions.
//
// One work-group of 256 or 512 threads per CU (4 or 8 waves, i.e. 1 or 2 waves per SIMD); every
// wave runs R iterations of a fixed instruction mix and reads the shader clock (s_memtime) around
// its loop. A group's span runs from its first wave's start to its last wave's end: one wave
// alone is no measure of a shared SIMD, because the older wave of a pair gets the issue slots
// first and finishes early. Reported: span cycles per iteration, and cycles per unit, a unit being
// one instruction of the timed kind issued on the SIMD (for mixes: one MFMA, whose own rate is
// 32 cycles). All LDS addresses stay
// inside the group's 64 KiB array; nothing is written to memory except one word per thread that
// the compiler cannot prove dead.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#define HC(x)                                                                   \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);     \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int R = 2048;
constexpr int LDS_BYTES = 65536;

enum : int { LDS128 = 1, LDSTR = 2, MFMA = 4, EXP = 8, FMA = 16, LDSBW = 32, LDSTRBW = 64, MAD64 = 128, BOP3 = 256,
             PHILOX = 1024 };

// MODE: a bit set of the instruction groups each iteration issues; SPLIT: waves 0-3 issue only the
// MFMA group and waves 4-7 only the VALU groups (so each SIMD pairs one MFMA wave with one VALU wave).
template <int MODE, bool SPLIT>
__global__ __launch_bounds__(512) void mix(float* out, long long* cyc, float seed) {
  __shared__ __attribute__((aligned(16))) uint8_t sm[LDS_BYTES];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int i = t; i < LDS_BYTES / 4; i += blockDim.x) ((uint32_t*)sm)[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const bool do_mfma = (MODE & MFMA) && (!SPLIT || w < 4);
  const bool do_valu = !SPLIT || w >= 4;
  u32x4 x = {0u, 0u, 0u, 0u};
  f32x16 acc[4];
  for (int j = 0; j < 4; ++j)
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{(uint32_t)t, 1u, 2u, 3u});
  float ev[16], fv[16];
  for (int e = 0; e < 16; ++e) {
    ev[e] = seed * (float)(e + lane) * 1e-3f;
    fv[e] = ev[e];
  }
  const long long c0 = clock64();
  for (int r = 0; r < R; ++r) {
    if (MODE & LDS128) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x ^= *(volatile u32x4*)(sm + ((lane * 16 + i * 1024 + r * 64) & (LDS_BYTES - 1)));
    }
    if (MODE & LDSTR) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const i16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(sm + ((lane * 8 + i * 512 + r * 64) & (LDS_BYTES - 1))));
        x[i & 3] ^= __builtin_bit_cast(uint2, y).x;
      }
    }
    if (MODE & LDSBW) {  // 16 independent ds_read_b128, combined only after all have been issued
      u32x4 y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = *(const u32x4*)(sm + ((lane * 16 + i * 1024 + r * 64) & (LDS_BYTES - 1)));
#pragma unroll
      for (int i = 0; i < 16; ++i) x ^= y[i];
    }
    if (MODE & LDSTRBW) {  // 16 independent ds_read_b64_tr_b16
      uint32_t y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        y[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                   (lds_i16x4*)(sm + ((lane * 8 + i * 512 + r * 64) & (LDS_BYTES - 1))))).x;
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i & 3] ^= y[i];
    }
    if ((MODE & MAD64) && do_valu) {  // 32 v_mad_u64_u32 in 8 independent chains
#pragma unroll
      for (int k = 0; k < 4; ++k)
  #pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint64_t pr = (uint64_t)0xD2511F53u * (uint32_t)__float_as_uint(fv[e]) + (uint32_t)__float_as_uint(fv[e + 8]);
          fv[e] = __uint_as_float((uint32_t)(pr >> 32));
          fv[e + 8] = __uint_as_float((uint32_t)pr);
        }
    }
    if ((MODE & BOP3) && do_valu) {  // 64 v_bitop3 in 16 chains
#pragma unroll
      for (int k = 0; k < 4; ++k)
  #pragma unroll
        for (int e = 0; e < 16; ++e)
          fv[e] = __uint_as_float(__builtin_amdgcn_bitop3_b32(__float_as_uint(fv[e]), (uint32_t)lane, (uint32_t)(e + k), 0x96));
    }
    if ((MODE & PHILOX) && do_valu) {  // 4 Philox4x32-10 calls (independent)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint32_t c0 = __float_as_uint(fv[4 * c]), c1 = __float_as_uint(fv[4 * c + 1]), c2 = __float_as_uint(fv[4 * c + 2]), c3 = __float_as_uint(fv[4 * c + 3]);
        uint32_t k0 = 0x12345u + (uint32_t)r, k1 = 0x6789u;
  #pragma unroll
        for (int rr = 0; rr < 10; ++rr) {
          const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
          const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
          c0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
          c1 = (uint32_t)p1;
          c2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
          c3 = (uint32_t)p0;
          k0 += 0x9E3779B9u;
          k1 += 0xBB67AE85u;
        }
        fv[4 * c] = __uint_as_float(c0); fv[4 * c + 1] = __uint_as_float(c1); fv[4 * c + 2] = __uint_as_float(c2); fv[4 * c + 3] = __uint_as_float(c3);
      }
    }
    if (do_mfma) {  // 16 MFMAs in 4 independent accumulator chains
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, acc[j], 0, 0, 0);
    }
    if ((MODE & EXP) && do_valu) {  // 32 v_exp_f32 in 16 independent chains (exp2(-x) stays in (0, 1])
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int e = 0; e < 16; ++e) ev[e] = __builtin_amdgcn_exp2f(-ev[e]);
    }
    if ((MODE & FMA) && do_valu) {  // 64 v_fma_f32 in 16 independent chains
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int e = 0; e < 16; ++e) fv[e] = fmaf(fv[e], 0.999f, 1e-3f);
    }
  }
  const long long c1 = clock64();
  float s = (float)(x[0] ^ x[1] ^ x[2] ^ x[3]);
  for (int j = 0; j < 4; ++j)
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  for (int e = 0; e < 16; ++e) s += ev[e] + fv[e];
  if (s == 1234.5f) out[t] = s;
  if (lane == 0) {
    cyc[(blockIdx.x * 8 + w) * 2] = c0;
    cyc[(blockIdx.x * 8 + w) * 2 + 1] = c1;
  }
}

// units: instructions of the timed kind per SIMD per iteration (for mixes: MFMAs per SIMD, so the
// last column is cycles per MFMA with the other work riding along; 32 is the MFMA-only rate)
template <int MODE, bool SPLIT>
int run(const char* name, int threads, int units, float* out, long long* cyc, int blocks) {
  for (int it = 0; it < 3; ++it) hipLaunchKernelGGL((mix<MODE, SPLIT>), dim3(blocks), dim3(threads), 0, 0, out, cyc, 1.0f);
  HC(hipGetLastError());
  HC(hipDeviceSynchronize());
  static long long h[1024 * 16];
  HC(hipMemcpy(h, cyc, (size_t)blocks * 16 * sizeof(long long), hipMemcpyDeviceToHost));
  const int waves = threads / 64;
  double avg = 0;
  for (int b = 0; b < blocks; ++b) {
    long long lo = h[b * 16], hi = h[b * 16 + 1];
    for (int w = 1; w < waves; ++w) {
      lo = h[(b * 8 + w) * 2] < lo ? h[(b * 8 + w) * 2] : lo;
      hi = h[(b * 8 + w) * 2 + 1] > hi ? h[(b * 8 + w) * 2 + 1] : hi;
    }
    avg += (double)(hi - lo);
  }
  avg /= blocks;
  const double per_iter = avg / R;
  printf("| %-46s | %d | %8.1f | %3d | %6.2f |\n", name, threads / 256, per_iter, units, per_iter / units);
  return 0;
}

int main() {
  float* out;
  long long* cyc;
  HC(hipMalloc(&out, 512 * sizeof(float)));
  HC(hipMalloc(&cyc, 1024 * 16 * sizeof(long long)));
  int dev = 0, ncu = 0;
  HC(hipGetDevice(&dev));
  HC(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  int khz = 0;
  HC(hipDeviceGetAttribute(&khz, hipDeviceAttributeClockRate, dev));
  const int B = ncu > 0 && ncu <= 1024 ? ncu : 256;  // one group per CU
  // dense bf16 peak = CUs x max engine clock x 4 SIMDs x (32768 FLOP per MFMA / its cycles)
  printf("compute units: %d; max engine clock %.0f MHz; %d iterations per wave\n", ncu, khz / 1e3, R);
  printf("bf16 MFMA peak at 32 cycles per 32x32x16 MFMA: %.1f TFLOP/s\n\n",
         (double)ncu * khz * 1e3 * 4 * (32768.0 / 32.0) / 1e12);
  printf("| mix (per wave per iteration) | waves/SIMD | cycles/iter | units/SIMD/iter | cycles/unit |\n"
         "|---|---|---|---|---|\n");
  int rc = 0;
  rc |= run<MFMA, false>("16 x mfma_f32_32x32x16_bf16", 256, 16, out, cyc, B);
  rc |= run<MFMA, false>("16 x mfma_f32_32x32x16_bf16", 512, 32, out, cyc, B);
  rc |= run<EXP, false>("32 x v_exp_f32", 256, 32, out, cyc, B);
  rc |= run<EXP, false>("32 x v_exp_f32", 512, 64, out, cyc, B);
  rc |= run<FMA, false>("64 x v_fma_f32", 256, 64, out, cyc, B);
  rc |= run<FMA, false>("64 x v_fma_f32", 512, 128, out, cyc, B);
  rc |= run<LDS128, false>("8 x ds_read_b128 (+ xor)", 512, 16, out, cyc, B);
  rc |= run<LDSTR, false>("8 x ds_read_b64_tr_b16 (+ xor)", 512, 16, out, cyc, B);
  rc |= run<MFMA | EXP, false>("16 mfma + 32 exp, same wave", 512, 32, out, cyc, B);
  rc |= run<MFMA | FMA, false>("16 mfma + 64 fma, same wave", 512, 32, out, cyc, B);
  rc |= run<MFMA | EXP, true>("16 mfma (waves 0-3) / 32 exp (waves 4-7)", 512, 16, out, cyc, B);
  rc |= run<MFMA | FMA, true>("16 mfma (waves 0-3) / 64 fma (waves 4-7)", 512, 16, out, cyc, B);
  rc |= run<MFMA | LDSTR, false>("16 mfma + 8 tr reads, same wave", 512, 32, out, cyc, B);
  // LDS bandwidth: bytes per CU per cycle = units/SIMD/iter x 4 SIMDs x 64 lanes x bytes per lane / cycles
  rc |= run<LDSBW, false>("16 x ds_read_b128, independent", 256, 16, out, cyc, B);
  rc |= run<LDSBW, false>("16 x ds_read_b128, independent", 512, 32, out, cyc, B);
  rc |= run<LDSTRBW, false>("16 x ds_read_b64_tr_b16, independent", 512, 32, out, cyc, B);
  rc |= run<MFMA | LDSBW, false>("16 mfma + 16 b128 reads, same wave", 512, 32, out, cyc, B);
  // the dropout generator: 32 x 32 -> 64-bit products, three-input xors, and whole calls
  rc |= run<MAD64, false>("32 x v_mad_u64_u32", 512, 64, out, cyc, B);
  rc |= run<BOP3, false>("64 x v_bitop3_b32", 512, 128, out, cyc, B);
  rc |= run<PHILOX, false>("4 x philox4x32-10 (units: calls)", 512, 8, out, cyc, B);
  rc |= run<MFMA | PHILOX, false>("16 mfma + 4 philox, same wave", 512, 32, out, cyc, B);
  rc |= run<MFMA | PHILOX, true>("16 mfma (waves 0-3) / 4 philox (waves 4-7)", 512, 16, out, cyc, B);
  return rc;
}
