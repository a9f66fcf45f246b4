// Throughput of float32 atomic adds into a dQ-shaped buffer on gfx950, the cost a backward that
// forms dQ inside the dK/dV pass (one dS K product per (query tile, key tile) pair, added into a
// float32 dQ accumulator) would pay on top of its matrix work.
//
// Shape: 32 heads of N = 4096 rows x d = 128 columns (float32, 64 MiB), causal. One work-group of
// 512 threads per (head, 128-key tile), as in the dK/dV kernel; it walks the 64-row query tiles
// from its diagonal to the end and adds one 64 x 128 float32 tile (32 KiB) into the accumulator
// for each: 1 GiB of adds per launch in all. Heads are dealt to XCDs in contiguous ranges (block x
// runs on XCD x % 8), so every add to one head comes from one XCD.
//
// Variants (all vector memory instructions, no return value used):
//   linear:  global_atomic_add_f32 at agent scope, each wave instruction on 64 consecutive floats
//   mfma:    the same adds in the layout a 32 x 32 MFMA accumulator leaves them in (wave w owns
//            the 32 x 32 block (w / 4, w % 4) of the tile; lane l holds rows 8j + 4(l / 32) + r of
//            column l % 32 in element 4j + r), so one instruction covers two 128-byte row pieces
//   store:   plain 4-byte stores of the linear pattern (not a sum; the rate to beat)
// (At work-group scope the compiler emits the same instruction for gfx950 as at agent scope.)
// Each variant is checked once: after one launch on a zeroed buffer, element (row r) must hold
// the number of key tiles that add into it, floor(r / 128) + 1 (exactly representable).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#define HC(x)                                                               \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                             \
    }                                                                       \
  } while (0)

constexpr int kHeads = 32, kN = 4096, kD = 128, kBK = 128, kBQ = 64, kNT = 512;
constexpr int kKeyTiles = kN / kBK, kQTiles = kN / kBQ;

template <int MODE>
__global__ __launch_bounds__(kNT) void add_tiles(float* __restrict__ acc) {
  const int bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int hpx = kHeads / 8;
  const int head = xcd * hpx + local / kKeyTiles;
  const int jt = local % kKeyTiles;
  float* base = acc + (size_t)head * kN * kD;
  const float one = 1.0f;
  for (int i = (jt * kBK) / kBQ; i < kQTiles; ++i) {
    float* tile = base + (size_t)i * kBQ * kD;
    // 64 x 128 floats = 16 per thread; each wave instruction covers 64 consecutive floats
#pragma unroll
    for (int t = 0; t < kBQ * kD / kNT; ++t) {
      if (MODE == 1) {
        const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
        const int row = 32 * (w >> 2) + 8 * (t >> 2) + 4 * (l >> 5) + (t & 3);
        const int col = 32 * (w & 3) + (l & 31);
        __hip_atomic_fetch_add(tile + row * kD + col, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        float* p = tile + t * kNT + threadIdx.x;
        if (MODE == 0)
          __hip_atomic_fetch_add(p, one, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          *p = one;
      }
    }
  }
}

template <int MODE>
static int run(const char* name, float* d_acc, std::vector<float>& host, hipEvent_t e0, hipEvent_t e1) {
  const size_t n = (size_t)kHeads * kN * kD;
  const dim3 grid(kHeads * kKeyTiles), block(kNT);
  // correctness: one launch on a zeroed buffer
  HC(hipMemset(d_acc, 0, n * sizeof(float)));
  hipLaunchKernelGGL(add_tiles<MODE>, grid, block, 0, 0, d_acc);
  HC(hipGetLastError());
  HC(hipDeviceSynchronize());
  HC(hipMemcpy(host.data(), d_acc, n * sizeof(float), hipMemcpyDeviceToHost));
  size_t bad = 0;
  for (size_t x = 0; x < n; ++x) {
    const int r = (int)((x / kD) % kN);
    const float want = MODE == 2 ? 1.0f : (float)(r / kBK + 1);
    bad += host[x] != want;
  }
  // timing: warm-up, then 20 launches
  for (int w = 0; w < 5; ++w) hipLaunchKernelGGL(add_tiles<MODE>, grid, block, 0, 0, d_acc);
  HC(hipDeviceSynchronize());
  const int reps = 20;
  HC(hipEventRecord(e0, 0));
  for (int w = 0; w < reps; ++w) hipLaunchKernelGGL(add_tiles<MODE>, grid, block, 0, 0, d_acc);
  HC(hipEventRecord(e1, 0));
  HC(hipEventSynchronize(e1));
  float ms = 0.f;
  HC(hipEventElapsedTime(&ms, e0, e1));
  ms /= reps;
  double adds = 0;
  for (int jt = 0; jt < kKeyTiles; ++jt) adds += (double)(kQTiles - (jt * kBK) / kBQ) * kBQ * kD;
  adds *= kHeads;
  printf("{\"variant\": \"%s\", \"ms\": %.4f, \"adds\": %.0f, \"payload_GB_s\": %.1f, \"wrong_elements\": %zu}\n", name,
         ms, adds, adds * 4 / (ms * 1e-3) / 1e9, bad);
  return 0;
}

int main() {
  const size_t n = (size_t)kHeads * kN * kD;
  float* d_acc = nullptr;
  HC(hipMalloc(&d_acc, n * sizeof(float)));
  std::vector<float> host(n);
  hipEvent_t e0, e1;
  HC(hipEventCreate(&e0));
  HC(hipEventCreate(&e1));
  if (run<0>("linear", d_acc, host, e0, e1)) return 1;
  if (run<1>("mfma", d_acc, host, e0, e1)) return 1;
  if (run<2>("store", d_acc, host, e0, e1)) return 1;
  HC(hipFree(d_acc));
  return 0;
}
