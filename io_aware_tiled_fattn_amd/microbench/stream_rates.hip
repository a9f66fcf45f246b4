// Streaming-read rates on gfx950 for the split-KV decode's access pattern: 1024 work-groups each
// reading 2 MiB (2 GiB in all), as the partial kernel's work-groups read one split of one head's
// K and V (B=8 H=32 Nk=16384 d=128 bf16, 4 splits), in 16 KiB tiles (K and V of 32 keys).
//
// Variants (no compute; one dword of each tile is read back so the loads are used):
//   dma ring:  one wave per work-group fills an NS-stage LDS ring with buffer_load_dwordx4 ... lds,
//              NS - 1 tiles in flight (16 load instructions per tile; a wave's vmcnt counts at most
//              63 outstanding loads, so at most 3 tiles beyond the current one);
//              the decode kernel's loads without its MFMA work. Tile orders: each work-group its own
//              contiguous 2 MiB (the decode kernel's), grid-stride (tile t of work-group b is
//              global tile t * 1024 + b), 4-way interleave (4 work-groups share 8 MiB, member s
//              takes tiles 4t + s), or each work-group its own 2 MiB starting at a tile that
//              depends on b and wrapping around (the same bytes per work-group, but work-groups
//              that run together read at different offsets within their regions).
//   vgpr:      16-byte global loads into registers, 1 or 4 waves per work-group, 2 or 4 tiles ahead.
// Each variant: 5 warm-up launches, then the mean of 20 (HIP events).
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#include "../csrc/fattn_device.hpp"
using namespace fattn;
#define HC(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { printf("HIP error %s line %d\n", hipGetErrorString(e_), __LINE__); return 1; } } while (0)

constexpr size_t REGION = 2u << 20;   // bytes per work-group
constexpr int TILE = 16384;           // bytes per tile (K+V of 32 keys at d=128 bf16)

// one wave; NS-stage LDS ring filled with buffer_load_dwordx4 ... lds (TILE/1024 instructions per tile)
template <int NS, int MODE = 0>
__global__ __launch_bounds__(64) void dma_ring(const uint8_t* src, uint32_t* out) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * TILE];
  const int lane = threadIdx.x;
  constexpr int LPT = TILE / 1024;
  const int ntiles = REGION / TILE;
  // MODE 0: work-group b streams its own 2 MiB region; MODE 1: tile t of work-group b is global
  // tile t * nwg + b (grid-stride); MODE 2: groups of 4 work-groups share an 8 MiB region, tile t
  // of member s is tile 4 t + s of the region; MODE 3 and 4: as MODE 0, but tile t of work-group b
  // is tile (t + r) mod 128 of its region, with r = 37 b mod 128 (MODE 3) or r = b mod 128 (MODE 4)
  const uint8_t* base = MODE == 0 || MODE >= 3 ? src + (size_t)blockIdx.x * REGION
                      : MODE == 1 ? src : src + (size_t)(blockIdx.x / 4) * 4 * REGION;
  const uint32_t nrec = MODE == 1 ? 0xffffffffu : (uint32_t)(MODE == 2 ? 4 * REGION : REGION);
  const int rot = MODE == 3 ? (int)((blockIdx.x * 37u) % (REGION / TILE)) : (int)(blockIdx.x % (REGION / TILE));
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, nrec);
  auto tile_off = [&](int t) -> size_t {
    return MODE == 0 ? (size_t)t * TILE
         : MODE == 1 ? ((size_t)t * gridDim.x + blockIdx.x) * TILE
         : MODE == 2 ? ((size_t)t * 4 + (blockIdx.x & 3)) * TILE
                     : (size_t)((t + rot) % ntiles) * TILE;
  };
  auto issue = [&](int t) {
    uint8_t* st = smem + (t % NS) * TILE;
    const size_t off = tile_off(t);
    if (MODE == 1) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) global_lds16(src + off + i * 1024 + lane * 16, st + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) buffer_lds16(r, st + i * 1024, (uint32_t)(lane * 16), (uint32_t)(off + i * 1024));
    }
  };
  uint32_t acc = 0;
  for (int t = 0; t < NS - 1; ++t) issue(t);
  for (int t = 0; t < ntiles; ++t) {
    if (t + NS - 2 < ntiles) wait_vmcnt<(NS - 2) * LPT>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
    // touch one dword of the tile so the data is "used"
    acc ^= *(const uint32_t*)(smem + (t % NS) * TILE + lane * 4);
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14));
    if (t + NS - 1 < ntiles) issue(t + NS - 1);
  }
  wait_vmcnt<0>();
  if (acc == 0x12345678u) out[blockIdx.x * 64 + lane] = acc;
}

// WAVES waves; each wave loads its share of each tile into VGPRs, DEPTH tiles ahead
template <int WAVES, int DEPTH>
__global__ __launch_bounds__(64 * WAVES) void vgpr_stream(const uint8_t* src, uint32_t* out) {
  const int tid = threadIdx.x;
  const uint8_t* base = src + (size_t)blockIdx.x * REGION;
  constexpr int PER = TILE / (64 * WAVES * 16);  // 16-B loads per thread per tile
  const int ntiles = REGION / TILE;
  u32x4 buf[DEPTH][PER];
  u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < DEPTH; ++t)
#pragma unroll
    for (int i = 0; i < PER; ++i) buf[t][i] = *(const u32x4*)(base + (size_t)t * TILE + (i * 64 * WAVES + tid) * 16);
  for (int t = 0; t < ntiles; t += DEPTH) {
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
#pragma unroll
      for (int i = 0; i < PER; ++i) acc ^= buf[u][i];
      const int tn = t + u + DEPTH;
      if (tn < ntiles) {
#pragma unroll
        for (int i = 0; i < PER; ++i) buf[u][i] = *(const u32x4*)(base + (size_t)tn * TILE + (i * 64 * WAVES + tid) * 16);
      }
    }
  }
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x12345678u) out[blockIdx.x * 64 * WAVES + tid] = x;
}

template <typename F>
int timeit(const char* name, F launch, double bytes) {
  hipEvent_t e0, e1;
  HC(hipEventCreate(&e0)); HC(hipEventCreate(&e1));
  for (int i = 0; i < 5; ++i) launch();
  HC(hipGetLastError());
  HC(hipDeviceSynchronize());
  HC(hipEventRecord(e0));
  for (int i = 0; i < 20; ++i) launch();
  HC(hipEventRecord(e1));
  HC(hipEventSynchronize(e1));
  float ms = 0; HC(hipEventElapsedTime(&ms, e0, e1));
  ms /= 20;
  printf("| %-40s | %.4f ms | %.0f GB/s |\n", name, ms, bytes / (ms * 1e-3) / 1e9);
  return 0;
}

int main() {
  const int nwg = 1024;
  const size_t total = (size_t)nwg * REGION;
  uint8_t* src; uint32_t* out;
  HC(hipMalloc(&src, total));
  HC(hipMalloc(&out, (size_t)nwg * 64 * 8 * 4));
  HC(hipMemset(src, 1, total));
  HC(hipDeviceSynchronize());
  printf("2 GiB read by %d work-groups of 2 MiB, 16 KiB tiles\n\n| variant | ms | GB/s |\n|---|---|---|\n", nwg);
  int rc = 0;
  rc |= timeit("dma ring 1 wave, 3 stages", [&] { hipLaunchKernelGGL((dma_ring<3>), dim3(nwg), dim3(64), 0, 0, src, out); }, (double)total);
  rc |= timeit("dma ring 1 wave, 4 stages", [&] { hipLaunchKernelGGL((dma_ring<4>), dim3(nwg), dim3(64), 0, 0, src, out); }, (double)total);
  rc |= timeit("dma ring 1 wave, 5 stages", [&] { hipLaunchKernelGGL((dma_ring<5>), dim3(nwg), dim3(64), 0, 0, src, out); }, (double)total);
  rc |= timeit("dma ring 1 wave, 4 stages, grid-stride", [&] { hipLaunchKernelGGL((dma_ring<4, 1>), dim3(nwg), dim3(64), 0, 0, src, out); }, (double)total);
  rc |= timeit("dma ring 1 wave, 4 stages, 4-way interleave", [&] { hipLaunchKernelGGL((dma_ring<4, 2>), dim3(nwg), dim3(64), 0, 0, src, out); }, (double)total);
  rc |= timeit("dma ring 1 wave, 4 stages, start 37b mod 128", [&] { hipLaunchKernelGGL((dma_ring<4, 3>), dim3(nwg), dim3(64), 0, 0, src, out); }, (double)total);
  rc |= timeit("dma ring 1 wave, 4 stages, start b mod 128", [&] { hipLaunchKernelGGL((dma_ring<4, 4>), dim3(nwg), dim3(64), 0, 0, src, out); }, (double)total);
  rc |= timeit("dma ring 1 wave, 4 stages (again)", [&] { hipLaunchKernelGGL((dma_ring<4>), dim3(nwg), dim3(64), 0, 0, src, out); }, (double)total);
  rc |= timeit("vgpr 1 wave, depth 2", [&] { hipLaunchKernelGGL((vgpr_stream<1, 2>), dim3(nwg), dim3(64), 0, 0, src, out); }, (double)total);
  rc |= timeit("vgpr 1 wave, depth 4", [&] { hipLaunchKernelGGL((vgpr_stream<1, 4>), dim3(nwg), dim3(64), 0, 0, src, out); }, (double)total);
  rc |= timeit("vgpr 4 waves, depth 2", [&] { hipLaunchKernelGGL((vgpr_stream<4, 2>), dim3(nwg), dim3(256), 0, 0, src, out); }, (double)total);
  rc |= timeit("vgpr 4 waves, depth 4", [&] { hipLaunchKernelGGL((vgpr_stream<4, 4>), dim3(nwg), dim3(256), 0, 0, src, out); }, (double)total);
  return rc;
}
