// The library's one static device buffer, for the entry point that allocates nothing
// (fattn_bwd_noalloc): the backward's float32 D vector lives here instead of in a caller
// workspace. Each GPU the library runs on holds its own copy of the array, resident until the
// process ends; every call on one GPU shares that GPU's copy.
//
// In host code `scratch` names a host-side stand-in, not device memory: the device address of a
// GPU's copy comes from hipGetSymbolAddress with that GPU current, resolved once per device and
// kept below, and only that address is ever handed to a kernel.
#include <mutex>

#include "fattn_launch.hpp"

namespace fattn {
namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;  // D of up to 4,194,304 rows (B * H * N)
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

hipError_t scratch_address(int device, void** out) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int current = -1;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (current != device) {
      const hipError_t e2 = hipSetDevice(current);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace fattn
