// Internal interface between the C-ABI layer (argument checks, dispatch) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "fattn_device.hpp"

namespace fattn {

struct FwdReq {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int causal;
  int dtype;  // fattn_dtype
  int Br, Bc; // resolved tile shape (never 0 here)
  bool dropout = false;  // dropout on P with `drop` (default tiles, 16-bit types only)
  DropParams drop = {0u, 0u, 0u, 1.0f};
  const uint8_t* bmask = nullptr;  // block mask [B*H][nb][nb], nb = ceil(N/128) (default tiles)
};

struct BwdReq {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, d;
  float scale;
  int causal;
  int dtype;
  float* dvec;  // workspace: D = rowsum(dO * O), float32 [B, H, N]
  bool dropout = false;
  DropParams drop = {0u, 0u, 0u, 1.0f};
  const uint8_t* bmask = nullptr;  // block-sparse backward: [B*H][nb][nb] mask over 128 x 128 blocks
};

// Default forward tile for (dtype, d, causal): returns false if none exists.
bool fwd_default_tile(int dtype, int d, int causal, int* Br, int* Bc);
// Whether a forward kernel instance exists for this combination.
bool fwd_tile_supported(int dtype, int d, int Br, int Bc);
hipError_t launch_fwd(const FwdReq& r, hipStream_t stream);

size_t bwd_workspace_bytes(int B, int H, int N, int d);

// The static device buffer of the no-allocation backward (fattn_noalloc.hip): its size, and the
// device address of `device`'s copy (resolved once per device, with that device current).
size_t scratch_capacity();
hipError_t scratch_address(int device, void** out);
// stage: 0 = preprocess, 1 = dK/dV, 2 = dQ; -1 = preprocess, dK/dV, dQ in order
hipError_t launch_bwd(const BwdReq& r, hipStream_t stream, int stage = -1);

// Split-KV forward (query rows Nq against Nk keys, the keys cut into num_splits ranges).
struct SplitReq {
  const void* q;     // [B, H, Nq, d]
  const void* k;     // [B, H, Nk, d]
  const void* v;
  float* o_part;     // [num_splits, B, H, Nq, d] float32
  float* lse_part;   // [num_splits, B, H, Nq] float32
  int B, H, Nq, Nk, d;
  float scale;
  int causal;
  int dtype;
  int num_splits;    // >= 1
};
struct CombineReq {
  const float* o_part;
  const float* lse_part;
  void* o;           // [B, H, Nq, d] in dtype
  float* lse;        // [B, H, Nq]
  int B, H, Nq, d;
  int dtype;
  int num_splits;
};
// Split s covers keys [s * L, min(Nk, (s + 1) * L)) with L = splitkv_split_len(Nk, S), the
// smallest multiple of kSplitAlign that is >= Nk / S.
constexpr int kSplitAlign = 64;
int splitkv_split_len(int Nk, int num_splits);
hipError_t launch_splitkv_partial(const SplitReq& r, hipStream_t stream);
hipError_t launch_combine(const CombineReq& r, hipStream_t stream);

// Causal grid order (causal_xcd_order): how many heads an XCD works on at once. Measured on
// MI355X at N = 4096, d = 128 against all of an XCD's heads at once: equal at 4 heads per XCD,
// forward +1.3% at 8, forward +4% and backward +6% at 16 (fewer heads' streamed tiles competing
// for the XCD's 4 MiB L2); one head at a time loses the balance across the causal triangle
// (up to -26%) when a head has fewer tiles than the XCD has CUs. So a group holds four heads,
// or fewer once their streamed tensors pass 8 MiB (`stream_bytes`: K and V per head in the
// forward and dQ kernels, Q and dO in the dK/dV kernel; 2 MiB at N = 4096, d = 128, 8 MiB at
// N = 16384, where one head is a group). Wherever the budget shrinks the group, a head has at
// least 32 tiles, so a group still gives each of an XCD's 32 CUs two or more.
inline int head_group(int bh_total, size_t stream_bytes) {
  const int hpx = bh_total / 8;
  if (hpx <= 1) return 1;
  const size_t budget = (size_t)8 << 20;
  int g = stream_bytes > 0 ? (int)(budget / stream_bytes) : 4;
  g = g < 1 ? 1 : (g > 4 ? 4 : g);
  return g > hpx ? hpx : g;
}

// K-outer (FA-1 order) forward, an ablation: one launch per key/value block.
struct KoReq {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  float scale;
  int causal;
  int dtype;
  float* workspace;  // running state: u [B*H*N*d], m [B*H*N], l [B*H*N], float32
};
size_t kouter_workspace_bytes(int B, int H, int N, int d);
hipError_t launch_kouter(const KoReq& r, hipStream_t stream);

}  // namespace fattn
