// C-ABI entry points of libfattn: argument checks (host only, before any HIP call) and dispatch.
#include "../../include/fattn.h"

#include <cmath>
#include <cstdint>

#include "fattn_launch.hpp"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr long long kMaxN = 16777216LL;
constexpr long long kMaxElems = 1LL << 46;

int elem_bytes(int dtype) { return dtype == FATTN_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int B, int H, int N, int d, int dtype) {
  if (dtype != FATTN_F32 && dtype != FATTN_F16 && dtype != FATTN_BF16) return FATTN_ERR_DTYPE;
  if (d != 64 && d != 128) return FATTN_ERR_HEADDIM;
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return FATTN_ERR_SHAPE;
  const long long bh = (long long)B * H;
  if (bh > (1LL << 31) - 1) return FATTN_ERR_SHAPE;
  if (bh * N > kMaxElems / d) return FATTN_ERR_SHAPE;
  // the forward grid is B*H*ceil(N/64) blocks at most; keep it in 32 bits
  if (bh * ((N + 63) / 64) > 0x7fffffffLL) return FATTN_ERR_SHAPE;
  return FATTN_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? FATTN_OK : FATTN_ERR_LAUNCH; }

// Keep threshold floor(p 2^16) of a 16-bit generator field and 1 / (1 - p), for a drop
// probability p in [0, 1).
fattn::DropParams drop_params(float p, unsigned long long seed) {
  fattn::DropParams d;
  d.seed_lo = (uint32_t)(seed & 0xffffffffull);
  d.seed_hi = (uint32_t)(seed >> 32);
  const double t = std::floor((double)p * 65536.0);
  d.thr = t >= 65535.0 ? 65535u : (uint32_t)t;
  d.inv_keep = (float)(1.0 / (1.0 - (double)p));
  return d;
}

bool drop_ok(float p) { return std::isfinite(p) && p >= 0.f && p < 1.f; }

constexpr int kMaxSplits = 1024;

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Shapes of the split-KV entry points: q [B,H,Nq,d], k/v [B,H,Nk,d], partials [S,B,H,Nq,d].
int check_split_shape(int B, int H, int Nq, int Nk, int d, int num_splits) {
  if (d != 64 && d != 128) return FATTN_ERR_HEADDIM;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || Nq > kMaxN || Nk > kMaxN) return FATTN_ERR_SHAPE;
  if (num_splits < 1 || num_splits > kMaxSplits) return FATTN_ERR_SHAPE;
  const long long bh = (long long)B * H;
  if (bh > (1LL << 31) - 1) return FATTN_ERR_SHAPE;
  if (bh * Nk > kMaxElems / d) return FATTN_ERR_SHAPE;
  if (bh * Nq * num_splits > kMaxElems / d) return FATTN_ERR_SHAPE;
  // partial-kernel grid: B*H*ceil(Nq/32)*S blocks
  if (bh * ((Nq + 31) / 32) * num_splits > 0x7fffffffLL) return FATTN_ERR_SHAPE;
  return FATTN_OK;
}

// Splits for num_splits = 0: about 1024 work-groups, i.e. two full rounds of the partial kernel's
// resident work-groups (two per CU on 256 CUs at d = 128), but at least 256 keys per split so each
// work-group's pipeline runs for several tiles.
int auto_splits(int B, int H, int Nq, int Nk) {
  const long long wgs = (long long)B * H * ((Nq + 31) / 32);
  long long s = (1024 + wgs - 1) / wgs;
  const long long useful = ((long long)Nk + 255) / 256;
  if (s > useful) s = useful;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : (int)s;
}

size_t split_o_bytes(int B, int H, int Nq, int d, int S) {
  return round256((size_t)S * B * H * Nq * d * sizeof(float));
}
size_t split_lse_bytes(int B, int H, int Nq, int S) {
  return round256((size_t)S * B * H * Nq * sizeof(float));
}

}  // namespace

extern "C" {

int fattn_version(void) { return kVersion; }

const char* fattn_strerror(int status) {
  switch (status) {
    case FATTN_OK: return "ok";
    case FATTN_ERR_NULL: return "a required pointer is NULL";
    case FATTN_ERR_SHAPE: return "B, H or N out of range";
    case FATTN_ERR_HEADDIM: return "head dim d must be 64 or 128";
    case FATTN_ERR_DTYPE: return "unsupported dtype for this entry point";
    case FATTN_ERR_TILE: return "unsupported tile shape (Br, Bc)";
    case FATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FATTN_ERR_SCALE: return "scale is not finite";
    case FATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case FATTN_ERR_UNSUPPORTED: return "not implemented in this library";
    case FATTN_ERR_LAUNCH: return "kernel launch failed";
    case FATTN_ERR_ALIAS: return "an output aliases an input";
    case FATTN_ERR_CAUSAL: return "causal must be 0 or 1";
    case FATTN_ERR_DROPOUT: return "dropout probability not in [0, 1)";
    case FATTN_ERR_SCRATCH: return "problem larger than the library's static scratch buffer";
    default: return "unknown status";
  }
}

int fattn_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal, int dtype,
                    int Br, int Bc, void* stream) {
  if (!q || !k || !v || !o || !lse) return FATTN_ERR_NULL;
  int st = check_common(B, H, N, d, dtype);
  if (st != FATTN_OK) return st;
  if (causal != 0 && causal != 1) return FATTN_ERR_CAUSAL;
  if (!std::isfinite(scale)) return FATTN_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FATTN_ERR_ALIGN;
  if (o == q || o == k || o == v || (const void*)lse == q || (const void*)lse == k ||
      (const void*)lse == v || (void*)lse == o)
    return FATTN_ERR_ALIAS;
  if (Br == 0 && Bc == 0) {
    if (!fattn::fwd_default_tile(dtype, d, causal, &Br, &Bc)) return FATTN_ERR_TILE;
  } else if (!fattn::fwd_tile_supported(dtype, d, Br, Bc)) {
    return FATTN_ERR_TILE;
  }
  fattn::FwdReq r{q, k, v, o, lse, B, H, N, d, scale, causal, dtype, Br, Bc};
  (void)elem_bytes;
  return launch_status(fattn::launch_fwd(r, (hipStream_t)stream));
}

int fattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  return fattn_fwd_tiled(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, 0, 0, stream);
}

int fattn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal, int dtype,
                          const unsigned char* block_mask, void* stream) {
  if (!q || !k || !v || !o || !lse || !block_mask) return FATTN_ERR_NULL;
  if (dtype == FATTN_F32) return FATTN_ERR_DTYPE;
  int st = check_common(B, H, N, d, dtype);
  if (st != FATTN_OK) return st;
  if (causal != 0 && causal != 1) return FATTN_ERR_CAUSAL;
  if (!std::isfinite(scale)) return FATTN_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FATTN_ERR_ALIGN;
  const void* outs[2] = {o, lse};
  const void* ins[4] = {q, k, v, block_mask};
  for (const void* p : outs)
    for (const void* i2 : ins)
      if (p == i2) return FATTN_ERR_ALIAS;
  if (o == (void*)lse) return FATTN_ERR_ALIAS;
  int Br = 0, Bc = 0;
  if (!fattn::fwd_default_tile(dtype, d, causal, &Br, &Bc)) return FATTN_ERR_TILE;
  fattn::FwdReq r{q, k, v, o, lse, B, H, N, d, scale, causal, dtype, Br, Bc};
  r.bmask = block_mask;
  return launch_status(fattn::launch_fwd(r, (hipStream_t)stream));
}

int fattn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal, int dtype,
                      float p_drop, unsigned long long seed, void* stream) {
  if (!drop_ok(p_drop)) return FATTN_ERR_DROPOUT;
  if (dtype == FATTN_F32) return FATTN_ERR_DTYPE;
  if (p_drop == 0.f) return fattn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream);
  if (!q || !k || !v || !o || !lse) return FATTN_ERR_NULL;
  int st = check_common(B, H, N, d, dtype);
  if (st != FATTN_OK) return st;
  if (causal != 0 && causal != 1) return FATTN_ERR_CAUSAL;
  if (!std::isfinite(scale)) return FATTN_ERR_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FATTN_ERR_ALIGN;
  if (o == q || o == k || o == v || (const void*)lse == q || (const void*)lse == k ||
      (const void*)lse == v || (void*)lse == o)
    return FATTN_ERR_ALIAS;
  int Br = 0, Bc = 0;
  if (!fattn::fwd_default_tile(dtype, d, causal, &Br, &Bc)) return FATTN_ERR_TILE;
  fattn::FwdReq r{q, k, v, o, lse, B, H, N, d, scale, causal, dtype, Br, Bc};
  r.dropout = true;
  r.drop = drop_params(p_drop, seed);
  return launch_status(fattn::launch_fwd(r, (hipStream_t)stream));
}

size_t fattn_bwd_workspace_size(int B, int H, int N, int d, int dtype) {
  if (check_common(B, H, N, d, dtype) != FATTN_OK) return 0;
  if (dtype == FATTN_F32) return 0;
  return fattn::bwd_workspace_bytes(B, H, N, d);
}

// Argument checks shared by the full backward entry points (extra: one more input, may be null),
// except for the workspace.
static int check_bwd_args(const void* q, const void* k, const void* v, const void* o, const void* dO,
                          const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                          float scale, int causal, int dtype, const void* extra) {
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FATTN_ERR_NULL;
  int st = check_common(B, H, N, d, dtype);
  if (st != FATTN_OK) return st;
  if (dtype == FATTN_F32) return FATTN_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FATTN_ERR_CAUSAL;
  if (!std::isfinite(scale)) return FATTN_ERR_SCALE;
  const void* ins[7] = {q, k, v, o, dO, lse, extra};
  void* outs[3] = {dq, dk, dv};
  for (int i = 0; i < 6; ++i)
    if (!aligned16(ins[i])) return FATTN_ERR_ALIGN;
  for (void* p : outs)
    if (!aligned16(p)) return FATTN_ERR_ALIGN;
  for (void* p : outs)
    for (const void* s2 : ins)
      if (s2 && p == s2) return FATTN_ERR_ALIAS;
  if (dq == dk || dq == dv || dk == dv) return FATTN_ERR_ALIAS;
  return FATTN_OK;
}

// ... and with the caller's workspace.
static int check_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                     float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
                     const void* extra) {
  int st = check_bwd_args(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, extra);
  if (st != FATTN_OK) return st;
  const size_t need = fattn::bwd_workspace_bytes(B, H, N, d);
  if (!workspace || workspace_bytes < need) return FATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FATTN_ERR_ALIGN;
  const void* all[10] = {dq, dk, dv, q, k, v, o, dO, lse, extra};
  for (const void* p : all)
    if (p && p == workspace) return FATTN_ERR_ALIAS;
  return FATTN_OK;
}

int fattn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const void* dO,
                          const float* lse, void* dq, void* dk, void* dv,
                          int B, int H, int N, int d, float scale, int causal, int dtype,
                          const unsigned char* block_mask, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (!block_mask) return FATTN_ERR_NULL;
  int st = check_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, workspace,
                     workspace_bytes, block_mask);
  if (st != FATTN_OK) return st;
  fattn::BwdReq r{q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, (float*)workspace};
  r.bmask = block_mask;
  return launch_status(fattn::launch_bwd(r, (hipStream_t)stream));
}

int fattn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
              const float* lse, void* dq, void* dk, void* dv,
              int B, int H, int N, int d, float scale, int causal, int dtype,
              void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, workspace,
                     workspace_bytes, nullptr);
  if (st != FATTN_OK) return st;
  fattn::BwdReq r{q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, (float*)workspace};
  return launch_status(fattn::launch_bwd(r, (hipStream_t)stream));
}

size_t fattn_bwd_noalloc_max_bytes(void) { return fattn::scratch_capacity(); }

int fattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  // fattn_bwd's checks, then the size of the static buffer, all before any HIP call
  int st = check_bwd_args(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, nullptr);
  if (st != FATTN_OK) return st;
  if (fattn::bwd_workspace_bytes(B, H, N, d) > fattn::scratch_capacity()) return FATTN_ERR_SCRATCH;
  int device = -1;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &device) : hipGetDevice(&device);
  if (e != hipSuccess) return FATTN_ERR_LAUNCH;
  void* ws = nullptr;
  if (fattn::scratch_address(device, &ws) != hipSuccess) return FATTN_ERR_LAUNCH;
  fattn::BwdReq r{q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, (float*)ws};
  return launch_status(fattn::launch_bwd(r, (hipStream_t)stream));
}

int fattn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, float scale, int causal, int dtype,
                      float p_drop, unsigned long long seed,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!drop_ok(p_drop)) return FATTN_ERR_DROPOUT;
  if (p_drop == 0.f)
    return fattn_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, workspace,
                     workspace_bytes, stream);
  int st = check_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, workspace,
                     workspace_bytes, nullptr);
  if (st != FATTN_OK) return st;
  fattn::BwdReq r{q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype, (float*)workspace};
  r.dropout = true;
  r.drop = drop_params(p_drop, seed);
  return launch_status(fattn::launch_bwd(r, (hipStream_t)stream));
}

int fattn_bwd_preprocess(const void* o, const void* dO, float* dvec, int B, int H, int N, int d,
                         int dtype, void* stream) {
  if (!o || !dO || !dvec) return FATTN_ERR_NULL;
  int st = check_common(B, H, N, d, dtype);
  if (st != FATTN_OK) return st;
  if (dtype == FATTN_F32) return FATTN_ERR_DTYPE;
  if (!aligned16(o) || !aligned16(dO) || !aligned16(dvec)) return FATTN_ERR_ALIGN;
  if ((const void*)dvec == o || (const void*)dvec == dO) return FATTN_ERR_ALIAS;
  fattn::BwdReq r{nullptr, nullptr, nullptr, o, dO, nullptr, nullptr, nullptr, nullptr,
                  B, H, N, d, 1.0f, 0, dtype, dvec};
  return launch_status(fattn::launch_bwd(r, (hipStream_t)stream, 0));
}

static int check_stage(const void* q, const void* k, const void* v, const void* dO,
                       const float* lse, const float* dvec, void* out0, void* out1,
                       int B, int H, int N, int d, float scale, int causal, int dtype) {
  if (!q || !k || !v || !dO || !lse || !dvec || !out0) return FATTN_ERR_NULL;
  int st = check_common(B, H, N, d, dtype);
  if (st != FATTN_OK) return st;
  if (dtype == FATTN_F32) return FATTN_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FATTN_ERR_CAUSAL;
  if (!std::isfinite(scale)) return FATTN_ERR_SCALE;
  const void* ins[6] = {q, k, v, dO, lse, dvec};
  for (const void* p : ins)
    if (!aligned16(p)) return FATTN_ERR_ALIGN;
  if (!aligned16(out0) || (out1 && !aligned16(out1))) return FATTN_ERR_ALIGN;
  for (const void* p : ins)
    if (p == out0 || (out1 && p == out1)) return FATTN_ERR_ALIAS;
  if (out1 && out0 == out1) return FATTN_ERR_ALIAS;
  return FATTN_OK;
}

int fattn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                   const float* dvec, void* dk, void* dv, int B, int H, int N, int d, float scale,
                   int causal, int dtype, void* stream) {
  if (!dv) return FATTN_ERR_NULL;
  int st = check_stage(q, k, v, dO, lse, dvec, dk, dv, B, H, N, d, scale, causal, dtype);
  if (st != FATTN_OK) return st;
  fattn::BwdReq r{q, k, v, nullptr, dO, lse, nullptr, dk, dv, B, H, N, d, scale, causal, dtype,
                  (float*)dvec};
  return launch_status(fattn::launch_bwd(r, (hipStream_t)stream, 1));
}

int fattn_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                 const float* dvec, void* dq, int B, int H, int N, int d, float scale, int causal,
                 int dtype, void* stream) {
  int st = check_stage(q, k, v, dO, lse, dvec, dq, nullptr, B, H, N, d, scale, causal, dtype);
  if (st != FATTN_OK) return st;
  fattn::BwdReq r{q, k, v, nullptr, dO, lse, dq, nullptr, nullptr, B, H, N, d, scale, causal, dtype,
                  (float*)dvec};
  return launch_status(fattn::launch_bwd(r, (hipStream_t)stream, 2));
}

size_t fattn_fwd_kouter_workspace_size(int B, int H, int N, int d, int dtype) {
  if (check_common(B, H, N, d, dtype) != FATTN_OK || dtype == FATTN_F32) return 0;
  return fattn::kouter_workspace_bytes(B, H, N, d);
}

int fattn_fwd_kouter(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, float scale, int causal, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FATTN_ERR_NULL;
  int st = check_common(B, H, N, d, dtype);
  if (st != FATTN_OK) return st;
  if (dtype == FATTN_F32) return FATTN_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FATTN_ERR_CAUSAL;
  if (!std::isfinite(scale)) return FATTN_ERR_SCALE;
  if (!workspace || workspace_bytes < fattn::kouter_workspace_bytes(B, H, N, d)) return FATTN_ERR_WORKSPACE;
  const void* all[6] = {q, k, v, o, lse, workspace};
  for (const void* p : all)
    if (!aligned16(p)) return FATTN_ERR_ALIGN;
  for (int i = 3; i < 6; ++i)
    for (int j = 0; j < 6; ++j)
      if (i != j && all[i] == all[j]) return FATTN_ERR_ALIAS;
  fattn::KoReq r{q, k, v, o, lse, B, H, N, d, scale, causal, dtype, (float*)workspace};
  return launch_status(fattn::launch_kouter(r, (hipStream_t)stream));
}

int fattn_splitkv_num_splits(int B, int H, int Nq, int Nk, int d) {
  if (check_split_shape(B, H, Nq, Nk, d, 1) != FATTN_OK) return 0;
  return auto_splits(B, H, Nq, Nk);
}

size_t fattn_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int d, int num_splits) {
  if (num_splits == 0 && check_split_shape(B, H, Nq, Nk, d, 1) == FATTN_OK)
    num_splits = auto_splits(B, H, Nq, Nk);
  if (check_split_shape(B, H, Nq, Nk, d, num_splits) != FATTN_OK) return 0;
  return split_o_bytes(B, H, Nq, d, num_splits) + split_lse_bytes(B, H, Nq, num_splits);
}

static int check_partial(const void* q, const void* k, const void* v, const void* o_parts,
                         const void* lse_parts, int B, int H, int Nq, int Nk, int d, float scale,
                         int causal, int dtype, int num_splits) {
  if (!q || !k || !v || !o_parts || !lse_parts) return FATTN_ERR_NULL;
  if (dtype != FATTN_F16 && dtype != FATTN_BF16) return FATTN_ERR_DTYPE;
  int st = check_split_shape(B, H, Nq, Nk, d, num_splits);
  if (st != FATTN_OK) return st;
  if (causal != 0 && causal != 1) return FATTN_ERR_CAUSAL;
  if (causal && Nq > Nk) return FATTN_ERR_SHAPE;
  if (!std::isfinite(scale)) return FATTN_ERR_SCALE;
  const void* ins[3] = {q, k, v};
  for (const void* p : ins) {
    if (!aligned16(p)) return FATTN_ERR_ALIGN;
    if (p == o_parts || p == lse_parts) return FATTN_ERR_ALIAS;
  }
  if (!aligned16(o_parts) || !aligned16(lse_parts)) return FATTN_ERR_ALIGN;
  if (o_parts == lse_parts) return FATTN_ERR_ALIAS;
  return FATTN_OK;
}

static int check_combine(const float* o_parts, const float* lse_parts, int num_splits, const void* o,
                         const float* lse, int B, int H, int Nq, int d, int dtype) {
  if (!o_parts || !lse_parts || !o || !lse) return FATTN_ERR_NULL;
  if (dtype != FATTN_F32 && dtype != FATTN_F16 && dtype != FATTN_BF16) return FATTN_ERR_DTYPE;
  int st = check_split_shape(B, H, Nq, 1, d, num_splits);
  if (st != FATTN_OK) return st;
  if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || !aligned16(lse))
    return FATTN_ERR_ALIGN;
  const void* ins[2] = {o_parts, lse_parts};
  for (const void* p : ins)
    if (p == o || p == (const void*)lse) return FATTN_ERR_ALIAS;
  if (o == (const void*)lse) return FATTN_ERR_ALIAS;
  return FATTN_OK;
}

int fattn_fwd_partial(const void* q, const void* k, const void* v, float* o_parts, float* lse_parts,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                      int num_splits, void* stream) {
  int st = check_partial(q, k, v, o_parts, lse_parts, B, H, Nq, Nk, d, scale, causal, dtype, num_splits);
  if (st != FATTN_OK) return st;
  fattn::SplitReq r{q, k, v, o_parts, lse_parts, B, H, Nq, Nk, d, scale, causal, dtype, num_splits};
  return launch_status(fattn::launch_splitkv_partial(r, (hipStream_t)stream));
}

int fattn_combine(const float* o_parts, const float* lse_parts, int num_splits, void* o, float* lse,
                  int B, int H, int Nq, int d, int dtype, void* stream) {
  int st = check_combine(o_parts, lse_parts, num_splits, o, lse, B, H, Nq, d, dtype);
  if (st != FATTN_OK) return st;
  fattn::CombineReq r{o_parts, lse_parts, o, lse, B, H, Nq, d, dtype, num_splits};
  return launch_status(fattn::launch_combine(r, (hipStream_t)stream));
}

int fattn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                      int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FATTN_ERR_NULL;
  if (dtype != FATTN_F16 && dtype != FATTN_BF16) return FATTN_ERR_DTYPE;
  if (num_splits == 0 && check_split_shape(B, H, Nq, Nk, d, 1) == FATTN_OK)
    num_splits = auto_splits(B, H, Nq, Nk);
  int st = check_split_shape(B, H, Nq, Nk, d, num_splits);
  if (st != FATTN_OK) return st;
  if (causal != 0 && causal != 1) return FATTN_ERR_CAUSAL;
  if (causal && Nq > Nk) return FATTN_ERR_SHAPE;
  if (!std::isfinite(scale)) return FATTN_ERR_SCALE;
  const size_t ob = split_o_bytes(B, H, Nq, d, num_splits);
  if (!workspace || workspace_bytes < ob + split_lse_bytes(B, H, Nq, num_splits))
    return FATTN_ERR_WORKSPACE;
  const void* all[6] = {q, k, v, o, lse, workspace};
  for (const void* p : all)
    if (!aligned16(p)) return FATTN_ERR_ALIGN;
  for (int i = 3; i < 6; ++i)
    for (int j = 0; j < 6; ++j)
      if (i != j && all[i] == all[j]) return FATTN_ERR_ALIAS;
  float* o_parts = (float*)workspace;
  float* lse_parts = (float*)((char*)workspace + ob);
  fattn::SplitReq r{q, k, v, o_parts, lse_parts, B, H, Nq, Nk, d, scale, causal, dtype, num_splits};
  hipError_t e = fattn::launch_splitkv_partial(r, (hipStream_t)stream);
  if (e != hipSuccess) return FATTN_ERR_LAUNCH;
  fattn::CombineReq c{o_parts, lse_parts, o, lse, B, H, Nq, d, dtype, num_splits};
  return launch_status(fattn::launch_combine(c, (hipStream_t)stream));
}

}  // extern "C"
