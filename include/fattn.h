/*
 * libfattn — exact scaled-dot-product attention computed tile by tile (FlashAttention style)
 * on AMD Instinct MI355X (gfx950).
 *
 * What is computed (page "FlashAttention为什么更快更省显存", opening formula; page
 * "从零实现 FlashAttention-2：分块在线 Softmax", sections on the rescale identity and on the
 * backward): for every batch b and head h, with S = scale * Q K^T,
 *
 *     O   = softmax(S) V          (row-wise softmax; S[i][j] = -inf for j > i when causal)
 *     LSE = log(sum_j exp(S[i][j]))   per query row, natural log, float32
 *
 * The forward never materialises S or P: it keeps a query tile on chip, streams key/value tiles
 * past it and merges each tile into a running row max, exp-sum and unnormalised output (page
 * "mianstack q-0277", section on keeping the blockwise softmax normalised). The backward rebuilds
 * the probability tiles from Q, K, V and the saved LSE instead of storing them (page 2, backward
 * section; page 1, section on why the backward recomputes).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensors are dense, contiguous [B, H, N, d] with d innermost, in the element type `dtype`.
 *    LSE (and the workspace's D vector) is float32 [B, H, N].
 *  - Every pointer is a caller-owned DEVICE pointer on the current HIP device, 16-byte aligned.
 *    The library allocates nothing and is re-entrant; its only state is the static device
 *    buffer of fattn_bwd_noalloc (below), which that entry point alone uses.
 *  - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream). Work is enqueued
 *    on it and the call returns at once; the caller synchronises.
 *  - Arguments are checked on the host before any HIP call: a call that returns an error has
 *    enqueued nothing and written nothing. The library never aborts or throws across this ABI.
 *    A launch failure returns FATTN_ERR_LAUNCH; faults inside a kernel surface at the caller's
 *    synchronisation.
 *  - Outputs must not overlap inputs (an exact pointer match is rejected with FATTN_ERR_ALIAS;
 *    partial overlap is undefined behaviour).
 *  - Supported: d in {64, 128}; 1 <= N <= 16777216; B, H >= 1 with B*H*N*d < 2^46; `scale`
 *    finite (0 gives uniform attention, negative values are allowed); causal in {0, 1}.
 *    Causal masks key j > query i (queries and keys share the same length N), except in the
 *    split-KV entry points below, where Nq and Nk may differ.
 */
#ifndef FATTN_H
#define FATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FATTN_F32 = 0, FATTN_F16 = 1, FATTN_BF16 = 2 } fattn_dtype;

typedef enum {
  FATTN_OK = 0,
  FATTN_ERR_NULL = -1,        /* a required pointer is NULL */
  FATTN_ERR_SHAPE = -2,       /* B, H or N out of range, or the sizes overflow */
  FATTN_ERR_HEADDIM = -3,     /* d not in {64, 128} */
  FATTN_ERR_DTYPE = -4,       /* unknown dtype, or a dtype this entry point does not support */
  FATTN_ERR_TILE = -5,        /* (Br, Bc) not a supported tile shape for this dtype and d */
  FATTN_ERR_ALIGN = -6,       /* a pointer is not 16-byte aligned */
  FATTN_ERR_SCALE = -7,       /* scale is NaN or infinite */
  FATTN_ERR_WORKSPACE = -8,   /* workspace NULL or smaller than fattn_bwd_workspace_size() */
  FATTN_ERR_UNSUPPORTED = -9, /* a valid request the library does not implement */
  FATTN_ERR_LAUNCH = -10,     /* the HIP runtime rejected a kernel launch */
  FATTN_ERR_ALIAS = -11,      /* an output pointer equals an input pointer */
  FATTN_ERR_CAUSAL = -12,     /* causal not 0 or 1 */
  FATTN_ERR_DROPOUT = -13,    /* dropout probability not in [0, 1) */
  FATTN_ERR_SCRATCH = -14     /* problem too large for fattn_bwd_noalloc's static buffer */
} fattn_status;

/*
 * Forward pass. Reads q, k, v [B,H,N,d] (dtype); writes o [B,H,N,d] (dtype, round-to-nearest-
 * even from the float32 accumulator) and lse [B,H,N] (float32, natural log of the row's exp-sum
 * of scaled logits). Picks the tile shape for (dtype, d, causal) itself.
 * Computation: page 2, hands-on section (query tiles outer, key/value tiles inner, causal mask
 * inside the tile loop); page 3's merge rule for the running statistics; final division by the
 * exp-sum after the last tile (page 2, rescale-identity section).
 */
int fattn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/*
 * fattn_fwd with an explicit tile shape: Br query rows per work-group, Bc key rows per step
 * (page 2, tips: the tile sizes change the on-chip working set, not the result). Br = Bc = 0
 * selects the default, so fattn_fwd(...) == fattn_fwd_tiled(..., 0, 0, stream).
 * Supported (Br, Bc): f16/bf16 — {64, 128, 256} x {64, 128}; f32 — (128, 32) and (64, 32).
 * Defaults: f16/bf16 (256, 128) at d = 128 and (128, 64) at d = 64; f32 (128, 32).
 */
int fattn_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal, int dtype,
                    int Br, int Bc, void* stream);

/*
 * Forward with dropout on the attention probabilities (page "mianstack q-0277", section on
 * whether the result changes, names dropout as a training-time source of difference; the pages
 * fix no convention, so this one is stated here). With P = softmax(S) and keep mask M:
 *     O = ((P * M) / (1 - p_drop)) V,   LSE = the undropped statistic (as fattn_fwd writes it).
 * M(b, h, i, j) = 1 iff x >= floor(p_drop * 2^16), where x is 16-bit field f = j % 8 of
 * Philox4x32-10 (Salmon et al., SC 2011) at counter (j / 8, i, b*H + h, 0) with key
 * (seed mod 2^32, seed / 2^32): the low half of output word f for f < 4, the high half of word
 * f - 4 otherwise. The same (seed, p_drop) reproduces the same mask in fattn_bwd_dropout. p_drop in [0, 1), else
 * FATTN_ERR_DROPOUT; p_drop = 0 is fattn_fwd. f16/bf16 only; uses the default tile shape.
 */
int fattn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int N, int d, float scale, int causal, int dtype,
                      float p_drop, unsigned long long seed, void* stream);

/*
 * Block-sparse forward: exact attention restricted to the allowed 128 x 128 (query, key) blocks
 * (page "FlashAttention为什么更快更省显存", section on computing in blocks, mentions the
 * block-sparse approximate variant without defining it; this is the reading stated here).
 * block_mask: device uint8 [B, H, nb, nb], nb = ceil(N / 128); block (r, c) covers queries
 * [128 r, 128 r + 128) and keys [128 c, 128 c + 128); nonzero = computed. Scores outside allowed
 * blocks (and above the diagonal when causal) are -inf; a row with no allowed key gets O = 0 and
 * LSE = -inf. Key tiles whose blocks are zero for a whole work-group are neither read nor
 * computed. f16/bf16 only; runs with 128 x 64 tiles (one mask row per work-group); same other
 * conventions as fattn_fwd.
 */
int fattn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, int d, float scale, int causal, int dtype,
                          const unsigned char* block_mask, void* stream);

/*
 * Bytes of device workspace fattn_bwd needs: the float32 row vector D = rowsum(dO * O) [B,H,N],
 * rounded up to 256 bytes. Returns 0 for arguments that fattn_bwd would reject on shape, head
 * dim or dtype grounds.
 */
size_t fattn_bwd_workspace_size(int B, int H, int N, int d, int dtype);

/*
 * Backward pass by recomputation (page 2, backward section; page 3, backward section).
 * Reads q, k, v, o, dO [B,H,N,d] (dtype) and lse [B,H,N] (float32, as written by fattn_fwd);
 * writes dq, dk, dv [B,H,N,d] (dtype, from float32 accumulators). P is rebuilt tile by tile as
 * exp(S - LSE) and never stored. `workspace` is caller-owned device memory of at least
 * fattn_bwd_workspace_size() bytes; its contents on entry are ignored and on exit unspecified.
 * dtype: FATTN_F16 or FATTN_BF16 (FATTN_F32 returns FATTN_ERR_DTYPE).
 */
int fattn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
              const float* lse, void* dq, void* dk, void* dv,
              int B, int H, int N, int d, float scale, int causal, int dtype,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * fattn_bwd without a workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving or training loops, harnesses that forbid allocation). The D
 * vector lives in a static device buffer of fattn_bwd_noalloc_max_bytes() bytes (16 MiB: D of
 * up to B * H * N = 4,194,304 rows) that every GPU the library runs on holds until the process
 * ends; larger problems return FATTN_ERR_SCRATCH before any HIP call. The call performs no
 * hipMalloc or hipFree. The buffer's device address on a GPU is looked up once, on the first
 * call there (the GPU of `stream`, or the current one for a NULL stream). Results are bit for bit
 * those of fattn_bwd. All calls on one GPU share its buffer: calls whose executions overlap on one
 * GPU (on different streams, or from different threads) race and give undefined results; calls
 * ordered on one stream are safe. Otherwise the same arguments, checks and results as fattn_bwd.
 */
int fattn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, float scale, int causal, int dtype, void* stream);

/* Size in bytes of fattn_bwd_noalloc's static buffer (the largest D it can hold). */
size_t fattn_bwd_noalloc_max_bytes(void);

/*
 * Backward of fattn_fwd_dropout (same p_drop and seed, hence the same mask M): with
 * Pd = P * M / (1 - p_drop), dV = Pd^T dO, dP = (dO V^T) * M / (1 - p_drop), D = rowsum(dO * O),
 * dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q. Same buffers and checks as fattn_bwd;
 * p_drop = 0 is fattn_bwd.
 */
int fattn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv,
                      int B, int H, int N, int d, float scale, int causal, int dtype,
                      float p_drop, unsigned long long seed,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of fattn_fwd_blocksparse (same block_mask, layout [B, H, nb, nb] uint8 on the device):
 * the chain rule through the block-restricted definition. Masked scores carry P = 0, so
 * dV = P^T dO, dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D), dQ = scale dS K,
 * dK = scale dS^T Q; a row with no allowed key (LSE = -inf) gets dQ = 0 and adds nothing to dK, dV.
 * Only (query, key) tiles whose mask block is set are read and computed: the dK/dV kernel visits
 * the query tiles of its key block's mask column, the dQ kernel the key tiles of its two mask
 * rows. Same buffers and checks as fattn_bwd, plus block_mask non-null (FATTN_ERR_NULL) and
 * distinct from the outputs and the workspace (FATTN_ERR_ALIAS). Not combinable with dropout.
 */
int fattn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const void* dO,
                          const float* lse, void* dq, void* dk, void* dv,
                          int B, int H, int N, int d, float scale, int causal, int dtype,
                          const unsigned char* block_mask, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * The backward split into three stages, for callers that want to schedule or time them
 * separately; run in this order they give fattn_bwd's results bit for bit (fattn_bwd itself runs
 * the dQ stage first, computing D on the way, then dK/dV). Same conventions and checks as
 * fattn_bwd; `dvec` is the float32 [B,H,N] row vector D = rowsum(dO * O) (the first bytes of
 * fattn_bwd's workspace).
 *   fattn_bwd_preprocess: reads o, dO; writes dvec.
 *   fattn_bwd_dkdv:       reads q, k, v, dO, lse, dvec; writes dk, dv (per key tile, recomputing
 *                         P = exp(S - LSE) once for every query tile on or below the diagonal;
 *                         dS = P (dP - D) takes P as rounded to the input type for dV = P^T dO).
 *   fattn_bwd_dq:         reads q, k, v, dO, lse, dvec; writes dq (per query tile).
 */
int fattn_bwd_preprocess(const void* o, const void* dO, float* dvec, int B, int H, int N, int d,
                         int dtype, void* stream);
int fattn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                   const float* dvec, void* dk, void* dv, int B, int H, int N, int d, float scale,
                   int causal, int dtype, void* stream);
int fattn_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                 const float* dvec, void* dq, int B, int H, int N, int d, float scale, int causal,
                 int dtype, void* stream);

/*
 * The forward in the K-outer loop order, an ablation (page 2, section on going from
 * FlashAttention-1 to FlashAttention-2: with key/value blocks outer, each query block and its
 * running statistics have to be reloaded for every key block). Same inputs, outputs and result
 * as fattn_fwd (f16/bf16 only); one kernel launch per key/value block, each work-group reading
 * its query tile and its float32 running state (u [B,H,N,d], m and l [B,H,N]) from `workspace`
 * and writing it back, or O and LSE at its last block. `workspace` holds at least
 * fattn_fwd_kouter_workspace_size() bytes; contents on entry are ignored, on exit unspecified.
 */
size_t fattn_fwd_kouter_workspace_size(int B, int H, int N, int d, int dtype);
int fattn_fwd_kouter(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, float scale, int causal, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split-KV forward: Nq query rows per head against an Nk-long key/value cache, computed as
 * per-range partial results merged afterwards. This is the decode shape (page "mianstack q-0277",
 * backward section, names the key/value cache): the keys of each row are cut into num_splits
 * ranges so that many work-groups stream K/V at once, then the partials are merged with the
 * two-state rule of page 3's section on keeping the blockwise softmax normalised (max, rescaled
 * exp-sums, rescaled outputs).
 *
 * Layout: q [B,H,Nq,d]; k, v [B,H,Nk,d] (dtype FATTN_F16 or FATTN_BF16); o [B,H,Nq,d] (dtype);
 * lse [B,H,Nq] (float32). Partials: o_parts [S,B,H,Nq,d] and lse_parts [S,B,H,Nq], float32, S =
 * num_splits. Limits: 1 <= Nq, Nk <= 16777216; 1 <= num_splits <= 1024; d in {64, 128}.
 *
 * Partition: split s covers keys [s*L, min(Nk, (s+1)*L)) with L = 64 * ceil(Nk / (64 * S)); splits
 * starting at or after Nk are empty.
 * Causal: query i is position i + Nk - Nq of the sequence and sees keys j <= i + Nk - Nq (the
 * queries are the last Nq positions; Nq == Nk is the ordinary causal mask). causal with Nq > Nk
 * returns FATTN_ERR_SHAPE.
 * Partial of split s for row i: O_s = softmax-weighted mean of the split's visible values and
 * LSE_s = natural log of the exp-sum of the split's visible scaled logits; a row that sees no key
 * of the split gets O_s = 0, LSE_s = -inf.
 */

/* num_splits that fattn_fwd_splitkv picks when given 0 (0 if the shape is invalid). */
int fattn_splitkv_num_splits(int B, int H, int Nq, int Nk, int d);

/*
 * Bytes of workspace fattn_fwd_splitkv needs for num_splits (0 = the automatic choice): the
 * float32 partials, o_parts then lse_parts, each rounded up to 256 bytes. 0 for invalid shapes.
 */
size_t fattn_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int d, int num_splits);

/*
 * O and LSE by fattn_fwd_partial into the workspace followed by fattn_combine, both enqueued on
 * `stream`. num_splits = 0 picks fattn_splitkv_num_splits(). The workspace is caller-owned device
 * memory of at least fattn_fwd_splitkv_workspace_size() bytes; contents on exit unspecified.
 */
int fattn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                      int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/* The partials alone (num_splits >= 1): writes o_parts and lse_parts as described above. */
int fattn_fwd_partial(const void* q, const void* k, const void* v, float* o_parts, float* lse_parts,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal, int dtype,
                      int num_splits, void* stream);

/*
 * Merge of S = num_splits float32 partials per row into o [B,H,Nq,d] (dtype: FATTN_F32, FATTN_F16
 * or FATTN_BF16, round-to-nearest-even) and lse [B,H,Nq] (float32). With M = max_s LSE_s and
 * w_s = exp(LSE_s - M): O = sum_s w_s O_s / sum_s w_s and LSE = M + ln sum_s w_s; partials with
 * LSE_s = -inf are skipped (their O_s is not read), and a row whose partials are all -inf gets
 * O = 0, LSE = -inf. Any partials in this layout can be merged, not only fattn_fwd_partial's.
 */
int fattn_combine(const float* o_parts, const float* lse_parts, int num_splits, void* o, float* lse,
                  int B, int H, int Nq, int d, int dtype, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fattn_strerror(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FATTN_H */
