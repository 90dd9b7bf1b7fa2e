/*
 * dictfs.h -- C ABI of the MI355X (gfx950) factored dictionary projection.
 *
 * A layer's weight W_l (d_in x d_out, rows of X are tokens) is stored as a
 * dense dictionary D_g (d_in x k, shared by the layers of a group) times a
 * sparse per-layer coefficient matrix C_l (k x d_out), and the layer computes
 *     Z_l = X_l D_g,    Y_l = Z_l C_l
 * ("DictLLM: Shared Dictionaries for Post-Training Compression", section
 * "Prerequisites: projections, rank and calibration", Eq. (1)).  Either
 * factor may be stored in NVFP4: 4-bit E2M1 values with one 8-bit E4M3 scale
 * per block of sixteen values (same review, "From retained values to measured
 * decoding"), plus one fp32 tensor scale.  The coefficients may also be
 * 8-bit codes, FP8 (E4M3) or INT8, each column with one fp32 scale: the
 * mixed-precision pairs of the paper's figures and tables page, Table 4
 * (NVFP4 dictionary with FP16, FP8 or INT8 coefficients).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     never allocates or frees device memory.  Scratch memory is passed in as
 *     a caller-owned workspace sized by the matching *_workspace_size call.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls
 *     enqueue their kernels on it and return without synchronising, except
 *     where a call says it synchronises.
 *   - Every argument is validated before anything is enqueued; on error the
 *     call returns a non-zero dfs_status and writes nothing.  No C++
 *     exception crosses this boundary.  DFS_E_HIP means the HIP runtime
 *     reported an error; dfs_last_hip_error() returns its hipError_t code.
 *   - Base pointers of X, D data, CSC row indices and values and NVFP4
 *     codes must be 16-byte aligned (DFS_E_ALIGN otherwise); leading
 *     dimensions of f16 X and D must be multiples of 8 elements and of f32
 *     ones multiples of 4, so that every row stays 16-byte aligned.  Y and
 *     the CSC column pointers need only the alignment of their element type
 *     (Y is written one element at a time; ldy is any value >= d_out).
 *   - Accumulation is always fp32.  Results are deterministic run to run
 *     (no floating-point atomics).  The intermediate Z = X D_g is held in
 *     fp32 whenever X or D_g is fp32 (every path keeps it unrounded then);
 *     with f16 X and an f16 or NVFP4 dictionary it is rounded to f16 where a
 *     path stages it so: the MFMA product for more than 16 stacked rows, and
 *     the f16 Z tiles the coefficient kernels use when an fp32 tile would
 *     not fit their LDS.
 *   - Thread safety: calls hold no mutable global state beyond a per-thread
 *     last-HIP-error code and per-device facts looked up once (the CU count,
 *     the address of the no-allocation workspace, under a lock); concurrent
 *     calls on different streams are safe when they do not share a
 *     workspace.  The one-launch decode runs one
 *     workgroup per CU and hands Z between them; if two such launches (or
 *     other kernels) share the GPU, the bounded waits described under
 *     dict_workspace_size keep the results right, at a cost in time.
 */
#ifndef DICTFS_H
#define DICTFS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DFS_OK = 0,
  DFS_E_INVALID = 1,     /* null pointer, bad dimension or leading dim, NaN/Inf input */
  DFS_E_UNSUPPORTED = 2, /* dtype combination or layout the library does not run */
  DFS_E_RANGE = 3,       /* k > 65536 (forward: k > 16384), nnz >= 2^31, capacity too small,
                            > 16 layers */
  DFS_E_ALIGN = 4,       /* a base pointer or leading dimension is misaligned */
  DFS_E_WORKSPACE = 5,   /* workspace missing or too small */
  DFS_E_HIP = 6          /* the HIP runtime returned an error */
} dfs_status;

/* Element types.  DFS_FP8 and DFS_INT8 are coefficient (dfs_csc) types only:
 *   DFS_FP8   one E4M3 code per value (sign bit 7, 4-bit exponent with bias
 *             7, 3-bit mantissa, exponent 0 subnormal; largest finite 448).
 *             The codes 0x7F and 0xFF (NaN in E4M3) are not supported: the
 *             kernels decode them as +-480.
 *   DFS_INT8  one two's-complement byte per value. */
enum { DFS_F32 = 0, DFS_F16 = 1, DFS_NVFP4 = 2, DFS_FP8 = 3, DFS_INT8 = 4 };

/* An NVFP4 tensor of n elements (device pointers):
 *   codes[(n+1)/2]   two E2M1 codes per byte, element 2i in the low nibble;
 *                    code bit 3 is the sign, bits 2..0 index the magnitudes
 *                    {0, 0.5, 1, 1.5, 2, 3, 4, 6};
 *   scales[(n+15)/16] one E4M3 (bias 7, no infinities, max 448) code per
 *                    block of 16 consecutive elements (last block may be short);
 *   tensor_scale[1]  fp32.
 * Element i decodes to e2m1(code_i) * e4m3(scales[i/16]) * tensor_scale[0]. */
typedef struct {
  uint8_t* codes;
  uint8_t* scales;
  float* tensor_scale;
} dfs_nvfp4;

/* Dictionary D_g, mathematically d_in x k, stored ATOM-MAJOR: atom a (column a
 * of D_g) is d_in contiguous elements starting at element a*ldd.  A row-major
 * (k, d_in) tensor, i.e. D_g transposed, has exactly this layout.
 *   dtype F16 / F32: `data` holds the elements, ldd >= d_in, ldd % 8 == 0 (F16)
 *                    or ldd % 4 == 0 (F32).
 *   dtype NVFP4:     `nv` holds the k*d_in elements in atom-major order,
 *                    ldd == d_in, d_in % 32 == 0 (so each 16-block lies inside
 *                    one atom and each atom starts on a 16-byte boundary). */
typedef struct {
  int32_t d_in;
  int32_t k;
  int32_t dtype;
  int32_t _pad;
  const void* data;
  int64_t ldd;
  dfs_nvfp4 nv;
} dfs_dict;

/* Coefficients C_l, k x d_out, column-compressed (CSC):
 *   colptr[d_out+1] int32, colptr[0] = 0, non-decreasing, colptr[d_out] = nnz;
 *   rowidx[nnz] uint16 atom indices, strictly increasing within a column;
 *   values in CSC order: `vals` (F16/F32), `nv` (NVFP4, blocks of 16 run
 *   over the flat CSC value array and may straddle column boundaries), or
 *   `vals` as one code byte per entry with `col_scale` (FP8/INT8): entry p
 *   of column j is value(code_p) * col_scale[j], col_scale[d_out] fp32.
 * k <= 65536 (16-bit indices), nnz < 2^31.
 * Padding: the forward kernels read rowidx and the values in aligned chunks
 * of 8 entries, so rowidx and vals must be allocated for
 * dict_csc_capacity(nnz) entries (NVFP4 codes: half that many bytes; block
 * scales: ceil(nnz / 16) bytes; FP8/INT8 codes: that many bytes).  Entries
 * past nnz are never used and may hold anything.  `capacity` states the
 * entries (blocks, with block_rows = 8) that rowidx and the values are
 * allocated for; every call that reads the arrays rejects capacity <
 * dict_csc_capacity(nnz) with DFS_E_RANGE.  The caller owns all arrays.
 * Block-structured support (block_rows = 8; 0 means one entry per stored
 * element): each column keeps whole blocks of 8 consecutive atoms (the
 * variant of "DictLLM: Shared Dictionaries for Post-Training Compression",
 * "Let the accelerator constrain the support").  Then colptr counts kept
 * blocks, nnz is the number of kept blocks, rowidx[nnz] holds block indices
 * b (atoms 8b .. 8b+7, strictly increasing within a column) and vals holds
 * 8 values per block, 8q .. 8q+7 for the q-th block (F16 or F32 only).
 * rowidx is allocated for dict_csc_capacity(nnz) blocks and vals for 8 times
 * that.  Such coefficients run for T <= 16 tokens per layer on the two-launch
 * path (DFS_E_UNSUPPORTED above that). */
typedef struct {
  int32_t k;
  int32_t d_out;
  int64_t nnz;
  int32_t dtype;
  int32_t block_rows; /* 0, or 8 for block-structured support */
  const int32_t* colptr;
  const uint16_t* rowidx;
  const void* vals;
  dfs_nvfp4 nv;
  const float* col_scale; /* FP8 / INT8 only: one scale per column */
  int64_t capacity;       /* entries (blocks) rowidx and the values hold */
} dfs_csc;

/* ---------------------------------------------------------------------- */
/* Packing                                                                */
/* ---------------------------------------------------------------------- */

/* Entries that rowidx and vals must be allocated for when a CSC with nnz
 * stored entries is passed to a forward call: nnz rounded up to a multiple
 * of 8, at least 8 (negative nnz gives 8). */
int64_t dict_csc_capacity(int64_t nnz);

/* Workspace bytes dict_pack_csc needs for a k x d_out matrix. */
dfs_status dict_pack_csc_workspace_size(int32_t k, int32_t d_out, size_t* bytes);

/* Dense row-major C (k x d_out, leading dimension ldc >= d_out, dtype F16 or
 * F32, device) -> CSC.  Column j keeps the rows r, in ascending order, whose
 * entry compares unequal to zero (+0 and -0 are dropped, NaN is kept); the
 * row goes to rowidx as uint16 and the value is bit-copied to vals (same
 * dtype as C).  This is the support-keeping export of the coefficients
 * ("DictLLM: Shared Dictionaries for Post-Training Compression", Algorithm 2:
 * export of dictionary, codes, scales and support, zeros preserved).
 *   rowidx == NULL and vals == NULL: fill colptr[d_out+1] and *nnz_host only.
 *   otherwise: fill colptr, rowidx[0..nnz), vals[0..nnz); capacity (elements
 *   of rowidx/vals) < dict_csc_capacity(nnz) gives DFS_E_RANGE with colptr
 *   written and rowidx/vals untouched.
 * Synchronises `stream` to return *nnz_host (host pointer, required). */
dfs_status dict_pack_csc(const void* C, int32_t dtype, int32_t k, int32_t d_out, int64_t ldc,
                         int32_t* colptr, uint16_t* rowidx, void* vals, int64_t capacity,
                         int64_t* nnz_host, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes dict_csc_quantize8 needs for d_out columns. */
dfs_status dict_csc_quantize8_workspace_size(int32_t d_out, size_t* bytes);

/* Quantise the values of a CSC (src->dtype F16 or F32, src->vals holding
 * nnz values in CSC order) to 8-bit codes, `dtype` DFS_FP8 or DFS_INT8, with
 * one scale per column: the coefficient formats of the mixed-precision rows
 * of Table 4 on the paper's figures and tables page.  The pages do not fix
 * the scaling; this library uses, each step a correctly rounded fp32
 * operation:
 *   amax_j = max |v| over column j's stored values;
 *   s_j = amax_j / 448 (FP8) or amax_j / 127 (INT8), or 1 if that is 0;
 *   q = v / s_j;
 *   FP8:  code = (sign bit of v) << 7 | E4M3 magnitude code nearest to |q|
 *         (ties to even, saturating at 448);
 *   INT8: code = integer nearest to q (ties to even), clamped to [-127, 127].
 * Writes codes[0..nnz) (device, 16-byte aligned; allocate
 * dict_csc_capacity(nnz) bytes to pass it to a forward call) and
 * col_scale[0..d_out) (device).  The support (colptr, rowidx) is unchanged
 * and shared with src.  Values holding NaN or Inf give DFS_E_INVALID and
 * nothing written; detecting it synchronises `stream`. */
dfs_status dict_csc_quantize8(const dfs_csc* src, int32_t dtype, uint8_t* codes, float* col_scale,
                              void* ws, size_t ws_bytes, void* stream);

/* Dense row-major C (as for dict_pack_csc) -> block-structured CSC, blocks
 * of 8 consecutive rows per column (see dfs_csc): a block is kept iff one of
 * its entries compares unequal to zero (rows past k count as zero); kept
 * block q stores its index in bidx[q] and its 8 values, bit-copied (rows past
 * k as +0), in vals[8q .. 8q+7].  Workspace: dict_pack_csc_workspace_size.
 * Otherwise as dict_pack_csc, with counts in blocks: bidx == NULL and vals
 * == NULL fill colptr and *nblk_host only; capacity (blocks that bidx holds;
 * vals holds 8 times as many elements) < dict_csc_capacity(nblk) gives
 * DFS_E_RANGE.  k <= 65536.  Synchronises `stream`. */
dfs_status dict_pack_bcsc(const void* C, int32_t dtype, int32_t k, int32_t d_out, int64_t ldc,
                          int32_t* colptr, uint16_t* bidx, void* vals, int64_t capacity,
                          int64_t* nblk_host, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes nvfp4_pack needs for n elements. */
dfs_status nvfp4_pack_workspace_size(int64_t n, size_t* bytes);

/* Quantise x[0..n) (fp32, device) to NVFP4 (see dfs_nvfp4): 4-bit values
 * with one 8-bit scale per block of sixteen ("DictLLM: Shared Dictionaries
 * for Post-Training Compression", "From retained values to measured
 * decoding"; the all-NVFP4 rows of the figures and tables page, Table 4).
 * The pages do not print the scale recipe; the one used here, applied with
 * correctly rounded fp32 operations:
 *   amax = max|x|;  ts = amax / 2688 (= 6 * 448), or 1 if that is 0;
 *   per block b: sf = amax_b / (6 * ts); scale code = E4M3 nearest to sf,
 *     ties to even, saturating at 448; s = its value; denom = s * ts;
 *   per element: magnitude code = E2M1 nearest to |x / denom| (ties to even,
 *     saturating at 6; 0 when denom == 0), sign bit = sign bit of x.
 * x holding NaN or Inf gives DFS_E_INVALID and writes nothing; detecting it
 * synchronises `stream`.  out.codes needs 16-byte alignment. */
dfs_status nvfp4_pack(const float* x, int64_t n, dfs_nvfp4 out, void* ws, size_t ws_bytes,
                      void* stream);

/* Decode n NVFP4 elements to fp32 (the inverse of nvfp4_pack's encoding,
 * same passages): y[i] = (e2m1(code_i) * e4m3(scale_{i/16})) * tensor_scale,
 * one fp32 rounding (the first product is exact).  n = 0 is a no-op and
 * n < 0 gives DFS_E_INVALID; in and y are device pointers owned by the
 * caller; enqueued on `stream`. */
dfs_status nvfp4_unpack(dfs_nvfp4 in, int64_t n, float* y, void* stream);

/* ---------------------------------------------------------------------- */
/* Forward                                                                */
/* ---------------------------------------------------------------------- */

/* Workspace bytes for dict_group_forward over n_layers layers of T tokens
 * (dict_proj_forward: n_layers = 1).  D and C describe the shapes and dtypes
 * (C may point at any one layer's descriptor; only k/d_out/dtype are read).
 *
 * The size does not depend on the activation dtype (the larger of the f16
 * and f32 layouts), so a workspace of this size serves either.
 *
 * Forward workspace contract: the whole workspace must be ZERO before the
 * first forward call that uses it (e.g. hipMemset once after allocation).
 * It starts with a 4096-byte control block followed by 64 * k bytes of
 * tagged Z words through which the workgroups of the one-launch decode hand
 * Z to each other instead of meeting at a grid barrier; every call leaves
 * both zero again when it completes (so zeroing them again between calls,
 * all or in part, is harmless).  The rest is scratch for the call.  Calls
 * sharing one workspace must not run concurrently.  The 32-bit word at byte
 * offset 128 becomes non-zero when a workgroup of the one-launch decode
 * (T = 1, <= 4 layers) gave up waiting for a published Z word after a
 * bounded number of polls and computed the missing words itself from X and
 * D_g, which happens when its grid is not resident all at once (for
 * instance, while other kernels hold some CUs).  The outputs are right
 * either way; the word is a diagnostic that stays set until the caller
 * clears it.  The bound is 2^20 polls of about a microsecond, or the value
 * of the environment variable DFS_SPIN_LIMIT, read at each call (0: no poll
 * at all, every workgroup computes every Z word it needs: slow, for tests). */
dfs_status dict_workspace_size(int32_t n_layers, int32_t T, const dfs_dict* D, const dfs_csc* C,
                               size_t* bytes);

/* One factored projection, Eq. (1): Z = X D_g, Y = Z C_l.
 *   X: T x d_in row-major, leading dimension ldx, dtype F16 or F32.
 *   Y: T x d_out row-major, leading dimension ldy, dtype F16 or F32.
 *   T = 0 is a no-op.  The intermediate Z (T x k) lives in the workspace.
 *   k <= 16384 (the product kernels stage Z tiles of every atom in LDS);
 *   a larger k gives DFS_E_RANGE.  The same limit holds for every forward call. */
dfs_status dict_proj_forward(const void* X, int32_t xdt, int32_t T, int64_t ldx, const dfs_dict* D,
                             const dfs_csc* C, void* Y, int32_t ydt, int64_t ldy, void* ws,
                             size_t ws_bytes, void* stream);

/* The projections of one layer group that share D_g
 * (same review, Figure 2: one dictionary, separate activations and codes):
 * for l in [0, n_layers): Y[l] = (X[l] D_g) C[l].  The n_layers * T rows are
 * contracted against D_g in one pass, so D_g is read from memory once per
 * group rather than once per layer; then one launch applies every C_l.
 * Decode (T = 1, <= 4 layers, f16 X, f16/NVFP4 D, f16/NVFP4/FP8/INT8 C)
 * runs both halves in a single launch, Z handed between workgroups through
 * the workspace
 * (environment variable DFS_DECODE_PATH=two selects the two-launch path).
 *   X, Y: host arrays of n_layers device pointers; C: host array of n_layers
 *   descriptors sharing k and d_out.  1 <= n_layers <= 16 (the largest
 *   group the pages study). */
dfs_status dict_group_forward(int32_t n_layers, const void* const* X, int32_t xdt, int32_t T,
                              int64_t ldx, const dfs_dict* D, const dfs_csc* C, void* const* Y,
                              int32_t ydt, int64_t ldy, void* ws, size_t ws_bytes, void* stream);

/* dict_group_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and results, with no workspace
 * argument.  Its workspace is a 64 MiB array inside the library, one per GPU
 * the library runs on, held until the process ends; shapes whose workspace
 * (dict_workspace_size) exceeds 64 MiB give DFS_E_WORKSPACE.  The call itself
 * allocates nothing; on its first use on a device it enqueues the zeroing of
 * the part of the array that must start at zero.  Every call on a GPU shares
 * that GPU's array, so calls that overlap in time on one GPU (other streams,
 * other threads) race and must not be made.  Arguments and errors as for
 * dict_group_forward. */
dfs_status dict_group_forward_noalloc(int32_t n_layers, const void* const* X, int32_t xdt,
                                      int32_t T, int64_t ldx, const dfs_dict* D, const dfs_csc* C,
                                      void* const* Y, int32_t ydt, int64_t ldy, void* stream);

/* Several layer groups that read the same activations, one dictionary each
 * (as the q, k and v projections of the same layers do; each group is the
 * factored projection of Eq. (1) with its own D_g, Figure 2):
 * for d in [0, n_dicts) and l in [0, n_layers):
 *   Y[d * n_layers + l] = (X[l] D[d]) C[d * n_layers + l].
 * D: host array of n_dicts descriptors sharing d_in, k, dtype and ldd;
 * C, Y: host arrays of n_dicts * n_layers descriptors / device pointers,
 * dictionary-major, sharing d_out and dtype; X: n_layers device pointers
 * shared by every dictionary.  1 <= n_dicts <= 8; each group obeys the
 * limits of dict_group_forward, and every argument is checked before
 * anything is launched.  At decode (T = 1, 2 or 3 dictionaries, at most 2
 * layers, f16 X, f16 or NVFP4 D and C, d_in <= 4096 for f16 D) the whole
 * set runs as one launch: one grid computes Z for the atoms of every
 * dictionary and applies every C, so the groups share one launch and one
 * latency chain.  Otherwise, or with DFS_DECODE_PATH=two, the groups run
 * in turn as dict_group_forward calls on the same workspace.  Results equal
 * those of dict_group_forward on each group.  The workspace (size from
 * dict_multi_workspace_size) starts with the 4096-byte control block of
 * dict_group_forward, zero before first use. */
dfs_status dict_multi_workspace_size(int32_t n_dicts, int32_t n_layers, int32_t T,
                                     const dfs_dict* D, const dfs_csc* C, size_t* bytes);
dfs_status dict_multi_forward(int32_t n_dicts, int32_t n_layers, const void* const* X,
                              int32_t xdt, int32_t T, int64_t ldx, const dfs_dict* D,
                              const dfs_csc* C, void* const* Y, int32_t ydt, int64_t ldy,
                              void* ws, size_t ws_bytes, void* stream);

/* The first half of Eq. (1) alone: Z = X D_g for every layer of a group.
 * Z is (n_layers*T) x k row-major (row l*T + t), dtype F32 or F16, 16-byte
 * aligned.  Dense-product choice: VALU dot products for n_layers*T <= 16 rows,
 * MFMA tiles above that (F16 or NVFP4 dictionary, F16 activations). */
dfs_status dict_xd_forward(int32_t n_layers, const void* const* X, int32_t xdt, int32_t T,
                           int64_t ldx, const dfs_dict* D, void* Z, int32_t zdt, void* ws,
                           size_t ws_bytes, void* stream);

/* Workspace bytes dict_xd_forward needs (non-zero only on the MFMA path:
 * the f16 expansion of an NVFP4 dictionary, and for at most 128 stacked rows
 * the fp32 partial products of the split K dimension). */
dfs_status dict_xd_workspace_size(int32_t n_layers, int32_t T, const dfs_dict* D, size_t* bytes);

/* The second half of Eq. (1) alone: Y[l] = Z_l C[l], Z as written by
 * dict_xd_forward (row l*T + t of a (n_layers*T) x k array, dtype zdt,
 * 16-byte aligned: DFS_E_ALIGN otherwise). */
dfs_status dict_zc_forward(int32_t n_layers, const void* Z, int32_t zdt, int32_t T,
                           const dfs_csc* C, void* const* Y, int32_t ydt, int64_t ldy,
                           void* stream);

/* ---------------------------------------------------------------------- */
/* Producer steps (offline, fp32)                                          */
/* ---------------------------------------------------------------------- */
/* The steps that produce D_g and C_l ("DictLLM: Shared Dictionaries for
 * Post-Training Compression", "Method II: prune in coefficient space" and
 * "Method III: refit the dictionary and quantize the factors").  All
 * matrices are fp32, row-major, device memory owned by the caller, with the
 * given leading dimensions (in elements).  k <= 8192. */

/* Workspace bytes of dict_gram_inverse for this dictionary. */
dfs_status dict_gram_inverse_workspace_size(const dfs_dict* D, size_t* bytes);

/* P = (D^T S D + lambda I)^-1 (Eq. (6); the fixed inverse of Eq. (7)).
 * D: F16 or F32 dictionary (atom-major, as for the forward); S: d_in x d_in
 * symmetric positive semidefinite (the group's calibration metric), leading
 * dimension lds; lambda >= 0; P: k x k, leading dimension ldp.  The inverse
 * is taken by Gauss-Jordan elimination without pivoting, blocked 64 pivots
 * at a time; if D^T S D + lambda I is not positive definite, the 32-bit word
 * at the start of the workspace is set non-zero and P is undefined.
 * NVFP4 dictionaries give DFS_E_UNSUPPORTED. */
dfs_status dict_gram_inverse(const dfs_dict* D, const float* S, int64_t lds, float lambda, float* P,
                             int64_t ldp, void* ws, size_t ws_bytes, void* stream);

/* Fixed-inverse pruning of every column of the coefficients (the review's
 * Algorithm 1, a reading of the paper's Algorithm 2, with the compensation
 * and saliency of Eq. (7)).  C: k x d_out (ldc), the unpruned coefficients;
 * P: k x k (ldp), symmetric, positive diagonal (from dict_gram_inverse).
 * Each column independently: score_i = (c_i * c_i) / P_ii in fp32 from the
 * column before any deletion; the n_prune rows of least score (ties to the
 * lower row) are deleted in that order, each by c -= P[i, :] * (c_i / P_ii)
 * with the current c_i; then the deleted entries are set to exactly 0.
 * Writes C_out (k x d_out, ldo; may not alias C) and keep (k x d_out bytes,
 * ldkeep: 1 = in the support, 0 = pruned).  0 <= n_prune <= k. */
dfs_status dict_obs_prune(int32_t k, int32_t d_out, const float* C, int64_t ldc, const float* P,
                          int64_t ldp, int32_t n_prune, float* C_out, int64_t ldo, uint8_t* keep,
                          int64_t ldkeep, void* stream);

/* Workspace bytes of dict_refit. */
dfs_status dict_refit_workspace_size(int32_t d_in, int32_t k, size_t* bytes);

/* Dictionary refit, Eq. (9): D (C C^T + lambda I) = W C^T.  W = [W_1 .. W_n]
 * (d_in x N, ldw: the group's dense weights side by side, N = n d_out);
 * C = [C_1 .. C_n] (k x N, ldc: the pruned coefficients, zeros included).
 * Writes D atom by atom, Dt (k x d_in, ldd), the layout the forward takes
 * for an F32 dictionary.  lambda >= 0; with lambda = 0 every atom must have
 * a coefficient somewhere (else the Gram matrix is singular: the 32-bit
 * word at the start of the workspace is set non-zero and Dt is undefined). */
dfs_status dict_refit(int32_t d_in, int32_t N, int32_t k, const float* W, int64_t ldw,
                      const float* C, int64_t ldc, float lambda, float* Dt, int64_t ldd, void* ws,
                      size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- */
/* Diagnostics                                                            */
/* ---------------------------------------------------------------------- */

const char* dfs_status_str(dfs_status s);
/* hipError_t of the last DFS_E_HIP returned on this thread (0 if none). */
int32_t dfs_last_hip_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int32_t dfs_version(void);

/* Matrix-core probe (measurement support, not a step of the method): blocks
 * workgroups of 256 threads; every wave runs iters rounds of 8 independent
 * v_mfma_f32_32x32x16_f16 on register operands, so the work is
 * blocks * 4 * iters * 8 * 32768 FLOP with no memory traffic except one
 * float per thread written to out (device memory, blocks * 256 floats,
 * caller-owned).  Two workgroups fit a CU.  Timed by the caller, it gives the
 * sustained fp16 MFMA rate of the device, the measured counterpart of the
 * nominal peak for the prefill GEMM (Eq. (1), Z = X D_g at prefill).  Every
 * thread's value is the same function of iters alone (exact in fp32 for
 * iters <= 2^16), so equal outputs across blocks and out(n) = n * out(1)
 * check it ran.  0 < blocks <= 2^20, iters > 0; enqueued on stream. */
dfs_status dfs_probe_mfma(int32_t blocks, int32_t iters, float* out, void* stream);

/* HBM read probe (measurement support, not a step of the method): reads the
 * `bytes` bytes at buf (device memory, caller-owned, read only) once with
 * blocks workgroups of 256 threads: thread t of the G = blocks * 256 threads
 * reads the 16-byte words t, t + G, t + 2G, ..., and writes the XOR of the
 * dwords it read to out[t] (device memory, G uint32, caller-owned; the XOR of
 * all of out is the XOR of every dword of the buffer, which checks that each
 * was read).  Timed by the caller on a buffer larger than the caches, it
 * gives the rate at which the device reads HBM, the measured counterpart of
 * the nominal 8 TB/s for the decode, which reads each factor byte once.
 * buf 16-byte aligned, bytes a positive multiple of 16 (DFS_E_ALIGN),
 * 0 < blocks <= 2^20; enqueued on stream. */
dfs_status dfs_probe_read(const void* buf, int64_t bytes, int32_t blocks, uint32_t* out,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DICTFS_H */
