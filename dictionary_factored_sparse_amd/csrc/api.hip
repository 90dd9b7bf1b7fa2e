// api.hip -- the C ABI of include/dictfs.h: validation, workspace layout,
// path choice and kernel launches on the caller's stream.
//
// Forward ("DictLLM: Shared Dictionaries for Post-Training Compression",
// Eq. (1)): Z = X D_g on VALU dot products for <= 16 stacked rows and on
// MFMA above that; Y_l = Z_l C_l on the CSC SpMV for T <= 16 tokens per
// layer and on the token-tiled SpMM above that.  Every argument is checked
// before anything is enqueued.
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "dfs_internal.hpp"

using namespace dfs;

namespace {

thread_local int32_t g_last_hip = 0;

dfs_status hip_fail(hipError_t e) {
  g_last_hip = (int32_t)e;
  return DFS_E_HIP;
}

#define DFS_HIP(x)                                  \
  do {                                              \
    hipError_t _e = (x);                            \
    if (_e != hipSuccess) return hip_fail(_e);      \
  } while (0)

#define DFS_TRY(x)                                  \
  do {                                              \
    dfs_status _s = (x);                            \
    if (_s != DFS_OK) return _s;                    \
  } while (0)

constexpr int32_t kMaxK = 65536;         // 16-bit row indices
constexpr int32_t kMaxKForward = 16384;  // Z tiles staged in LDS
constexpr int64_t kMaxNnz = (int64_t)1 << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t esize(int32_t dt) { return dt == DFS_F32 ? 4 : 2; }
size_t round256(size_t x) { return (x + 255) / 256 * 256; }
bool is_act_dtype(int32_t dt) { return dt == DFS_F16 || dt == DFS_F32; }
bool is_code8(int32_t dt) { return dt == DFS_FP8 || dt == DFS_INT8; }

dfs_status check_nvfp4(const dfs_nvfp4& nv) {
  if (!nv.codes || !nv.scales || !nv.tensor_scale) return DFS_E_INVALID;
  if (!aligned16(nv.codes)) return DFS_E_ALIGN;
  return DFS_OK;
}

dfs_status check_dict(const dfs_dict* D) {
  if (!D) return DFS_E_INVALID;
  if (D->d_in <= 0 || D->k <= 0) return DFS_E_INVALID;
  if (D->k > kMaxKForward) return DFS_E_RANGE;
  if (D->dtype == DFS_NVFP4) {
    DFS_TRY(check_nvfp4(D->nv));
    if (D->ldd != D->d_in) return DFS_E_UNSUPPORTED;
    if (D->d_in % 32 != 0) return DFS_E_UNSUPPORTED;
    return DFS_OK;
  }
  if (!is_act_dtype(D->dtype)) return DFS_E_UNSUPPORTED;
  if (!D->data) return DFS_E_INVALID;
  if (D->ldd < D->d_in) return DFS_E_INVALID;
  if (!aligned16(D->data) || (D->ldd * (int64_t)esize(D->dtype)) % 16 != 0) return DFS_E_ALIGN;
  return DFS_OK;
}

dfs_status check_csc(const dfs_csc* C, int32_t k, int32_t d_out) {
  if (!C) return DFS_E_INVALID;
  if (C->k != k || C->d_out != d_out || d_out <= 0) return DFS_E_INVALID;
  if (C->nnz < 0) return DFS_E_INVALID;
  if (C->nnz >= kMaxNnz) return DFS_E_RANGE;
  if (!C->colptr) return DFS_E_INVALID;
  if ((uintptr_t)C->colptr % 4 != 0) return DFS_E_ALIGN;
  if (C->nnz > 0) {
    if (!C->rowidx) return DFS_E_INVALID;
    if (!aligned16(C->rowidx)) return DFS_E_ALIGN;
    // the kernels read whole 8-entry chunks
    if (C->capacity < dict_csc_capacity(C->nnz)) return DFS_E_RANGE;
  }
  if (C->block_rows != 0 && C->block_rows != 8) return DFS_E_UNSUPPORTED;
  if (C->block_rows == 8 && !is_act_dtype(C->dtype)) return DFS_E_UNSUPPORTED;
  if (C->dtype == DFS_NVFP4) {
    if (C->nnz > 0) DFS_TRY(check_nvfp4(C->nv));
    else if (!C->nv.tensor_scale) return DFS_E_INVALID;
    return DFS_OK;
  }
  if (!is_act_dtype(C->dtype) && !is_code8(C->dtype)) return DFS_E_UNSUPPORTED;
  if (is_code8(C->dtype) && !C->col_scale) return DFS_E_INVALID;
  if (C->nnz > 0) {
    if (!C->vals) return DFS_E_INVALID;
    if (!aligned16(C->vals)) return DFS_E_ALIGN;
  }
  return DFS_OK;
}

dfs_status check_x(const void* const* X, int32_t n, int32_t xdt, int64_t ldx, int32_t d_in) {
  if (!is_act_dtype(xdt)) return DFS_E_UNSUPPORTED;
  if (ldx < d_in) return DFS_E_INVALID;
  if ((ldx * (int64_t)esize(xdt)) % 16 != 0) return DFS_E_ALIGN;
  for (int i = 0; i < n; ++i) {
    if (!X[i]) return DFS_E_INVALID;
    if (!aligned16(X[i])) return DFS_E_ALIGN;
  }
  return DFS_OK;
}

dfs_status check_y(void* const* Y, int32_t n, int32_t ydt, int64_t ldy, int32_t d_out) {
  if (!is_act_dtype(ydt)) return DFS_E_UNSUPPORTED;
  if (ldy < d_out) return DFS_E_INVALID;
  for (int i = 0; i < n; ++i) {
    if (!Y[i]) return DFS_E_INVALID;
    if ((uintptr_t)Y[i] % esize(ydt) != 0) return DFS_E_ALIGN;  // element stores
  }
  return DFS_OK;
}

bool mfma_path(int64_t rows, int32_t xdt, const dfs_dict* D) {
  return rows > kGemvMaxRows && xdt == DFS_F16 && D->dtype != DFS_F32 && D->d_in % 8 == 0;
}

// Workspace of the MFMA path: the f16 expansion of an NVFP4 dictionary, then
// the split-K partial products (few stacked rows).
size_t xd_expand_bytes(int64_t rows, int32_t xdt, const dfs_dict* D) {
  if (D->dtype == DFS_NVFP4 && mfma_path(rows, xdt, D))
    return round256((size_t)D->k * D->d_in * 2);
  return 0;
}
size_t xd_ws_bytes(int64_t rows, int32_t xdt, const dfs_dict* D) {
  if (!mfma_path(rows, xdt, D)) return 0;
  const int ks = gemm_split_k(rows, D->k, D->d_in);
  const size_t part = ks > 1 ? round256((size_t)ks * rows * D->k * 4) : 0;
  return xd_expand_bytes(rows, xdt, D) + part;
}

XdLaunch make_xd(int32_t n, const void* const* X, int32_t xdt, int32_t T, int64_t ldx,
                 const dfs_dict* D, void* Z, int32_t zdt) {
  XdLaunch a;
  std::memset(&a, 0, sizeof(a));
  for (int i = 0; i < n; ++i) a.X[i] = X[i];
  a.n_layers = n;
  a.T = T;
  a.ldx = ldx;
  a.xdt = xdt;
  a.d_in = D->d_in;
  a.k = D->k;
  a.ddt = D->dtype;
  a.D = D->data;
  a.ldd = D->ldd;
  a.dcodes = D->nv.codes;
  a.dscales = D->nv.scales;
  a.dts = D->nv.tensor_scale;
  a.Z = Z;
  a.zdt = zdt;
  return a;
}

ZcLaunch make_zc(int32_t n, const void* Z, int32_t zdt, int32_t T, const dfs_csc* C,
                 void* const* Y, int32_t ydt, int64_t ldy) {
  ZcLaunch a;
  std::memset(&a, 0, sizeof(a));
  a.Z = Z;
  a.zdt = zdt;
  a.n_layers = n;
  a.T = T;
  a.k = C[0].k;
  a.d_out = C[0].d_out;
  a.vdt = C[0].dtype;
  for (int i = 0; i < n; ++i) {
    a.colptr[i] = C[i].colptr;
    a.nnz[i] = C[i].nnz;
    a.rowidx[i] = C[i].rowidx;
    if (C[i].dtype == DFS_NVFP4) {
      a.vals[i] = C[i].nv.codes;
      a.vscales[i] = C[i].nv.scales;
      a.vts[i] = C[i].nv.tensor_scale;
    } else if (is_code8(C[i].dtype)) {
      a.vals[i] = C[i].vals;
      a.vts[i] = C[i].col_scale;
    } else {
      a.vals[i] = C[i].vals;
    }
    a.Y[i] = Y[i];
  }
  a.ydt = ydt;
  a.ldy = ldy;
  a.block_rows = C[0].block_rows;
  return a;
}

// Z = X D for the stacked rows; Z row-major (rows x k) of dtype zdt.
dfs_status run_xd(int32_t n, const void* const* X, int32_t xdt, int32_t T, int64_t ldx,
                  const dfs_dict* D, void* Z, int32_t zdt, void* ws, hipStream_t s) {
  XdLaunch a = make_xd(n, X, xdt, T, ldx, D, Z, zdt);
  const int64_t rows = (int64_t)n * T;
  if (mfma_path(rows, xdt, D)) {
    a.zpart = (float*)((char*)ws + xd_expand_bytes(rows, xdt, D));
    if (D->dtype == DFS_NVFP4) {
      _Float16* dh = (_Float16*)ws;
      DFS_HIP(launch_nvfp4_to_f16(D->nv.codes, D->nv.scales, D->nv.tensor_scale,
                                  (int64_t)D->k * D->d_in, dh, s));
      a.D = dh;
      a.ldd = D->d_in;
      a.ddt = DFS_F16;
    }
    DFS_HIP(launch_gemm_xd_mfma(a, s));
  } else {
    DFS_HIP(launch_gemv_xd(a, s));
  }
  return DFS_OK;
}

dfs_status run_zc(int32_t n, const void* Z, int32_t zdt, int32_t T, const dfs_csc* C,
                  void* const* Y, int32_t ydt, int64_t ldy, hipStream_t s) {
  ZcLaunch a = make_zc(n, Z, zdt, T, C, Y, ydt, ldy);
  // fp32 Z (fp32 activations or dictionary) stays fp32 in LDS: the SpMVs,
  // which pass over the tokens in fp32 tiles, serve any T; the SpMMs stage
  // f16 tiles and take only f16 Z (the MFMA path's)
  const bool spmv = T <= kGemvMaxRows || zdt == DFS_F32;
  if (a.block_rows != 0 && spmv)
    DFS_HIP(launch_spmv_bcsc(a, s));
  else if (a.block_rows != 0)
    DFS_HIP(launch_spmm_bcsc(a, s));
  else if (spmv)
    DFS_HIP(launch_spmv_csc(a, s));
  else
    DFS_HIP(launch_spmm_csc(a, s));
  return DFS_OK;
}

// DFS_DECODE_PATH=two forces the two-launch decode (for comparisons).
bool fused_allowed() {
  const char* v = std::getenv("DFS_DECODE_PATH");
  return !(v && std::strcmp(v, "two") == 0);
}

constexpr size_t kCtrlBytes = kCtrlBlockBytes;  // control block at the start of the workspace

// Layout of a forward workspace, one definition for the size query and the
// calls: the control block; the tagged Z words of the one-launch decode
// (fixed size for the dictionary's k, so no other path ever writes there);
// the plain Z rows of the two-launch paths (fp32 on the dot-product path,
// f16 on the MFMA path); the MFMA path's own workspace.
struct FwdLayout {
  size_t zwords, zplain, xd, total;
};
FwdLayout fwd_layout(int64_t rows, int32_t xdt, const dfs_dict* D) {
  FwdLayout w;
  w.zwords = round256(fused_z_words_bytes(D->k));
  w.zplain = round256((size_t)rows * D->k * (mfma_path(rows, xdt, D) ? 2 : 4));
  w.xd = xd_ws_bytes(rows, xdt, D);
  w.total = kCtrlBytes + w.zwords + w.zplain + w.xd;
  return w;
}
// The size query knows no activation dtype: the larger of the two layouts.
size_t fwd_ws_bytes(int64_t rows, const dfs_dict* D) {
  const size_t a = fwd_layout(rows, DFS_F16, D).total, b = fwd_layout(rows, DFS_F32, D).total;
  return a > b ? a : b;
}

constexpr int32_t kMaxProducerK = 8192;  // the pruning kernel keeps a column's sort keys in LDS
size_t gram_ws_bytes(const dfs_dict* D) {
  size_t b = spd_inverse_ws_bytes(D->k) + round256((size_t)D->k * D->d_in * 4);  // U = D^T S
  if (D->dtype == DFS_F16) b += round256((size_t)D->k * D->d_in * 4);            // f32 atoms
  return b;
}
size_t refit_ws_bytes(int32_t d_in, int32_t k) {
  return spd_inverse_ws_bytes(k) + round256((size_t)k * k * 4) + round256((size_t)d_in * k * 4);
}

}  // namespace

extern "C" {

const char* dfs_status_str(dfs_status st) {
  switch (st) {
    case DFS_OK:
      return "ok";
    case DFS_E_INVALID:
      return "invalid argument";
    case DFS_E_UNSUPPORTED:
      return "unsupported dtype or layout";
    case DFS_E_RANGE:
      return "value out of range";
    case DFS_E_ALIGN:
      return "misaligned pointer or leading dimension";
    case DFS_E_WORKSPACE:
      return "workspace missing or too small";
    case DFS_E_HIP:
      return "HIP runtime error";
  }
  return "unknown status";
}

int32_t dfs_last_hip_error(void) { return g_last_hip; }

int32_t dfs_version(void) { return 301; }

dfs_status dfs_probe_mfma(int32_t blocks, int32_t iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return DFS_E_INVALID;
  if (blocks > (1 << 20)) return DFS_E_RANGE;
  DFS_HIP(launch_mfma_peak(blocks, iters, out, (hipStream_t)stream));
  return DFS_OK;
}

dfs_status dfs_probe_read(const void* buf, int64_t bytes, int32_t blocks, uint32_t* out,
                          void* stream) {
  if (!buf || !out || blocks <= 0 || bytes <= 0) return DFS_E_INVALID;
  if ((uintptr_t)buf % 16 != 0 || bytes % 16 != 0) return DFS_E_ALIGN;
  if (blocks > (1 << 20)) return DFS_E_RANGE;
  DFS_HIP(launch_read_probe(buf, bytes / 16, blocks, out, (hipStream_t)stream));
  return DFS_OK;
}

int64_t dict_csc_capacity(int64_t nnz) {
  if (nnz < 8) return 8;
  return (nnz + 7) / 8 * 8;
}

// ------------------------------------------------------------------ packing

dfs_status dict_pack_csc_workspace_size(int32_t k, int32_t d_out, size_t* bytes) {
  if (!bytes) return DFS_E_INVALID;
  if (k <= 0 || d_out <= 0) return DFS_E_INVALID;
  if (k > kMaxK) return DFS_E_RANGE;
  *bytes = pack_csc_ws_bytes(k, d_out);
  return DFS_OK;
}

dfs_status dict_pack_csc(const void* C, int32_t dtype, int32_t k, int32_t d_out, int64_t ldc,
                         int32_t* colptr, uint16_t* rowidx, void* vals, int64_t capacity,
                         int64_t* nnz_host, void* ws, size_t ws_bytes, void* stream) {
  if (!C || !colptr || !nnz_host) return DFS_E_INVALID;
  if (dtype != DFS_F16 && dtype != DFS_F32) return DFS_E_UNSUPPORTED;
  if (k <= 0 || d_out <= 0 || ldc < d_out) return DFS_E_INVALID;
  if (k > kMaxK) return DFS_E_RANGE;
  if ((rowidx == nullptr) != (vals == nullptr)) return DFS_E_INVALID;
  if (capacity < 0) return DFS_E_INVALID;
  // the layout every reader of the arrays takes (see check_csc)
  if ((uintptr_t)colptr % 4 != 0) return DFS_E_ALIGN;
  if (rowidx && (!aligned16(rowidx) || !aligned16(vals))) return DFS_E_ALIGN;
  if (!ws || ws_bytes < pack_csc_ws_bytes(k, d_out)) return DFS_E_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  DFS_HIP(launch_pack_csc_count(C, dtype, k, d_out, ldc, colptr, ws, s));
  int64_t total = 0;
  DFS_HIP(hipMemcpyAsync(&total, ws, sizeof(total), hipMemcpyDeviceToHost, s));
  DFS_HIP(hipStreamSynchronize(s));
  *nnz_host = total;
  if (total >= kMaxNnz) return DFS_E_RANGE;
  if (!rowidx) return DFS_OK;
  if (capacity < dict_csc_capacity(total)) return DFS_E_RANGE;
  DFS_HIP(launch_pack_csc_scatter(C, dtype, k, d_out, ldc, rowidx, vals, ws, s));
  return DFS_OK;
}

dfs_status dict_csc_quantize8_workspace_size(int32_t d_out, size_t* bytes) {
  if (!bytes || d_out <= 0) return DFS_E_INVALID;
  *bytes = quant8_ws_bytes(d_out);
  return DFS_OK;
}

dfs_status dict_csc_quantize8(const dfs_csc* src, int32_t dtype, uint8_t* codes, float* col_scale,
                              void* ws, size_t ws_bytes, void* stream) {
  if (!src || !col_scale) return DFS_E_INVALID;
  if (!is_code8(dtype)) return DFS_E_UNSUPPORTED;
  if (!is_act_dtype(src->dtype)) return DFS_E_UNSUPPORTED;
  if (src->k <= 0) return DFS_E_INVALID;
  if (src->k > kMaxK) return DFS_E_RANGE;
  DFS_TRY(check_csc(src, src->k, src->d_out));
  if (src->nnz > 0) {
    if (!codes) return DFS_E_INVALID;
    if (!aligned16(codes)) return DFS_E_ALIGN;
  }
  if (!ws || ws_bytes < quant8_ws_bytes(src->d_out)) return DFS_E_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  DFS_HIP(launch_quant8_amax(src->vals, src->dtype, src->colptr, src->nnz, src->d_out, ws, s));
  uint32_t bad = 0;
  DFS_HIP(hipMemcpyAsync(&bad, ws, sizeof(bad), hipMemcpyDeviceToHost, s));
  DFS_HIP(hipStreamSynchronize(s));
  if (bad != 0) return DFS_E_INVALID;
  DFS_HIP(launch_quant8_encode(src->vals, src->dtype, src->colptr, src->nnz, src->d_out, dtype,
                               ws, codes, col_scale, s));
  return DFS_OK;
}

dfs_status dict_pack_bcsc(const void* C, int32_t dtype, int32_t k, int32_t d_out, int64_t ldc,
                          int32_t* colptr, uint16_t* bidx, void* vals, int64_t capacity,
                          int64_t* nblk_host, void* ws, size_t ws_bytes, void* stream) {
  if (!C || !colptr || !nblk_host) return DFS_E_INVALID;
  if (dtype != DFS_F16 && dtype != DFS_F32) return DFS_E_UNSUPPORTED;
  if (k <= 0 || d_out <= 0 || ldc < d_out) return DFS_E_INVALID;
  if (k > kMaxK) return DFS_E_RANGE;
  if ((bidx == nullptr) != (vals == nullptr)) return DFS_E_INVALID;
  if (capacity < 0) return DFS_E_INVALID;
  // the layout every reader of the arrays takes (see check_csc)
  if ((uintptr_t)colptr % 4 != 0) return DFS_E_ALIGN;
  if (bidx && (!aligned16(bidx) || !aligned16(vals))) return DFS_E_ALIGN;
  if (!ws || ws_bytes < pack_csc_ws_bytes(k, d_out)) return DFS_E_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  DFS_HIP(launch_pack_csc_count(C, dtype, k, d_out, ldc, colptr, ws, s, 8));
  int64_t total = 0;
  DFS_HIP(hipMemcpyAsync(&total, ws, sizeof(total), hipMemcpyDeviceToHost, s));
  DFS_HIP(hipStreamSynchronize(s));
  *nblk_host = total;
  if (!bidx) return DFS_OK;
  if (capacity < dict_csc_capacity(total)) return DFS_E_RANGE;
  DFS_HIP(launch_pack_csc_scatter(C, dtype, k, d_out, ldc, bidx, vals, ws, s, 8));
  return DFS_OK;
}

dfs_status nvfp4_pack_workspace_size(int64_t n, size_t* bytes) {
  if (!bytes || n < 0) return DFS_E_INVALID;
  *bytes = nvfp4_ws_bytes(n);
  return DFS_OK;
}

dfs_status nvfp4_pack(const float* x, int64_t n, dfs_nvfp4 out, void* ws, size_t ws_bytes,
                      void* stream) {
  if (n < 0) return DFS_E_INVALID;
  if (!out.tensor_scale) return DFS_E_INVALID;
  if (n > 0) {
    if (!x) return DFS_E_INVALID;
    DFS_TRY(check_nvfp4(out));
  }
  if (!ws || ws_bytes < nvfp4_ws_bytes(n)) return DFS_E_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (n == 0) {
    DFS_HIP(hipMemsetD32Async((hipDeviceptr_t)out.tensor_scale, 0x3F800000u, 1, s));  // 1.0f
    return DFS_OK;
  }
  DFS_HIP(launch_nvfp4_amax(x, n, ws, s));
  uint32_t res[2] = {0, 0};
  DFS_HIP(hipMemcpyAsync(res, ws, sizeof(res), hipMemcpyDeviceToHost, s));
  DFS_HIP(hipStreamSynchronize(s));
  if (res[1] != 0) return DFS_E_INVALID;
  DFS_HIP(launch_nvfp4_encode(x, n, out, ws, s));
  return DFS_OK;
}

dfs_status nvfp4_unpack(dfs_nvfp4 in, int64_t n, float* y, void* stream) {
  if (n < 0) return DFS_E_INVALID;
  if (n == 0) return DFS_OK;
  if (!y) return DFS_E_INVALID;
  DFS_TRY(check_nvfp4(in));
  DFS_HIP(launch_nvfp4_decode(in, n, y, (hipStream_t)stream));
  return DFS_OK;
}

// ------------------------------------------------------------------ producer steps

dfs_status dict_gram_inverse_workspace_size(const dfs_dict* D, size_t* bytes) {
  if (!bytes || !D) return DFS_E_INVALID;
  if (D->d_in <= 0 || D->k <= 0) return DFS_E_INVALID;
  if (D->k > kMaxProducerK) return DFS_E_RANGE;
  if (D->dtype != DFS_F16 && D->dtype != DFS_F32) return DFS_E_UNSUPPORTED;
  *bytes = gram_ws_bytes(D);
  return DFS_OK;
}

dfs_status dict_gram_inverse(const dfs_dict* D, const float* S, int64_t lds, float lambda, float* P,
                             int64_t ldp, void* ws, size_t ws_bytes, void* stream) {
  if (!D || !S || !P) return DFS_E_INVALID;
  if (D->d_in <= 0 || D->k <= 0 || !D->data) return DFS_E_INVALID;
  if (D->k > kMaxProducerK) return DFS_E_RANGE;
  if (D->dtype != DFS_F16 && D->dtype != DFS_F32) return DFS_E_UNSUPPORTED;
  if (D->ldd < D->d_in || lds < D->d_in || ldp < D->k) return DFS_E_INVALID;
  if (!(lambda >= 0.0f) || !(lambda < __builtin_inff())) return DFS_E_INVALID;
  if (!ws || ws_bytes < gram_ws_bytes(D)) return DFS_E_WORKSPACE;
  if (!aligned16(ws)) return DFS_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const int d_in = D->d_in, k = D->k;
  char* w = (char*)ws;
  void* inv_ws = w;
  w += spd_inverse_ws_bytes(k);
  float* U = (float*)w;
  w += round256((size_t)k * d_in * 4);
  const float* Dt = (const float*)D->data;
  int64_t ldd = D->ldd;
  if (D->dtype == DFS_F16) {
    float* Df = (float*)w;
    DFS_HIP(launch_atoms_to_f32((const _Float16*)D->data, D->ldd, d_in, k, Df, s));
    Dt = Df;
    ldd = d_in;
  }
  // U = D^T S (S symmetric: S^T = S), then K = U D + lambda I into P, then P = K^-1
  DFS_HIP(launch_gemm_nt_f32(Dt, ldd, S, lds, U, d_in, k, d_in, d_in, 1.0f, 0.0f, 0.0f, s));
  DFS_HIP(launch_gemm_nt_f32(U, d_in, Dt, ldd, P, ldp, k, k, d_in, 1.0f, 0.0f, lambda, s));
  DFS_HIP(launch_spd_inverse(P, ldp, k, inv_ws, s));
  return DFS_OK;
}

dfs_status dict_obs_prune(int32_t k, int32_t d_out, const float* C, int64_t ldc, const float* P,
                          int64_t ldp, int32_t n_prune, float* C_out, int64_t ldo, uint8_t* keep,
                          int64_t ldkeep, void* stream) {
  if (!C || !P || !C_out || !keep) return DFS_E_INVALID;
  if (k <= 0 || d_out <= 0 || n_prune < 0 || n_prune > k) return DFS_E_INVALID;
  if (k > kMaxProducerK) return DFS_E_RANGE;
  if (ldc < d_out || ldo < d_out || ldkeep < d_out || ldp < k) return DFS_E_INVALID;
  DFS_HIP(launch_obs_prune(C, ldc, P, ldp, k, d_out, n_prune, C_out, ldo, keep, ldkeep,
                           (hipStream_t)stream));
  return DFS_OK;
}

dfs_status dict_refit_workspace_size(int32_t d_in, int32_t k, size_t* bytes) {
  if (!bytes || d_in <= 0 || k <= 0) return DFS_E_INVALID;
  if (k > kMaxProducerK) return DFS_E_RANGE;
  *bytes = refit_ws_bytes(d_in, k);
  return DFS_OK;
}

dfs_status dict_refit(int32_t d_in, int32_t N, int32_t k, const float* W, int64_t ldw,
                      const float* C, int64_t ldc, float lambda, float* Dt, int64_t ldd, void* ws,
                      size_t ws_bytes, void* stream) {
  if (!W || !C || !Dt) return DFS_E_INVALID;
  if (d_in <= 0 || N <= 0 || k <= 0) return DFS_E_INVALID;
  if (k > kMaxProducerK) return DFS_E_RANGE;
  if (ldw < N || ldc < N || ldd < d_in) return DFS_E_INVALID;
  if (!(lambda >= 0.0f) || !(lambda < __builtin_inff())) return DFS_E_INVALID;
  if (!ws || ws_bytes < refit_ws_bytes(d_in, k)) return DFS_E_WORKSPACE;
  if (!aligned16(ws)) return DFS_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  char* w = (char*)ws;
  void* inv_ws = w;
  w += spd_inverse_ws_bytes(k);
  float* G = (float*)w;
  w += round256((size_t)k * k * 4);
  float* R = (float*)w;
  // G = C C^T + lambda I, R = W C^T (d_in x k), G <- G^-1, D^T = G^-1 R^T
  DFS_HIP(launch_gemm_nt_f32(C, ldc, C, ldc, G, k, k, k, N, 1.0f, 0.0f, lambda, s));
  DFS_HIP(launch_gemm_nt_f32(W, ldw, C, ldc, R, k, d_in, k, N, 1.0f, 0.0f, 0.0f, s));
  DFS_HIP(launch_spd_inverse(G, k, k, inv_ws, s));
  DFS_HIP(launch_gemm_nt_f32(G, k, R, k, Dt, ldd, k, d_in, k, 1.0f, 0.0f, 0.0f, s));
  return DFS_OK;
}

// ------------------------------------------------------------------ forward

dfs_status dict_xd_workspace_size(int32_t n_layers, int32_t T, const dfs_dict* D, size_t* bytes) {
  if (!bytes || n_layers <= 0 || T < 0) return DFS_E_INVALID;
  if (n_layers > kMaxLayers) return DFS_E_RANGE;
  DFS_TRY(check_dict(D));
  *bytes = xd_ws_bytes((int64_t)n_layers * T, DFS_F16, D);
  return DFS_OK;
}

dfs_status dict_workspace_size(int32_t n_layers, int32_t T, const dfs_dict* D, const dfs_csc* C,
                               size_t* bytes) {
  if (!bytes || n_layers <= 0 || T < 0) return DFS_E_INVALID;
  if (n_layers > kMaxLayers) return DFS_E_RANGE;
  DFS_TRY(check_dict(D));
  if (!C || C->k != D->k || C->d_out <= 0) return DFS_E_INVALID;
  *bytes = fwd_ws_bytes((int64_t)n_layers * T, D);
  return DFS_OK;
}

dfs_status dict_xd_forward(int32_t n_layers, const void* const* X, int32_t xdt, int32_t T,
                           int64_t ldx, const dfs_dict* D, void* Z, int32_t zdt, void* ws,
                           size_t ws_bytes, void* stream) {
  if (n_layers <= 0 || T < 0 || !X) return DFS_E_INVALID;
  if (n_layers > kMaxLayers) return DFS_E_RANGE;
  DFS_TRY(check_dict(D));
  if (zdt != DFS_F16 && zdt != DFS_F32) return DFS_E_UNSUPPORTED;
  if (!is_act_dtype(xdt)) return DFS_E_UNSUPPORTED;
  if (T == 0) return DFS_OK;
  DFS_TRY(check_x(X, n_layers, xdt, ldx, D->d_in));
  if (!Z) return DFS_E_INVALID;
  if (!aligned16(Z)) return DFS_E_ALIGN;
  const size_t need = xd_ws_bytes((int64_t)n_layers * T, xdt, D);
  if (need && (!ws || ws_bytes < need)) return DFS_E_WORKSPACE;
  if (need && !aligned16(ws)) return DFS_E_ALIGN;
  return run_xd(n_layers, X, xdt, T, ldx, D, Z, zdt, ws, (hipStream_t)stream);
}

dfs_status dict_zc_forward(int32_t n_layers, const void* Z, int32_t zdt, int32_t T,
                           const dfs_csc* C, void* const* Y, int32_t ydt, int64_t ldy,
                           void* stream) {
  if (n_layers <= 0 || T < 0 || !C || !Y) return DFS_E_INVALID;
  if (n_layers > kMaxLayers) return DFS_E_RANGE;
  if (zdt != DFS_F16 && zdt != DFS_F32) return DFS_E_UNSUPPORTED;
  if (C[0].k <= 0) return DFS_E_INVALID;
  if (C[0].k > kMaxKForward) return DFS_E_RANGE;
  for (int i = 0; i < n_layers; ++i) {
    DFS_TRY(check_csc(&C[i], C[0].k, C[0].d_out));
    if (C[i].dtype != C[0].dtype || C[i].block_rows != C[0].block_rows)
      return DFS_E_UNSUPPORTED;
  }
  if (!is_act_dtype(ydt)) return DFS_E_UNSUPPORTED;
  if (T == 0) return DFS_OK;
  DFS_TRY(check_y(Y, n_layers, ydt, ldy, C[0].d_out));
  if (!Z) return DFS_E_INVALID;
  if (!aligned16(Z)) return DFS_E_ALIGN;  // Z rows are staged in 16-byte pieces
  return run_zc(n_layers, Z, zdt, T, C, Y, ydt, ldy, (hipStream_t)stream);
}

}  // extern "C"

namespace {
// Every argument of a group forward, checked before anything is launched.
dfs_status check_group(int32_t n_layers, const void* const* X, int32_t xdt, int32_t T,
                       int64_t ldx, const dfs_dict* D, const dfs_csc* C, void* const* Y,
                       int32_t ydt, int64_t ldy) {
  if (n_layers <= 0 || T < 0 || !X || !C || !Y) return DFS_E_INVALID;
  if (n_layers > kMaxLayers) return DFS_E_RANGE;
  DFS_TRY(check_dict(D));
  for (int i = 0; i < n_layers; ++i) {
    DFS_TRY(check_csc(&C[i], D->k, C[0].d_out));
    if (C[i].dtype != C[0].dtype || C[i].block_rows != C[0].block_rows)
      return DFS_E_UNSUPPORTED;
  }
  if (!is_act_dtype(xdt) || !is_act_dtype(ydt)) return DFS_E_UNSUPPORTED;
  if (T == 0) return DFS_OK;  // no rows: the activation pointers may be null
  DFS_TRY(check_x(X, n_layers, xdt, ldx, D->d_in));
  DFS_TRY(check_y(Y, n_layers, ydt, ldy, C[0].d_out));
  return DFS_OK;
}

constexpr int32_t kMaxMultiDicts = 8;

// ---- the workspace of dict_group_forward_noalloc: a file-scope device
// array, one copy per GPU the library runs on, held until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is ever passed on.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device
bool g_scratch_zeroed[kMaxDevices];

// Zeroes the control block and the tagged region (the part of a forward
// workspace that must start at zero) without a memset, so that a call under
// graph capture records a kernel node.
__global__ void zero_words(u4* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = u4{0u, 0u, 0u, 0u};
}

// Device address of the current device's `scratch`; on the first call for a
// device, also enqueues on `s` the zeroing of the part that must start at 0.
dfs_status scratch_of_current_device(void** out, hipStream_t s) {
  int dev = -1;
  DFS_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return DFS_E_RANGE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    DFS_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return DFS_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  if (!g_scratch_zeroed[dev]) {
    const size_t zero_bytes = kCtrlBytes + round256(fused_z_words_bytes(kMaxKForward));
    hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, s, (u4*)g_scratch_ptr[dev],
                       (int64_t)(zero_bytes / 16));
    DFS_HIP(hipGetLastError());
    g_scratch_zeroed[dev] = true;
  }
  *out = g_scratch_ptr[dev];
  return DFS_OK;
}
}  // namespace

extern "C" {

dfs_status dict_group_forward(int32_t n_layers, const void* const* X, int32_t xdt, int32_t T,
                              int64_t ldx, const dfs_dict* D, const dfs_csc* C, void* const* Y,
                              int32_t ydt, int64_t ldy, void* ws, size_t ws_bytes,
                              void* stream) {
  DFS_TRY(check_group(n_layers, X, xdt, T, ldx, D, C, Y, ydt, ldy));
  if (T == 0) return DFS_OK;
  const int64_t rows = (int64_t)n_layers * T;
  const bool mfma = mfma_path(rows, xdt, D);
  const int32_t zdt = mfma ? DFS_F16 : DFS_F32;
  const FwdLayout w = fwd_layout(rows, xdt, D);
  if (!ws || ws_bytes < w.total) return DFS_E_WORKSPACE;
  if (!aligned16(ws)) return DFS_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* ctrl = (uint32_t*)ws;
  uint8_t* tagged = (uint8_t*)ws + kCtrlBytes;
  void* Z = (char*)ws + kCtrlBytes + w.zwords;
  void* xws = (char*)Z + w.zplain;
  if (!mfma && fused_allowed()) {
    XdLaunch xa = make_xd(n_layers, X, xdt, T, ldx, D, Z, zdt);
    ZcLaunch za = make_zc(n_layers, Z, zdt, T, C, Y, ydt, ldy);
    if (fused_decode_supported(xa, za)) {
      DFS_HIP(launch_fused_decode(xa, za, tagged, ctrl, s));
      return DFS_OK;
    }
  }
  DFS_TRY(run_xd(n_layers, X, xdt, T, ldx, D, Z, zdt, xws, s));
  return run_zc(n_layers, Z, zdt, T, C, Y, ydt, ldy, s);
}

dfs_status dict_multi_workspace_size(int32_t n_dicts, int32_t n_layers, int32_t T,
                                     const dfs_dict* D, const dfs_csc* C, size_t* bytes) {
  if (!bytes || !D || !C || n_dicts <= 0) return DFS_E_INVALID;
  if (n_dicts > kMaxMultiDicts) return DFS_E_RANGE;
  // one group at a time; the tagged Z words of the one-launch decode hold
  // every (dictionary, layer) unit it runs
  return dict_workspace_size(n_layers, T, D, C, bytes);
}

dfs_status dict_multi_forward(int32_t n_dicts, int32_t n_layers, const void* const* X,
                              int32_t xdt, int32_t T, int64_t ldx, const dfs_dict* D,
                              const dfs_csc* C, void* const* Y, int32_t ydt, int64_t ldy,
                              void* ws, size_t ws_bytes, void* stream) {
  if (n_dicts <= 0 || !D || !C || !Y) return DFS_E_INVALID;
  if (n_dicts > kMaxMultiDicts) return DFS_E_RANGE;
  // every group valid, one shape and type for all dictionaries and for all
  // coefficient matrices, before anything is launched
  for (int d = 0; d < n_dicts; ++d) {
    DFS_TRY(check_group(n_layers, X, xdt, T, ldx, &D[d], C + (size_t)d * n_layers,
                        Y + (size_t)d * n_layers, ydt, ldy));
    if (D[d].d_in != D[0].d_in || D[d].k != D[0].k || D[d].dtype != D[0].dtype ||
        D[d].ldd != D[0].ldd)
      return DFS_E_INVALID;
    const dfs_csc& c = C[(size_t)d * n_layers];
    if (c.d_out != C[0].d_out || c.dtype != C[0].dtype || c.block_rows != C[0].block_rows)
      return DFS_E_INVALID;
  }
  if (T == 0) return DFS_OK;
  size_t need = 0;
  DFS_TRY(dict_multi_workspace_size(n_dicts, n_layers, T, D, C, &need));
  if (!ws || ws_bytes < need) return DFS_E_WORKSPACE;
  if (!aligned16(ws)) return DFS_E_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  // the launch structs hold at most kFusedMaxLayers X rows and
  // kFusedMaxUnits (dictionary, layer) units: checked before they are filled
  if (n_dicts > 1 && n_dicts <= kFusedMaxDicts && n_layers <= kFusedMaxLayers &&
      n_dicts * n_layers <= kFusedMaxUnits && fused_allowed()) {
    uint32_t* ctrl = (uint32_t*)ws;
    uint8_t* tagged = (uint8_t*)ws + kCtrlBytes;
    void* Z = (char*)ws + kCtrlBytes + round256(fused_z_words_bytes(D[0].k));
    XdLaunch xa = make_xd(n_layers, X, xdt, T, ldx, &D[0], Z, DFS_F32);
    xa.n_dicts = n_dicts;
    for (int d = 1; d < n_dicts; ++d)
      xa.more[d - 1] = {D[d].data, D[d].nv.codes, D[d].nv.scales, D[d].nv.tensor_scale};
    ZcLaunch za = make_zc(n_dicts * n_layers, Z, DFS_F32, T, C, Y, ydt, ldy);
    if (fused_decode_supported(xa, za)) {
      DFS_HIP(launch_fused_decode(xa, za, tagged, ctrl, s));
      return DFS_OK;
    }
  }
  for (int d = 0; d < n_dicts; ++d)
    DFS_TRY(dict_group_forward(n_layers, X, xdt, T, ldx, &D[d], C + (size_t)d * n_layers,
                               Y + (size_t)d * n_layers, ydt, ldy, ws, ws_bytes, stream));
  return DFS_OK;
}

dfs_status dict_group_forward_noalloc(int32_t n_layers, const void* const* X, int32_t xdt,
                                      int32_t T, int64_t ldx, const dfs_dict* D, const dfs_csc* C,
                                      void* const* Y, int32_t ydt, int64_t ldy, void* stream) {
  DFS_TRY(check_group(n_layers, X, xdt, T, ldx, D, C, Y, ydt, ldy));
  if (T == 0) return DFS_OK;
  if (fwd_layout((int64_t)n_layers * T, xdt, D).total > kScratchBytes) return DFS_E_WORKSPACE;
  void* ws = nullptr;
  DFS_TRY(scratch_of_current_device(&ws, (hipStream_t)stream));
  return dict_group_forward(n_layers, X, xdt, T, ldx, D, C, Y, ydt, ldy, ws, kScratchBytes,
                            stream);
}

dfs_status dict_proj_forward(const void* X, int32_t xdt, int32_t T, int64_t ldx, const dfs_dict* D,
                             const dfs_csc* C, void* Y, int32_t ydt, int64_t ldy, void* ws,
                             size_t ws_bytes, void* stream) {
  const void* xs[1] = {X};
  void* ys[1] = {Y};
  return dict_group_forward(1, xs, xdt, T, ldx, D, C, ys, ydt, ldy, ws, ws_bytes, stream);
}

}  // extern "C"
