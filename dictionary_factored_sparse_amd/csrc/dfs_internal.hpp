// dfs_internal.hpp -- device helpers and kernel-launcher interfaces shared by
// the translation units of libdictfs (the HIP path only).
//
// Target: gfx950 (CDNA4), wave64.  Nothing here is used by the CPU oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dictfs.h"

namespace dfs {

constexpr int kWave = 64;
constexpr int kMaxLayers = 16;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ DPP
// Cross-lane moves inside a 16-lane DPP row.  Controls: quad_perm [1,0,3,2]
// = 0xB1, quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141,
// row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets the sum.
// The combination order is fixed, so results are run-to-run identical.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

// Sum over the whole wave; every lane gets the sum.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16, kWave);
  v += __shfl_xor(v, 32, kWave);
  return v;
}

// ------------------------------------------------------------------ formats
// E4M3 (bias 7, no infinities) code -> fp32, from the format definition.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e == 0 ? (float)m * 0x1p-9f : __builtin_ldexpf((float)(8u + m), (int)e - 10);
  return (c & 0x80u) ? -mag : mag;
}

// Nearest E4M3 code for s >= 0 (finite), ties to even, saturating at 448
// (the NVFP4 block scales and the FP8 coefficient codes).
__device__ __forceinline__ uint32_t e4m3_rne_satfinite(float s) {
  if (s >= 448.0f) return 0x7Eu;
  const uint32_t b = __float_as_uint(s);
  const int e = (int)(b >> 23) - 127;
  if (e < -6) {
    // subnormal range of E4M3 (and fp32 subnormals): multiples of 2^-9;
    // the scaling by 2^9 is exact and rintf rounds half to even.  A result
    // of 8 is the smallest normal, code 0x08.
    return (uint32_t)__builtin_rintf(s * 512.0f);
  }
  const uint32_t mant = b & 0x7FFFFFu;
  const uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
  uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1;  // may carry
  return code > 0x7Eu ? 0x7Eu : code;
}

// Two E2M1 codes (byte SEL of `word`: low nibble -> .x, high nibble -> .y)
// to f16 / f32, unscaled: the hardware conversion with scale 1.0 is exact
// because every E2M1 value is an f16 value.
template <int SEL>
__device__ __forceinline__ h2 e2m1x2_h2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, SEL);
}
template <int SEL>
__device__ __forceinline__ f2 e2m1x2_f2(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

__device__ __forceinline__ float h2f(_Float16 h) { return (float)h; }

// View of a pointer in the global address space.  Loads through it are
// global_load (vector-memory counter only); through a generic pointer whose
// origin the compiler cannot see (e.g. read back from LDS) they would be
// flat_load, which also holds the LDS counter.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gptr(const T* p) {
  return (const __attribute__((address_space(1))) T*)p;
}
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gptr_w(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// 16-byte global load through the vector path.
template <typename T>
__device__ __forceinline__ T ld16(const void* p) {
  return *gptr(reinterpret_cast<const T*>(p));
}

// ------------------------------------------------------------------ launches
// Rows of the stacked X: row r = l*T + t is token t of layer l.
struct XdLaunch {
  const void* X[kMaxLayers];
  int32_t n_layers, T;
  int64_t ldx;
  int32_t xdt;
  int32_t d_in, k;
  int32_t ddt;
  const void* D;        // f16 / f32 atom-major, or f16 expansion for MFMA
  int64_t ldd;
  const uint8_t* dcodes;
  const uint8_t* dscales;
  const float* dts;
  void* Z;              // (n_layers*T) x k row-major
  int32_t zdt;
  float* zpart;         // MFMA path with split K: [ksplit][rows][k] fp32 partials
  // Further dictionaries over the same X rows (the one-launch decode of
  // several projections that share their input, e.g. q, k and v): same
  // d_in, k, dtype and ldd as D; 0 means one dictionary.
  int32_t n_dicts;
  struct {
    const void* D;
    const uint8_t* dcodes;
    const uint8_t* dscales;
    const float* dts;
  } more[2];
};

struct ZcLaunch {
  const void* Z;        // (n_layers*T) x k row-major
  int32_t zdt;
  int32_t n_layers, T, k, d_out;
  int32_t vdt;
  const int32_t* colptr[kMaxLayers];
  int64_t nnz[kMaxLayers];
  const uint16_t* rowidx[kMaxLayers];
  const void* vals[kMaxLayers];       // f16/f32 values, or NVFP4 codes
  const uint8_t* vscales[kMaxLayers]; // NVFP4 block scales
  const float* vts[kMaxLayers];       // NVFP4 tensor scale, or FP8/INT8 column scales
  void* Y[kMaxLayers];
  int32_t ydt;
  int64_t ldy;
  int32_t block_rows;  // 0, or 8: colptr counts blocks of 8 atoms, rowidx holds block indices
};

// Rows at or below which X.D runs on VALU dot products instead of MFMA.
constexpr int kGemvMaxRows = 16;

// One-launch decode of a group (T == 1, up to 4 layers), or of up to 3
// dictionaries over the same X rows (up to 2 layers; the ZcLaunch then holds
// one unit per (dictionary, layer), dictionary-major).
constexpr int kFusedMaxLayers = 4;
constexpr int kFusedMaxDicts = 3;
constexpr int kFusedMaxUnits = 8;
static_assert(kFusedMaxUnits <= kMaxLayers, "units fit the launch structs");
constexpr int kCtrlBlockBytes = 4096;   // forward workspace control block
constexpr int kMaxFusedGroups = 1024;   // workgroups of the one-launch decode (one per CU)
bool fused_decode_supported(const XdLaunch& xd, const ZcLaunch& zc);
// Bytes of the tagged region of the one-launch decode (one epoch word per
// workgroup, then kFusedMaxUnits rows of k tagged Z words), kept at a fixed
// place after the control block: zero before first use, then kept by the
// calls (no other path writes there).
size_t fused_z_words_bytes(int32_t k);
hipError_t launch_fused_decode(const XdLaunch& xd, const ZcLaunch& zc, uint8_t* tagged,
                               uint32_t* ctrl, hipStream_t s);

hipError_t launch_gemv_xd(const XdLaunch& a, hipStream_t s);
hipError_t launch_gemm_xd_mfma(const XdLaunch& a, hipStream_t s);
// Slices of K the MFMA GEMM splits into for rows x n_atoms x d_in (1 = no
// split); with more than one, it needs ksplit * rows * n_atoms fp32 of
// workspace for the partial products.
int gemm_split_k(int64_t rows, int n_atoms, int d_in);
hipError_t launch_nvfp4_to_f16(const uint8_t* codes, const uint8_t* scales, const float* ts,
                               int64_t n, _Float16* out, hipStream_t s);
hipError_t launch_spmv_csc(const ZcLaunch& a, hipStream_t s);
// Tokens per LDS pass of the SpMV (power of two, <= 16); *half: the tile is
// f16 (never for fp32 Z).
int spmv_token_tile(int T, int k, bool fp32_z, bool* half);
hipError_t launch_spmm_csc(const ZcLaunch& a, hipStream_t s);
// Tokens per workgroup tile of the SpMM (32, 16, 8 or 4; f16 Z tile <= 128 KiB).
int spmm_token_tile(int k);

// CSC packing
size_t pack_csc_ws_bytes(int32_t k, int32_t d_out);
// block_rows: 0 (one entry per stored element) or 8 (blocks of 8 atoms)
hipError_t launch_pack_csc_count(const void* C, int32_t dtype, int32_t k, int32_t d_out,
                                 int64_t ldc, int32_t* colptr, void* ws, hipStream_t s,
                                 int block_rows = 0);
hipError_t launch_pack_csc_scatter(const void* C, int32_t dtype, int32_t k, int32_t d_out,
                                   int64_t ldc, uint16_t* rowidx, void* vals, const void* ws,
                                   hipStream_t s, int block_rows = 0);
// Y_l = Z_l C_l for block-structured C: T <= 16 tokens per layer (SpMV),
// and any T with the Z tile staged as f16 (SpMM)
hipError_t launch_spmv_bcsc(const ZcLaunch& a, hipStream_t s);
hipError_t launch_spmm_bcsc(const ZcLaunch& a, hipStream_t s);

// 8-bit coefficient codes (FP8 / INT8), one scale per column
size_t quant8_ws_bytes(int32_t d_out);
hipError_t launch_quant8_amax(const void* vals, int32_t dt, const int32_t* colptr, int64_t nnz,
                              int32_t d_out, void* ws, hipStream_t s);
hipError_t launch_quant8_encode(const void* vals, int32_t dt, const int32_t* colptr, int64_t nnz,
                                int32_t d_out, int32_t kind, const void* ws, uint8_t* codes,
                                float* col_scale, hipStream_t s);

// producer steps (fp32): C = alpha A B^T + beta C (+ diag on m == n), the
// in-place inverse of a symmetric positive definite matrix, coefficient
// pruning with a fixed inverse
hipError_t launch_gemm_nt_f32(const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
                              int64_t ldc, int M, int N, int K, float alpha, float beta, float diag,
                              hipStream_t s);
size_t spd_inverse_ws_bytes(int n);
// matrix-core probe (measurement support)
hipError_t launch_mfma_peak(int32_t blocks, int32_t iters, float* out, hipStream_t s);
hipError_t launch_read_probe(const void* buf, int64_t n16, int32_t blocks, uint32_t* out,
                             hipStream_t s);
hipError_t launch_spd_inverse(float* A, int64_t lda, int n, void* ws, hipStream_t s);
size_t obs_prune_smem(int k);
hipError_t launch_obs_prune(const float* C, int64_t ldc, const float* P, int64_t ldp, int k,
                            int d_out, int n_prune, float* Co, int64_t ldo, uint8_t* keep,
                            int64_t ldkeep, hipStream_t s);
hipError_t launch_atoms_to_f32(const _Float16* D, int64_t ldd, int d_in, int k, float* out,
                               hipStream_t s);

// NVFP4 packing
size_t nvfp4_ws_bytes(int64_t n);
hipError_t launch_nvfp4_amax(const float* x, int64_t n, void* ws, hipStream_t s);
hipError_t launch_nvfp4_encode(const float* x, int64_t n, dfs_nvfp4 out, const void* ws,
                               hipStream_t s);
hipError_t launch_nvfp4_decode(dfs_nvfp4 in, int64_t n, float* y, hipStream_t s);

}  // namespace dfs
