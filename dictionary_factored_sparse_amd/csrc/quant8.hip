// quant8.hip -- 8-bit coefficient codes (E4M3 or INT8), one fp32 scale per
// column of C.
//
// The mixed-precision rows of Table 4 on the paper's figures and tables page
// ("DictLLM: Post-training Compression of Large Language Model with
// Dictionary Kernels") pair an NVFP4 dictionary with FP8 or INT8
// coefficients.  The pages do not give the scaling of those codes; this
// library scales each column of C on its own (a CSC column is contiguous, and
// the forward kernels apply the scale once to the column's finished dot
// product):
//   amax_j = max |v| over column j;  s_j = amax_j / 448 (E4M3) or
//   amax_j / 127 (INT8), or 1 if that quotient is 0;
//   code = E4M3 nearest to |v / s_j| with v's sign bit, or the integer
//   nearest to v / s_j clamped to [-127, 127]; ties to even.
// Each step is one correctly rounded fp32 operation (this file is compiled
// without FMA contraction; fp32 division is correctly rounded).
// One wave per column: the column's values are read with unit stride, twice
// (max, then codes), and the codes are written with unit stride.
#include "dfs_internal.hpp"

namespace dfs {
namespace {

constexpr int kThreads = 256;
constexpr int kColsPerBlock = kThreads / kWave;

__device__ __forceinline__ float load_val(const void* vals, int dt, int64_t p) {
  return dt == DFS_F32 ? ((const float*)vals)[p] : (float)((const _Float16*)vals)[p];
}

// [s, e) of column j, clamped to [0, nnz] so a malformed colptr cannot index
// out of bounds.
__device__ __forceinline__ void col_range(const int32_t* colptr, int64_t nnz, int j, int64_t* s,
                                          int64_t* e) {
  *s = min<int64_t>(max<int64_t>(colptr[j], 0), nnz);
  *e = min<int64_t>(max<int64_t>(colptr[j + 1], *s), nnz);
}

// Per column: the bits of max |v| (for non-negative floats bit order is value
// order) and whether any value is NaN or infinite.
__global__ __launch_bounds__(kThreads) void q8_amax_kernel(const void* vals, int dt,
                                                           const int32_t* colptr, int64_t nnz,
                                                           int d_out, uint32_t* amax,
                                                           uint32_t* bad) {
  const int j = blockIdx.x * kColsPerBlock + (int)threadIdx.x / kWave;
  if (j >= d_out) return;  // a whole wave leaves together
  const int lane = threadIdx.x & (kWave - 1);
  int64_t s, e;
  col_range(colptr, nnz, j, &s, &e);
  uint32_t m = 0, nf = 0;
  for (int64_t p = s + lane; p < e; p += kWave) {
    const uint32_t b = __float_as_uint(load_val(vals, dt, p)) & 0x7FFFFFFFu;
    nf |= b >= 0x7F800000u ? 1u : 0u;
    m = b > m ? b : m;
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const uint32_t om = (uint32_t)__shfl_xor((int)m, off, kWave);
    m = om > m ? om : m;
    nf |= (uint32_t)__shfl_xor((int)nf, off, kWave);
  }
  if (lane == 0) {
    amax[j] = m;
    if (nf) atomicOr(bad, 1u);
  }
}

template <int KIND>
__global__ __launch_bounds__(kThreads) void q8_encode_kernel(const void* vals, int dt,
                                                             const int32_t* colptr, int64_t nnz,
                                                             int d_out, const uint32_t* amax,
                                                             uint8_t* codes, float* col_scale) {
  const int j = blockIdx.x * kColsPerBlock + (int)threadIdx.x / kWave;
  if (j >= d_out) return;
  const int lane = threadIdx.x & (kWave - 1);
  const float qmax = KIND == DFS_FP8 ? 448.0f : 127.0f;
  float sc = __uint_as_float(amax[j]) / qmax;
  if (sc == 0.0f) sc = 1.0f;
  if (lane == 0) col_scale[j] = sc;
  int64_t s, e;
  col_range(colptr, nnz, j, &s, &e);
  for (int64_t p = s + lane; p < e; p += kWave) {
    const float v = load_val(vals, dt, p);
    const float q = v / sc;
    uint32_t code;
    if constexpr (KIND == DFS_FP8) {
      code = e4m3_rne_satfinite(fabsf(q)) | ((__float_as_uint(v) >> 24) & 0x80u);
    } else {
      const float r = fminf(fmaxf(__builtin_rintf(q), -127.0f), 127.0f);
      code = (uint32_t)(uint8_t)(int8_t)(int)r;
    }
    codes[p] = (uint8_t)code;
  }
}

}  // namespace

size_t quant8_ws_bytes(int32_t d_out) { return 256 + ((size_t)d_out * 4 + 255) / 256 * 256; }

hipError_t launch_quant8_amax(const void* vals, int32_t dt, const int32_t* colptr, int64_t nnz,
                              int32_t d_out, void* ws, hipStream_t s) {
  uint32_t* bad = (uint32_t*)ws;
  uint32_t* amax = (uint32_t*)((char*)ws + 256);
  hipError_t err = hipMemsetAsync(bad, 0, 4, s);
  if (err != hipSuccess) return err;
  const int blocks = (d_out + kColsPerBlock - 1) / kColsPerBlock;
  hipLaunchKernelGGL(q8_amax_kernel, dim3(blocks), dim3(kThreads), 0, s, vals, (int)dt, colptr,
                     nnz, (int)d_out, amax, bad);
  return hipGetLastError();
}

hipError_t launch_quant8_encode(const void* vals, int32_t dt, const int32_t* colptr, int64_t nnz,
                                int32_t d_out, int32_t kind, const void* ws, uint8_t* codes,
                                float* col_scale, hipStream_t s) {
  const uint32_t* amax = (const uint32_t*)((const char*)ws + 256);
  const int blocks = (d_out + kColsPerBlock - 1) / kColsPerBlock;
  if (kind == DFS_FP8)
    hipLaunchKernelGGL(q8_encode_kernel<DFS_FP8>, dim3(blocks), dim3(kThreads), 0, s, vals,
                       (int)dt, colptr, nnz, (int)d_out, amax, codes, col_scale);
  else
    hipLaunchKernelGGL(q8_encode_kernel<DFS_INT8>, dim3(blocks), dim3(kThreads), 0, s, vals,
                       (int)dt, colptr, nnz, (int)d_out, amax, codes, col_scale);
  return hipGetLastError();
}

}  // namespace dfs
