// nvfp4.hip -- NVFP4 quantisation and decoding of fp32 tensors.
//
// NVFP4 stores a 4-bit E2M1 value per element with one 8-bit scale per block
// of sixteen consecutive values ("DictLLM: Shared Dictionaries for
// Post-Training Compression", "From retained values to measured decoding";
// the paper's figures and tables page, Table 4) plus one fp32 tensor scale.
// Recipe (each step one correctly rounded fp32 operation; this file is
// compiled without FMA contraction):
//   ts = amax / 2688, or 1 if that quotient is 0
//   block b: sf = amax_b / (6 * ts); scale code = nearest E4M3 (ties to
//            even, saturating at 448); s = its value; denom = s * ts
//   element: magnitude code = nearest E2M1 to |x / denom| (ties to even,
//            saturating at 6; 0 if denom == 0); sign bit copied from x.
// The E4M3 rounding works on the fp32 bit pattern; the E2M1 rounding
// compares |v| with the midpoints of the value grid, where a tie goes to the
// neighbour with the even code.
#include "dfs_internal.hpp"

namespace dfs {
namespace {

constexpr int kThreads = 256;
constexpr int kAmaxBlocks = 1024;

struct Nv4Ws {
  uint32_t* result;   // [0] amax bits, [1] non-finite flag
  uint32_t* partial;  // [kAmaxBlocks][2]
};

__host__ __device__ inline Nv4Ws carve(void* ws) {
  Nv4Ws w;
  w.result = (uint32_t*)ws;
  w.partial = (uint32_t*)((char*)ws + 256);
  return w;
}

__global__ __launch_bounds__(kThreads) void amax_partial_kernel(const float* x, int64_t n,
                                                                uint32_t* partial) {
  __shared__ uint32_t smax[kThreads], sbad[kThreads];
  uint32_t m = 0, bad = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const uint32_t b = __float_as_uint(x[i]) & 0x7FFFFFFFu;
    bad |= (b >= 0x7F800000u) ? 1u : 0u;  // Inf or NaN
    m = b > m ? b : m;                      // |x| order == bit order
  }
  smax[threadIdx.x] = m;
  sbad[threadIdx.x] = bad;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      smax[threadIdx.x] = max(smax[threadIdx.x], smax[threadIdx.x + w]);
      sbad[threadIdx.x] |= sbad[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    partial[2 * blockIdx.x] = smax[0];
    partial[2 * blockIdx.x + 1] = sbad[0];
  }
}

__global__ __launch_bounds__(kThreads) void amax_final_kernel(const uint32_t* partial, int nb,
                                                              uint32_t* result) {
  __shared__ uint32_t smax[kThreads], sbad[kThreads];
  uint32_t m = 0, bad = 0;
  for (int i = threadIdx.x; i < nb; i += kThreads) {
    m = max(m, partial[2 * i]);
    bad |= partial[2 * i + 1];
  }
  smax[threadIdx.x] = m;
  sbad[threadIdx.x] = bad;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      smax[threadIdx.x] = max(smax[threadIdx.x], smax[threadIdx.x + w]);
      sbad[threadIdx.x] |= sbad[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    result[0] = smax[0];
    result[1] = sbad[0];
  }
}

// Nearest E2M1 magnitude code to a = |v| (ties to even code, saturating at 6).
__device__ __forceinline__ uint32_t e2m1_rne_sat(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
         (uint32_t)(a > 5.0f);
}

__device__ __forceinline__ float tensor_scale(uint32_t amax_bits) {
  const float ts = __uint_as_float(amax_bits) / 2688.0f;
  return ts == 0.0f ? 1.0f : ts;
}

// One thread per 16-element block.
__global__ __launch_bounds__(kThreads) void encode_kernel(const float* x, int64_t n,
                                                          const uint32_t* result, uint8_t* codes,
                                                          uint8_t* scales, float* ts_out) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t lo = b * 16;
  if (lo >= n) return;
  const float ts = tensor_scale(result[0]);
  if (b == 0) *ts_out = ts;
  const int cnt = n - lo < 16 ? (int)(n - lo) : 16;
  float v[16];
  if (cnt == 16 && ((uintptr_t)(x + lo) & 15u) == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f4 t = *reinterpret_cast<const f4*>(x + lo + 4 * q);
      v[4 * q] = t[0]; v[4 * q + 1] = t[1]; v[4 * q + 2] = t[2]; v[4 * q + 3] = t[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = i < cnt ? x[lo + i] : 0.0f;
  }
  float bmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bmax = fmaxf(bmax, fabsf(v[i]));
  const float six_ts = 6.0f * ts;
  const float sf = bmax / six_ts;
  const uint32_t sc = e4m3_rne_satfinite(sf);
  const float s = e4m3_to_f32(sc);
  const float denom = s * ts;
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t mag = denom != 0.0f ? e2m1_rne_sat(fabsf(v[i] / denom)) : 0u;
    c[i] = mag | ((__float_as_uint(v[i]) >> 28) & 8u);
  }
  scales[b] = (uint8_t)sc;
  uint8_t* out = codes + lo / 2;
  if (cnt == 16) {
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w0 |= c[i] << (4 * i);
      w1 |= c[8 + i] << (4 * i);
    }
    *reinterpret_cast<uint32_t*>(out) = w0;
    *reinterpret_cast<uint32_t*>(out + 4) = w1;
  } else {
    for (int i = 0; i < cnt; i += 2) {
      const uint32_t hi = i + 1 < cnt ? c[i + 1] : 0u;
      out[i / 2] = (uint8_t)(c[i] | (hi << 4));
    }
  }
}

// y[i] = (e2m1 * e4m3) * ts: the first product is exact, one rounding after.
__global__ __launch_bounds__(kThreads) void decode_kernel(const uint8_t* codes,
                                                          const uint8_t* scales, const float* ts,
                                                          int64_t n, float* y) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const uint32_t byte = codes[i / 2];
  const uint32_t code = (i & 1) ? (byte >> 4) : (byte & 15u);
  const f2 v = e2m1x2_f2<0>(code);  // low nibble of byte 0
  y[i] = (v[0] * e4m3_to_f32(scales[i / 16])) * (*ts);
}

}  // namespace

size_t nvfp4_ws_bytes(int64_t) { return 256 + (size_t)kAmaxBlocks * 8; }

hipError_t launch_nvfp4_amax(const float* x, int64_t n, void* ws, hipStream_t s) {
  Nv4Ws w = carve(ws);
  int64_t nb = (n + kThreads - 1) / kThreads;
  if (nb > kAmaxBlocks) nb = kAmaxBlocks;
  if (nb < 1) nb = 1;
  hipLaunchKernelGGL(amax_partial_kernel, dim3((unsigned)nb), dim3(kThreads), 0, s, x, n,
                     w.partial);
  hipLaunchKernelGGL(amax_final_kernel, dim3(1), dim3(kThreads), 0, s, w.partial, (int)nb,
                     w.result);
  return hipGetLastError();
}

hipError_t launch_nvfp4_encode(const float* x, int64_t n, dfs_nvfp4 out, const void* ws,
                               hipStream_t s) {
  Nv4Ws w = carve(const_cast<void*>(ws));
  const int64_t blocks16 = (n + 15) / 16;
  const unsigned grid = (unsigned)((blocks16 + kThreads - 1) / kThreads);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(encode_kernel, dim3(grid), dim3(kThreads), 0, s, x, n, w.result, out.codes,
                     out.scales, out.tensor_scale);
  return hipGetLastError();
}

hipError_t launch_nvfp4_decode(dfs_nvfp4 in, int64_t n, float* y, hipStream_t s) {
  const unsigned grid = (unsigned)((n + kThreads - 1) / kThreads);
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_kernel, dim3(grid), dim3(kThreads), 0, s, in.codes, in.scales,
                     in.tensor_scale, n, y);
  return hipGetLastError();
}

}  // namespace dfs
