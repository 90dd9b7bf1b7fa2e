// probes.hip -- measurement support, not a step of the method: the sustained
// rate of the matrix cores on this device, against which the prefill GEMM
// (Z = X D_g on v_mfma_f32_32x32x16_f16) is reported beside the nominal peak,
// and the rate at which it reads HBM, against which the decode (which reads
// every factor byte once) is reported beside the nominal 8 TB/s.
//
// Every wave runs `iters` rounds of kProbeAcc independent MFMAs on register
// operands (each accumulator is reused kProbeAcc MFMAs later, well past the
// instruction's latency), so the only limit is the issue rate of the matrix
// cores at the clock the device holds under that load.  One float per
// thread is written at the end so the work cannot be dropped.
#include "dfs_internal.hpp"

namespace dfs {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeAcc = 8;

__global__ __launch_bounds__(kProbeThreads, 2) void mfma_peak_kernel(int iters, float* out) {
  const int lane = threadIdx.x & (kWave - 1);
  // operands with exact products (quarters times one), so every round adds
  // the same exactly representable block
  h8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)((float)((lane + i) & 3) * 0.25f);
    b[i] = (_Float16)1.0f;
  }
  f16v acc[kProbeAcc];
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[j][v];
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

// Reads n16 16-byte words: thread t of a grid of G threads reads words t,
// t + G, t + 2G, ... (each step of the grid is one contiguous run of 16 G
// bytes) and writes the XOR of its words' four dwords to out[t].
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u4* p, int64_t n16,
                                                                   uint32_t* out) {
  const int64_t t = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  const int64_t step = (int64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  for (int64_t i = t; i < n16; i += step) {
    const u4 v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[t] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* buf, int64_t n16, int32_t blocks, uint32_t* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                     (const u4*)buf, n16, out);
  return hipGetLastError();
}

hipError_t launch_mfma_peak(int32_t blocks, int32_t iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0, s,
                     (int)iters, out);
  return hipGetLastError();
}

}  // namespace dfs
