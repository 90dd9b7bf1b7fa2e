// gemm_xd.hip -- Z = X D_g on MFMA for many stacked rows (prefill).
//
// First half of the factored projection ("DictLLM: Shared Dictionaries for
// Post-Training Compression", Eq. (1): Z_l = X_l D_g) when the group brings
// enough rows (n_layers * T > 16) that the dense contraction, not the
// dictionary's bytes, sets the time (same review, "From retained values to
// measured decoding": at larger batch or prefill the multiply-adds dominate).
//
// C[M x N] = A[M x K] * B[K x N] with A = stacked X rows (row-major, K = d_in
// contiguous; row l*T + t read from layer l's pointer), B = D_g stored
// atom-major (each of the N = k atoms has its K elements contiguous), f16
// operands, fp32 accumulation in v_mfma_f32_32x32x16_f16.
//
// Tiling: 128 x 128 output tile per workgroup of 4 waves (2 x 2), each wave
// 64 x 64 = 2 x 2 MFMA blocks; K advances 64 at a time through two LDS
// buffers (rows padded by 16 bytes so the 16-byte fragment reads of 16
// consecutive rows fall in distinct banks).  The next K tile is fetched into
// registers while the current one is multiplied.
#include "dfs_internal.hpp"

namespace dfs {
namespace {

constexpr int kThreads = 256;
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;               // padded row length (halfs)
constexpr int kChunks = BM * BK / 8;      // 16-byte chunks per operand tile
constexpr int kPerThread = kChunks / kThreads;

template <int ZT>
__global__ __launch_bounds__(kThreads) void gemm_xd_kernel(XdLaunch a) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][BN * LDK];

  const int M = a.n_layers * a.T, N = a.k, K = a.d_in;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  // Row pointers of the chunks this thread loads (fixed across K tiles).
  const _Float16* arow[kPerThread];
  const _Float16* brow[kPerThread];
  int kc[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int c = tid + i * kThreads;
    const int r = c / (BK / 8);
    kc[i] = (c % (BK / 8)) * 8;
    const int m = m0 + r;
    arow[i] = nullptr;
    if (m < M) {
      const int l = m / a.T, t = m - l * a.T;
      arow[i] = (const _Float16*)a.X[l] + (int64_t)t * a.ldx;
    }
    const int n = n0 + r;
    brow[i] = n < N ? (const _Float16*)a.D + (int64_t)n * a.ldd : nullptr;
  }

  u4 ra[kPerThread], rb[kPerThread];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int kk = k0 + kc[i];
      ra[i] = (arow[i] && kk < K) ? ld16<u4>(arow[i] + kk) : u4{0u, 0u, 0u, 0u};
      rb[i] = (brow[i] && kk < K) ? ld16<u4>(brow[i] + kk) : u4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int c = tid + i * kThreads;
      const int r = c / (BK / 8);
      *reinterpret_cast<u4*>(&As[buf][r * LDK + kc[i]]) = ra[i];
      *reinterpret_cast<u4*>(&Bs[buf][r * LDK + kc[i]]) = rb[i];
    }
  };

  f16v acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      h8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const h8*>(&As[cur][(wm + 32 * i + fr) * LDK + ks + fk]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const h8*>(&Bs[cur][(wn + 32 * j + fr) * LDK + ks + fk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // Accumulator layout of a 32 x 32 block: lane l holds column l % 32 and
  // rows 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M && n < N) {
          if constexpr (ZT == DFS_F32)
            ((float*)a.Z)[(int64_t)m * N + n] = acc[i][j][v];
          else
            ((_Float16*)a.Z)[(int64_t)m * N + n] = (_Float16)acc[i][j][v];
        }
      }
    }
}

// Expand an atom-major NVFP4 dictionary to f16 (element i = e2m1 * e4m3 *
// ts, rounded once to f16) so the MFMA path can consume it.
__global__ __launch_bounds__(256) void nvfp4_to_f16_kernel(const uint8_t* codes,
                                                           const uint8_t* scales, const float* ts,
                                                           int64_t n, _Float16* out) {
  const int64_t i8 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i8 >= n) return;
  const float t = *ts;
  const float s = e4m3_to_f32(scales[i8 / 16]) * t;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + i8 / 2);
  const f2 v0 = e2m1x2_f2<0>(w), v1 = e2m1x2_f2<1>(w), v2 = e2m1x2_f2<2>(w),
           v3 = e2m1x2_f2<3>(w);
  h8 o = {(_Float16)(v0[0] * s), (_Float16)(v0[1] * s), (_Float16)(v1[0] * s),
          (_Float16)(v1[1] * s), (_Float16)(v2[0] * s), (_Float16)(v2[1] * s),
          (_Float16)(v3[0] * s), (_Float16)(v3[1] * s)};
  *reinterpret_cast<h8*>(out + i8) = o;
}

}  // namespace

hipError_t launch_gemm_xd_mfma(const XdLaunch& a, hipStream_t s) {
  const int M = a.n_layers * a.T;
  dim3 grid((a.k + BN - 1) / BN, (M + BM - 1) / BM);
  if (a.zdt == DFS_F32)
    hipLaunchKernelGGL(gemm_xd_kernel<DFS_F32>, grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_xd_kernel<DFS_F16>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

// n must be a multiple of 8 (the caller checks d_in % 32 == 0).
hipError_t launch_nvfp4_to_f16(const uint8_t* codes, const uint8_t* scales, const float* ts,
                               int64_t n, _Float16* out, hipStream_t s) {
  const int64_t threads = n / 8;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(nvfp4_to_f16_kernel, dim3(blocks), dim3(256), 0, s, codes, scales, ts, n,
                     out);
  return hipGetLastError();
}

}  // namespace dfs
