// spmv_bcsc.hip -- Y_l = Z_l C_l for block-structured coefficients, T <= 16.
//
// The variant the Review asks for under "Let the accelerator constrain the
// support" ("DictLLM: Shared Dictionaries for Post-Training Compression"):
// a column of C_l keeps whole blocks of 8 consecutive atoms.  A kept block is
// one 16-bit block index b and 8 values, so the index stream shrinks eightfold
// and a block's Z operands are 8 contiguous rows of the Z tile: one index
// load, one 16-byte value load (32 for f32) and contiguous LDS reads per
// block, where the unstructured SpMV gathers one Z row per entry.
//
// Mapping as in the unstructured SpMV: a 16-lane DPP row per column, lane g
// taking the column's blocks g, g + 16, ...; a workgroup stages a token tile
// of Z (fp32, [k8][TT], rows past k zero) once for a run of column groups.
#include "dfs_internal.hpp"

namespace dfs {
namespace {

constexpr int kTh = 256;
constexpr int kCPG = kTh / 16;  // columns per group: 4 per wave, one per DPP row
constexpr int kUB = 4;          // blocks in flight per lane

template <int VT>
struct BlockVals;

template <>
struct BlockVals<DFS_F16> {
  u4 w;
  __device__ __forceinline__ void load(const void* vals, int64_t q) {
    w = ld16<u4>((const uint16_t*)vals + 8 * q);
  }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t bits = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  }
};

template <>
struct BlockVals<DFS_F32> {
  u4 w0, w1;
  __device__ __forceinline__ void load(const void* vals, int64_t q) {
    const uint32_t* v = (const uint32_t*)vals + 8 * q;
    w0 = ld16<u4>(v);
    w1 = ld16<u4>(v + 4);
  }
  __device__ __forceinline__ float get(int e) const {
    return __uint_as_float(e < 4 ? w0[e] : w1[e - 4]);
  }
};

template <int VT, int ZT, int TT>
__global__ __launch_bounds__(kTh) void spmv_bcsc_kernel(ZcLaunch a, int groups_per_block) {
  extern __shared__ __attribute__((aligned(16))) float zs[];  // [k8][TT]
  const int layer = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane & 15;
  const int k = a.k;
  const int k8 = (k + 7) / 8 * 8;
  const int ngroups = (a.d_out + kCPG - 1) / kCPG;
  const int gb = blockIdx.x * groups_per_block;
  const int gend = min(gb + groups_per_block, ngroups);
  const int64_t nblk = a.nnz[layer];
  const uint16_t* bidx = a.rowidx[layer];
  const void* vals = a.vals[layer];

  for (int t0 = 0; t0 < a.T; t0 += TT) {
    const int rows = a.T - t0 < TT ? a.T - t0 : TT;
    if (t0 > 0) __syncthreads();
    for (int i = threadIdx.x; i < k8 * TT; i += kTh) {
      const int r = i / TT, t = i - r * TT;
      float v = 0.0f;
      if (r < k && t < rows) {
        const int64_t src = ((int64_t)layer * a.T + t0 + t) * k + r;
        v = ZT == DFS_F32 ? ((const float*)a.Z)[src] : (float)((const _Float16*)a.Z)[src];
      }
      zs[i] = v;
    }
    __syncthreads();

    for (int cg = gb; cg < gend; ++cg) {
      const int col = cg * kCPG + wave * 4 + (lane >> 4);
      int s = 0, e = 0;
      if (col < a.d_out) {  // clamp to [0, nblk]: a malformed colptr cannot index out of bounds
        s = (int)min<int64_t>(max(a.colptr[layer][col], 0), nblk);
        e = (int)min<int64_t>(max(a.colptr[layer][col + 1], s), nblk);
      }
      // lanes past the column's end reload its last block (masked); the
      // arrays hold at least 8 blocks, so block 0 is valid for empty columns
      const int64_t lastb = e > 0 ? e - 1 : 0;
      float acc[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
      for (int p0 = s + g; p0 < e; p0 += 16 * kUB) {
        uint32_t b[kUB];
        BlockVals<VT> v[kUB];
#pragma unroll
        for (int u = 0; u < kUB; ++u) {
          const int64_t q = min<int64_t>(p0 + 16 * u, lastb);
          b[u] = *gptr(bidx + q);
          v[u].load(vals, q);
        }
#pragma unroll
        for (int u = 0; u < kUB; ++u) {
          if (p0 + 16 * u < e) {
            const float* zr = zs + (int)min(b[u], (uint32_t)(k8 / 8 - 1)) * 8 * TT;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const float c = v[u].get(q);
#pragma unroll
              for (int t = 0; t < TT; ++t) acc[t] = __builtin_fmaf(zr[q * TT + t], c, acc[t]);
            }
          }
        }
      }
      float out = 0.0f;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float r = row16_sum(acc[t]);
        if (g == t) out = r;
      }
      if (col < a.d_out && g < rows) {
        const int64_t o = (int64_t)(t0 + g) * a.ldy + col;
        if (a.ydt == DFS_F16)
          ((_Float16*)a.Y[layer])[o] = (_Float16)out;
        else
          ((float*)a.Y[layer])[o] = out;
      }
    }
  }
}

template <int VT, int ZT, int TT>
hipError_t launch3(const ZcLaunch& a, hipStream_t s) {
  const int k8 = (a.k + 7) / 8 * 8;
  const size_t smem = (size_t)k8 * TT * sizeof(float);
  auto kern = spmv_bcsc_kernel<VT, ZT, TT>;
  if (smem > 64 * 1024) {
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
  }
  const int ngroups = (a.d_out + kCPG - 1) / kCPG;
  const int per = (ngroups * a.n_layers + 511) / 512;
  const int gpb = per < 1 ? 1 : per;
  dim3 grid((ngroups + gpb - 1) / gpb, a.n_layers);
  hipLaunchKernelGGL(kern, grid, dim3(kTh), smem, s, a, gpb);
  return hipGetLastError();
}

// Largest power-of-two token tile <= 16 (and <= the next power of two of T)
// whose fp32 Z tile fits in 64 KiB (k <= 16384 fits at TT = 1).
int bcsc_token_tile(int T, int k) {
  const int k8 = (k + 7) / 8 * 8;
  int tt = 1;
  while (tt < T && tt < 16) tt *= 2;
  while (tt > 1 && (size_t)k8 * tt * 4 > 64 * 1024) tt /= 2;
  return tt;
}

template <int VT, int ZT>
hipError_t launch2(const ZcLaunch& a, hipStream_t s) {
  switch (bcsc_token_tile(a.T, a.k)) {
    case 1: return launch3<VT, ZT, 1>(a, s);
    case 2: return launch3<VT, ZT, 2>(a, s);
    case 4: return launch3<VT, ZT, 4>(a, s);
    case 8: return launch3<VT, ZT, 8>(a, s);
    default: return launch3<VT, ZT, 16>(a, s);
  }
}

template <int VT>
hipError_t launch1(const ZcLaunch& a, hipStream_t s) {
  return a.zdt == DFS_F32 ? launch2<VT, DFS_F32>(a, s) : launch2<VT, DFS_F16>(a, s);
}

}  // namespace

hipError_t launch_spmv_bcsc(const ZcLaunch& a, hipStream_t s) {
  return a.vdt == DFS_F32 ? launch1<DFS_F32>(a, s) : launch1<DFS_F16>(a, s);
}

}  // namespace dfs
