// spmv_csc.hip -- Y_l = Z_l C_l for a few tokens (decode), C_l in CSC.
//
// Second half of the factored projection ("DictLLM: Shared Dictionaries for
// Post-Training Compression", Eq. (1): Y_l = Z_l C_l).  Each output column
// uses its own subset of atoms, so the access is irregular (same review,
// "Prerequisites: projections, rank and calibration"): the kernel streams
// the column's row indices and values from HBM with coalesced 16-byte loads
// and gathers the matching Z entries from LDS.
//
// Mapping: a workgroup is 4 waves; each wave serves 4 columns at once, one
// per 16-lane DPP row.  Lane g of a row reads the 8-entry chunks g, g+16, ...
// of its column (128 entries per step), U steps in flight per batch, every
// lane issuing the same loads (past its column it reloads the last chunk of
// the arrays, masked).  The first batch is issued before Z is staged into
// LDS (C does not depend on Z).  The Z tile is [k][TT] fp32 (TT tokens per pass); the partial sums are
// reduced over the 16 lanes of the row with DPP, in a fixed order.
// grid = (ceil(d_out / 16), n_layers); one launch covers a whole group.
#include "csc_chunks.hpp"

namespace dfs {
namespace {

constexpr int kThreads = 256;
constexpr int kColsPerBlock = 16;  // 4 waves x 4 DPP rows

// 8-entry chunks in flight per lane per batch: with 16 lanes per column a
// batch covers 128 * U entries, enough for a whole column at the densities of
// the decode workloads (mean 410-615 stored entries per column).  Wide token
// tiles keep fewer chunks so that the accumulators and Z reads fit.
template <int VT, int TT>
struct Unroll {
  static constexpr int U = TT >= 16 ? 1 : TT >= 8 ? 2 : TT >= 4 ? 4 : (VT == DFS_F32 ? 3 : 6);
};

// Z rows [row0, row0 + rows) -> LDS [k][TT] fp32 (zero rows past `rows`).
// TT == 1 with k % 8 == 0 is a straight vector copy with every load issued
// before the first store.
template <int ZT, int TT>
__device__ __forceinline__ void stage_z(float* zs, const void* Z, int64_t row0, int rows, int k) {
  if constexpr (TT == 1) {
    if (rows <= 0) return;
    if (k % 8 == 0) {
      constexpr int kUnr = 4;
      constexpr int kW = ZT == DFS_F32 ? 2 : 1;
      const int n8 = k / 8;
      for (int base = 0; base < n8; base += kThreads * kUnr) {
        u4 v[kUnr][kW];
#pragma unroll
        for (int j = 0; j < kUnr; ++j) {
          const int i8 = base + j * kThreads + threadIdx.x;
          if (i8 < n8) {
            if constexpr (ZT == DFS_F32) {
              const float* z = (const float*)Z + row0 * k + i8 * 8;
              v[j][0] = ld16<u4>(z);
              v[j][1] = ld16<u4>(z + 4);
            } else {
              v[j][0] = ld16<u4>((const _Float16*)Z + row0 * k + i8 * 8);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < kUnr; ++j) {
          const int i8 = base + j * kThreads + threadIdx.x;
          if (i8 < n8) {
            float* dst = zs + i8 * 8;
            if constexpr (ZT == DFS_F32) {
              *reinterpret_cast<u4*>(dst) = v[j][0];
              *reinterpret_cast<u4*>(dst + 4) = v[j][1];
            } else {
              const h8 h = __builtin_bit_cast(h8, v[j][0]);
              *reinterpret_cast<f4*>(dst) = f4{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
              *reinterpret_cast<f4*>(dst + 4) = f4{(float)h[4], (float)h[5], (float)h[6], (float)h[7]};
            }
          }
        }
      }
    } else {
      for (int i = threadIdx.x; i < k; i += kThreads)
        zs[i] = ZT == DFS_F32 ? ((const float*)Z)[row0 * k + i]
                              : (float)((const _Float16*)Z)[row0 * k + i];
    }
  } else {
    for (int idx = threadIdx.x; idx < k * TT; idx += kThreads) {
      const int t = idx / k, at = idx - t * k;  // read rows contiguously
      float v = 0.0f;
      if (t < rows) {
        const int64_t g = (row0 + t) * k + at;
        v = ZT == DFS_F32 ? ((const float*)Z)[g] : (float)((const _Float16*)Z)[g];
      }
      zs[at * TT + t] = v;
    }
  }
}

template <int VT, int ZT, int TT>
__global__ __launch_bounds__(kThreads) void spmv_csc_kernel(ZcLaunch a) {
  constexpr int U = Unroll<VT, TT>::U;
  extern __shared__ __attribute__((aligned(16))) float zs[];  // [k][TT]

  const int layer = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane & 15;
  const int col = blockIdx.x * kColsPerBlock + wave * 4 + (lane >> 4);
  const bool col_ok = col < a.d_out;
  const int64_t nnz = a.nnz[layer];
  int s = 0, e = 0;
  if (col_ok) {  // clamp to [0, nnz] so a malformed colptr cannot index out of bounds
    s = (int)min<int64_t>(max(a.colptr[layer][col], 0), nnz);
    e = (int)min<int64_t>(max(a.colptr[layer][col + 1], s), nnz);
  }
  const uint16_t* rowidx = a.rowidx[layer];
  const void* vals = a.vals[layer];
  const uint8_t* vsc = a.vscales[layer];
  const int first = (s & ~7) + g * 8;
  const int64_t lastc = last_chunk(e);
  float ts = 1.0f;
  if constexpr (VT == DFS_NVFP4) ts = *a.vts[layer];

  for (int t0 = 0; t0 < a.T; t0 += TT) {
    IdxChunk ic[U];
    ValChunk<VT> vc[U];
    int p0 = first;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = min<int64_t>(p0 + 128 * u, lastc);
      ic[u].load(rowidx, p);
      vc[u].load(vals, vsc, p);
    }
    if (t0 > 0) __syncthreads();
    const int rows = a.T - t0 < TT ? a.T - t0 : TT;
    stage_z<ZT, TT>(zs, a.Z, (int64_t)layer * a.T + t0, rows, a.k);
    __syncthreads();

    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
    const uint32_t len = (uint32_t)(e - s);
    while (p0 < e) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int base = p0 + 128 * u - s;
        // entries outside [s, e) are masked without a branch (index 0, zero
        // product), so the LDS gathers of a chunk issue back to back
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool ok = (uint32_t)(base + i) < len;
          const float v = ok ? vc[u].get(i) : 0.0f;
          const float* zr = zs + (ok ? ic[u].get(i) : 0u) * TT;
          if constexpr (TT % 4 == 0) {
#pragma unroll
            for (int t = 0; t < TT; t += 4) {
              const f4 z4 = *reinterpret_cast<const f4*>(zr + t);
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[t + q] += ok ? z4[q] * v : 0.0f;
            }
          } else {
#pragma unroll
            for (int t = 0; t < TT; ++t) acc[t] += ok ? zr[t] * v : 0.0f;
          }
        }
      }
      p0 += 128 * U;
      if (p0 < e) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t p = min<int64_t>(p0 + 128 * u, lastc);
          ic[u].load(rowidx, p);
          vc[u].load(vals, vsc, p);
        }
      }
    }

    float out = 0.0f;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float r = row16_sum(acc[t]);
      if (g == t) out = r;
    }
    if (col_ok && g < rows) {
      const int64_t o = (int64_t)(t0 + g) * a.ldy + col;
      out *= ts;
      if (a.ydt == DFS_F16)
        ((_Float16*)a.Y[layer])[o] = (_Float16)out;
      else
        ((float*)a.Y[layer])[o] = out;
    }
  }
}

template <int VT, int ZT, int TT>
hipError_t launch3(const ZcLaunch& a, hipStream_t s) {
  const size_t smem = (size_t)a.k * TT * sizeof(float);
  auto kern = spmv_csc_kernel<VT, ZT, TT>;
  if (smem > 64 * 1024) {
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
  }
  dim3 grid((a.d_out + kColsPerBlock - 1) / kColsPerBlock, a.n_layers);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, s, a);
  return hipGetLastError();
}

template <int VT, int ZT>
hipError_t launch2(const ZcLaunch& a, hipStream_t s) {
  const int tt = spmv_token_tile(a.T, a.k);
  switch (tt) {
    case 1:
      return launch3<VT, ZT, 1>(a, s);
    case 2:
      return launch3<VT, ZT, 2>(a, s);
    case 4:
      return launch3<VT, ZT, 4>(a, s);
    case 8:
      return launch3<VT, ZT, 8>(a, s);
    default:
      return launch3<VT, ZT, 16>(a, s);
  }
}

template <int VT>
hipError_t launch1(const ZcLaunch& a, hipStream_t s) {
  return a.zdt == DFS_F32 ? launch2<VT, DFS_F32>(a, s) : launch2<VT, DFS_F16>(a, s);
}

}  // namespace

int spmv_token_tile(int T, int k) {
  int tt = 1;
  while (tt < T && tt < 16 && (size_t)k * (tt * 2) * sizeof(float) <= 64 * 1024) tt *= 2;
  return tt;
}

hipError_t launch_spmv_csc(const ZcLaunch& a, hipStream_t s) {
  switch (a.vdt) {
    case DFS_F16:
      return launch1<DFS_F16>(a, s);
    case DFS_F32:
      return launch1<DFS_F32>(a, s);
    default:
      return launch1<DFS_NVFP4>(a, s);
  }
}

}  // namespace dfs
