// spmm_csc.hip -- Y_l = Z_l C_l for many tokens (prefill), C_l in CSC, VALU.
//
// Second half of the factored projection ("DictLLM: Shared Dictionaries for
// Post-Training Compression", Eq. (1)) when T is large.  The product stays on
// VALU: the coefficients are unstructured, so the work is a gather-FMA over
// each column's stored entries, not a dense contraction.
//
// Mapping: a workgroup owns a tile of TT tokens and a block of CB output
// columns.  It stages the tile's Z (TT x k) into LDS once as f16 [k][TT],
// with the 4-token quads of each atom row XOR-swizzled by the atom index so
// that staging writes spread over the banks.  A lane owns 4 consecutive
// tokens; TT/4 lanes share one column and read the same 8-entry C chunks
// (broadcast loads), so a wave works on 64/(TT/4) columns at once.  Per stored
// entry a lane does one 8-byte LDS read and four fp32 FMAs.  The next batch of
// C chunks is loaded before the current one is consumed.
// grid = (ceil(d_out / CB), ceil(T / TT), n_layers).
#include "csc_chunks.hpp"

namespace dfs {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kCB = 256;  // columns per workgroup
constexpr int kU = 4;     // 8-entry chunks per batch

typedef _Float16 h4 __attribute__((ext_vector_type(4)));

// Byte offset of token quad `tq` of atom `a` in the [k][TT] f16 tile.
template <int TT>
__device__ __forceinline__ int zoff(int a, int tq) {
  constexpr int NQ = TT / 4;
  return a * (TT * 2) + ((tq ^ ((a >> 2) & (NQ - 1))) * 8);
}

template <int VT, int ZT, int TT>
__global__ __launch_bounds__(kThreads) void spmm_csc_kernel(ZcLaunch a) {
  constexpr int LPC = TT / 4;        // lanes per column
  constexpr int CPW = kWave / LPC;   // columns per wave at once
  extern __shared__ __attribute__((aligned(16))) char zraw[];

  const int layer = blockIdx.z;
  const int t0 = blockIdx.y * TT;
  const int k = a.k;
  const int rows = a.T - t0 < TT ? a.T - t0 : TT;
  const int64_t zrow0 = (int64_t)layer * a.T + t0;

  // ---- stage Z tile: thread (atom a, quad tq) gathers 4 tokens
  for (int idx = threadIdx.x; idx < k * LPC; idx += kThreads) {
    const int at = idx % k, tq = idx / k;
    h4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tq * 4 + i;
      float v = 0.0f;
      if (t < rows) {
        const int64_t gi = (zrow0 + t) * k + at;
        v = ZT == DFS_F32 ? ((const float*)a.Z)[gi] : (float)((const _Float16*)a.Z)[gi];
      }
      q[i] = (_Float16)v;
    }
    *reinterpret_cast<h4*>(zraw + zoff<TT>(at, tq)) = q;
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int cg = lane / LPC, sub = lane % LPC;
  const int64_t nnz = a.nnz[layer];
  const uint16_t* rowidx = a.rowidx[layer];
  const void* vals = a.vals[layer];
  const uint8_t* vsc = a.vscales[layer];
  float ts = 1.0f;
  if constexpr (VT == DFS_NVFP4) ts = *a.vts[layer];
  const int cend = min(a.d_out, (blockIdx.x + 1) * kCB);

  for (int cbase = blockIdx.x * kCB; cbase < cend; cbase += kWaves * CPW) {
    const int col = cbase + wave * CPW + cg;
    int s = 0, e = 0;
    if (col < cend) {  // clamped to [0, nnz] like the SpMV
      s = (int)min<int64_t>(max(a.colptr[layer][col], 0), nnz);
      e = (int)min<int64_t>(max(a.colptr[layer][col + 1], s), nnz);
    }
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    IdxChunk ia[kU], ib[kU];
    ValChunk<VT> va[kU], vb[kU];
    auto load = [&](IdxChunk* ic, ValChunk<VT>* vc, int p) {
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (p + 8 * u < e) {
          ic[u].load(rowidx, p + 8 * u, nnz);
          vc[u].load(vals, vsc, p + 8 * u, nnz);
        }
    };
    const uint32_t len = (uint32_t)(e - s);
    auto consume = [&](const IdxChunk* ic, const ValChunk<VT>* vc, int p) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        // entries outside [s, e) are masked without a branch (atom 0, zero
        // product) so that the LDS gathers of a chunk issue back to back
        const int base = p + 8 * u - s;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool ok = (uint32_t)(base + i) < len;
          const int r = ok ? (int)ic[u].get(i) : 0;
          const float v = vc[u].get(i);
          const h4 z = *reinterpret_cast<const h4*>(zraw + zoff<TT>(r, sub));
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[t] += ok ? (float)z[t] * v : 0.0f;
        }
      }
    };
    // two register buffers with static names, alternating: the loads of the
    // next batch are in flight while the current one is consumed
    int p = s & ~7;
    load(ia, va, p);
    while (p < e) {
      load(ib, vb, p + 8 * kU);
      consume(ia, va, p);
      p += 8 * kU;
      if (p >= e) break;
      load(ia, va, p + 8 * kU);
      consume(ib, vb, p);
      p += 8 * kU;
    }
    if (col < cend) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = sub * 4 + i;
        if (t < rows) {
          const int64_t o = (int64_t)(t0 + t) * a.ldy + col;
          const float out = acc[i] * ts;
          if (a.ydt == DFS_F16)
            ((_Float16*)a.Y[layer])[o] = (_Float16)out;
          else
            ((float*)a.Y[layer])[o] = out;
        }
      }
    }
  }
}

template <int VT, int ZT, int TT>
hipError_t launch3(const ZcLaunch& a, hipStream_t s) {
  const size_t smem = (size_t)a.k * TT * 2;
  auto kern = spmm_csc_kernel<VT, ZT, TT>;
  if (smem > 64 * 1024) {
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
  }
  dim3 grid((a.d_out + kCB - 1) / kCB, (a.T + TT - 1) / TT, a.n_layers);
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, s, a);
  return hipGetLastError();
}

template <int VT, int ZT>
hipError_t launch2(const ZcLaunch& a, hipStream_t s) {
  switch (spmm_token_tile(a.k)) {
    case 32:
      return launch3<VT, ZT, 32>(a, s);
    case 16:
      return launch3<VT, ZT, 16>(a, s);
    case 8:
      return launch3<VT, ZT, 8>(a, s);
    default:
      return launch3<VT, ZT, 4>(a, s);
  }
}

template <int VT>
hipError_t launch1(const ZcLaunch& a, hipStream_t s) {
  return a.zdt == DFS_F32 ? launch2<VT, DFS_F32>(a, s) : launch2<VT, DFS_F16>(a, s);
}

}  // namespace

// Largest token tile (32, 16, 8 or 4) whose f16 Z tile fits in 128 KiB.
int spmm_token_tile(int k) {
  int tt = 32;
  while (tt > 4 && (size_t)k * tt * 2 > 128 * 1024) tt /= 2;
  return tt;
}

hipError_t launch_spmm_csc(const ZcLaunch& a, hipStream_t s) {
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
