// spmm_csc.hip -- Y_l = Z_l C_l for many tokens (prefill), C_l in CSC, VALU.
//
// Second half of the factored projection ("DictLLM: Shared Dictionaries for
// Post-Training Compression", Eq. (1)) when T is large.  The product stays on
// VALU: the coefficients are unstructured, so the work is a gather-FMA over
// each column's stored entries, not a dense contraction.
//
// Mapping: a workgroup owns a tile of TT tokens and a block of output
// columns, LPC lanes per column, each lane NT = TT / LPC of the tokens (at
// most 16, which bounds the registers).  It stages the tile's Z into LDS
// once as f16 [k + 1][TT] (row k is zero: masked entries point there).  For
// every stored entry (r, v) of its column a lane reads its NT tokens of Z
// row r (NT * 2 contiguous bytes) and does NT fused multiply-adds, f16 times
// f32 into f32 (v_fma_mix), so a C entry fetched once serves the whole tile.
// Chunks of 8 entries are loaded kU at a time, double-buffered, every lane
// issuing the same loads (past its column it reloads the column's last
// chunk, masked), so the compiler can wait for exactly the batch it needs.
// Costs per MAC: one VALU op and 2 bytes of LDS.
// grid = (ceil(d_out / (threads / LPC)), ceil(T / TT), n_layers).
#include "csc_chunks.hpp"

namespace dfs {
namespace {

// Threads per workgroup.  The Z tile holds most of a CU's LDS at the sizes
// that matter (k = 2048: 131 KiB), so a CU runs one workgroup, and its waves
// must cover the latency of each entry's chain (LDS gather, then NT
// multiply-adds): 1024 threads (four waves per SIMD) measured 683 -> 586 us
// against 512 for the q_proj group's prefill.  NVFP4 and 8-bit codes decode
// on use and would not fit the 128 registers of four waves per SIMD: 512.
template <int VT>
constexpr int spmm_threads() { return (VT == DFS_F16 || VT == DFS_F32) ? 1024 : 512; }
// 8-entry chunks per batch (double-buffered): two, which fits the registers
// of four waves per SIMD
template <int VT>
constexpr int kUnroll = 2;

typedef _Float16 h4 __attribute__((ext_vector_type(4)));

// NT f16 tokens of one Z row, read from LDS in 16-byte pieces (8 bytes for
// NT = 4).  The two pieces of a 16-token read come from `p0` and `p1`, which
// point at the lane's first and second 8 tokens of the row, or the other way
// round (see the piece order in the kernel); `p1` is unused for NT < 16.
template <int NT>
struct ZRow {
  h8 v[NT / 8];
  __device__ __forceinline__ void read(const _Float16* p0, const _Float16* p1) {
    v[0] = *reinterpret_cast<const h8*>(p0);
    if constexpr (NT == 16) v[1] = *reinterpret_cast<const h8*>(p1);
  }
  __device__ __forceinline__ float get(int t) const { return (float)v[t / 8][t % 8]; }
};
template <>
struct ZRow<4> {
  h4 v;
  __device__ __forceinline__ void read(const _Float16* p0, const _Float16*) {
    v = *reinterpret_cast<const h4*>(p0);
  }
  __device__ __forceinline__ float get(int t) const { return (float)v[t]; }
};

// Stage Z rows [row0, row0 + rows) (tokens) into the f16 tile [k + 1][TT].
// Thread (token t, atom group) converts 8 atoms of token t per step: one
// 16-byte load (32 for f32 Z) when k % 8 == 0, elementwise otherwise.
template <int ZT, int TT, int kThreads>
__device__ __forceinline__ void stage_z(_Float16* zt, const void* Z, int64_t row0, int rows,
                                        int k) {
  constexpr int kGroups = kThreads / TT;
  const int t = threadIdx.x % TT;
  const bool live = t < rows;
  const int64_t zrow = (row0 + (live ? t : 0)) * k;
  if (k % 8 == 0) {
    for (int a0 = (threadIdx.x / TT) * 8; a0 < k; a0 += kGroups * 8) {
      float v[8];
      if constexpr (ZT == DFS_F32) {
        const u4 w0 = ld16<u4>((const float*)Z + zrow + a0);
        const u4 w1 = ld16<u4>((const float*)Z + zrow + a0 + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = __uint_as_float(w0[i]);
          v[4 + i] = __uint_as_float(w1[i]);
        }
      } else {
        const h8 h = __builtin_bit_cast(h8, ld16<u4>((const _Float16*)Z + zrow + a0));
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)h[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) zt[(a0 + i) * TT + t] = live ? (_Float16)v[i] : (_Float16)0.0f;
    }
  } else {
    for (int a0 = (threadIdx.x / TT) * 8; a0 < k; a0 += kGroups * 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (a0 + i < k) {
          const float v = ZT == DFS_F32 ? ((const float*)Z)[zrow + a0 + i]
                                        : (float)((const _Float16*)Z)[zrow + a0 + i];
          zt[(a0 + i) * TT + t] = live ? (_Float16)v : (_Float16)0.0f;
        }
      }
    }
  }
  for (int i = threadIdx.x; i < TT; i += kThreads) zt[k * TT + i] = (_Float16)0.0f;
}

template <int VT, int TT>
struct Split {
  static constexpr int kThreads = spmm_threads<VT>();
  static constexpr int LPC = TT > 16 ? TT / 16 : 1;  // lanes per column
  static constexpr int NT = TT / LPC;                // tokens per lane
  static constexpr int CPB = kThreads / LPC;         // columns per workgroup
};

template <int VT, int ZT, int TT>
__global__ __launch_bounds__(spmm_threads<VT>()) void spmm_csc_kernel(ZcLaunch a) {
  constexpr int LPC = Split<VT, TT>::LPC, NT = Split<VT, TT>::NT, CPB = Split<VT, TT>::CPB;
  constexpr int kU = kUnroll<VT>;
  extern __shared__ __attribute__((aligned(16))) char zraw[];
  _Float16* zt = reinterpret_cast<_Float16*>(zraw);

  const int layer = blockIdx.z;
  const int t0 = blockIdx.y * TT;
  const int k = a.k;
  const int rows = a.T - t0 < TT ? a.T - t0 : TT;
  const int sub = threadIdx.x % LPC;  // this lane's tokens: sub * NT ...
  const int col = blockIdx.x * CPB + threadIdx.x / LPC;
  const bool col_ok = col < a.d_out;
  const int64_t nnz = a.nnz[layer];
  int s = 0, e = 0;
  if (col_ok) {  // clamped to [0, nnz] like the SpMV
    s = (int)min<int64_t>(max(a.colptr[layer][col], 0), nnz);
    e = (int)min<int64_t>(max(a.colptr[layer][col + 1], s), nnz);
  }
  const uint16_t* rowidx = a.rowidx[layer];
  const void* vals = a.vals[layer];
  const uint8_t* vsc = a.vscales[layer];
  const int64_t lastc = last_chunk(e);
  // 8-bit codes: the column's scale, loaded with the column bounds
  float cs = 1.0f;
  if constexpr (kIsCode8<VT>)
    if (col_ok) cs = a.vts[layer][col] * kCodeScale<VT>;

  IdxChunk ia[kU], ib[kU];
  ValChunk<VT> va[kU], vb[kU];
  auto load = [&](IdxChunk* ic, ValChunk<VT>* vc, int p) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t pc = min<int64_t>(p + 8 * u, lastc);
      ic[u].load(rowidx, pc);
      vc[u].load(vals, vsc, pc);
    }
  };
  // the first batch does not depend on Z: in flight while the tile is staged
  int p = s & ~7;
  load(ia, va, p);
  stage_z<ZT, TT, spmm_threads<VT>()>(zt, a.Z, (int64_t)layer * a.T + t0, rows, k);
  __syncthreads();

  float acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = 0.0f;
  // Piece order.  A 16-token read is two 16-byte pieces of a row; rows are
  // gathered at random atoms, and a row's bank window depends only on the
  // atom's low bits, so neighbouring columns reading the same piece of their
  // rows collide in the LDS banks.  Odd columns read their second piece
  // first: acc[t] then holds token t ^ 8 of the lane's 16, for the whole
  // kernel, so each sum keeps its order and the result is unchanged.
  const int swp = NT == 16 ? ((threadIdx.x / LPC) & 1) * 8 : 0;
  const _Float16* zl0 = zt + sub * NT + swp;
  const _Float16* zl1 = zt + sub * NT + (8 - swp);
  const uint32_t len = (uint32_t)(e - s);
  auto consume = [&](const IdxChunk* ic, const ValChunk<VT>* vc, int pb) {
    // A batch that lies inside every active lane's column (all but the
    // first and the last one or two of a column) needs no mask: the index
    // is the row and the value enters the multiply-add as stored.
    if (__all(pb >= s && pb + 8 * kU <= e)) {
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        ValChunk<VT> vu = vc[u];
        vu.touch();
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          ZRow<NT> z;
          const uint32_t ro = ic[u].get(i) * TT;
          z.read(zl0 + ro, zl1 + ro);
          const float v = vu.get(i);
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(z.get(t), v, acc[t]);
        }
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      ValChunk<VT> vu = vc[u];
      vu.touch();
      const int base = pb + 8 * u - s;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // entries outside [s, e) read the zero row with a zero value
        const bool ok = (uint32_t)(base + i) < len;
        const uint32_t r = ok ? ic[u].get(i) : (uint32_t)k;
        const float v = ok ? vu.get(i) : 0.0f;
        ZRow<NT> z;
        z.read(zl0 + r * TT, zl1 + r * TT);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = __builtin_fmaf(z.get(t), v, acc[t]);
      }
    }
  };
  // two register buffers with static names, alternating: the next batch is
  // in flight while the current one is consumed
  while (p < e) {
    load(ib, vb, p + 8 * kU);
    consume(ia, va, p);
    p += 8 * kU;
    if (p >= e) break;
    load(ia, va, p + 8 * kU);
    consume(ib, vb, p);
    p += 8 * kU;
  }

  if (col_ok) {
    float ts = cs;
    if constexpr (VT == DFS_NVFP4) ts = *a.vts[layer];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int t = sub * NT + (i ^ swp);
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

template <int VT, int ZT, int TT>
hipError_t launch3(const ZcLaunch& a, hipStream_t s) {
  const size_t smem = (size_t)(a.k + 1) * TT * 2;
  auto kern = spmm_csc_kernel<VT, ZT, TT>;
  if (smem > 64 * 1024) {
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
  }
  constexpr int CPB = Split<VT, TT>::CPB;
  dim3 grid((a.d_out + CPB - 1) / CPB, (a.T + TT - 1) / TT, a.n_layers);
  hipLaunchKernelGGL(kern, grid, dim3(spmm_threads<VT>()), smem, s, a);
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

// Largest token tile (32, 16, 8 or 4) whose f16 Z tile [k + 1][TT] fits in
// 144 KiB of LDS (k <= 16384 always fits at TT = 4).
int spmm_token_tile(int k) {
  int tt = 32;
  while (tt > 4 && (size_t)(k + 1) * tt * 2 > 144 * 1024) tt /= 2;
  return tt;
}

hipError_t launch_spmm_csc(const ZcLaunch& a, hipStream_t s) {
  switch (a.vdt) {
    case DFS_F16:
      return launch1<DFS_F16>(a, s);
    case DFS_F32:
      return launch1<DFS_F32>(a, s);
    case DFS_FP8:
      return launch1<DFS_FP8>(a, s);
    case DFS_INT8:
      return launch1<DFS_INT8>(a, s);
    default:
      return launch1<DFS_NVFP4>(a, s);
  }
}

}  // namespace dfs
