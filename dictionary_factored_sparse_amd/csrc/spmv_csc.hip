// spmv_csc.hip -- Y_l = Z_l C_l for a few tokens (decode), C_l in CSC.
//
// Second half of the factored projection ("DictLLM: Shared Dictionaries for
// Post-Training Compression", Eq. (1): Y_l = Z_l C_l).  Each output column
// uses its own subset of atoms, so the access is irregular (same review,
// "Prerequisites: projections, rank and calibration"): the kernel streams
// the column's row indices and values from HBM with coalesced 16-byte loads
// and gathers the matching Z entries from LDS.
//
// Mapping: a workgroup is 4 waves (8 with the f16 tile, 16 with its 16-token
// form); each wave serves 4 columns at once, one per 16-lane DPP row.  Lane
// g of a row reads the 8-entry chunks g, g+16, ... of its column (128
// entries per step), U steps in flight per batch, every
// lane issuing the same loads (past its column it reloads the column's last
// chunk, masked).  The first batch is issued before Z is staged into
// LDS (C does not depend on Z).  The Z tile is [k][TT] fp32 (TT tokens per
// pass), or f16 [k + 1][TT] when fp32 would not fit and Z is f16 already
// (see spmv_token_tile),
// so that up to 16 tokens take one pass over C; the partial sums are
// reduced over the 16 lanes of the row with DPP, in a fixed order.  A
// workgroup serves an equal run of 4-column quads (256 or 512 workgroups
// per launch), so one staging of Z serves many columns.
// grid = (workgroups per layer, n_layers).
#include "csc_chunks.hpp"

namespace dfs {
namespace {

constexpr int kThreads = 256;      // fp32 Z tile (small T)
// f16 Z tile: one large tile per CU, shared by 2 waves per SIMD, or by 4 for
// the 16-token tile, whose gather chains (LDS read, then 16 multiply-adds per
// entry) need the extra waves to cover LDS latency (MLP group of 4 at
// b = 16: gate 68.6 -> 63.8 us, down 52.8 -> 48.5 us); it then holds one
// chunk per lane to fit 128 registers.
template <bool ZH, int TT>
constexpr int threads_of() { return ZH ? (TT >= 16 ? 1024 : 512) : kThreads; }

// 8-entry chunks in flight per lane per batch: with 16 lanes per column a
// batch covers 128 * U entries, enough for a whole column at the densities of
// the decode workloads (mean 410-615 stored entries per column).  Wide token
// tiles keep fewer chunks so that the accumulators and Z reads fit.
template <int VT, int TT, bool ZH>
struct Unroll {
  static constexpr int U = ZH ? (TT >= 16 ? 1 : TT >= 8 ? 3 : (VT == DFS_F32 || VT == DFS_INT8 ? 3 : 4))
                              : TT >= 16 ? 1 : TT >= 8 ? 2 : TT >= 4 ? 4 : (VT == DFS_F32 ? 3 : 6);
};

typedef _Float16 h4 __attribute__((ext_vector_type(4)));

// Z rows [row0, row0 + rows) -> LDS [k + 1][TT] f16, row k zero (masked
// entries read it).  Used when the fp32 tile would not fit: the token tile
// then still covers the whole call (T <= 16) in one pass over C.  Thread
// (token t, atom group) converts 8 atoms of token t per step.
template <int ZT, int TT, int NTH>
__device__ __forceinline__ void stage_zh(_Float16* zh, const void* Z, int64_t row0, int rows,
                                         int k) {
  constexpr int kGroups = NTH / TT;
  const int t = threadIdx.x % TT;
  const bool live = t < rows;
  const int64_t zrow = (row0 + (live ? t : 0)) * k;
  if (k % 8 == 0) {  // 16-byte loads of 8 atoms (32 bytes for fp32 Z)
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
      for (int i = 0; i < 8; ++i) zh[(a0 + i) * TT + t] = live ? (_Float16)v[i] : (_Float16)0.0f;
    }
  } else {
    for (int a0 = (threadIdx.x / TT) * 8; a0 < k; a0 += kGroups * 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (a0 + i < k) {
          const float v = ZT == DFS_F32 ? ((const float*)Z)[zrow + a0 + i]
                                        : (float)((const _Float16*)Z)[zrow + a0 + i];
          zh[(a0 + i) * TT + t] = live ? (_Float16)v : (_Float16)0.0f;
        }
      }
    }
  }
  for (int i = threadIdx.x; i < TT; i += NTH) zh[k * TT + i] = (_Float16)0.0f;
}

// TT f16 tokens of one staged Z row (16-byte pieces; 8 bytes for TT = 4).
// For TT = 16 the two pieces come from `p0` and `p1`: the row's first and
// second 8 tokens, or the other way round (see the piece order in the
// kernel); `p1` is unused for TT < 16.
template <int TT>
struct ZRowH {
  h8 v[TT / 8];
  __device__ __forceinline__ void read(const _Float16* p0, const _Float16* p1) {
    v[0] = *reinterpret_cast<const h8*>(p0);
    if constexpr (TT == 16) v[1] = *reinterpret_cast<const h8*>(p1);
  }
  __device__ __forceinline__ float get(int t) const { return (float)v[t / 8][t % 8]; }
};
template <>
struct ZRowH<4> {
  h4 v;
  __device__ __forceinline__ void read(const _Float16* p0, const _Float16*) {
    v = *reinterpret_cast<const h4*>(p0);
  }
  __device__ __forceinline__ float get(int t) const { return (float)v[t]; }
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

template <int VT, int ZT, int TT, bool ZH>
__global__ __launch_bounds__((threads_of<ZH, TT>())) void spmv_csc_kernel(ZcLaunch a) {
  constexpr int NTH = threads_of<ZH, TT>();
  constexpr int NW = NTH / kWave;  // waves; each serves 4 columns (a quad) at a time
  constexpr int U = Unroll<VT, TT, ZH>::U;
  extern __shared__ __attribute__((aligned(16))) float zs[];  // [k][TT] fp32, or f16 (ZH)
  _Float16* zh = reinterpret_cast<_Float16*>(zs);

  const int layer = blockIdx.y;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane & 15;
  // this workgroup's run [qb, qe) of the layer's column quads, an equal
  // share within one quad: one staging of Z serves all of them.  In step j
  // wave w serves quad qb + j * NW + w, so the NW waves work on NW adjacent
  // quads at a time, and in the last step only the waves with a quad left.
  // (Whole groups of NW quads per workgroup gave some workgroups a third
  // more quads than others: 48 against 32 in the MLP gate layer.)
  const int nquads = (a.d_out + 3) / 4;
  const int qb = (int)((int64_t)blockIdx.x * nquads / gridDim.x);
  const int qe = (int)((int64_t)(blockIdx.x + 1) * nquads / gridDim.x);
  const int nsteps = (qe - qb + NW - 1) / NW;
  const int64_t nnz = a.nnz[layer];
  const uint16_t* rowidx = a.rowidx[layer];
  const void* vals = a.vals[layer];
  const uint8_t* vsc = a.vscales[layer];
  float ts = 1.0f;
  if constexpr (VT == DFS_NVFP4) ts = *a.vts[layer];
  // Piece order of the 16-token f16 rows.  The lanes of a row gather rows
  // at random atoms, and a row's LDS bank window depends only on the atom's
  // low bits, so lanes reading the same piece collide in the banks.  Odd
  // lanes read the second piece first; their acc[t] then holds token t ^ 8
  // until the halves are swapped back before the reduction, so every sum
  // keeps its order.
  const int swp = (ZH && TT == 16) ? (g & 1) * 8 : 0;

  struct Col {
    int col, s, e, first;
    int64_t lastc;
    float cs;  // 8-bit codes: the column's scale (times kCodeScale)
  };
  auto col_of = [&](int cg) {
    Col c;
    const int quad = qb + cg * NW + wave;
    c.col = quad < qe ? quad * 4 + (lane >> 4) : a.d_out;  // past the run: no column
    c.s = c.e = 0;
    c.cs = 1.0f;
    if (c.col < a.d_out) {  // clamp to [0, nnz]: a malformed colptr cannot index out of bounds
      c.s = (int)min<int64_t>(max(a.colptr[layer][c.col], 0), nnz);
      c.e = (int)min<int64_t>(max(a.colptr[layer][c.col + 1], c.s), nnz);
      if constexpr (kIsCode8<VT>) c.cs = a.vts[layer][c.col] * kCodeScale<VT>;
    }
    c.first = (c.s & ~7) + g * 8;
    c.lastc = last_chunk(c.e);
    return c;
  };
  // Batches of coefficient chunks in registers.  The 16-token f16 tile
  // (one chunk per batch) keeps two batches in flight: the next batch is
  // loaded (clamped to the column's last chunk, masked on use) while the
  // current one is consumed, so a column's batches do not each wait a full
  // memory round trip.  The other forms hold several chunks per batch and
  // one batch.
  constexpr bool kTwo = ZH && TT >= 16;
  IdxChunk ia[U], ib[kTwo ? U : 1];
  ValChunk<VT> va[U], vb[kTwo ? U : 1];
  auto load_batch = [&](IdxChunk* ic, ValChunk<VT>* vc, const Col& c, int p0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = min<int64_t>(p0 + 128 * u, c.lastc);
      ic[u].load(rowidx, p);
      vc[u].load(vals, vsc, p);
    }
  };

  for (int t0 = 0; t0 < a.T; t0 += TT) {
    Col c = col_of(0);
    load_batch(ia, va, c, c.first);  // does not depend on Z: in flight while Z is staged
    if (t0 > 0) __syncthreads();
    const int rows = a.T - t0 < TT ? a.T - t0 : TT;
    if constexpr (ZH)
      stage_zh<ZT, TT, NTH>(zh, a.Z, (int64_t)layer * a.T + t0, rows, a.k);
    else
      stage_z<ZT, TT>(zs, a.Z, (int64_t)layer * a.T + t0, rows, a.k);
    __syncthreads();

    for (int cg = 0; cg < nsteps; ++cg) {
      float acc[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
      const uint32_t len = (uint32_t)(c.e - c.s);
      auto consume = [&](const IdxChunk* ic, const ValChunk<VT>* vcb, int p0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          ValChunk<VT> vu = vcb[u];
          vu.touch();
          const int base = p0 + 128 * u - c.s;
          // entries outside [s, e) are masked without a branch, so the LDS
          // gathers of a chunk issue back to back
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const bool ok = (uint32_t)(base + i) < len;
            const float v = ok ? vu.get(i) : 0.0f;
            if constexpr (ZH) {
              // masked entries read the zero row with a zero value
              ZRowH<TT> z;
              const _Float16* zr = zh + (ok ? ic[u].get(i) : (uint32_t)a.k) * TT;
              z.read(zr + swp, zr + (8 - swp));
#pragma unroll
              for (int t = 0; t < TT; ++t) acc[t] = __builtin_fmaf(z.get(t), v, acc[t]);
            } else {
              // masked entries read row 0 and add a zero product
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
        }
      };
      int p0 = c.first;
      if constexpr (kTwo) {
        // the next batch is loaded before this one is consumed and moved
        // into place after it (a loop-exit branch between the two halves of
        // an unrolled pair would let the compiler sink the load past the
        // first consume)
        while (p0 < c.e) {
          load_batch(ib, vb, c, p0 + 128 * U);
          consume(ia, va, p0);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            ia[u] = ib[u];
            va[u] = vb[u];
          }
          p0 += 128 * U;
        }
      } else {
        while (p0 < c.e) {
          consume(ia, va, p0);
          p0 += 128 * U;
          if (p0 < c.e) load_batch(ia, va, c, p0);
        }
      }
      // the next group's first batch goes out before this group's reduction
      Col n = c;
      if (cg + 1 < nsteps) {
        n = col_of(cg + 1);
        load_batch(ia, va, n, n.first);
      }
      if constexpr (ZH && TT == 16) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float lo = acc[t], hi = acc[t + 8];
          acc[t] = swp ? hi : lo;
          acc[t + 8] = swp ? lo : hi;
        }
      }
      float out = 0.0f;
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float r = row16_sum(acc[t]);
        if (g == t) out = r;
      }
      if (c.col < a.d_out && g < rows) {
        const int64_t o = (int64_t)(t0 + g) * a.ldy + c.col;
        if constexpr (kIsCode8<VT>)
          out *= c.cs;
        else
          out *= ts;
        if (a.ydt == DFS_F16)
          ((_Float16*)a.Y[layer])[o] = (_Float16)out;
        else
          ((float*)a.Y[layer])[o] = out;
      }
      c = n;
    }
  }
}

template <int VT, int ZT, int TT, bool ZH>
hipError_t launch3(const ZcLaunch& a, hipStream_t s) {
  const size_t smem = ZH ? (size_t)(a.k + 1) * TT * 2 : (size_t)a.k * TT * sizeof(float);
  auto kern = spmv_csc_kernel<VT, ZT, TT, ZH>;
  if (smem > 64 * 1024) {
    hipError_t err = hipFuncSetAttribute((const void*)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (err != hipSuccess) return err;
  }
  // a fixed number of workgroups (one per CU when the f16 tile limits the
  // CU to one workgroup, two per CU otherwise), split evenly over the
  // layers; each stages Z once for an equal run of column quads
  constexpr int NTH = threads_of<ZH, TT>();
  const int ngroups = (a.d_out + NTH / 16 - 1) / (NTH / 16);
  const int target = ZH ? 256 : 512;
  int per_layer = target / a.n_layers;
  per_layer = per_layer < 1 ? 1 : (per_layer > ngroups ? ngroups : per_layer);
  dim3 grid(per_layer, a.n_layers);
  hipLaunchKernelGGL(kern, grid, dim3(NTH), smem, s, a);
  return hipGetLastError();
}

template <int VT, int ZT>
hipError_t launch2(const ZcLaunch& a, hipStream_t s) {
  bool half = false;
  const int tt = spmv_token_tile(a.T, a.k, ZT == DFS_F32, &half);
  switch (tt) {
    case 1:
      return launch3<VT, ZT, 1, false>(a, s);
    case 2:
      return launch3<VT, ZT, 2, false>(a, s);
    case 4:
      return half ? launch3<VT, ZT, 4, true>(a, s) : launch3<VT, ZT, 4, false>(a, s);
    case 8:
      return half ? launch3<VT, ZT, 8, true>(a, s) : launch3<VT, ZT, 8, false>(a, s);
    default:
      return half ? launch3<VT, ZT, 16, true>(a, s) : launch3<VT, ZT, 16, false>(a, s);
  }
}

template <int VT>
hipError_t launch1(const ZcLaunch& a, hipStream_t s) {
  return a.zdt == DFS_F32 ? launch2<VT, DFS_F32>(a, s) : launch2<VT, DFS_F16>(a, s);
}

}  // namespace

// Token tile of the SpMV: the smallest power of two covering T (at most 16),
// staged as fp32 when that fits in 64 KiB of LDS, else as f16 (with a zero
// row) when that fits in 144 KiB, else a smaller tile (fp32 at TT = 1 holds
// any k <= 16384).  fp32 Z (fp32 activations or dictionary) always keeps an
// fp32 tile, so that such callers get Z unrounded: a smaller tile, and more
// passes over C.
int spmv_token_tile(int T, int k, bool fp32_z, bool* half) {
  int tt = 1;
  while (tt < T && tt < 16) tt *= 2;
  for (;;) {
    if ((size_t)k * tt * sizeof(float) <= 64 * 1024 || tt == 1) {
      *half = false;
      return tt;
    }
    if (!fp32_z && tt >= 4 && (size_t)(k + 1) * tt * 2 <= 144 * 1024) {
      *half = true;
      return tt;
    }
    tt /= 2;
  }
}

hipError_t launch_spmv_csc(const ZcLaunch& a, hipStream_t s) {
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
