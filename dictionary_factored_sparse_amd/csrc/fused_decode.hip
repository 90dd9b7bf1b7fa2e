// fused_decode.hip -- one launch for a decode group: Z = X D_g, then every
// Y_l = Z_l C_l ("DictLLM: Shared Dictionaries for Post-Training
// Compression", Eq. (1) and Figure 2: one dictionary, separate activations).
//
// At decode both halves stream bytes from HBM: D_g (read once for the whole
// group) and each C_l.  Run as two kernels, C_l's stream cannot start until
// the Z kernel ends.  Here one persistent grid (one workgroup per CU) does
// both:
//   1. each workgroup stages X and the [start, end) of its output columns;
//   2. it issues the loads of its first two rounds of C chunks (they do not
//      depend on Z) and of its slice of D_g's atoms;
//   3. it computes its atoms' Z, writes them to the workspace and arrives at
//      a grid barrier;
//   4. after the barrier it stages all of Z into LDS and finishes its
//      columns, later rounds of C double-buffered in registers.
// So the C stream overlaps the D stream and the Z dependency costs one
// barrier instead of a second launch.
//
// Grid barrier: a counter and a generation word in the workspace control
// block (the counter is zero before first use; the last arriver resets it,
// so it is zero again after every launch; the generation word only grows).  The grid never exceeds one
// workgroup per CU, so every workgroup is resident; the wait is bounded
// anyway: after `spin_limit` polls a workgroup sets the error word and goes
// on, so the kernel always terminates.
#include "csc_chunks.hpp"
#include "gemv_common.hpp"

namespace dfs {
namespace {

using namespace gemv;

constexpr int kU = 6;  // 8-entry C chunks per lane per batch
constexpr int kLayerTableBytes = 256;

// Per-layer pointers live in a small LDS table: looking one up for a
// lane-dependent layer is an LDS read (LGKM counter), not a vector load
// from the kernel arguments that would have to wait behind the C stream.
struct LayerRow {
  const int32_t* colptr;
  const uint16_t* rowidx;
  const void* vals;
  const uint8_t* vsc;
  const float* vts;
  void* Y;
  int64_t nnz;
};

// Release: every wave waits for its own Z stores to complete (they reach the
// XCD's L2; L1 is write-through), then one thread per workgroup performs the
// agent-scope release (write back the L2 for other XCDs) with its arrival.
// Acquire: the same thread's agent-scope acquire invalidates this CU's L1
// and the XCD's L2 before any wave reads Z.  One fence pair per workgroup,
// not per thread: agent-scope fences are cache-wide operations.
__device__ void grid_barrier(uint32_t* ctrl, uint32_t G, uint32_t spin_limit) {
  uint32_t* count = ctrl;
  uint32_t* gen = ctrl + 16;
  uint32_t* err = ctrl + 32;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t g0 = __hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t old = __hip_atomic_fetch_add(count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (old == G - 1) {
      __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_fetch_add(gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      uint32_t it = 0;
      while (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0) {
        if (++it > spin_limit) {
          __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __atomic_thread_fence(__ATOMIC_ACQUIRE);  // agent-scope acquire (system in HIP => >= agent)
  }
  __syncthreads();
}

template <int DT, int VT, int RT, int A>
__global__ __launch_bounds__(kThreads, 1) void fused_decode_kernel(FusedLaunch f) {
  using Cf = Cfg<DT, DFS_F16, RT>;
  constexpr int CE = Cf::CE, SEGC = Cf::SEGC, SEG = Cf::SEG;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const XdLaunch& a = f.xd;
  const ZcLaunch& z = f.zc;
  LayerRow* lt = reinterpret_cast<LayerRow*>(smem);            // [kFusedMaxLayers]
  int2* cse = reinterpret_cast<int2*>(smem + kLayerTableBytes);  // [ncols] column [start, end)
  char* big = smem + kLayerTableBytes + f.col_bytes;           // X rows, later all of Z
  _Float16* xs = reinterpret_cast<_Float16*>(big);
  float* zs = reinterpret_cast<float*>(big);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int g = lane & 15;
  const int G = gridDim.x;
  const int d_in = a.d_in, k = a.k, d_out = z.d_out, nl = z.n_layers;
  const int NC = nl * d_out;
  const int c0 = (int)((int64_t)blockIdx.x * NC / G);
  const int c1 = (int)((int64_t)(blockIdx.x + 1) * NC / G);
  const int ncols = c1 - c0;
  const int rounds = (ncols + 15) / 16;
  const int ld = (d_in + SEG - 1) / SEG * SEG;

  // ---- 1. layer table, column ranges and X rows into LDS
  if (threadIdx.x < kFusedMaxLayers) {
    const int l = threadIdx.x;
    lt[l] = LayerRow{z.colptr[l], z.rowidx[l], z.vals[l], z.vscales[l], z.vts[l], z.Y[l], z.nnz[l]};
  }
  __syncthreads();
  for (int i = threadIdx.x; i < ncols; i += kThreads) {
    const int c = c0 + i, l = c / d_out, j = c - l * d_out;
    const auto* cp = gptr(lt[l].colptr);
    const int64_t nnz = lt[l].nnz;
    const int s = (int)min<int64_t>(max(cp[j], 0), nnz);
    const int e = (int)min<int64_t>(max(cp[j + 1], s), nnz);
    cse[i] = make_int2(s, e);
  }
  stage_x<DFS_F16, RT, _Float16>(xs, a, 0, 0, ld, ld);
  __syncthreads();

  // ---- 2. first two rounds of C chunks in flight
  const int slot = wave * 4 + (lane >> 4);
  auto load_round = [&](IdxChunk* ic, ValChunk<VT>* vc, int r) {
    const int ci = r * 16 + slot;
    if (ci < ncols) {
      const int2 se = cse[ci];
      const LayerRow& L = lt[(c0 + ci) / d_out];
      const uint16_t* rowidx = L.rowidx;
      const void* vals = L.vals;
      const uint8_t* vsc = L.vsc;
      const int64_t nnz = L.nnz;
      const int p0 = (se.x & ~7) + g * 8;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int p = p0 + 128 * u;
        if (p < se.y) {
          ic[u].load(rowidx, p, nnz);
          vc[u].load(vals, vsc, p, nnz);
        }
      }
    }
  };
  IdxChunk ia[kU], ib[kU];
  ValChunk<VT> va[kU], vb[kU];
  load_round(ia, va, 0);
  load_round(ib, vb, 1);

  // ---- 3. Z for this workgroup's atoms
  const int atom0 = (blockIdx.x * kWaves + wave) * A;
  float acc[A][RT];
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[i][r] = 0.0f;
  for (int seg = 0; seg < d_in; seg += SEG) {
    u4 dreg[A][SEGC];
    uint32_t sreg[A][SEGC];
#pragma unroll
    for (int i = 0; i < A; ++i) {
      const int atom = atom0 + i;
#pragma unroll
      for (int c = 0; c < SEGC; ++c) {
        const int e0 = seg + (c * kWave + lane) * CE;
        dreg[i][c] = u4{0u, 0u, 0u, 0u};
        sreg[i][c] = 0u;
        if (atom < k && e0 < d_in) {
          if constexpr (DT == DFS_NVFP4) {
            const int64_t el = (int64_t)atom * d_in + e0;
            dreg[i][c] = ld16<u4>(a.dcodes + el / 2);
            sreg[i][c] = (uint32_t)a.dscales[el / 16] | ((uint32_t)a.dscales[el / 16 + 1] << 8);
          } else {
            dreg[i][c] = ld16<u4>((const _Float16*)a.D + (int64_t)atom * a.ldd + e0);
          }
        }
      }
    }
    const _Float16* xseg = xs + seg;
#pragma unroll
    for (int c = 0; c < SEGC; ++c) {
      const int el = (c * kWave + lane) * CE;
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int i = 0; i < A; ++i)
          acc[i][r] = dot_chunk<DT, true, _Float16>(dreg[i][c], sreg[i][c], xseg + r * ld + el,
                                                    acc[i][r]);
    }
  }
  float dts = 1.0f;
  if constexpr (DT == DFS_NVFP4) dts = *a.dts;
#pragma unroll
  for (int i = 0; i < A; ++i) {
    const int atom = atom0 + i;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float v = wave_sum(acc[i][r]) * dts;
      if (lane == r && atom < k && r < nl) f.zws[(int64_t)r * k + atom] = v;
    }
  }

  // ---- 4. every workgroup's Z is written
  grid_barrier(f.ctrl, (uint32_t)G, f.spin_limit);

  // ---- 5. all of Z (nl x k fp32) into LDS
  {
    const int n4 = nl * k / 4;  // k % 4 == 0 on this path
    constexpr int kUnr = 4;
    for (int base = 0; base < n4; base += kThreads * kUnr) {
      u4 v[kUnr];
#pragma unroll
      for (int j = 0; j < kUnr; ++j) {
        const int i4 = base + j * kThreads + threadIdx.x;
        if (i4 < n4) v[j] = ld16<u4>(f.zws + 4 * i4);
      }
#pragma unroll
      for (int j = 0; j < kUnr; ++j) {
        const int i4 = base + j * kThreads + threadIdx.x;
        if (i4 < n4) *reinterpret_cast<u4*>(zs + 4 * i4) = v[j];
      }
    }
  }
  __syncthreads();

  // ---- 6. the columns, two rounds in flight
  auto consume = [&](const IdxChunk* ic, const ValChunk<VT>* vc, int r) {
    const int ci = r * 16 + slot;
    int s = 0, e = 0, l = 0;
    if (ci < ncols) {
      const int2 se = cse[ci];
      s = se.x;
      e = se.y;
      l = (c0 + ci) / d_out;
    }
    const float* zl = zs + l * k;
    float sum = 0.0f;
    int p0 = (s & ~7) + g * 8;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p = p0 + 128 * u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = p + i;
        if (q >= s && q < e) sum = __builtin_fmaf(zl[ic[u].get(i)], vc[u].get(i), sum);
      }
    }
    // columns longer than one batch continue with plain loads
    p0 += 128 * kU;
    if (p0 < e) {
      const uint16_t* rowidx = lt[l].rowidx;
      const void* vals = lt[l].vals;
      const uint8_t* vsc = lt[l].vsc;
      const int64_t nnz = lt[l].nnz;
      while (p0 < e) {
        IdxChunk tc[kU];
        ValChunk<VT> tv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (p0 + 128 * u < e) {
            tc[u].load(rowidx, p0 + 128 * u, nnz);
            tv[u].load(vals, vsc, p0 + 128 * u, nnz);
          }
#pragma unroll
        for (int u = 0; u < kU; ++u)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int q = p0 + 128 * u + i;
            if (q < e) sum = __builtin_fmaf(zl[tc[u].get(i)], tv[u].get(i), sum);
          }
        p0 += 128 * kU;
      }
    }
    sum = row16_sum(sum);
    if (ci < ncols && g == 0) {
      float ts = 1.0f;
      if constexpr (VT == DFS_NVFP4) ts = *gptr(lt[l].vts);
      const int j = c0 + ci - l * d_out;
      void* y = lt[l].Y;
      if (z.ydt == DFS_F16)
        gptr_w((_Float16*)y)[j] = (_Float16)(sum * ts);
      else
        gptr_w((float*)y)[j] = sum * ts;
    }
  };
  for (int r = 0; r < rounds; r += 2) {
    consume(ia, va, r);
    if (r + 2 < rounds) load_round(ia, va, r + 2);
    if (r + 1 < rounds) {
      consume(ib, vb, r + 1);
      if (r + 3 < rounds) load_round(ib, vb, r + 3);
    }
  }
}

int g_cus[64];  // CU count per device, filled on first use

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

struct Plan {
  int G, A, RT;
  size_t col_bytes, smem;
};

bool plan(const XdLaunch& xd, const ZcLaunch& zc, Plan* p) {
  const int G = device_cus();
  if (G <= 0) return false;
  const int nl = zc.n_layers;
  const int A = (xd.k + 4 * G - 1) / (4 * G);
  if (A < 1 || A > 4) return false;
  const int RT = nl <= 1 ? 1 : (nl <= 2 ? 2 : 4);
  const int seg = xd.ddt == DFS_NVFP4 ? kWave * 2 * 32 : kWave * 8 * 8;  // Cfg<.., F16, RT<=4>::SEG
  const size_t ld = (size_t)(xd.d_in + seg - 1) / seg * seg;
  const size_t xbytes = (size_t)RT * ld * 2;
  const size_t zbytes = (size_t)nl * xd.k * 4;
  const int max_cols = (nl * zc.d_out + G - 1) / G + 1;
  p->G = G;
  p->A = A;
  p->RT = RT;
  p->col_bytes = ((size_t)max_cols * 8 + 15) / 16 * 16;
  p->smem = kLayerTableBytes + p->col_bytes + (xbytes > zbytes ? xbytes : zbytes);
  return p->smem <= 128 * 1024;
}

template <int DT, int VT, int RT, int A>
hipError_t launch4(FusedLaunch f, const Plan& p, hipStream_t s) {
  auto kern = fused_decode_kernel<DT, VT, RT, A>;
  hipError_t err = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.smem);
  if (err != hipSuccess) return err;
  int per_cu = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, p.smem);
  if (err != hipSuccess) return err;
  if (per_cu < 1) return hipErrorInvalidConfiguration;  // grid must be co-resident
  f.col_bytes = (int)p.col_bytes;
  hipLaunchKernelGGL(kern, dim3(p.G), dim3(kThreads), p.smem, s, f);
  return hipGetLastError();
}

template <int DT, int VT, int RT>
hipError_t launch3(FusedLaunch f, const Plan& p, hipStream_t s) {
  switch (p.A) {
    case 1: return launch4<DT, VT, RT, 1>(f, p, s);
    case 2: return launch4<DT, VT, RT, 2>(f, p, s);
    case 3: return launch4<DT, VT, RT, 3>(f, p, s);
    default: return launch4<DT, VT, RT, 4>(f, p, s);
  }
}

template <int DT, int VT>
hipError_t launch2(FusedLaunch f, const Plan& p, hipStream_t s) {
  switch (p.RT) {
    case 1: return launch3<DT, VT, 1>(f, p, s);
    case 2: return launch3<DT, VT, 2>(f, p, s);
    default: return launch3<DT, VT, 4>(f, p, s);
  }
}

}  // namespace

bool fused_decode_supported(const XdLaunch& xd, const ZcLaunch& zc) {
  if (xd.T != 1 || zc.T != 1) return false;
  if (zc.n_layers < 1 || zc.n_layers > kFusedMaxLayers) return false;
  if (xd.xdt != DFS_F16) return false;
  if (xd.ddt != DFS_F16 && xd.ddt != DFS_NVFP4) return false;
  if (zc.vdt != DFS_F16 && zc.vdt != DFS_NVFP4) return false;
  if (xd.d_in % (xd.ddt == DFS_NVFP4 ? 32 : 8) != 0 || xd.k % 4 != 0) return false;
  Plan p;
  return plan(xd, zc, &p);
}

hipError_t launch_fused_decode(const XdLaunch& xd, const ZcLaunch& zc, float* zws,
                               uint32_t* ctrl, hipStream_t s) {
  Plan p;
  if (!plan(xd, zc, &p)) return hipErrorInvalidValue;
  FusedLaunch f;
  f.xd = xd;
  f.zc = zc;
  f.zws = zws;
  f.ctrl = ctrl;
  f.spin_limit = 1u << 22;
  f.col_bytes = 0;
  if (xd.ddt == DFS_NVFP4)
    return zc.vdt == DFS_NVFP4 ? launch2<DFS_NVFP4, DFS_NVFP4>(f, p, s)
                               : launch2<DFS_NVFP4, DFS_F16>(f, p, s);
  return zc.vdt == DFS_NVFP4 ? launch2<DFS_F16, DFS_NVFP4>(f, p, s)
                             : launch2<DFS_F16, DFS_F16>(f, p, s);
}

}  // namespace dfs
