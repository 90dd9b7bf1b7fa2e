// gemv_xd.hip -- Z = X D_g for a few stacked rows (decode), on VALU.
//
// First half of the factored projection ("DictLLM: Shared Dictionaries for
// Post-Training Compression", Eq. (1): Z_l = X_l D_g).  At decode a group
// has n_layers * T <= 16 rows, so every dictionary element is used at most
// 16 times: the kernel is a bandwidth-bound stream of D_g, which is read
// exactly once per launch however many layers share it (the group reuse of
// the review's Figure 2).
//
// Layout: D_g atom-major (atom a = d_in contiguous elements), X rows
// row-major.  One wave owns A atoms; lane l reads 16-byte chunks
// l, l+64, l+128, ... of each atom, so a wave-wide load is one fully
// coalesced 1 KiB segment.  The X rows are staged into LDS first (their
// loads must not queue behind the D stream: vector loads retire in order),
// then every chunk load of a d_in segment is issued before the first
// multiply.  The lane partial sums are reduced across the wave with DPP.
//
// Products: f16 x f16 (and E2M1 decoded to f16 x f16) use v_dot2_f32_f16,
// which multiplies exactly and accumulates in fp32; f32 operands use FMA.
#include "gemv_common.hpp"

namespace dfs {
namespace {

using namespace gemv;

// kWholeX: all of X[row0 .. row0+RT) is staged once (LDS row stride = d_in
// rounded up to SEG); otherwise one SEG-wide slice is staged per segment.
// In both cases the X loads complete before any D load is issued, and the D
// loads of a segment are all in flight before its first multiply.
template <int DT, int XT, int RT, bool kTail, bool kWholeX>
__global__ __launch_bounds__(kThreads) void gemv_xd_kernel(XdLaunch a) {
  using C = Cfg<DT, XT, RT>;
  using XS = typename C::XS;
  constexpr int CE = C::CE, A = C::A, SEGC = C::SEGC, SEG = C::SEG;
  extern __shared__ __attribute__((aligned(16))) char xs_raw[];
  XS* xs = reinterpret_cast<XS*>(xs_raw);

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int atom0 = (blockIdx.x * kWaves + wave) * A;
  const int R = a.n_layers * a.T;
  const int row0 = blockIdx.y * RT;
  const int d_in = a.d_in;
  const int ld = kWholeX ? (d_in + SEG - 1) / SEG * SEG : SEG;

  if constexpr (kWholeX) {
    stage_x<XT, RT, XS>(xs, a, row0, 0, ld, ld);
    __syncthreads();
  }

  float acc[A][RT];
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[i][r] = 0.0f;

  for (int seg = 0; seg < d_in; seg += SEG) {
    if constexpr (!kWholeX) {
      if (seg > 0) __syncthreads();
      stage_x<XT, RT, XS>(xs, a, row0, seg, SEG, SEG);
    }
    // issue every D chunk load of this segment
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
        if (atom < a.k && e0 < d_in) {
          if constexpr (DT == DFS_NVFP4) {
            const int64_t el = (int64_t)atom * d_in + e0;
            dreg[i][c] = ld16<u4>(a.dcodes + el / 2);
            sreg[i][c] = (uint32_t)a.dscales[el / 16] | ((uint32_t)a.dscales[el / 16 + 1] << 8);
          } else {
            const char* p = (const char*)a.D + ((int64_t)atom * a.ldd + e0) * (DT == DFS_F32 ? 4 : 2);
            if (!kTail || e0 + CE <= d_in)
              dreg[i][c] = ld16<u4>(p);
            else
              dreg[i][c] = load_chunk_tail<DT>(p, d_in - e0);
          }
        }
      }
    }
    if constexpr (!kWholeX) __syncthreads();

    const XS* xseg = xs + (kWholeX ? seg : 0);
#pragma unroll
    for (int c = 0; c < SEGC; ++c) {
      const int el = (c * kWave + lane) * CE;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
#pragma unroll
        for (int i = 0; i < A; ++i)
          acc[i][r] = dot_chunk<DT, C::kDot2, XS>(dreg[i][c], sreg[i][c], xseg + r * ld + el, acc[i][r]);
      }
    }
  }

  float ts = 1.0f;
  if constexpr (DT == DFS_NVFP4) ts = *a.dts;
#pragma unroll
  for (int i = 0; i < A; ++i) {
    const int atom = atom0 + i;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float v = wave_sum(acc[i][r]) * ts;
      const int row = row0 + r;
      if (lane == r && atom < a.k && row < R) {
        if (a.zdt == DFS_F32)
          ((float*)a.Z)[(int64_t)row * a.k + atom] = v;
        else
          ((_Float16*)a.Z)[(int64_t)row * a.k + atom] = (_Float16)v;
      }
    }
  }
}

template <int DT, int XT, int RT, bool kTail>
hipError_t launch_w(const XdLaunch& a, hipStream_t s, dim3 grid) {
  using C = Cfg<DT, XT, RT>;
  const size_t whole = (size_t)RT * ((a.d_in + C::SEG - 1) / C::SEG * C::SEG) * sizeof(typename C::XS);
  if (whole <= (size_t)kLdsBudget) {
    hipLaunchKernelGGL((gemv_xd_kernel<DT, XT, RT, kTail, true>), grid, dim3(kThreads), whole, s, a);
  } else {
    const size_t seg = (size_t)RT * C::SEG * sizeof(typename C::XS);
    hipLaunchKernelGGL((gemv_xd_kernel<DT, XT, RT, kTail, false>), grid, dim3(kThreads), seg, s, a);
  }
  return hipGetLastError();
}

template <int DT, int XT, int RT>
hipError_t launch_rt(const XdLaunch& a, hipStream_t s) {
  constexpr int A = DTraits<DT>::A;
  const int R = a.n_layers * a.T;
  dim3 grid((a.k + kWaves * A - 1) / (kWaves * A), (R + RT - 1) / RT);
  if (a.d_in % DTraits<DT>::CE == 0) return launch_w<DT, XT, RT, false>(a, s, grid);
  return launch_w<DT, XT, RT, true>(a, s, grid);
}

template <int DT, int XT>
hipError_t launch_xt(const XdLaunch& a, hipStream_t s) {
  // NVFP4 with f32 activations keeps 32 fp32 X values per chunk in flight:
  // cap its row tile at 2 so that nothing spills.
  constexpr int kMax = (DT == DFS_NVFP4 && XT == DFS_F32) ? 2 : DTraits<DT>::kMaxRT;
  const int R = a.n_layers * a.T;
  if (R <= 1) return launch_rt<DT, XT, 1>(a, s);
  if (R <= 2 || kMax == 2) return launch_rt<DT, XT, 2>(a, s);
  if constexpr (kMax >= 4) {
    if (R <= 4 || kMax == 4) return launch_rt<DT, XT, 4>(a, s);
  }
  if constexpr (kMax >= 16) {
    if (R <= 8) return launch_rt<DT, XT, 8>(a, s);
    return launch_rt<DT, XT, 16>(a, s);  // tiles of 16 rows over grid.y
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_dt(const XdLaunch& a, hipStream_t s) {
  return a.xdt == DFS_F16 ? launch_xt<DT, DFS_F16>(a, s) : launch_xt<DT, DFS_F32>(a, s);
}

}  // namespace

hipError_t launch_gemv_xd(const XdLaunch& a, hipStream_t s) {
  switch (a.ddt) {
    case DFS_F16:
      return launch_dt<DFS_F16>(a, s);
    case DFS_F32:
      return launch_dt<DFS_F32>(a, s);
    default:
      return launch_dt<DFS_NVFP4>(a, s);
  }
}

}  // namespace dfs
