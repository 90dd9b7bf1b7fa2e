// gemv_common.hpp -- device pieces of Z = X D_g on VALU, shared by the
// decode GEMV and the fused decode kernel (HIP path only).
//
// A 16-byte chunk of an atom holds CE elements (f32: 4, f16: 8, NVFP4: 32
// codes = two 16-element blocks).  dot_chunk multiplies one chunk with the
// matching X elements staged in LDS: f16 x f16 (and E2M1 decoded to f16)
// with v_dot2_f32_f16, which multiplies exactly and accumulates in fp32;
// f32 operands with FMA.
#pragma once

#include "dfs_internal.hpp"

namespace dfs {
namespace gemv {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kLdsBudget = 64 * 1024;

template <int DT>
struct DTraits;
template <>
struct DTraits<DFS_F32> {
  static constexpr int CE = 4;       // elements per 16-byte chunk
  static constexpr int A = 2;        // atoms per wave
  static constexpr int kMaxRT = 16;  // rows per launch tile
};
template <>
struct DTraits<DFS_F16> {
  static constexpr int CE = 8;
  static constexpr int A = 2;
  static constexpr int kMaxRT = 16;
};
template <>
struct DTraits<DFS_NVFP4> {
  static constexpr int CE = 32;
  static constexpr int A = 4;
  static constexpr int kMaxRT = 4;   // 32-element chunks: keep registers and LDS bounded
};


template <int DT, int XT, int RT>
struct Cfg {
  static constexpr bool kDot2 = (DT != DFS_F32) && (XT == DFS_F16);
  using XS = typename std::conditional<kDot2, _Float16, float>::type;
  static constexpr int CE = DTraits<DT>::CE;
  static constexpr int A = DTraits<DT>::A;
  static constexpr int kSegcDefault = DT == DFS_NVFP4 ? 2 : 8;
  static constexpr int kSegcFit = kLdsBudget / (RT * (int)sizeof(XS) * kWave * CE);
  static constexpr int SEGC = kSegcFit < 1 ? 1 : (kSegcFit < kSegcDefault ? kSegcFit : kSegcDefault);
  static constexpr int SEG = kWave * SEGC * CE;  // elements of d_in per segment
};

// Elementwise-guarded load of the last, partial chunk of an atom.
template <int DT>
__device__ __forceinline__ u4 load_chunk_tail(const void* base, int valid) {
  u4 r = {0u, 0u, 0u, 0u};
  if constexpr (DT == DFS_F32) {
    const uint32_t* p = (const uint32_t*)base;
    for (int i = 0; i < valid; ++i) r[i] = p[i];
  } else if constexpr (DT == DFS_F16) {
    const uint16_t* p = (const uint16_t*)base;
    uint16_t tmp[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < valid; ++i) tmp[i] = p[i];
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)tmp[2 * i] | ((uint32_t)tmp[2 * i + 1] << 16);
  }
  return r;  // NVFP4 dictionaries have d_in % 32 == 0: no partial chunk
}

// Dot product of one 16-byte D chunk with the matching X elements in LDS.
template <int DT, bool kDot2, typename XS>
__device__ __forceinline__ float dot_chunk(u4 d, uint32_t sc2, const XS* x, float acc) {
  if constexpr (DT == DFS_F16 && kDot2) {
    const h8 xv = *reinterpret_cast<const h8*>(x);
    const h2* dh = reinterpret_cast<const h2*>(&d);
    acc = __builtin_amdgcn_fdot2(dh[0], h2{xv[0], xv[1]}, acc, false);
    acc = __builtin_amdgcn_fdot2(dh[1], h2{xv[2], xv[3]}, acc, false);
    acc = __builtin_amdgcn_fdot2(dh[2], h2{xv[4], xv[5]}, acc, false);
    acc = __builtin_amdgcn_fdot2(dh[3], h2{xv[6], xv[7]}, acc, false);
    return acc;
  } else if constexpr (DT == DFS_F16) {
    const f4 x0 = *reinterpret_cast<const f4*>(x);
    const f4 x1 = *reinterpret_cast<const f4*>(x + 4);
    const _Float16* dh = reinterpret_cast<const _Float16*>(&d);
    acc = __builtin_fmaf((float)dh[0], x0[0], acc);
    acc = __builtin_fmaf((float)dh[1], x0[1], acc);
    acc = __builtin_fmaf((float)dh[2], x0[2], acc);
    acc = __builtin_fmaf((float)dh[3], x0[3], acc);
    acc = __builtin_fmaf((float)dh[4], x1[0], acc);
    acc = __builtin_fmaf((float)dh[5], x1[1], acc);
    acc = __builtin_fmaf((float)dh[6], x1[2], acc);
    acc = __builtin_fmaf((float)dh[7], x1[3], acc);
    return acc;
  } else if constexpr (DT == DFS_F32) {
    const f4 x0 = *reinterpret_cast<const f4*>(x);
    acc = __builtin_fmaf(__uint_as_float(d[0]), x0[0], acc);
    acc = __builtin_fmaf(__uint_as_float(d[1]), x0[1], acc);
    acc = __builtin_fmaf(__uint_as_float(d[2]), x0[2], acc);
    acc = __builtin_fmaf(__uint_as_float(d[3]), x0[3], acc);
    return acc;
  } else {
    // NVFP4: 32 elements = two 16-element blocks, words 0-1 and 2-3.
    const float s0 = e4m3_to_f32(sc2 & 0xFFu);
    const float s1 = e4m3_to_f32((sc2 >> 8) & 0xFFu);
    float b[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float p = 0.0f;
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t word = d[2 * h + w];
        const XS* xw = x + 16 * h + 8 * w;
        if constexpr (kDot2) {
          const h8 xv = *reinterpret_cast<const h8*>(xw);
          p = __builtin_amdgcn_fdot2(e2m1x2_h2<0>(word), h2{xv[0], xv[1]}, p, false);
          p = __builtin_amdgcn_fdot2(e2m1x2_h2<1>(word), h2{xv[2], xv[3]}, p, false);
          p = __builtin_amdgcn_fdot2(e2m1x2_h2<2>(word), h2{xv[4], xv[5]}, p, false);
          p = __builtin_amdgcn_fdot2(e2m1x2_h2<3>(word), h2{xv[6], xv[7]}, p, false);
        } else {
          const f4 x0 = *reinterpret_cast<const f4*>(xw);
          const f4 x1 = *reinterpret_cast<const f4*>(xw + 4);
          f2 v;
          v = e2m1x2_f2<0>(word);
          p = __builtin_fmaf(v[0], x0[0], p);
          p = __builtin_fmaf(v[1], x0[1], p);
          v = e2m1x2_f2<1>(word);
          p = __builtin_fmaf(v[0], x0[2], p);
          p = __builtin_fmaf(v[1], x0[3], p);
          v = e2m1x2_f2<2>(word);
          p = __builtin_fmaf(v[0], x1[0], p);
          p = __builtin_fmaf(v[1], x1[1], p);
          v = e2m1x2_f2<3>(word);
          p = __builtin_fmaf(v[0], x1[2], p);
          p = __builtin_fmaf(v[1], x1[3], p);
        }
      }
      b[h] = p;
    }
    acc = __builtin_fmaf(b[0], s0, acc);
    acc = __builtin_fmaf(b[1], s1, acc);
    return acc;
  }
}

// Stage rows [row0, row0 + RT) x elements [e_begin, e_begin + n_el) of the
// stacked X into LDS rows of stride `ld` (zero padded past d_in and past the
// last row), 8 elements per item, kUnr items per thread in flight.  Row base
// pointers are wave-uniform and come from scalar loads, so the vector-memory
// counter only ever waits on these X loads here.
template <int XT, int RT, typename XS>
__device__ __forceinline__ void stage_x(XS* xs, const XdLaunch& a, int row0, int e_begin,
                                        int n_el, int ld) {
  constexpr int kUnr = 4;
  constexpr int kWords = XT == DFS_F16 ? 4 : 8;  // 32-bit words per 8 elements
  constexpr int esz = XT == DFS_F16 ? 2 : 4;
  const int R = a.n_layers * a.T;
  const char* rowp[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int row = row0 + r;
    rowp[r] = nullptr;
    if (row < R) {
      const int l = row / a.T, t = row - l * a.T;
      rowp[r] = (const char*)a.X[l] + (int64_t)t * a.ldx * esz;
    }
  }
  const int per_row = n_el / 8;
  const int n_items = RT * per_row;
  for (int base = 0; base < n_items; base += kThreads * kUnr) {
    uint32_t v[kUnr][kWords];
#pragma unroll
    for (int j = 0; j < kUnr; ++j) {
      const int item = base + j * kThreads + threadIdx.x;
      const int r = item / per_row;
      const int ge = e_begin + (item - r * per_row) * 8;
      const char* p = rowp[0];
#pragma unroll
      for (int rr = 1; rr < RT; ++rr)
        if (r == rr) p = rowp[rr];
#pragma unroll
      for (int w = 0; w < kWords; ++w) v[j][w] = 0u;
      if (item < n_items && p != nullptr && ge < a.d_in) {
        p += (int64_t)ge * esz;
        if (ge + 8 <= a.d_in) {
          const u4 q0 = ld16<u4>(p);
          v[j][0] = q0[0]; v[j][1] = q0[1]; v[j][2] = q0[2]; v[j][3] = q0[3];
          if constexpr (XT == DFS_F32) {
            const u4 q1 = ld16<u4>(p + 16);
            v[j][4] = q1[0]; v[j][5] = q1[1]; v[j][6] = q1[2]; v[j][7] = q1[3];
          }
        } else {
          for (int e = 0; e < a.d_in - ge; ++e) {
            if constexpr (XT == DFS_F16) {
              const uint32_t h = ((const uint16_t*)p)[e];
              v[j][e >> 1] |= (e & 1) ? (h << 16) : h;
            } else {
              v[j][e] = ((const uint32_t*)p)[e];
            }
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kUnr; ++j) {
      const int item = base + j * kThreads + threadIdx.x;
      if (item < n_items) {
        const int r = item / per_row;
        XS* dst = xs + r * ld + (item - r * per_row) * 8;
        if constexpr (sizeof(XS) == 2) {
          *reinterpret_cast<u4*>(dst) = u4{v[j][0], v[j][1], v[j][2], v[j][3]};
        } else if constexpr (XT == DFS_F16) {  // f16 -> f32 in LDS
          f4 lo, hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t wl = v[j][e >> 1], wh = v[j][2 + (e >> 1)];
            lo[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)((e & 1) ? wl >> 16 : wl));
            hi[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)((e & 1) ? wh >> 16 : wh));
          }
          *reinterpret_cast<f4*>(dst) = lo;
          *reinterpret_cast<f4*>(dst + 4) = hi;
        } else {  // f32 -> f32
          *reinterpret_cast<u4*>(dst) = u4{v[j][0], v[j][1], v[j][2], v[j][3]};
          *reinterpret_cast<u4*>(dst + 4) = u4{v[j][4], v[j][5], v[j][6], v[j][7]};
        }
      }
    }
  }
}

}  // namespace gemv
}  // namespace dfs
