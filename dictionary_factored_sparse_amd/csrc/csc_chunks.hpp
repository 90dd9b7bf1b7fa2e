// csc_chunks.hpp -- 8-entry chunks of a CSC coefficient stream (HIP path).
//
// The coefficient kernels read C_l as aligned groups of 8 consecutive stored
// entries: 16 bytes of uint16 row indices plus the matching values (16 bytes
// of f16, 32 bytes of f32, or 4 bytes of E2M1 codes and the one E4M3 block
// scale that covers them: 8 divides the 16-entry NVFP4 block).  A chunk that
// would run past the end of the arrays is read entry by entry.
#pragma once

#include "dfs_internal.hpp"

namespace dfs {

struct IdxChunk {
  u4 w;
  __device__ __forceinline__ void load(const uint16_t* rowidx, int64_t p, int64_t nnz) {
    if (p + 8 <= nnz) {
      w = ld16<u4>(rowidx + p);
    } else {
      uint32_t t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int i = 0; i < 8; ++i)
        if (p + i < nnz) t[i] = gptr(rowidx)[p + i];
      w = u4{t[0] | (t[1] << 16), t[2] | (t[3] << 16), t[4] | (t[5] << 16), t[6] | (t[7] << 16)};
    }
  }
  __device__ __forceinline__ uint32_t get(int i) const {
    return (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
  }
};

template <int VT>
struct ValChunk;

template <>
struct ValChunk<DFS_F16> {
  u4 w;
  __device__ __forceinline__ void load(const void* vals, const uint8_t*, int64_t p, int64_t nnz) {
    const uint16_t* v = (const uint16_t*)vals;
    if (p + 8 <= nnz) {
      w = ld16<u4>(v + p);
    } else {
      uint32_t t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int i = 0; i < 8; ++i)
        if (p + i < nnz) t[i] = gptr(v)[p + i];
      w = u4{t[0] | (t[1] << 16), t[2] | (t[3] << 16), t[4] | (t[5] << 16), t[6] | (t[7] << 16)};
    }
  }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  }
};

template <>
struct ValChunk<DFS_F32> {
  u4 w0, w1;
  __device__ __forceinline__ void load(const void* vals, const uint8_t*, int64_t p, int64_t nnz) {
    const uint32_t* v = (const uint32_t*)vals;
    if (p + 8 <= nnz) {
      w0 = ld16<u4>(v + p);
      w1 = ld16<u4>(v + p + 4);
    } else {
      uint32_t t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int i = 0; i < 8; ++i)
        if (p + i < nnz) t[i] = gptr(v)[p + i];
      w0 = u4{t[0], t[1], t[2], t[3]};
      w1 = u4{t[4], t[5], t[6], t[7]};
    }
  }
  __device__ __forceinline__ float get(int i) const {
    return __uint_as_float(i < 4 ? w0[i] : w1[i - 4]);
  }
};

// NVFP4: decoded value = e2m1 * e4m3(block scale); the tensor scale is
// applied once to the finished dot product.  The chunk keeps the raw code
// word and decodes on use (hardware E2M1 conversion, exact with scale 1).
template <>
struct ValChunk<DFS_NVFP4> {
  uint32_t word;
  float s;
  __device__ __forceinline__ void load(const void* vals, const uint8_t* scales, int64_t p,
                                       int64_t nnz) {
    const uint8_t* codes = (const uint8_t*)vals;
    if (p + 8 <= nnz) {
      word = *gptr(reinterpret_cast<const uint32_t*>(codes + p / 2));
    } else {
      word = 0;
      for (int i = 0; i < 8; i += 2)
        if (p + i < nnz) word |= (uint32_t)gptr(codes)[(p + i) / 2] << (4 * i);
    }
    s = e4m3_to_f32(gptr(scales)[p / 16]);
  }
  // i is a compile-time constant after unrolling, so the switch folds away.
  __device__ __forceinline__ float get(int i) const {
    f2 v;
    switch (i >> 1) {
      case 0: v = e2m1x2_f2<0>(word); break;
      case 1: v = e2m1x2_f2<1>(word); break;
      case 2: v = e2m1x2_f2<2>(word); break;
      default: v = e2m1x2_f2<3>(word); break;
    }
    return v[i & 1] * s;
  }
};

}  // namespace dfs
