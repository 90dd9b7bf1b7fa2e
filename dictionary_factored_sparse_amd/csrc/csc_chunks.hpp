// csc_chunks.hpp -- 8-entry chunks of a CSC coefficient stream (HIP path).
//
// The coefficient kernels read C_l as aligned groups of 8 consecutive stored
// entries: 16 bytes of uint16 row indices plus the matching values (16 bytes
// of f16, 32 bytes of f32, 8 bytes of FP8 or INT8 codes, or 4 bytes of E2M1
// codes and the one E4M3 block scale that covers them: 8 divides the
// 16-entry NVFP4 block).  The arrays
// are allocated for a whole number of chunks (dict_csc_capacity), so every
// chunk is one unconditional load; entries past nnz are masked by the caller.
// `p` is always a multiple of 8 below the capacity.
//
// Chunks are loaded well before they are used, often under a branch.  Any
// arithmetic on a loaded word that the compiler places next to its load (a
// byte shift, a scale conversion) makes the wave wait for that load there,
// and since loads retire in order, for every load before it: the stream is
// then issued one round trip at a time.  So a chunk keeps its raw words
// until use, and the kernels call touch() on it first.  For the INT8 and
// NVFP4 chunks, whose decode the compiler otherwise moved up to the load
// (INT8 C took 12.7 us instead of 10.7 in the q_proj decode group), touch()
// is an empty asm that marks the words as redefined at the use; for the
// other chunks it is empty (measured: an asm there costs about 0.1 us).
#pragma once

#include "dfs_internal.hpp"

namespace dfs {

// Start of the chunk that holds entry e - 1 (the last entry of a column that
// ends at e; 0 when e == 0).  A lane whose chunk lies past its column loads
// this one instead (in bounds, fully masked, and already fetched by a
// neighbouring lane), so every lane issues the same loads.
__device__ __forceinline__ int64_t last_chunk(int64_t e) {
  return e > 0 ? (e - 1) & ~(int64_t)7 : 0;
}

struct IdxChunk {
  u4 w;
  __device__ __forceinline__ void load(const uint16_t* rowidx, int64_t p) {
    w = ld16<u4>(rowidx + p);
  }
  __device__ __forceinline__ void touch() {}
  __device__ __forceinline__ uint32_t get(int i) const {
    return (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
  }
};

template <int VT>
struct ValChunk;

template <>
struct ValChunk<DFS_F16> {
  u4 w;
  __device__ __forceinline__ void load(const void* vals, const uint8_t*, int64_t p) {
    w = ld16<u4>((const uint16_t*)vals + p);
  }
  __device__ __forceinline__ void touch() {}
  __device__ __forceinline__ float get(int i) const {
    const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  }
};

template <>
struct ValChunk<DFS_F32> {
  u4 w0, w1;
  __device__ __forceinline__ void load(const void* vals, const uint8_t*, int64_t p) {
    const uint32_t* v = (const uint32_t*)vals;
    w0 = ld16<u4>(v + p);
    w1 = ld16<u4>(v + p + 4);
  }
  __device__ __forceinline__ void touch() {}
  __device__ __forceinline__ float get(int i) const {
    return __uint_as_float(i < 4 ? w0[i] : w1[i - 4]);
  }
};

// NVFP4: decoded value = e2m1 * e4m3(block scale); the tensor scale is
// applied once to the finished dot product.  The chunk keeps the raw code
// word and scale byte and decodes on use (hardware E2M1 conversion, exact
// with scale 1).
template <>
struct ValChunk<DFS_NVFP4> {
  uint32_t word, sc;
  __device__ __forceinline__ void load(const void* vals, const uint8_t* scales, int64_t p) {
    word = *gptr(reinterpret_cast<const uint32_t*>((const uint8_t*)vals + p / 2));
    sc = gptr(scales)[p / 16];
  }
  __device__ __forceinline__ void touch() { asm volatile("" : "+v"(word), "+v"(sc)); }
  // i is a compile-time constant after unrolling, so the switch folds away.
  __device__ __forceinline__ float get(int i) const {
    f2 v;
    switch (i >> 1) {
      case 0: v = e2m1x2_f2<0>(word); break;
      case 1: v = e2m1x2_f2<1>(word); break;
      case 2: v = e2m1x2_f2<2>(word); break;
      default: v = e2m1x2_f2<3>(word); break;
    }
    return v[i & 1] * e4m3_to_f32(sc);
  }
};

// FP8 (E4M3) and INT8 codes: 8 bytes per chunk.  get() returns the code's
// value without its column scale; the kernels multiply the finished dot
// product by col_scale[j] * kCodeScale<VT>.  An E4M3 code, its exponent and
// mantissa bits moved into the matching positions of an f16 (exponent field
// e, top three fraction bits m), is the f16 value 2^(e-15) (1 + m/8), or
// 2^-14 m/8 when e = 0: exactly 2^-8 times the E4M3 value, subnormals
// included.  So the decode is two bit operations and an f16 that multiplies
// straight into fp32 (v_fma_mix), and kCodeScale<DFS_FP8> = 256 restores the
// factor, exactly.  INT8 codes are exact in f16 and fp32.
template <int VT>
constexpr bool kIsCode8 = VT == DFS_FP8 || VT == DFS_INT8;
template <int VT>
constexpr float kCodeScale = VT == DFS_FP8 ? 256.0f : 1.0f;

template <>
struct ValChunk<DFS_FP8> {
  u2 w;
  __device__ __forceinline__ void load(const void* vals, const uint8_t*, int64_t p) {
    w = *gptr(reinterpret_cast<const u2*>((const uint8_t*)vals + p));
  }
  __device__ __forceinline__ void touch() {}
  __device__ __forceinline__ float get(int i) const {
    const uint32_t b = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
    const uint32_t h = ((b & 0x7Fu) << 7) | ((b & 0x80u) << 8);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  }
};

template <>
struct ValChunk<DFS_INT8> {
  u2 w;
  __device__ __forceinline__ void load(const void* vals, const uint8_t*, int64_t p) {
    w = *gptr(reinterpret_cast<const u2*>((const uint8_t*)vals + p));
  }
  __device__ __forceinline__ void touch() { asm volatile("" : "+v"(w)); }
  __device__ __forceinline__ float get(int i) const {
    return (float)(int8_t)(uint8_t)(w[i >> 2] >> (8 * (i & 3)));
  }
};

// Block-structured support with f16 values (blocks of 8 consecutive atoms,
// see dfs_csc): in the one-launch decode a lane's unit of the coefficient
// stream is one kept block, its 16-bit block index and its 8 values.
// kBlockF16 is a value-type code used only inside the kernels.
constexpr int kBlockF16 = 16;

template <>
struct ValChunk<kBlockF16> {
  u4 w;
  uint32_t b;
  __device__ __forceinline__ void load_block(const uint16_t* bidx, const void* vals, int64_t q) {
    b = *gptr(bidx + q);
    w = ld16<u4>((const uint16_t*)vals + 8 * q);
  }
  __device__ __forceinline__ void touch() {}
  __device__ __forceinline__ float get(int i) const {
    const uint32_t bits = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  }
};

}  // namespace dfs
