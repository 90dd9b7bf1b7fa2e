// pack_csc.hip -- dense coefficients -> CSC with 16-bit atom indices.
//
// The support-keeping export of C_l ("DictLLM: Shared Dictionaries for
// Post-Training Compression", Algorithm 2: export of dictionary, codes,
// scales and support, zeros preserved): column j keeps the rows r, in
// ascending order, whose entry is nonzero (tested on the bits, so +-0 are
// dropped and NaN and subnormals are kept), stores r as uint16 and copies
// the value bits.
//
// Three phases, all deterministic:
//   count    thread (column j, chunk of 64 rows) counts its nonzeros;
//            counts are laid out [j][chunk], i.e. in CSC order;
//   scan     exclusive scan of the counts (block sums in int64) gives every
//            (j, chunk) its output offset, colptr[j] = offset of (j, 0);
//   scatter  thread (j, chunk) rewrites its nonzeros at its offset, rows
//            ascending, so the result is the unique canonical CSC.
// The same phases pack the block-structured variant (blocks of BR = 8
// consecutive rows of a column, kept whole when one entry is nonzero; the
// Review's "Let the accelerator constrain the support"): counts are of kept
// blocks, and the scatter writes the block index and its 8 values.
#include "dfs_internal.hpp"

namespace dfs {
namespace {

constexpr int kRowChunk = 64;
constexpr int kScanThreads = 256;
constexpr int kScanItems = 8;
constexpr int kScanTile = kScanThreads * kScanItems;

// Workspace: the int64 total first (the host reads it back), then the tile
// sums, then the per-(column, chunk) counts.
struct PackWs {
  int32_t* counts;   // [d_out * n_rc], scanned in place into offsets
  int64_t* bsum;     // [n_tiles + 1]
  int64_t* total;    // [1], at the start of the workspace
  int64_t n_items;
  int n_tiles;
};

__host__ __device__ inline int n_row_chunks(int k) { return (k + kRowChunk - 1) / kRowChunk; }

__host__ __device__ inline PackWs carve(void* ws, int k, int d_out) {
  PackWs w;
  const int n_rc = n_row_chunks(k);
  w.n_items = (int64_t)d_out * n_rc;
  w.n_tiles = (int)((w.n_items + kScanTile - 1) / kScanTile);
  char* p = (char*)ws;
  w.total = (int64_t*)p;
  p += 256;
  w.bsum = (int64_t*)p;
  p += ((size_t)(w.n_tiles + 1) * 8 + 255) / 256 * 256;
  w.counts = (int32_t*)p;
  return w;
}

template <int DT>
__device__ __forceinline__ bool nonzero_at(const void* C, int64_t i) {
  if constexpr (DT == DFS_F32)
    return (((const uint32_t*)C)[i] & 0x7FFFFFFFu) != 0u;
  else
    return (((const uint16_t*)C)[i] & 0x7FFFu) != 0u;
}

// Whether block [r, r + BR) of column j (rows past k count as 0) holds a
// nonzero; BR = 1 is a single entry.
template <int DT, int BR>
__device__ __forceinline__ bool block_nonzero(const void* C, int r, int k, int64_t ldc, int j) {
  bool any = false;
#pragma unroll
  for (int e = 0; e < BR; ++e)
    if (r + e < k) any |= nonzero_at<DT>(C, (int64_t)(r + e) * ldc + j);
  return any;
}

template <int DT, int BR>
__global__ __launch_bounds__(256) void count_kernel(const void* C, int k, int d_out, int64_t ldc,
                                                    int32_t* counts) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int rc = blockIdx.y;
  if (j >= d_out) return;
  const int r1 = min(k, (rc + 1) * kRowChunk);
  int c = 0;
  for (int r = rc * kRowChunk; r < r1; r += BR) c += block_nonzero<DT, BR>(C, r, k, ldc, j);
  counts[(int64_t)j * gridDim.y + rc] = c;
}

// Phase 1 of the scan: per-tile sums.
__global__ __launch_bounds__(kScanThreads) void tile_sum_kernel(const int32_t* counts,
                                                                int64_t n, int64_t* bsum) {
  __shared__ int64_t red[kScanThreads];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * kScanItems;
  int64_t s = 0;
  for (int i = 0; i < kScanItems; ++i)
    if (base + i < n) s += counts[base + i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = kScanThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) bsum[blockIdx.x] = red[0];
}

// Phase 2: exclusive scan of the tile sums in one workgroup; total out.
__global__ __launch_bounds__(kScanThreads) void tile_scan_kernel(int64_t* bsum, int n_tiles,
                                                                 int64_t* total) {
  __shared__ int64_t buf[kScanThreads];
  int64_t carry = 0;
  for (int base = 0; base < n_tiles; base += kScanThreads) {
    const int i = base + threadIdx.x;
    const int64_t v = i < n_tiles ? bsum[i] : 0;
    buf[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {  // inclusive Hillis-Steele
      const int64_t add = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
      __syncthreads();
      buf[threadIdx.x] += add;
      __syncthreads();
    }
    if (i < n_tiles) bsum[i] = carry + buf[threadIdx.x] - v;
    const int64_t tile_total = buf[kScanThreads - 1];
    __syncthreads();
    carry += tile_total;
  }
  if (threadIdx.x == 0) total[0] = carry;
}

// Phase 3: scan inside each tile, write offsets in place and colptr.
__global__ __launch_bounds__(kScanThreads) void tile_apply_kernel(int32_t* counts, int64_t n,
                                                                  const int64_t* bsum,
                                                                  const int64_t* total, int n_rc,
                                                                  int d_out, int32_t* colptr) {
  __shared__ int64_t buf[kScanThreads];
  const int64_t base = (int64_t)blockIdx.x * kScanTile + threadIdx.x * kScanItems;
  int32_t v[kScanItems];
  int64_t s = 0;
  for (int i = 0; i < kScanItems; ++i) {
    v[i] = base + i < n ? counts[base + i] : 0;
    s += v[i];
  }
  buf[threadIdx.x] = s;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int64_t add = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
    __syncthreads();
    buf[threadIdx.x] += add;
    __syncthreads();
  }
  int64_t run = bsum[blockIdx.x] + buf[threadIdx.x] - s;
  for (int i = 0; i < kScanItems; ++i) {
    const int64_t idx = base + i;
    if (idx < n) {
      counts[idx] = (int32_t)run;  // offsets stay < 2^31 whenever they are used
      if (idx % n_rc == 0) colptr[idx / n_rc] = (int32_t)run;
    }
    run += v[i];
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) colptr[d_out] = (int32_t)total[0];
}

template <int DT, int BR>
__global__ __launch_bounds__(256) void scatter_kernel(const void* C, int k, int d_out, int64_t ldc,
                                                      const int32_t* offsets, uint16_t* rowidx,
                                                      void* vals) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int rc = blockIdx.y;
  if (j >= d_out) return;
  int64_t o = offsets[(int64_t)j * gridDim.y + rc];
  const int r1 = min(k, (rc + 1) * kRowChunk);
  for (int r = rc * kRowChunk; r < r1; r += BR) {
    if (!block_nonzero<DT, BR>(C, r, k, ldc, j)) continue;
    rowidx[o] = (uint16_t)(r / BR);
#pragma unroll
    for (int e = 0; e < BR; ++e) {
      const int64_t i = (int64_t)(r + e) * ldc + j;
      const bool in = r + e < k;
      if constexpr (DT == DFS_F32)
        ((uint32_t*)vals)[o * BR + e] = in ? ((const uint32_t*)C)[i] : 0u;
      else
        ((uint16_t*)vals)[o * BR + e] = in ? ((const uint16_t*)C)[i] : (uint16_t)0;
    }
    ++o;
  }
}

}  // namespace

size_t pack_csc_ws_bytes(int32_t k, int32_t d_out) {
  const int n_rc = n_row_chunks(k);
  const int64_t items = (int64_t)d_out * n_rc;
  const int64_t tiles = (items + kScanTile - 1) / kScanTile;
  return 256 + (size_t)((tiles + 1) * 8 + 255) / 256 * 256 + (size_t)items * 4 + 256;
}

hipError_t launch_pack_csc_count(const void* C, int32_t dtype, int32_t k, int32_t d_out,
                                 int64_t ldc, int32_t* colptr, void* ws, hipStream_t s,
                                 int block_rows) {
  PackWs w = carve(ws, k, d_out);
  const int n_rc = n_row_chunks(k);
  dim3 grid((d_out + 255) / 256, n_rc);
  auto kern = count_kernel<DFS_F16, 1>;
  if (dtype == DFS_F32)
    kern = block_rows == 8 ? count_kernel<DFS_F32, 8> : count_kernel<DFS_F32, 1>;
  else if (block_rows == 8)
    kern = count_kernel<DFS_F16, 8>;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, C, k, d_out, ldc, w.counts);
  hipLaunchKernelGGL(tile_sum_kernel, dim3(w.n_tiles), dim3(kScanThreads), 0, s, w.counts,
                     w.n_items, w.bsum);
  hipLaunchKernelGGL(tile_scan_kernel, dim3(1), dim3(kScanThreads), 0, s, w.bsum, w.n_tiles,
                     w.total);
  hipLaunchKernelGGL(tile_apply_kernel, dim3(w.n_tiles), dim3(kScanThreads), 0, s, w.counts,
                     w.n_items, w.bsum, w.total, n_rc, d_out, colptr);
  return hipGetLastError();
}

hipError_t launch_pack_csc_scatter(const void* C, int32_t dtype, int32_t k, int32_t d_out,
                                   int64_t ldc, uint16_t* rowidx, void* vals, const void* ws,
                                   hipStream_t s, int block_rows) {
  PackWs w = carve(const_cast<void*>(ws), k, d_out);
  dim3 grid((d_out + 255) / 256, n_row_chunks(k));
  auto kern = scatter_kernel<DFS_F16, 1>;
  if (dtype == DFS_F32)
    kern = block_rows == 8 ? scatter_kernel<DFS_F32, 8> : scatter_kernel<DFS_F32, 1>;
  else if (block_rows == 8)
    kern = scatter_kernel<DFS_F16, 8>;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, C, k, d_out, ldc, w.counts, rowidx, vals);
  return hipGetLastError();
}

}  // namespace dfs
