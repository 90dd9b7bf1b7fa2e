// gemm_xd.hip -- Z = X D_g on MFMA for many stacked rows (prefill).
//
// First half of the factored projection ("DictLLM: Shared Dictionaries for
// Post-Training Compression", Eq. (1): Z_l = X_l D_g) when the group brings
// enough rows (n_layers * T > 16) that the dense contraction, not the
// dictionary's bytes, sets the time (same review, "From retained values to
// measured decoding": at larger batch or prefill the multiply-adds dominate).
//
// C[M x N] = A[M x K] * B[K x N] with A = stacked X rows (row-major, K = d_in
// contiguous; row l*T + t read from layer l's pointer), B = D_g stored
// atom-major (each of the N = k atoms has its K elements contiguous), f16
// operands, fp32 accumulation in v_mfma_f32_32x32x16_f16.
//
// Tiling: a 256 x 128 output tile per workgroup of 4 waves (2 x 2), each
// wave 128 x 64 = 4 x 2 MFMA blocks of 32 x 32, so that one 16-wide slice of
// K costs a wave 6 fragment reads from LDS for 8 MFMAs.  K advances 64 at a
// time through three LDS stages filled straight from global memory
// (global_load_lds_dwordx4: each wave instruction writes 1 KiB = 8 tile rows
// of 128 bytes), so two K tiles are in flight while one is multiplied and
// no registers stage the operands.  Rows are unpadded; the eight 16-byte
// chunks of a row are stored in an XOR-swizzled slot order (see swz) that
// keeps the fragment reads free of bank conflicts.  Rows past M or N
// read a valid row and are never stored; a K tail (K % 64 != 0, K % 8 == 0)
// is zeroed in LDS after its loads land.  One workgroup per CU; tiles are
// numbered so that the workgroups that share an XCD (dispatch is
// round-robin over the 8 XCDs) cover a compact 4 x 8 block of tiles and so
// share A and B panels in their L2.
#include <type_traits>

#include "dfs_internal.hpp"

namespace dfs {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesG = kThreads / kWave;
constexpr int BK = 64;
constexpr int kRowBytes = BK * 2;  // 128
constexpr int kStages = 3;
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

// Workgroup tile BM x BN: 2 x 2 waves of (BM / 2) x (BN / 2), i.e. MI x NJ
// MFMA blocks of 32 x 32 per wave.  256 x 128 for large M; 64 x 64 when M
// (the stacked rows) is at most 128, where the large tile would leave most
// CUs idle (a 4-layer group at b = 16 has M = 64).
template <int BM, int BN>
struct Tile {
  static constexpr int kStageBytes = (BM + BN) * kRowBytes;
  static constexpr int kAInst = BM * kRowBytes / 1024 / kWavesG;  // 1 KiB loads per wave (A)
  static constexpr int kBInst = BN * kRowBytes / 1024 / kWavesG;  // (B)
  static constexpr int kLoadsPerStage = kAInst + kBInst;
  static constexpr int MI = BM / 64, NJ = BN / 64;
  static constexpr size_t kSmemBytes = (size_t)kStages * kStageBytes;
};

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8): wait until at most n vector memory ops are pending
// (and every LDS op has completed).
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// Workgroup barrier without the release/acquire fences of __syncthreads:
// those would wait for every vector memory op, i.e. for the K tiles still
// in flight.  The waits the pipeline needs are issued explicitly before it
// (the compiler does not track the LDS writes of global_load_lds), and the
// memory clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Tile (mb, nb) of workgroup `bid`: workgroups bid = x, x + 8, x + 16, ...
// run on XCD x, so consecutive positions of the tile order go to one XCD,
// and the order walks groups of kGroupM m-tiles column by column.
__device__ __forceinline__ void tile_of(int bid, int G, int MB, int NB, int* mb, int* nb) {
  int t = bid;
  if (G % kXcds == 0) t = (bid % kXcds) * (G / kXcds) + bid / kXcds;
  const int per_group = kGroupM * NB;
  const int g = t / per_group;
  const int first = g * kGroupM;
  const int gm = MB - first < kGroupM ? MB - first : kGroupM;
  const int r = t - g * per_group;
  *mb = first + r % gm;
  *nb = r / gm;
}

// Slot of K chunk c of tile row r is c ^ swz(r).  A fragment read serves
// 32 consecutive rows at one chunk; with swz(r) = (r >> 1) & 7 the rows that
// share a bank window (every 2nd row in 8, every 4th row in 16) land in
// distinct slots, so the reads are conflict-free whether the LDS serves 8 or
// 16 lanes of a 16-byte read per clock.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef const __attribute__((address_space(1))) void* glob_ptr;

// Split K (few stacked rows): a tile's K range is cut into `ks` slices of
// `kslice` elements (a multiple of BK), each done by its own workgroup, which
// writes an fp32 partial tile; a second kernel sums the slices in order.
// Without the split, 64 rows over 3072 atoms are 48 workgroups on 256 CUs.
template <int ZT, int BM, int BN>
__global__ __launch_bounds__(kThreads, 1) void gemm_xd_kernel(XdLaunch a, int ks, int kslice) {
  using TC = Tile<BM, BN>;
  constexpr int kStageBytes = TC::kStageBytes, kAInst = TC::kAInst, kBInst = TC::kBInst;
  constexpr int kLoadsPerStage = TC::kLoadsPerStage, MI = TC::MI, NJ = TC::NJ;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int M = a.n_layers * a.T, N = a.k;
  const int MB = (M + BM - 1) / BM, NB = (N + BN - 1) / BN;
  const int split = (int)blockIdx.x % ks;
  const int kbeg = split * kslice;
  const int K = min(a.d_in - kbeg, kslice);  // this workgroup's K extent
  int mb, nb;
  tile_of((int)blockIdx.x / ks, (int)gridDim.x / ks, MB, NB, &mb, &nb);
  const int m0 = mb * BM, n0 = nb * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS addresses in SGPRs
  const int wm = (wave >> 1) * (MI * 32), wn = (wave & 1) * (NJ * 32);

  // Each load instruction fills 8 tile rows; lane j writes row rr = 8 * q +
  // j / 8 (q = instruction index in the tile), LDS slot j % 8, and so reads
  // the global chunk (j % 8) ^ swz(rr) of that row.
  const _Float16* arow[kAInst];
  const _Float16* brow[kBInst];
#pragma unroll
  for (int i = 0; i < kAInst; ++i) {
    const int m = min(m0 + 8 * (wave * kAInst + i) + (lane >> 3), M - 1);
    const int l = m / a.T, t = m - l * a.T;
    arow[i] = (const _Float16*)a.X[l] + (int64_t)t * a.ldx + kbeg;
  }
#pragma unroll
  for (int i = 0; i < kBInst; ++i) {
    const int n = min(n0 + 8 * (wave * kBInst + i) + (lane >> 3), N - 1);
    brow[i] = (const _Float16*)a.D + (int64_t)n * a.ldd + kbeg;
  }
  const int nk = (K + BK - 1) / BK;
  const int nkf = K / BK;  // whole K tiles
  // Loads of K tile kt into LDS stage kt % 3.  A chunk past K (only in a
  // short last tile; K % 8 == 0 on this path) reads the row's last chunk and
  // is zeroed once it has landed.
  // K offset (elements) of this lane's chunk in load instruction q
  auto chunk_of = [&](int q) { return ((lane & 7) ^ swz(8 * q + (lane >> 3))) * 8; };
  auto issue = [&](int kt) {
    char* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int i = 0; i < kAInst; ++i) {
      const int q = wave * kAInst + i;
      const int kk = min(kt * BK + chunk_of(q), K - 8);
      __builtin_amdgcn_global_load_lds((glob_ptr)(arow[i] + kk), (lds_ptr)(st + q * 1024), 16, 0,
                                       0);
    }
#pragma unroll
    for (int i = 0; i < kBInst; ++i) {
      const int q = wave * kBInst + i;
      const int kk = min(kt * BK + chunk_of(q), K - 8);
      __builtin_amdgcn_global_load_lds((glob_ptr)(brow[i] + kk),
                                       (lds_ptr)(st + BM * kRowBytes + q * 1024), 16, 0, 0);
    }
  };
  // Whole tiles from stage 2 on: one pointer per load instruction, advanced
  // by one tile per issue (no clamp, no per-load index arithmetic).  Loads
  // [lo, hi) of the stage's list (A loads first, then B).
  const _Float16* gp[kLoadsPerStage];
#pragma unroll
  for (int i = 0; i < kAInst; ++i) gp[i] = arow[i] + 2 * BK + chunk_of(wave * kAInst + i);
#pragma unroll
  for (int i = 0; i < kBInst; ++i)
    gp[kAInst + i] = brow[i] + 2 * BK + chunk_of(wave * kBInst + i);
  auto issue_fast = [&](int kt, auto lo_c, auto hi_c) {
    constexpr int lo = decltype(lo_c)::value, hi = decltype(hi_c)::value;
    char* st = smem + (kt % kStages) * kStageBytes;
#pragma unroll
    for (int i = lo; i < hi; ++i) {
      char* dst = i < kAInst ? st + (wave * kAInst + i) * 1024
                             : st + BM * kRowBytes + (wave * kBInst + i - kAInst) * 1024;
      __builtin_amdgcn_global_load_lds((glob_ptr)gp[i], (lds_ptr)dst, 16, 0, 0);
      gp[i] += BK;
    }
  };
  auto zero_tail = [&](int kt) {
    char* st = smem + (kt % kStages) * kStageBytes;
    const u4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kAInst; ++i) {
      const int q = wave * kAInst + i;
      if (kt * BK + chunk_of(q) >= K) *reinterpret_cast<u4*>(st + q * 1024 + lane * 16) = z;
    }
#pragma unroll
    for (int i = 0; i < kBInst; ++i) {
      const int q = wave * kBInst + i;
      if (kt * BK + chunk_of(q) >= K)
        *reinterpret_cast<u4*>(st + BM * kRowBytes + q * 1024 + lane * 16) = z;
    }
  };

  f16v acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int fr = lane & 31, fc = lane >> 5;
  // Fragments of 16-wide K slice ks (lane: row fr of each 32-row block, K
  // chunk 2 * ks + fc).
  auto frags = [&](const char* as, const char* bs, int ks, h8* fa, h8* fb) {
    const int c = 2 * ks + fc;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wm + 32 * i + fr;
      fa[i] = *reinterpret_cast<const h8*>(as + r * kRowBytes + ((c ^ swz(r)) * 16));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = wn + 32 * j + fr;
      fb[j] = *reinterpret_cast<const h8*>(bs + r * kRowBytes + ((c ^ swz(r)) * 16));
    }
  };
  auto mma = [&](const h8* fa, const h8* fb) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  // Issue order of one slice for the scheduler: each MFMA followed by one
  // fragment read (masks: 0x008 MFMA, 0x100 LDS read); the slice's tile
  // loads are left to the scheduler.  A slice is a scheduling region of its
  // own (sched_barrier 0 on both sides).
  constexpr int kReads = MI + NJ, kMfma = MI * NJ;
  auto interleave = [&]() {
#pragma unroll
    for (int r = 0; r < kMfma; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (r < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Stage s's tiles are in LDS for every wave: this wave waits for its own
  // loads of s (`newer` loads issued after them may stay in flight) and for
  // its LDS reads, zero-fills a short last tile, then meets the others.
  auto stage_ready = [&](int s, int newer) {
    if (newer > 0) {
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kLoadsPerStage));
    } else {
      __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
      if (s == nk - 1 && K % BK != 0) {
        zero_tail(s);
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
      }
    }
    lds_barrier();
  };

  // Software pipeline over K tiles, three LDS stages, one barrier per tile.
  // Within tile kt: the MFMAs of slice j run while the fragments of slice
  // j + 1 are read and a quarter of tile kt + 2's loads go out (into the
  // stage tile kt - 1 used); after slice 2, tile kt + 1 is made ready (this
  // wave's loads of it have landed: only the three quarters of tile kt + 2
  // issued since may be pending), and slice 3's MFMAs cover the reads of
  // its first slice.  Reading slice 3 of
  // tile kt - 1 finished before the previous barrier, so the loads of
  // tile kt + 2 never overwrite data a wave still reads.
  issue(0);
  if (nk > 1) issue(1);
  stage_ready(0, nk > 1 ? 1 : 0);
  h8 fa0[MI], fb0[NJ], fa1[MI], fb1[NJ];
  frags(smem, smem + BM * kRowBytes, 0, fa0, fb0);
  int kt = 0;
  for (; kt + 2 < nkf; ++kt) {  // tile kt + 2 is whole: loads on advancing pointers
    __builtin_amdgcn_sched_barrier(0);
    const char* as = smem + (kt % kStages) * kStageBytes;
    const char* bs = as + BM * kRowBytes;
    constexpr int q = kLoadsPerStage / 4;
    static_assert(4 * q == kLoadsPerStage, "a quarter of the tile's loads per slice");
    frags(as, bs, 1, fa1, fb1);
    mma(fa0, fb0);
    issue_fast(kt + 2, std::integral_constant<int, 0>{}, std::integral_constant<int, q>{});
    interleave();
    frags(as, bs, 2, fa0, fb0);
    mma(fa1, fb1);
    issue_fast(kt + 2, std::integral_constant<int, q>{}, std::integral_constant<int, 2 * q>{});
    interleave();
    frags(as, bs, 3, fa1, fb1);
    mma(fa0, fb0);
    issue_fast(kt + 2, std::integral_constant<int, 2 * q>{}, std::integral_constant<int, 3 * q>{});
    interleave();
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(3 * q));
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const char* an = smem + ((kt + 1) % kStages) * kStageBytes;
    frags(an, an + BM * kRowBytes, 0, fa0, fb0);
    mma(fa1, fb1);
    issue_fast(kt + 2, std::integral_constant<int, 3 * q>{}, std::integral_constant<int, kLoadsPerStage>{});
    interleave();
  }
  for (; kt < nk; ++kt) {  // the last two tiles (and a short one): plain issue
    const char* as = smem + (kt % kStages) * kStageBytes;
    const char* bs = as + BM * kRowBytes;
    if (kt + 2 < nk) issue(kt + 2);
    frags(as, bs, 1, fa1, fb1);
    mma(fa0, fb0);
    frags(as, bs, 2, fa0, fb0);
    mma(fa1, fb1);
    frags(as, bs, 3, fa1, fb1);
    mma(fa0, fb0);
    if (kt + 1 < nk) {
      stage_ready(kt + 1, kt + 2 < nk ? 1 : 0);
      const char* an = smem + ((kt + 1) % kStages) * kStageBytes;
      frags(an, an + BM * kRowBytes, 0, fa0, fb0);
    }
    mma(fa1, fb1);
  }

  // Accumulator layout of a 32 x 32 block: lane l holds column l % 32 and
  // rows 8*(v/4) + 4*(l/32) + v%4 for v = 0..15.
  // The tile leaves through LDS when its rows are whole 16-byte pieces (f16
  // Z, fp32 Z, or the fp32 partial of a K slice): the stages are free once
  // every wave has read the last K tile, the waves write their accumulators
  // there in the output's type, and the workgroup stores 16-byte pieces,
  // whole rows per wave, instead of 2- or 4-byte stores scattered over the
  // tile's rows.  Rows are padded by 16 bytes so that the two row groups a
  // wave writes at once fall into different banks.
  auto staged_store = [&](auto tag, void* base) {
    using E = decltype(tag);
    constexpr int kPer = 16 / (int)sizeof(E);
    constexpr int RS = BN * (int)sizeof(E) + 16;  // bytes per staged row
    static_assert((size_t)BM * RS <= (size_t)kStages * kStageBytes, "tile fits the stages");
    __syncthreads();
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = wn + 32 * j + (lane & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          *reinterpret_cast<E*>(smem + r * RS + c * (int)sizeof(E)) = (E)acc[i][j][v];
        }
      }
    __syncthreads();
    constexpr int kRowPieces = BN / kPer, kPieces = BM * kRowPieces;
#pragma unroll 4
    for (int q = tid; q < kPieces; q += kThreads) {
      const int r = q / kRowPieces, c = q - r * kRowPieces;
      const int m = m0 + r, n = n0 + kPer * c;
      if (m < M && n < N)
        *reinterpret_cast<u4*>((E*)base + (int64_t)m * N + n) =
            *reinterpret_cast<const u4*>(smem + r * RS + c * 16);
    }
  };
  auto aligned = [](const void* p) { return (((uintptr_t)p) & 15) == 0; };
  if (ks > 1) {
    float* zp = a.zpart + (int64_t)split * M * N;
    if (N % 4 == 0 && aligned(zp)) {
      staged_store(0.0f, zp);
      return;
    }
  } else if constexpr (ZT == DFS_F16) {
    if (N % 8 == 0 && aligned(a.Z)) {
      staged_store((_Float16)0.0f, a.Z);
      return;
    }
  } else {
    if (N % 4 == 0 && aligned(a.Z)) {
      staged_store(0.0f, a.Z);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M && n < N) {
          if (ks > 1)
            a.zpart[((int64_t)split * M + m) * N + n] = acc[i][j][v];
          else if constexpr (ZT == DFS_F32)
            ((float*)a.Z)[(int64_t)m * N + n] = acc[i][j][v];
          else
            ((_Float16*)a.Z)[(int64_t)m * N + n] = (_Float16)acc[i][j][v];
        }
      }
    }
}

// ------------------------------------------------------------------ wide tile
// 256 x 256 outputs per workgroup of 4 waves (2 x 2), each wave 128 x 128 =
// 4 x 4 MFMA blocks: a 16-wide K slice costs a wave 8 fragment reads for 16
// MFMAs, two thirds of the reads per MFMA of the 128 x 64 wave tile, and the
// tile loads per MFMA fall by a third.  K advances 32 at a time (rows of
// 64 bytes, 4 chunks) through four LDS stages of 32 KiB, loads issued three
// tiles ahead; one barrier per 32 MFMAs of a wave, as above.
constexpr int WBK = 32, kWRowBytes = WBK * 2, kWStages = 4;
constexpr int kWAhead = kWStages - 1;  // tiles in flight ahead of the one multiplied
template <int TM, int TN>
struct WTile {
  static constexpr int kStageBytes = (TM + TN) * kWRowBytes;   // 32 KiB for 256 x 256
  static constexpr int kAInst = TM * kWRowBytes / 1024 / kWavesG;
  static constexpr int kBInst = TN * kWRowBytes / 1024 / kWavesG;
  static constexpr int kLoads = kAInst + kBInst;              // per wave per tile
  static constexpr size_t kSmemBytes = (size_t)kWStages * kStageBytes;
  static constexpr int MI = TM / 64, NJ = TN / 64;            // 32 x 32 blocks per wave
};

// Slot of chunk c of a 64-byte row r is c ^ wswz(r): the 32 rows of a
// fragment read land in distinct 16-byte bank slots for 8- and for 16-lane
// windows (two rows share a 128-byte window, four a 256-byte one).
__device__ __forceinline__ int wswz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

template <int ZT, int WBM, int WBN, int OCC>
__global__ __launch_bounds__(kThreads, OCC) void gemm_xd_wide_kernel(XdLaunch a) {
  using WT = WTile<WBM, WBN>;
  constexpr int MI = WT::MI, NJ = WT::NJ, kWAInst = WT::kAInst, kWBInst = WT::kBInst;
  constexpr int kWLoads = WT::kLoads, kWStageBytes = WT::kStageBytes;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int M = a.n_layers * a.T, N = a.k, K = a.d_in;
  const int MB = (M + WBM - 1) / WBM, NB = (N + WBN - 1) / WBN;
  int mb, nb;
  tile_of((int)blockIdx.x, (int)gridDim.x, MB, NB, &mb, &nb);
  const int m0 = mb * WBM, n0 = nb * WBN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = (wave >> 1) * (WBM / 2), wn = (wave & 1) * (WBN / 2);

  // Load instruction q fills 16 rows: lane j writes
  // row 16 q + j / 4, slot j % 4, and reads that row's chunk (j % 4) ^ wswz.
  const _Float16* arow[kWAInst];
  const _Float16* brow[kWBInst];
#pragma unroll
  for (int i = 0; i < kWAInst; ++i) {
    const int m = min(m0 + 16 * (wave * kWAInst + i) + (lane >> 2), M - 1);
    const int l = m / a.T, t = m - l * a.T;
    arow[i] = (const _Float16*)a.X[l] + (int64_t)t * a.ldx;
  }
#pragma unroll
  for (int i = 0; i < kWBInst; ++i) {
    const int n = min(n0 + 16 * (wave * kWBInst + i) + (lane >> 2), N - 1);
    brow[i] = (const _Float16*)a.D + (int64_t)n * a.ldd;
  }
  const int nk = (K + WBK - 1) / WBK;
  const int nkf = K / WBK;
  auto chunk_of = [&](int q) { return ((lane & 3) ^ wswz(16 * q + (lane >> 2))) * 8; };
  auto issue = [&](int kt) {  // clamped: any tile, a short last one included
    char* st = smem + (kt % kWStages) * kWStageBytes;
#pragma unroll
    for (int i = 0; i < kWAInst; ++i) {
      const int q = wave * kWAInst + i;
      const int kk = min(kt * WBK + chunk_of(q), K - 8);
      __builtin_amdgcn_global_load_lds((glob_ptr)(arow[i] + kk), (lds_ptr)(st + q * 1024), 16, 0,
                                       0);
    }
#pragma unroll
    for (int i = 0; i < kWBInst; ++i) {
      const int q = wave * kWBInst + i;
      const int kk = min(kt * WBK + chunk_of(q), K - 8);
      __builtin_amdgcn_global_load_lds((glob_ptr)(brow[i] + kk),
                                       (lds_ptr)(st + WBM * kWRowBytes + q * 1024), 16, 0, 0);
    }
  };
  // whole tiles from tile 3 on: pointers advanced by one tile per issue
  const _Float16* gp[kWLoads];
#pragma unroll
  for (int i = 0; i < kWAInst; ++i) gp[i] = arow[i] + kWAhead * WBK + chunk_of(wave * kWAInst + i);
#pragma unroll
  for (int i = 0; i < kWBInst; ++i)
    gp[kWAInst + i] = brow[i] + kWAhead * WBK + chunk_of(wave * kWBInst + i);
  auto issue_fast = [&](int kt, auto lo_c, auto hi_c) {
    constexpr int lo = decltype(lo_c)::value, hi = decltype(hi_c)::value;
    char* st = smem + (kt % kWStages) * kWStageBytes;
#pragma unroll
    for (int i = lo; i < hi; ++i) {
      char* dst = i < kWAInst ? st + (wave * kWAInst + i) * 1024
                              : st + WBM * kWRowBytes + (wave * kWBInst + i - kWAInst) * 1024;
      __builtin_amdgcn_global_load_lds((glob_ptr)gp[i], (lds_ptr)dst, 16, 0, 0);
      gp[i] += WBK;
    }
  };
  auto zero_tail = [&](int kt) {
    char* st = smem + (kt % kWStages) * kWStageBytes;
    const u4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kWAInst; ++i) {
      const int q = wave * kWAInst + i;
      if (kt * WBK + chunk_of(q) >= K) *reinterpret_cast<u4*>(st + q * 1024 + lane * 16) = z;
    }
#pragma unroll
    for (int i = 0; i < kWBInst; ++i) {
      const int q = wave * kWBInst + i;
      if (kt * WBK + chunk_of(q) >= K)
        *reinterpret_cast<u4*>(st + WBM * kWRowBytes + q * 1024 + lane * 16) = z;
    }
  };

  f16v acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const int fr = lane & 31, fc = lane >> 5;
  auto frags = [&](const char* st, int ks, h8* fa, h8* fb) {
    const int c = 2 * ks + fc;
    const char* bs = st + WBM * kWRowBytes;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int r = wm + 32 * i + fr;
      fa[i] = *reinterpret_cast<const h8*>(st + r * kWRowBytes + ((c ^ wswz(r)) * 16));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int r = wn + 32 * j + fr;
      fb[j] = *reinterpret_cast<const h8*>(bs + r * kWRowBytes + ((c ^ wswz(r)) * 16));
    }
  };
  auto mma = [&](const h8* fa, const h8* fb) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };
  auto interleave = [&]() {  // each MFMA followed by one fragment read
#pragma unroll
    for (int r = 0; r < MI * NJ; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (r < MI + NJ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // stage s ready for every wave: own loads of s landed (`newer` loads of
  // later tiles may be pending), LDS reads done, short tile zero-filled
  auto stage_ready = [&](int s, int newer) {
    static_assert(kWAhead <= 4, "wait counts below cover up to 3 newer tiles");
    switch (newer) {
      case 0:
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
        if (s == nk - 1 && K % WBK != 0) {
          zero_tail(s);
          __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
        }
        break;
      case 1: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(kWLoads)); break;
      case 2: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * kWLoads)); break;
      default: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(3 * kWLoads)); break;
    }
    lds_barrier();
  };

  // Pipeline: tile kt in stage kt % 4.  Slice 0's MFMAs run while slice 1 is
  // read and half of tile kt + 3 goes out (into the stage tile kt - 1 used,
  // which every wave finished reading before the previous barrier); then
  // tile kt + 1 is made ready (this wave's loads of it have landed: tile
  // kt + 2 and half of kt + 3 may be pending) and slice 1's MFMAs cover the
  // reads of its first slice while the other half of tile kt + 3 goes out.
  for (int t = 0; t < kWAhead; ++t)
    if (t < nk) issue(t);
  stage_ready(0, min(nk, kWAhead) - 1);
  h8 fa0[MI], fb0[NJ], fa1[MI], fb1[NJ];
  frags(smem, 0, fa0, fb0);
  int kt = 0;
  for (; kt + kWAhead < nkf; ++kt) {
    __builtin_amdgcn_sched_barrier(0);
    const char* st = smem + (kt % kWStages) * kWStageBytes;
    frags(st, 1, fa1, fb1);
    mma(fa0, fb0);
    issue_fast(kt + kWAhead, std::integral_constant<int, 0>{},
               std::integral_constant<int, kWLoads / 2>{});
    interleave();
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((kWAhead - 2) * kWLoads + kWLoads / 2));
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    frags(smem + ((kt + 1) % kWStages) * kWStageBytes, 0, fa0, fb0);
    mma(fa1, fb1);
    issue_fast(kt + kWAhead, std::integral_constant<int, kWLoads / 2>{},
               std::integral_constant<int, kWLoads>{});
    interleave();
  }
  for (; kt < nk; ++kt) {  // the last tiles (and a short one): plain issue
    const char* st = smem + (kt % kWStages) * kWStageBytes;
    if (kt + kWAhead < nk) issue(kt + kWAhead);
    frags(st, 1, fa1, fb1);
    mma(fa0, fb0);
    if (kt + 1 < nk) {
      stage_ready(kt + 1, min(nk - 1, kt + kWAhead) - (kt + 1));
      frags(smem + ((kt + 1) % kWStages) * kWStageBytes, 0, fa0, fb0);
    }
    mma(fa1, fb1);
  }

  // f16 Z with whole 16-byte pieces per row leaves through LDS, half a tile
  // (one row of waves) per pass, as in gemm_xd_kernel: 2-byte stores
  // scattered over the tile's rows would sit at the end of every workgroup.
  if constexpr (ZT == DFS_F16) {
    if (N % 8 == 0 && (((uintptr_t)a.Z) & 15) == 0) {
      constexpr int HR = WBM / 2;       // rows per pass
      constexpr int RS = WBN * 2 + 16;  // bytes per staged row, padded
      static_assert((size_t)HR * RS <= WT::kSmemBytes, "half a tile fits the stages");
      constexpr int kRowPieces = WBN / 8, kPieces = HR * kRowPieces;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        __syncthreads();
        if ((wave >> 1) == pass) {
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              const int c = wn + 32 * j + (lane & 31);
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                const int r = 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                *reinterpret_cast<_Float16*>(smem + r * RS + c * 2) = (_Float16)acc[i][j][v];
              }
            }
        }
        __syncthreads();
#pragma unroll 4
        for (int q = tid; q < kPieces; q += kThreads) {
          const int r = q / kRowPieces, c = q - r * kRowPieces;
          const int m = m0 + pass * HR + r, n = n0 + 8 * c;
          if (m < M && n < N)
            *reinterpret_cast<u4*>((_Float16*)a.Z + (int64_t)m * N + n) =
                *reinterpret_cast<const u4*>(smem + r * RS + c * 16);
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int n = n0 + wn + 32 * j + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M && n < N) {
          if constexpr (ZT == DFS_F32)
            ((float*)a.Z)[(int64_t)m * N + n] = acc[i][j][v];
          else
            ((_Float16*)a.Z)[(int64_t)m * N + n] = (_Float16)acc[i][j][v];
        }
      }
    }
}

// Z = the sum of the ks partial products, in slice order (deterministic).
template <int ZT>
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float* part, int ks, int64_t n,
                                                         void* Z) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = part[i];
  for (int q = 1; q < ks; ++q) v += part[q * n + i];
  if constexpr (ZT == DFS_F32)
    ((float*)Z)[i] = v;
  else
    ((_Float16*)Z)[i] = (_Float16)v;
}

// Expand an atom-major NVFP4 dictionary to f16 (element i = e2m1 * e4m3 *
// ts, rounded once to f16) so the MFMA path can consume it.
__global__ __launch_bounds__(256) void nvfp4_to_f16_kernel(const uint8_t* codes,
                                                           const uint8_t* scales, const float* ts,
                                                           int64_t n, _Float16* out) {
  const int64_t i8 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i8 >= n) return;
  const float t = *ts;
  const float s = e4m3_to_f32(scales[i8 / 16]) * t;
  const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + i8 / 2);
  const f2 v0 = e2m1x2_f2<0>(w), v1 = e2m1x2_f2<1>(w), v2 = e2m1x2_f2<2>(w),
           v3 = e2m1x2_f2<3>(w);
  h8 o = {(_Float16)(v0[0] * s), (_Float16)(v0[1] * s), (_Float16)(v1[0] * s),
          (_Float16)(v1[1] * s), (_Float16)(v2[0] * s), (_Float16)(v2[1] * s),
          (_Float16)(v3[0] * s), (_Float16)(v3[1] * s)};
  *reinterpret_cast<h8*>(out + i8) = o;
}

int gemm_wide_tiles(int64_t rows, int n_atoms) {
  return (int)((rows + 255) / 256) * ((n_atoms + 255) / 256);
}

template <int ZT, int BM, int BN>
hipError_t launch_tile(const XdLaunch& a, hipStream_t s) {
  auto kern = gemm_xd_kernel<ZT, BM, BN>;
  constexpr size_t smem = Tile<BM, BN>::kSmemBytes;
  hipError_t err = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int M = a.n_layers * a.T;
  const int tiles = ((M + BM - 1) / BM) * ((a.k + BN - 1) / BN);
  const int ks = BM == 64 ? gemm_split_k(M, a.k, a.d_in) : 1;
  const int nkt = (a.d_in + BK - 1) / BK;
  const int kslice = (nkt + ks - 1) / ks * BK;
  hipLaunchKernelGGL(kern, dim3((unsigned)(tiles * ks)), dim3(kThreads), smem, s, a, ks, kslice);
  if (ks > 1) {
    const int64_t n = (int64_t)M * a.k;
    hipLaunchKernelGGL(splitk_sum_kernel<ZT>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       a.zpart, ks, n, a.Z);
  }
  return hipGetLastError();
}

template <int ZT, int TM, int TN, int OCC>
hipError_t launch_wide(const XdLaunch& a, hipStream_t s) {
  auto kern = gemm_xd_wide_kernel<ZT, TM, TN, OCC>;
  constexpr size_t smem = WTile<TM, TN>::kSmemBytes;
  hipError_t err = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int64_t M = (int64_t)a.n_layers * a.T;
  const int tiles = (int)((M + TM - 1) / TM) * ((a.k + TN - 1) / TN);
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(kThreads), smem, s, a);
  return hipGetLastError();
}

template <int ZT>
hipError_t launch_z(const XdLaunch& a, hipStream_t s) {
  if (a.n_layers * a.T <= 128) return launch_tile<ZT, 64, 64>(a, s);
  if (gemm_wide_tiles(a.n_layers * a.T, a.k) >= 256) return launch_wide<ZT, 256, 256, 1>(a, s);
  return launch_tile<ZT, 256, 128>(a, s);
}

}  // namespace

// Enough slices that tiles * slices reaches about one workgroup per CU (256),
// each slice at least 4 K tiles; only for the 64 x 64 tile (<= 128 rows).
int gemm_split_k(int64_t rows, int n_atoms, int d_in) {
  if (rows > 128) return 1;
  const int tiles = (int)((rows + 63) / 64) * ((n_atoms + 63) / 64);
  const int nkt = (d_in + BK - 1) / BK;
  int ks = (256 + tiles - 1) / tiles;
  ks = min(ks, nkt / 4);
  ks = max(ks, 1);
  // equal slices of whole K tiles: no slice may come out empty
  while (ks > 1 && (int64_t)((nkt + ks - 1) / ks) * (ks - 1) >= nkt) --ks;
  return ks;
}

hipError_t launch_gemm_xd_mfma(const XdLaunch& a, hipStream_t s) {
  return a.zdt == DFS_F32 ? launch_z<DFS_F32>(a, s) : launch_z<DFS_F16>(a, s);
}

// n must be a multiple of 8 (the caller checks d_in % 32 == 0).
hipError_t launch_nvfp4_to_f16(const uint8_t* codes, const uint8_t* scales, const float* ts,
                               int64_t n, _Float16* out, hipStream_t s) {
  const int64_t threads = n / 8;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(nvfp4_to_f16_kernel, dim3(blocks), dim3(256), 0, s, codes, scales, ts, n,
                     out);
  return hipGetLastError();
}

}  // namespace dfs
