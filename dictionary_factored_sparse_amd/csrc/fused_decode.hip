// fused_decode.hip -- one launch for a decode group: Z = X D_g, then every
// Y_l = Z_l C_l ("DictLLM: Shared Dictionaries for Post-Training
// Compression", Eq. (1) and Figure 2: one dictionary, separate activations).
//
// At decode both halves stream bytes from HBM: D_g (read once for the whole
// group) and each C_l.  Run as two kernels, C_l's stream cannot start until
// the Z kernel ends.  Here one persistent grid (one workgroup per CU) does
// both:
//   1. each workgroup puts its X rows and its slice of D_g's atoms in flight;
//   2. it computes its atoms' Z and publishes them as epoch-tagged words;
//   3. it issues the loads of its coefficient columns (they do not depend on
//      Z), then receives the Z rows of its layers (polling for the current
//      epoch) into LDS while those loads arrive;
//   4. it finishes its columns, later rounds of C double-buffered in
//      registers.
// So the Z dependency costs one round trip through memory, hidden under the
// C stream, instead of a second launch.  The grid never exceeds one
// workgroup per CU.  Should the grid still not be resident all at once
// (other kernels holding CUs), a bounded wait gives up and the workgroup
// computes the Z words it lacks itself, so the result stays right and the
// kernel always terminates.
#include <cstdlib>
#include <type_traits>

#include "csc_chunks.hpp"
#include "gemv_common.hpp"

namespace dfs {
namespace {

using namespace gemv;

constexpr int kU = 6;  // 8-entry C chunks per lane per batch
constexpr int kLayerTableBytes = 256;
constexpr int kFT = 512;          // threads per workgroup (2 waves per SIMD)
constexpr int kFW = kFT / kWave;  // waves per workgroup
constexpr int kSlots = kFW * 4;   // columns per round (4 per wave)

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

// Hand-off of Z between workgroups without a grid barrier.  Each Z entry is
// one 64-bit word (epoch << 32 | fp32 bits) written with a single agent-scope
// atomic store, so a reader that sees the current epoch also sees the value;
// readers poll exactly the entries they need with agent-scope loads (these
// bypass the non-coherent caches), so no cache-wide fence is needed.
// The tagged region (caller's workspace after the control block, zero before
// first use and kept by the calls): one epoch word per workgroup, then the
// tagged Z words.  Workgroup w reads its epoch word, uses epoch + 1 and
// stores it back; every launch advances every word once, so all workgroups
// of a launch agree on the epoch, and every word a call reads carries its
// epoch only once this call has published it.  The control block holds only
// the diagnostic word at byte 128 (set when a wait gave up), so re-zeroing
// it between calls is harmless.
constexpr int kCtrlErr = 32;  // in 32-bit words


__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_agent64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Launder a kernel-argument pointer through SGPRs so that a lane-dependent
// choice among a few of them stays a register select (the compiler would
// otherwise turn the select chain into a vector load from the argument
// segment, which then waits behind every load already in flight).
template <typename T>
__device__ __forceinline__ T* sreg_ptr(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// sum += Z[idx] * v over the 8 entries of a chunk whose positions p..p+7 lie
// in [s, e); the other entries are masked without a branch, so the 8 LDS
// gathers of a chunk are issued back to back.
template <int VT>
__device__ __forceinline__ float gather_chunk(const float* zl, IdxChunk ic, ValChunk<VT> vc,
                                              int p, int s, int e, float sum) {
  ic.touch();
  vc.touch();
  const uint32_t len = (uint32_t)(e - s);
  const int base = p - s;
  float z[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool ok = (uint32_t)(base + i) < len;
    z[i] = zl[ok ? ic.get(i) : 0u];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const bool ok = (uint32_t)(base + i) < len;
    const float prod = z[i] * vc.get(i);
    sum += ok ? prod : 0.0f;
  }
  return sum;
}

// sum += Z[8b .. 8b + 7] . v for one kept block at position q of a column
// whose blocks lie in [s, e) (block-structured coefficients): the block's 8
// Z words are contiguous in LDS, two 16-byte reads.  A block outside the
// column (or not loaded) reads block 0 and adds nothing.
__device__ __forceinline__ float gather_block(const float* zl, const ValChunk<kBlockF16>& vc,
                                              int q, int s, int e, float sum) {
  const bool ok = (uint32_t)(q - s) < (uint32_t)(e - s);
  const float* zb = zl + 8 * (ok ? vc.b : 0u);
  const f4 z0 = *reinterpret_cast<const f4*>(zb);
  const f4 z1 = *reinterpret_cast<const f4*>(zb + 4);
  float d = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) d = __builtin_fmaf(z0[i], vc.get(i), d);
#pragma unroll
  for (int i = 0; i < 4; ++i) d = __builtin_fmaf(z1[i], vc.get(4 + i), d);
  return sum + (ok ? d : 0.0f);
}

// Kernel arguments, compact so that they fit a few scalar-cache lines: the
// first line holds everything the first loads need.  NU units (the outputs:
// one coefficient matrix and Y each), 4 for one dictionary (one unit per
// layer) and 8 for several (one per dictionary and layer).
template <int NU>
struct FusedArgs {
  const void* D;  // f16 atoms, or NVFP4 codes
  const uint8_t* dscales;
  int64_t ldd;
  int32_t d_in, k;
  const void* X[kFusedMaxLayers];
  const int32_t* colptr[NU];
  const uint16_t* rowidx[NU];
  const void* vals[NU];
  const uint8_t* vscales[NU];
  const float* vts[NU];  // NVFP4 tensor scale, or FP8/INT8 column scales
  void* Y[NU];
  int64_t nnz[NU];
  const float* dts;
  uint64_t* zz;        // units x k epoch-tagged Z words
  uint32_t* epochs;    // one epoch word per workgroup
  uint32_t* ctrl;      // control block (diagnostic word)
  int32_t n_layers, d_out, ydt;
  uint32_t spin_limit;  // polls of one Z word before it is computed locally
  int32_t col_bytes;
  int32_t G;  // workgroups in the grid
  int32_t z_off;  // byte offset of the received Z from the X rows in LDS
  // several dictionaries over the same X rows: their count, and the codes,
  // block scales and tensor scale of dictionaries 1 and 2 (same d_in, k, ldd
  // and dtype as dictionary 0)
  int32_t n_dicts;
  const void* Dx[kFusedMaxDicts - 1];
  const uint8_t* dscalesx[kFusedMaxDicts - 1];
  const float* dtsx[kFusedMaxDicts - 1];
};

// A column's entry in LDS: [start, end) of its stored entries, and for 8-bit
// codes the bits of its scale (times kCodeScale).
template <int VT>
using ColEntry = typename std::conditional<kIsCode8<VT>, int4, int2>::type;

// Units of the argument struct and bytes of the LDS unit table for ND
// dictionaries.
template <int ND>
constexpr int units_of() { return ND == 1 ? kFusedMaxLayers : kFusedMaxUnits; }
template <int ND>
constexpr int table_bytes_of() { return ND == 1 ? kLayerTableBytes : 2 * kLayerTableBytes; }
static_assert(sizeof(LayerRow) * kFusedMaxLayers <= kLayerTableBytes, "unit table");
static_assert(sizeof(LayerRow) * kFusedMaxUnits <= 2 * kLayerTableBytes, "unit table");

// ND dictionaries over the same X rows: atoms [d k, (d + 1) k) of the atom
// space are dictionary d's, and unit d * n_layers + l (coefficients and Y)
// reads Z row l of dictionary d.  ND = 1 is the group of one dictionary.
template <int DT, int VT, int RT, int A, int NX, int ND>
__global__ __launch_bounds__(kFT, 1) void fused_decode_kernel(FusedArgs<units_of<ND>()> f) {
  using Cf = Cfg<DT, DFS_F16, RT>;
  using CE_t = ColEntry<VT>;
  constexpr bool Q8 = kIsCode8<VT>;
  constexpr bool BLK = VT == kBlockF16;  // 8-atom blocks: a lane's unit is one block
  constexpr int CE = Cf::CE, SEGC = Cf::SEGC, SEG = Cf::SEG;
  constexpr int NU = units_of<ND>(), kTable = table_bytes_of<ND>();
  // Rounds of columns in flight before Z is received, and chunks per lane
  // per batch.  Several dictionaries give a workgroup more columns (q, k, v
  // over two layers: three rounds), so all three go out ahead, with batches
  // of 5 chunks (640 entries per column) to fit the registers.
  constexpr int NB = ND > 1 ? 3 : 2;
  // 8-atom blocks: 9 blocks per lane per batch (the registers of 6 chunks)
  constexpr int KU = BLK ? 9 : (ND > 1 ? 5 : kU);
  // positions a lane's batch entries are apart, and the lane's first one
  constexpr int STEP = BLK ? 16 : 128;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  LayerRow* lt = reinterpret_cast<LayerRow*>(smem);            // [NU]
  CE_t* cse = reinterpret_cast<CE_t*>(smem + kTable);          // [ncols]
  char* big = smem + kTable + f.col_bytes;                     // X rows, then Z
  _Float16* xs = reinterpret_cast<_Float16*>(big);
  float* zs = reinterpret_cast<float*>(big + f.z_off);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int g = lane & 15;
  // Every kernel argument needed before the first wait is fetched in one
  // batch of scalar loads (one round trip instead of one per first use).
  const int d_in = f.d_in, k = f.k, d_out = f.d_out, nl = f.n_layers;
  if constexpr (Q8)  // the column scales are read with the column bounds
    asm volatile("" ::"s"(d_in), "s"(k), "s"(d_out), "s"(nl), "s"(f.D), "s"(f.ldd), "s"(f.X[0]),
                 "s"(f.X[RT > 1 ? 1 : 0]), "s"(f.epochs), "s"(f.colptr[0]), "s"(f.colptr[1]),
                 "s"(f.colptr[2]), "s"(f.colptr[3]), "s"(f.col_bytes), "s"(f.G), "s"(f.vts[0]),
                 "s"(f.vts[1]), "s"(f.vts[2]), "s"(f.vts[3]));
  else if constexpr (DT == DFS_NVFP4)
    // an NVFP4 dictionary streams in a quarter of the time, so a kernel
    // argument line first touched after it (the value pointers, before the
    // coefficient loads) shows in the step: fetch every line up front
    // (measured 0.2-0.3 us faster; no gain with an f16 dictionary)
    asm volatile("" ::"s"(d_in), "s"(k), "s"(d_out), "s"(nl), "s"(f.D), "s"(f.ldd), "s"(f.X[0]),
                 "s"(f.X[RT > 1 ? 1 : 0]), "s"(f.epochs), "s"(f.colptr[0]), "s"(f.colptr[1]),
                 "s"(f.colptr[2]), "s"(f.colptr[3]), "s"(f.col_bytes), "s"(f.G), "s"(f.vals[0]),
                 "s"(f.vts[0]), "s"(f.z_off));
  else
    asm volatile("" ::"s"(d_in), "s"(k), "s"(d_out), "s"(nl), "s"(f.D), "s"(f.ldd), "s"(f.X[0]),
                 "s"(f.X[RT > 1 ? 1 : 0]), "s"(f.epochs), "s"(f.colptr[0]), "s"(f.colptr[1]),
                 "s"(f.colptr[2]), "s"(f.colptr[3]), "s"(f.col_bytes), "s"(f.G));
  if constexpr (ND > 1)
    asm volatile("" ::"s"(f.Dx[0]), "s"(f.Dx[ND > 2 ? 1 : 0]), "s"(f.dscalesx[0]),
                 "s"(f.dscalesx[ND > 2 ? 1 : 0]), "s"(f.colptr[4]), "s"(f.colptr[5]));
  static_assert(SEG % (8 * kFT) == 0, "an X row is a whole number of 512-thread passes");
  constexpr int NR = NX / RT;  // passes of the workgroup per X row
  static_assert(NR * RT == NX, "X register count");
  const int ld = (d_in + SEG - 1) / SEG * SEG;  // == NR * 8 * kFT

  // Order of the loads.  Vector loads retire in order, so a wait for one
  // load also waits for every older one.  Issued first are the small loads
  // whose values are needed early (X, the epoch word, the column bounds),
  // then this workgroup's atoms of D_g.  The coefficient columns are issued
  // only once the workgroup's own atoms have arrived and Z is published:
  // the memory system serves requests roughly in arrival order, so D_g is
  // never queued behind C, Z is ready after about half of the stream, and
  // the Z hand-off runs while the C half is arriving.  Loads are issued
  // without branches (out-of-range addresses are clamped and the values
  // masked), so the compiler can count exactly how many are in flight.
  // ---- 1. X rows (all of d_in, zero padded to ld), held in registers
  u4 xr[NX];
#pragma unroll
  for (int jx = 0; jx < NX; ++jx) {
    const int r = jx / NR;
    const int ge = ((jx % NR) * kFT + tid) * 8;
    const _Float16* xrow = (const _Float16*)(r < nl ? sreg_ptr(f.X[r]) : sreg_ptr(f.X[0]));
    const bool ok = r < nl && ge < d_in;
    const u4 v = ld16<u4>(xrow + (ok ? ge : 0));  // d_in % 8 == 0 on this path
    xr[jx] = ok ? v : u4{0u, 0u, 0u, 0u};
  }
  // ---- 2. this launch's epoch word and the bounds of this workgroup's columns
  const int nu = ND == 1 ? nl : ND * nl;  // units: (dictionary, layer) pairs
  const uint32_t NC = (uint32_t)(nu * d_out);  // NC * (G + 1) < 2^32 (host check)
  const int c0 = (int)(blockIdx.x * NC / (uint32_t)f.G);
  const int c1 = (int)((blockIdx.x + 1) * NC / (uint32_t)f.G);
  const int ncols = c1 - c0;  // <= kFT (checked on the host)
  const int rounds = (ncols + kSlots - 1) / kSlots;
  const uint32_t epoch_old = ld_agent(f.epochs + blockIdx.x);
  // this lane's columns in the first NB rounds (16 lanes per column)
  const int slot = wave * 4 + (lane >> 4);
  int rs_raw[NB], re_raw[NB], rl[NB];
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    const int ci = r * kSlots + slot < ncols ? r * kSlots + slot : 0;
    const int l = (c0 + ci) / d_out, j = c0 + ci - l * d_out;
    const int32_t* cpr = sreg_ptr(f.colptr[0]);
#pragma unroll
    for (int i = 1; i < NU; ++i)
      if (l == i) cpr = sreg_ptr(f.colptr[i]);
    rs_raw[r] = gptr(cpr)[j];
    re_raw[r] = gptr(cpr)[j + 1];
    rl[r] = l;
  }
  // this thread's column (one per thread, for the LDS table of later rounds)
  const int cidx = tid < ncols ? tid : 0;
  const int cl = (c0 + cidx) / d_out, cj = c0 + cidx - cl * d_out;
  const int32_t* cp = sreg_ptr(f.colptr[0]);
#pragma unroll
  for (int i = 1; i < NU; ++i)
    if (cl == i) cp = sreg_ptr(f.colptr[i]);
  const int s_raw = gptr(cp)[cj], e_raw = gptr(cp)[cj + 1];
  float cs_raw = 1.0f;
  if constexpr (Q8) {
    const float* vp = sreg_ptr(f.vts[0]);
#pragma unroll
    for (int i = 1; i < NU; ++i)
      if (cl == i) vp = sreg_ptr(f.vts[i]);
    cs_raw = gptr(vp)[cj];
  }

  // ---- 3. this workgroup's atoms of D_g.  Out-of-range reads are clamped,
  // not masked: an atom past k reads atom k - 1 (its Z is never published),
  // a chunk past d_in reads the atom's last chunk and meets the zero padding
  // of X, so it adds 0 (or propagates a non-finite value of that same atom).
  const int atom0 = (blockIdx.x * kFW + wave) * A;
  u4 dreg[A][SEGC];
  uint32_t sreg[A][SEGC];
  // atom i of this wave: dictionary dict_of(i), index atom_of(i) within it
  // (ND = 1: dictionary 0; past the last atom, the last atom is read)
  auto dict_of = [&](int i) {
    if constexpr (ND == 1) return 0;
    else return min(atom0 + i, ND * k - 1) / k;
  };
  auto atom_of = [&](int i) {
    if constexpr (ND == 1) return min(atom0 + i, k - 1);
    else return min(atom0 + i, ND * k - 1) - dict_of(i) * k;
  };
  auto load_d = [&](int seg) {
#pragma unroll
    for (int i = 0; i < A; ++i) {
      const int atom = atom_of(i);
      const int dd = dict_of(i);
      // constant indices only: a computed index into the argument arrays
      // would make the compiler copy them to private memory
      const void* Dd = f.D;
      const uint8_t* Sd = f.dscales;
      if constexpr (ND > 1) {
        Dd = dd == 1 ? f.Dx[0] : Dd;
        Sd = dd == 1 ? f.dscalesx[0] : Sd;
      }
      if constexpr (ND > 2) {
        Dd = dd == 2 ? f.Dx[1] : Dd;
        Sd = dd == 2 ? f.dscalesx[1] : Sd;
      }
#pragma unroll
      for (int c = 0; c < SEGC; ++c) {
        const int e0 = min(seg + (c * kWave + lane) * CE, d_in - CE);
        if constexpr (DT == DFS_NVFP4) {
          const int64_t el = (int64_t)atom * d_in + e0;
          dreg[i][c] = ld16<u4>((const uint8_t*)Dd + el / 2);
          sreg[i][c] = (uint32_t)gptr(Sd)[el / 16] | ((uint32_t)gptr(Sd)[el / 16 + 1] << 8);
        } else {
          dreg[i][c] = ld16<u4>((const _Float16*)Dd + (int64_t)atom * f.ldd + e0);
          sreg[i][c] = 0u;
        }
      }
    }
  };
  load_d(0);

  // ---- 4. layer table (scalar loads) and X into LDS (waits for X only)
  if (tid == 0) {
#pragma unroll
    for (int l = 0; l < NU; ++l)
      lt[l] = LayerRow{f.colptr[l], f.rowidx[l], f.vals[l], f.vscales[l], f.vts[l], f.Y[l], f.nnz[l]};
  }
#pragma unroll
  for (int jx = 0; jx < NX; ++jx)
    *reinterpret_cast<u4*>(xs + (jx / NR) * ld + ((jx % NR) * kFT + tid) * 8) = xr[jx];
  __syncthreads();

  // ---- 5. Z for this workgroup's atoms; 6. published as epoch-tagged words
  float acc[A][RT];
#pragma unroll
  for (int i = 0; i < A; ++i)
#pragma unroll
    for (int r = 0; r < RT; ++r) acc[i][r] = 0.0f;
  for (int seg = 0; seg < d_in; seg += SEG) {
    if (seg > 0) load_d(seg);
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
  float dts[ND];
  dts[0] = 1.0f;
  if constexpr (DT == DFS_NVFP4) dts[0] = *gptr(f.dts);
  if constexpr (ND > 1) dts[1] = DT == DFS_NVFP4 ? *gptr(f.dtsx[0]) : 1.0f;
  if constexpr (ND > 2) dts[2] = DT == DFS_NVFP4 ? *gptr(f.dtsx[1]) : 1.0f;
  const uint32_t epoch = epoch_old + 1u;
#pragma unroll
  for (int i = 0; i < A; ++i) {
    const int dd = dict_of(i), atom = atom_of(i);
    const bool live = atom0 + i < ND * k;  // atoms past the last one publish nothing
    float ts = dts[0];
#pragma unroll
    for (int d = 1; d < ND; ++d) ts = dd == d ? dts[d] : ts;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const float v = wave_sum(acc[i][r]) * ts;
      // Z row of unit dd * nl + r (ND = 1: row r)
      if (lane == r && live && r < nl)
        st_agent64(f.zz + (int64_t)(dd * nl + r) * k + atom,
                   ((uint64_t)epoch << 32) | __float_as_uint(v));
    }
  }

  // Groups of 4 layers: the waves meet once every one has issued its Z
  // stores, before any coefficient load of the workgroup goes out.  The
  // stores then leave the CU ahead of that stream instead of queueing behind
  // it; with 4 layers the C stream is large and a late publication delays
  // every workgroup's receive (MLP gate group 34.5 -> 32.0 us, down 30.9 ->
  // 30.0 us).  For smaller groups the receive waits for the coefficients
  // either way, and the barrier only delays them.
  if constexpr (ND == 1 && RT == 4) asm volatile("s_barrier" ::: "memory");

  // ---- 7. the column ranges into LDS; the first NB rounds of C in flight (their
  // bounds are older than D, so nothing here waits)
  if (tid < ncols) {
    const int nz = (int)lt[cl].nnz;
    const int s0 = min(max(s_raw, 0), nz);
    const int e0 = min(max(e_raw, s0), nz);
    if constexpr (Q8)
      cse[tid] = make_int4(s0, e0, __float_as_int(cs_raw * kCodeScale<VT>), 0);
    else
      cse[tid] = make_int2(s0, e0);
  }
  // A lane loads only the chunks inside its column: here nothing waits for
  // an exact count of these loads (the Z polls issued after them wait for
  // all of them), and skipping the lanes past the column's end saves their
  // share of the memory pipeline.
  auto lane_first = [&](int s0) -> int { return BLK ? s0 + g : (s0 & ~7) + g * 8; };
  auto load_chunks = [&](IdxChunk* ic, ValChunk<VT>* vc, int s0, int e0, const uint16_t* rowidx,
                         const void* vals, const uint8_t* vsc) {
    const int p0 = lane_first(s0);
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const int p = p0 + STEP * u;
      if (p < e0) {
        if constexpr (BLK) {
          vc[u].load_block(rowidx, vals, p);
        } else {
          ic[u].load(rowidx, p);
          vc[u].load(vals, vsc, p);
        }
      }
    }
  };
  IdxChunk ia[KU], ib[KU], ie[NB > 2 ? KU : 1];
  ValChunk<VT> va[KU], vb[KU], ve[NB > 2 ? KU : 1];
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    const int l = rl[r];
    const uint16_t* rowidx = sreg_ptr(f.rowidx[0]);
    const void* vals = sreg_ptr(f.vals[0]);
    const uint8_t* vsc = sreg_ptr(f.vscales[0]);
    int64_t nnz = f.nnz[0];
#pragma unroll
    for (int i = 1; i < NU; ++i)
      if (l == i) {
        rowidx = sreg_ptr(f.rowidx[i]);
        vals = sreg_ptr(f.vals[i]);
        vsc = sreg_ptr(f.vscales[i]);
        nnz = f.nnz[i];
      }
    const bool live = r * kSlots + slot < ncols;
    const int s0 = live ? (int)min<int64_t>(max(rs_raw[r], 0), nnz) : 0;
    const int e0 = live ? (int)min<int64_t>(max(re_raw[r], s0), nnz) : 0;
    if (r == 0)
      load_chunks(ia, va, s0, e0, rowidx, vals, vsc);
    else if (r == 1 && rounds > 1)
      load_chunks(ib, vb, s0, e0, rowidx, vals, vsc);
    else if (r == 2 && rounds > 2)
      load_chunks(ie, ve, s0, e0, rowidx, vals, vsc);
  }
  auto load_round = [&](IdxChunk* ic, ValChunk<VT>* vc, int r) {
    const int ci = r * kSlots + slot;
    if (ci < ncols) {
      const CE_t se = cse[ci];
      const LayerRow& L = lt[(c0 + ci) / d_out];
      load_chunks(ic, vc, se.x, se.y, L.rowidx, L.vals, L.vsc);
    }
  };

  // ---- 8. receive the Z rows of this workgroup's units into LDS, 16 words
  // per thread at a time.  A word still missing after spin_limit polls (at
  // once when spin_limit is 0) is computed here from the X rows in LDS and
  // D_g (same definition, another summation order), and the diagnostic word
  // is set.
  {
    const int l_first = c0 / d_out, l_last = (c1 - 1) / d_out;
    const int n = (l_last - l_first + 1) * k;
    const uint64_t* zsrc = f.zz + (int64_t)l_first * k;
    float* zdst = zs + l_first * k;
    auto local_z = [&](int idx) {
      const int u = l_first + idx / k, atom = idx - (idx / k) * k;
      const int dd = ND == 1 ? 0 : u / nl;
      const void* Dd = f.D;
      const uint8_t* Sd = f.dscales;
      if constexpr (ND > 1) {
        Dd = dd == 1 ? f.Dx[0] : Dd;
        Sd = dd == 1 ? f.dscalesx[0] : Sd;
      }
      if constexpr (ND > 2) {
        Dd = dd == 2 ? f.Dx[1] : Dd;
        Sd = dd == 2 ? f.dscalesx[1] : Sd;
      }
      const _Float16* x = xs + (u - dd * nl) * ld;
      float acc = 0.0f;
#pragma unroll 1
      for (int e0 = 0; e0 < d_in; e0 += CE) {
        u4 dv;
        uint32_t sc = 0u;
        if constexpr (DT == DFS_NVFP4) {
          const int64_t el = (int64_t)atom * d_in + e0;
          dv = ld16<u4>((const uint8_t*)Dd + el / 2);
          sc = (uint32_t)gptr(Sd)[el / 16] | ((uint32_t)gptr(Sd)[el / 16 + 1] << 8);
        } else {
          dv = ld16<u4>((const _Float16*)Dd + (int64_t)atom * f.ldd + e0);
        }
        acc = dot_chunk<DT, true, _Float16>(dv, sc, x + e0, acc);
      }
      float ts = dts[0];
#pragma unroll
      for (int d = 1; d < ND; ++d) ts = dd == d ? dts[d] : ts;
      return acc * ts;
    };
    constexpr int kPer = 16;
    for (int base = 0; base < n; base += kFT * kPer) {
      uint32_t pending = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (base + j * kFT + tid < n) pending |= 1u << j;
      for (uint32_t it = 0; pending; ++it) {
        if (it >= f.spin_limit) {
          st_agent(f.ctrl + kCtrlErr, 1u);
#pragma unroll 1
          for (int j = 0; j < kPer; ++j)
            if (pending & (1u << j)) zdst[base + j * kFT + tid] = local_z(base + j * kFT + tid);
          break;
        }
        if (it > 0) __builtin_amdgcn_s_sleep(1);
        uint64_t w[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (pending & (1u << j)) w[j] = ld_agent64(zsrc + base + j * kFT + tid);
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if ((pending & (1u << j)) && (uint32_t)(w[j] >> 32) == epoch) {
            zdst[base + j * kFT + tid] = __uint_as_float((uint32_t)w[j]);
            pending &= ~(1u << j);
          }
      }
    }
  }
  __syncthreads();
  // every wave has published and received: advance this workgroup's epoch
  if (tid == 0) st_agent(f.epochs + blockIdx.x, epoch);

  // ---- 9. the columns, NB rounds in flight
  auto consume = [&](const IdxChunk* ic, const ValChunk<VT>* vc, int r) {
    const int ci = r * kSlots + slot;
    int s = 0, e = 0, l = 0;
    float ts = 1.0f;
    if (ci < ncols) {
      const CE_t se = cse[ci];
      s = se.x;
      e = se.y;
      l = (c0 + ci) / d_out;
      if constexpr (Q8) ts = __int_as_float(se.z);
    }
    const float* zl = zs + l * k;
    float sum = 0.0f;
    int p0 = lane_first(s);
    auto gather = [&](const IdxChunk& ic1, const ValChunk<VT>& vc1, int p, float acc) {
      if constexpr (BLK)
        return gather_block(zl, vc1, p, s, e, acc);
      else
        return gather_chunk<VT>(zl, ic1, vc1, p, s, e, acc);
    };
#pragma unroll
    for (int u = 0; u < KU; ++u) sum = gather(ic[u], vc[u], p0 + STEP * u, sum);
    // columns longer than one batch continue with plain loads
    p0 += STEP * KU;
    if (p0 < e) {
      const LayerRow& L = lt[l];
      while (p0 < e) {
        IdxChunk tc[KU];
        ValChunk<VT> tv[KU];
#pragma unroll
        for (int u = 0; u < KU; ++u)
          if (p0 + STEP * u < e) {
            if constexpr (BLK) {
              tv[u].load_block(L.rowidx, L.vals, p0 + STEP * u);
            } else {
              tc[u].load(L.rowidx, p0 + STEP * u);
              tv[u].load(L.vals, L.vsc, p0 + STEP * u);
            }
          }
#pragma unroll
        for (int u = 0; u < KU; ++u) sum = gather(tc[u], tv[u], p0 + STEP * u, sum);
        p0 += STEP * KU;
      }
    }
    sum = row16_sum(sum);
    if (ci < ncols && g == 0) {
      if constexpr (VT == DFS_NVFP4) ts = *gptr(lt[l].vts);
      const int j = c0 + ci - l * d_out;
      void* y = lt[l].Y;
      if (f.ydt == DFS_F16)
        gptr_w((_Float16*)y)[j] = (_Float16)(sum * ts);
      else
        gptr_w((float*)y)[j] = sum * ts;
    }
  };
  if constexpr (NB == 2) {
    for (int r = 0; r < rounds; r += 2) {
      consume(ia, va, r);
      if (r + 2 < rounds) load_round(ia, va, r + 2);
      if (r + 1 < rounds) {
        consume(ib, vb, r + 1);
        if (r + 3 < rounds) load_round(ib, vb, r + 3);
      }
    }
  } else {
    for (int r = 0; r < rounds; r += 3) {
      consume(ia, va, r);
      if (r + 3 < rounds) load_round(ia, va, r + 3);
      if (r + 1 < rounds) {
        consume(ib, vb, r + 1);
        if (r + 4 < rounds) load_round(ib, vb, r + 4);
      }
      if (r + 2 < rounds) {
        consume(ie, ve, r + 2);
        if (r + 5 < rounds) load_round(ie, ve, r + 5);
      }
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

// Polls of one Z word before a workgroup computes it itself: 2^20 polls of
// about a microsecond each, unless DFS_SPIN_LIMIT sets another count (0: no
// poll, every workgroup computes every Z word it needs).
uint32_t spin_limit() {
  const char* v = std::getenv("DFS_SPIN_LIMIT");
  if (v && *v) {
    char* end = nullptr;
    const unsigned long n = std::strtoul(v, &end, 10);
    if (end && *end == '\0') return n > 0xFFFFFFFFul ? 0xFFFFFFFFu : (uint32_t)n;
  }
  return 1u << 20;
}

constexpr size_t kEpochBytes = (size_t)kMaxFusedGroups * 4;  // one epoch word per workgroup

struct Plan {
  int G, A, RT, NX;  // NX = RT, 2 * RT or 3 * RT (X passes per row)
  int ND;            // dictionaries over the X rows
  size_t col_bytes, smem;
  int z_off;         // byte offset of Z from the X rows in LDS
};

bool plan(const XdLaunch& xd, const ZcLaunch& zc, Plan* p) {
  const bool q8 = zc.vdt == DFS_FP8 || zc.vdt == DFS_INT8;
  const int G = device_cus();
  if (G <= 0 || G > kMaxFusedGroups) return false;
  const int nd = xd.n_dicts <= 1 ? 1 : xd.n_dicts;
  if (nd > kFusedMaxDicts) return false;
  const int nl = xd.n_layers;  // X rows
  const int nu = zc.n_layers;  // units: one per (dictionary, layer)
  if (nu != nd * nl) return false;
  int A = (nd * xd.k + kFW * G - 1) / (kFW * G);  // atoms per wave
  if (A > (nd == 1 ? 2 : 3)) return false;
  A = A < 1 ? 1 : A;
  const int RT = nl <= 1 ? 1 : (nl <= 2 ? 2 : 4);
  if (xd.ddt == DFS_NVFP4 && RT == 4 && A == 2) return false;  // would spill registers
  if (nd > 1) {  // the instantiated multi-dictionary forms
    if (RT > 2) return false;
    if (xd.ddt != DFS_F16 && xd.ddt != DFS_NVFP4) return false;
    if (zc.vdt != DFS_F16 && zc.vdt != DFS_NVFP4) return false;
  }
  const int seg = xd.ddt == DFS_NVFP4 ? kWave * 2 * 32 : kWave * 8 * 8;  // Cfg<.., F16, RT<=4>::SEG
  const size_t ld = (size_t)(xd.d_in + seg - 1) / seg * seg;
  const size_t xbytes = (size_t)RT * ld * 2;
  const size_t zbytes = (size_t)nu * xd.k * 4;
  const int max_cols = (nu * zc.d_out + G - 1) / G + 1;
  if (max_cols > kFT) return false;  // one column range per thread
  if ((uint64_t)nu * (uint64_t)zc.d_out * (uint64_t)(G + 1) >= (1ull << 32)) return false;
  const int x_items = (int)((size_t)RT * ld / 8);
  const int NX = (x_items + kFT - 1) / kFT;
  // X rows pass through registers: 1, 2 or 3 passes of the workgroup per
  // row (ld <= 12288), at most 12 16-byte registers per thread
  if (NX != RT && NX != 2 * RT && NX != 3 * RT) return false;
  if (NX > 12) return false;
  if (nd > 1 && NX != RT) return false;  // d_in <= 4096 (f16) or 8192 (NVFP4)
  p->G = G;
  p->A = A;
  p->RT = RT;
  p->NX = NX;
  p->ND = nd;
  p->col_bytes = ((size_t)max_cols * (q8 ? 16 : 8) + 15) / 16 * 16;
  // X rows and Z side by side in LDS (X stays readable for a Z word that a
  // workgroup computes itself)
  constexpr size_t kMaxSmem = 160 * 1024;
  const size_t table = nd == 1 ? table_bytes_of<1>() : table_bytes_of<2>();
  const size_t xalign = (xbytes + 15) / 16 * 16;
  p->z_off = (int)xalign;
  p->smem = table + p->col_bytes + xalign + zbytes;
  return p->smem <= kMaxSmem;
}

template <int ND>
using ArgsFor = FusedArgs<units_of<ND>()>;

template <int DT, int VT, int RT, int A, int NX, int ND>
hipError_t launch5(ArgsFor<ND> f, const Plan& p, hipStream_t s) {
  auto kern = fused_decode_kernel<DT, VT, RT, A, NX, ND>;
  hipError_t err = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)p.smem);
  if (err != hipSuccess) return err;
  int per_cu = 0;
  err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kFT, p.smem);
  if (err != hipSuccess) return err;
  if (per_cu < 1) return hipErrorInvalidConfiguration;  // grid must be co-resident
  f.col_bytes = (int)p.col_bytes;
  f.G = p.G;
  f.z_off = p.z_off;
  hipLaunchKernelGGL(kern, dim3(p.G), dim3(kFT), p.smem, s, f);
  return hipGetLastError();
}

// ---- one dictionary: every format, up to 4 layers, d_in up to 12288
template <int DT, int VT, int RT, int A>
hipError_t launch4(ArgsFor<1> f, const Plan& p, hipStream_t s) {
  if (p.NX == 3 * RT) return launch5<DT, VT, RT, A, 3 * RT, 1>(f, p, s);
  if (p.NX == 2 * RT) return launch5<DT, VT, RT, A, 2 * RT, 1>(f, p, s);
  return launch5<DT, VT, RT, A, RT, 1>(f, p, s);
}

template <int DT, int VT, int RT>
hipError_t launch3(ArgsFor<1> f, const Plan& p, hipStream_t s) {
  return p.A == 1 ? launch4<DT, VT, RT, 1>(f, p, s) : launch4<DT, VT, RT, 2>(f, p, s);
}

template <int DT, int VT>
hipError_t launch2(ArgsFor<1> f, const Plan& p, hipStream_t s) {
  switch (p.RT) {
    case 1: return launch3<DT, VT, 1>(f, p, s);
    case 2: return launch3<DT, VT, 2>(f, p, s);
    default: return launch3<DT, VT, 4>(f, p, s);
  }
}

template <int DT>
hipError_t launch1(ArgsFor<1> f, const Plan& p, int vdt, hipStream_t s) {
  switch (vdt) {
    case kBlockF16: return launch2<DT, kBlockF16>(f, p, s);
    case DFS_NVFP4: return launch2<DT, DFS_NVFP4>(f, p, s);
    case DFS_FP8: return launch2<DT, DFS_FP8>(f, p, s);
    case DFS_INT8: return launch2<DT, DFS_INT8>(f, p, s);
    default: return launch2<DT, DFS_F16>(f, p, s);
  }
}

// ---- 2 or 3 dictionaries: f16 or NVFP4 factors, 1 or 2 layers, NX = RT
template <int DT, int VT, int ND, int RT>
hipError_t mlaunch4(ArgsFor<ND> f, const Plan& p, hipStream_t s) {
  switch (p.A) {
    case 1: return launch5<DT, VT, RT, 1, RT, ND>(f, p, s);
    case 2: return launch5<DT, VT, RT, 2, RT, ND>(f, p, s);
    default: return launch5<DT, VT, RT, 3, RT, ND>(f, p, s);
  }
}

template <int DT, int VT, int ND>
hipError_t mlaunch3(ArgsFor<ND> f, const Plan& p, hipStream_t s) {
  return p.RT == 1 ? mlaunch4<DT, VT, ND, 1>(f, p, s) : mlaunch4<DT, VT, ND, 2>(f, p, s);
}

template <int DT, int ND>
hipError_t mlaunch2(ArgsFor<ND> f, const Plan& p, int vdt, hipStream_t s) {
  return vdt == DFS_NVFP4 ? mlaunch3<DT, DFS_NVFP4, ND>(f, p, s) : mlaunch3<DT, DFS_F16, ND>(f, p, s);
}

template <int ND>
ArgsFor<ND> make_args(const XdLaunch& xd, const ZcLaunch& zc, uint8_t* tagged, uint32_t* ctrl) {
  ArgsFor<ND> f = {};
  f.D = xd.ddt == DFS_NVFP4 ? (const void*)xd.dcodes : xd.D;
  f.dscales = xd.dscales;
  f.ldd = xd.ldd;
  f.d_in = xd.d_in;
  f.k = xd.k;
  for (int l = 0; l < xd.n_layers; ++l) f.X[l] = xd.X[l];
  for (int u = 0; u < zc.n_layers; ++u) {
    f.colptr[u] = zc.colptr[u];
    f.rowidx[u] = zc.rowidx[u];
    f.vals[u] = zc.vals[u];
    f.vscales[u] = zc.vscales[u];
    f.vts[u] = zc.vts[u];
    f.Y[u] = zc.Y[u];
    f.nnz[u] = zc.nnz[u];
  }
  f.dts = xd.dts;
  f.epochs = reinterpret_cast<uint32_t*>(tagged);
  f.zz = reinterpret_cast<uint64_t*>(tagged + kEpochBytes);
  f.ctrl = ctrl;
  f.n_layers = xd.n_layers;
  f.d_out = zc.d_out;
  f.ydt = zc.ydt;
  f.spin_limit = spin_limit();
  f.col_bytes = 0;
  f.n_dicts = ND;
  for (int d = 1; d < ND; ++d) {
    f.Dx[d - 1] = xd.ddt == DFS_NVFP4 ? (const void*)xd.more[d - 1].dcodes : xd.more[d - 1].D;
    f.dscalesx[d - 1] = xd.more[d - 1].dscales;
    f.dtsx[d - 1] = xd.more[d - 1].dts;
  }
  return f;
}

}  // namespace

bool fused_decode_supported(const XdLaunch& xd, const ZcLaunch& zc) {
  if (xd.T != 1 || zc.T != 1) return false;
  // block-structured C: f16 values, 8-atom blocks that never cross k
  if (zc.block_rows != 0 && (zc.block_rows != 8 || zc.vdt != DFS_F16 || xd.k % 8 != 0 ||
                             xd.n_dicts > 1))
    return false;
  if (xd.n_layers < 1 || xd.n_layers > kFusedMaxLayers) return false;
  if (zc.n_layers < 1 || zc.n_layers > kFusedMaxUnits) return false;
  if (xd.xdt != DFS_F16) return false;
  if (xd.ddt != DFS_F16 && xd.ddt != DFS_NVFP4) return false;
  if (zc.vdt != DFS_F16 && zc.vdt != DFS_NVFP4 && zc.vdt != DFS_FP8 && zc.vdt != DFS_INT8)
    return false;
  if (xd.d_in % (xd.ddt == DFS_NVFP4 ? 32 : 8) != 0 || xd.k % 4 != 0) return false;
  Plan p;
  return plan(xd, zc, &p);
}

size_t fused_z_words_bytes(int32_t k) { return kEpochBytes + (size_t)kFusedMaxUnits * k * 8; }

hipError_t launch_fused_decode(const XdLaunch& xd, const ZcLaunch& zc, uint8_t* tagged,
                               uint32_t* ctrl, hipStream_t s) {
  Plan p;
  if (!plan(xd, zc, &p)) return hipErrorInvalidValue;
  const bool nv = xd.ddt == DFS_NVFP4;
  switch (p.ND) {
    case 1: {
      const ArgsFor<1> f = make_args<1>(xd, zc, tagged, ctrl);
      const int vt = zc.block_rows != 0 ? kBlockF16 : zc.vdt;
      return nv ? launch1<DFS_NVFP4>(f, p, vt, s) : launch1<DFS_F16>(f, p, vt, s);
    }
    case 2: {
      const ArgsFor<2> f = make_args<2>(xd, zc, tagged, ctrl);
      return nv ? mlaunch2<DFS_NVFP4, 2>(f, p, zc.vdt, s) : mlaunch2<DFS_F16, 2>(f, p, zc.vdt, s);
    }
    default: {
      const ArgsFor<3> f = make_args<3>(xd, zc, tagged, ctrl);
      return nv ? mlaunch2<DFS_NVFP4, 3>(f, p, zc.vdt, s) : mlaunch2<DFS_F16, 3>(f, p, zc.vdt, s);
    }
  }
}

}  // namespace dfs
