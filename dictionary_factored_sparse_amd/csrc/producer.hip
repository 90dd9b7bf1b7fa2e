// producer.hip -- the steps that produce D_g and C_l, on the GPU:
//   * P = (D^T S D + lambda I)^-1, the fixed inverse of coefficient-space
//     pruning ("DictLLM: Shared Dictionaries for Post-Training Compression",
//     "Method II: prune in coefficient space", Eq. (6)-(7));
//   * fixed-inverse pruning of each coefficient column with compensation
//     (same section, Algorithm 1 and Eq. (7));
//   * the dictionary refit D (C C^T + lambda I) = W C^T (same review,
//     "Method III: refit the dictionary", Eq. (9)).
// These run once per group, offline, in fp32.  The products use one VALU
// GEMM, C = A B^T or C = A B with row-major operands; the symmetric positive
// definite inverses use Gauss-Jordan elimination without pivoting (stable for
// such matrices), blocked: 64 pivots per step, the update as one GEMM.
#include "dfs_internal.hpp"

namespace dfs {
namespace {

// ------------------------------------------------------------------ GEMM
// C[m][n] = alpha * sum_k A[m][k] B'[k][n] + beta * C[m][n] + (m == n ? diag : 0)
// with B'[k][n] = B[n][k] (NN == false) or B[k][n] (NN == true).
// 128 x 128 tiles, 256 threads, 8 x 8 outputs per thread, K in steps of 16
// through LDS (stored k-major, rows padded by 4 floats).
constexpr int kBM = 128, kBN = 128, kBK = 16, kGT = 256;

template <bool NN>
__global__ __launch_bounds__(kGT) void gemm_kernel(const float* A, int64_t lda, const float* B,
                                                   int64_t ldb, float* C, int64_t ldc, int M,
                                                   int N, int K, float alpha, float beta,
                                                   float diag) {
  __shared__ __attribute__((aligned(16))) float As[kBK][kBM + 4];
  __shared__ __attribute__((aligned(16))) float Bs[kBK][kBN + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
  const int tm = tid / 16, tn = tid % 16;
  const int lk = tid % 16, lr = tid / 16;  // loader: k column, first row
  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += kBK) {
    const int gk = k0 + lk;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = lr + 16 * q;
      const int gm = m0 + r, gn = n0 + r;
      As[lk][r] = (gm < M && gk < K) ? A[(int64_t)gm * lda + gk] : 0.0f;
      if constexpr (!NN) Bs[lk][r] = (gn < N && gk < K) ? B[(int64_t)gn * ldb + gk] : 0.0f;
    }
    if constexpr (NN) {  // B rows run along n: consecutive threads, consecutive n
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int kk = tid / 128 + 2 * q, r = tid % 128;
        const int gn = n0 + r, gk2 = k0 + kk;
        Bs[kk][r] = (gn < N && gk2 < K) ? B[(int64_t)gk2 * ldb + gn] : 0.0f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kBK; ++k) {
      const f4 a0 = *reinterpret_cast<const f4*>(&As[k][tm * 4]);
      const f4 a1 = *reinterpret_cast<const f4*>(&As[k][64 + tm * 4]);
      const f4 b0 = *reinterpret_cast<const f4*>(&Bs[k][tn * 4]);
      const f4 b1 = *reinterpret_cast<const f4*>(&Bs[k][64 + tn * 4]);
      const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  // all loads of C before any store, so that they are in flight together
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + (i < 4 ? tm * 4 + i : 64 + tm * 4 + i - 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + (j < 4 ? tn * 4 + j : 64 + tn * 4 + j - 4);
      float v = alpha * acc[i][j];
      if (beta != 0.0f && m < M && n < N) v += beta * C[(int64_t)m * ldc + n];
      if (m == n) v += diag;
      acc[i][j] = v;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + (i < 4 ? tm * 4 + i : 64 + tm * 4 + i - 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + (j < 4 ? tn * 4 + j : 64 + tn * 4 + j - 4);
      if (m < M && n < N) C[(int64_t)m * ldc + n] = acc[i][j];
    }
  }
}

// ------------------------------------------------------------------ inverse
// Blocked in-place Gauss-Jordan inversion of an n x n symmetric positive
// definite matrix, pivot blocks P of kNB rows.  With Q = A_PP^-1, the scalar
// step's block form is
//   A_IJ -= A_IP Q A_PJ,  A_PJ <- Q A_PJ,  A_IP <- -A_IP Q,  A_PP <- Q
// (I, J != P).  With R = Q A_P,: whose block P is replaced by I + Q, the
// first and third are one product, A -= A_:,P R (A_IP - A_IP (I + Q) =
// -A_IP Q); row block P is then written as Q A_P,: with Q in its block P.
// A pivot of the small inverse that is not positive and finite sets *err.
constexpr int kNB = 64;

__global__ __launch_bounds__(256) void panel_copy_kernel(const float* A, int64_t lda, int n, int P0,
                                                         int m, float* Cp, float* Rr) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)n * m) return;
  const int i = (int)(e / m), c = (int)(e % m);
  Cp[(int64_t)i * m + c] = A[(int64_t)i * lda + P0 + c];  // column panel, n x m
  const int r = (int)(e / n), j = (int)(e % n);
  Rr[(int64_t)r * n + j] = A[(int64_t)(P0 + r) * lda + j];  // row panel, m x n
}

// Q = A_PP^-1 by scalar Gauss-Jordan steps, the 64 x 64 block (identity past
// m) in registers: thread t holds row t / 4, columns 16 (t % 4) .. + 15.
// Per pivot p the owners of row p and of column p publish them to LDS (two
// buffers by the parity of p, so one barrier per pivot suffices), then every
// element takes its step: a_ij - a_ip a_pj / a_pp off row and column p,
// a_pj / a_pp on row p, -a_ip / a_pp on column p, 1 / a_pp at the pivot.
// Padding pivots (p >= m) are unit rows and columns: their steps change
// nothing.
__global__ __launch_bounds__(256) void block_inverse_kernel(const float* Rr, int n, int P0, int m,
                                                            float* Q, uint32_t* err) {
  __shared__ __attribute__((aligned(16))) float rp[2][kNB];
  __shared__ float cp[2][kNB];
  const int tid = threadIdx.x;
  const int r = tid >> 2, cb = tid & 3;
  float s[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int c = cb * 16 + q;
    s[q] = (r < m && c < m) ? Rr[(int64_t)r * n + P0 + c] : (r == c ? 1.0f : 0.0f);
  }
  bool bad = false;
  for (int pb = 0; pb < kNB / 16; ++pb) {
#pragma unroll
    for (int pi = 0; pi < 16; ++pi) {
      const int p = pb * 16 + pi, buf = pi & 1;
      if (r == p) {
#pragma unroll
        for (int q = 0; q < 16; q += 4)
          *reinterpret_cast<f4*>(&rp[buf][cb * 16 + q]) = f4{s[q], s[q + 1], s[q + 2], s[q + 3]};
      }
      if (cb == pb) cp[buf][r] = s[pi];
      __syncthreads();
      const float piv = rp[buf][p];
      bad |= !(piv > 0.0f && piv < __builtin_inff());
      const float inv = 1.0f / piv;
      const float a = cp[buf][r];
      float row[16];
#pragma unroll
      for (int q = 0; q < 16; q += 4) {
        const f4 v = *reinterpret_cast<const f4*>(&rp[buf][cb * 16 + q]);
        row[q] = v[0], row[q + 1] = v[1], row[q + 2] = v[2], row[q + 3] = v[3];
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float rq = row[q] * inv;
        float v = r == p ? rq : s[q] - a * rq;
        if (q == pi && cb == pb) v = r == p ? inv : -a * inv;
        s[q] = v;
      }
    }
  }
  if (tid == 0 && bad) atomicOr(err, 1u);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int c = cb * 16 + q;
    if (r < m && c < m) Q[r * m + c] = s[q];
  }
}

// R[:, P] = I + Q (m x n panel, block P at columns P0 .. P0 + m)
__global__ __launch_bounds__(256) void fix_panel_kernel(float* R, int n, int P0, int m,
                                                        const float* Q) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= m * m) return;
  const int r = e / m, c = e % m;
  R[(int64_t)r * n + P0 + c] = Q[e] + (r == c ? 1.0f : 0.0f);
}

// row block P of A: Q A_P,: outside block P, Q inside it
__global__ __launch_bounds__(256) void write_row_kernel(float* A, int64_t lda, int n, int P0, int m,
                                                        const float* R, const float* Q) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (int64_t)m * n) return;
  const int r = (int)(e / n), j = (int)(e % n);
  const bool inP = j >= P0 && j < P0 + m;
  A[(int64_t)(P0 + r) * lda + j] = inP ? Q[r * m + (j - P0)] : R[(int64_t)r * n + j];
}

// ------------------------------------------------------------------ pruning
// One workgroup per coefficient column j.  Scores c_i^2 / P_ii in fp32 (the
// product and the quotient each rounded once: no contraction can fuse them)
// from the column before any deletion; rows sorted by (score, row) with a
// bitonic network over 64-bit keys (a non-negative float's bits order like
// its value); then the n_prune first rows are deleted in that order, each
// with the Eq. (7) move c -= P[i, :] * (c_i / P_ii) (P symmetric, row i
// contiguous); finally the deleted entries are set to exactly 0.
constexpr int kPT = 256;

__global__ __launch_bounds__(kPT) void obs_prune_kernel(const float* C, int64_t ldc, const float* P,
                                                        int64_t ldp, int k, int kp, int n_prune,
                                                        float* Co, int64_t ldo, uint8_t* keep,
                                                        int64_t ldkeep) {
  extern __shared__ __attribute__((aligned(16))) char sm[];
  uint64_t* key = reinterpret_cast<uint64_t*>(sm);  // [kp]
  float* c = reinterpret_cast<float*>(key + kp);    // [k]
  float* pd = c + k;                                // [k] diagonal of P
  uint8_t* gone = reinterpret_cast<uint8_t*>(pd + k);  // [k]
  const int j = blockIdx.x;
  const int tid = threadIdx.x;
  for (int i = tid; i < k; i += kPT) {
    const float ci = C[(int64_t)i * ldc + j];
    const float pii = P[(int64_t)i * ldp + i];
    c[i] = ci;
    pd[i] = pii;
    gone[i] = 0;
    const float sq = ci * ci;
    const float s = sq / pii;
    key[i] = ((uint64_t)__float_as_uint(s) << 32) | (uint32_t)i;
  }
  for (int i = k + tid; i < kp; i += kPT) key[i] = ~(uint64_t)0;
  __syncthreads();
  for (int size = 2; size <= kp; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int q = tid; q < kp / 2; q += kPT) {
        const int lo = 2 * q - (q & (stride - 1));
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const uint64_t a = key[lo], b = key[hi];
        if ((a > b) == asc) {
          key[lo] = b;
          key[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int t = 0; t < n_prune; ++t) {
    const int i = (int)(uint32_t)key[t];
    const float f = c[i] / pd[i];
    __syncthreads();  // every thread has read c_i before it moves
    const float* pr = P + (int64_t)i * ldp;
    for (int a = tid; a < k; a += kPT) c[a] = __builtin_fmaf(-pr[a], f, c[a]);
    __syncthreads();
  }
  for (int t = tid; t < n_prune; t += kPT) gone[(uint32_t)key[t]] = 1;
  __syncthreads();
  for (int i = tid; i < k; i += kPT) {
    Co[(int64_t)i * ldo + j] = gone[i] ? 0.0f : c[i];
    keep[(int64_t)i * ldkeep + j] = gone[i] ? 0 : 1;
  }
}

// f16 atoms -> f32 (k x d_in, row stride ldd -> d_in)
__global__ __launch_bounds__(256) void atoms_to_f32_kernel(const _Float16* D, int64_t ldd, int d_in,
                                                           int64_t total, float* out) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int64_t a = e / d_in, i = e - a * d_in;
  out[e] = (float)D[a * ldd + i];
}

}  // namespace

template <bool NN>
hipError_t launch_gemm(const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
                       int64_t ldc, int M, int N, int K, float alpha, float beta, float diag,
                       hipStream_t s) {
  dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
  hipLaunchKernelGGL(gemm_kernel<NN>, grid, dim3(kGT), 0, s, A, lda, B, ldb, C, ldc, M, N, K,
                     alpha, beta, diag);
  return hipGetLastError();
}

hipError_t launch_gemm_nt_f32(const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
                              int64_t ldc, int M, int N, int K, float alpha, float beta, float diag,
                              hipStream_t s) {
  return launch_gemm<false>(A, lda, B, ldb, C, ldc, M, N, K, alpha, beta, diag, s);
}

// error word, column panel (n x kNB), row panel and its product (kNB x n), Q
size_t spd_inverse_ws_bytes(int n) {
  const size_t panel = ((size_t)n * kNB * 4 + 255) / 256 * 256;
  return 256 + 3 * panel + (size_t)kNB * kNB * 4;
}

hipError_t launch_spd_inverse(float* A, int64_t lda, int n, void* ws, hipStream_t s) {
  uint32_t* err = (uint32_t*)ws;
  const size_t panel = ((size_t)n * kNB * 4 + 255) / 256 * 256;
  float* Cp = (float*)((char*)ws + 256);
  float* Rr = (float*)((char*)Cp + panel);
  float* R = (float*)((char*)Rr + panel);
  float* Q = (float*)((char*)R + panel);
  hipError_t e = hipMemsetAsync(err, 0, 4, s);
  if (e != hipSuccess) return e;
  for (int P0 = 0; P0 < n; P0 += kNB) {
    const int m = n - P0 < kNB ? n - P0 : kNB;
    const int64_t nm = (int64_t)n * m;
    const unsigned gb = (unsigned)((nm + 255) / 256);
    hipLaunchKernelGGL(panel_copy_kernel, dim3(gb), dim3(256), 0, s, A, lda, n, P0, m, Cp, Rr);
    hipLaunchKernelGGL(block_inverse_kernel, dim3(1), dim3(256), 0, s, Rr, n, P0, m, Q, err);
    e = launch_gemm<true>(Q, m, Rr, n, R, n, m, n, m, 1.0f, 0.0f, 0.0f, s);  // R = Q A_P,:
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fix_panel_kernel, dim3((m * m + 255) / 256), dim3(256), 0, s, R, n, P0, m,
                       Q);
    e = launch_gemm<true>(Cp, m, R, n, A, lda, n, n, m, -1.0f, 1.0f, 0.0f, s);  // A -= A_:,P R
    if (e != hipSuccess) return e;
    // R's block P now holds I + Q; write_row takes Q there, R elsewhere
    hipLaunchKernelGGL(write_row_kernel, dim3(gb), dim3(256), 0, s, A, lda, n, P0, m, R, Q);
  }
  return hipGetLastError();
}

size_t obs_prune_smem(int k) {
  int kp = 1;
  while (kp < k) kp <<= 1;
  return (size_t)kp * 8 + (size_t)k * 9;
}

hipError_t launch_obs_prune(const float* C, int64_t ldc, const float* P, int64_t ldp, int k,
                            int d_out, int n_prune, float* Co, int64_t ldo, uint8_t* keep,
                            int64_t ldkeep, hipStream_t s) {
  int kp = 1;
  while (kp < k) kp <<= 1;
  const size_t smem = obs_prune_smem(k);
  if (smem > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)obs_prune_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(obs_prune_kernel, dim3(d_out), dim3(kPT), smem, s, C, ldc, P, ldp, k, kp,
                     n_prune, Co, ldo, keep, ldkeep);
  return hipGetLastError();
}

hipError_t launch_atoms_to_f32(const _Float16* D, int64_t ldd, int d_in, int k, float* out,
                               hipStream_t s) {
  const int64_t total = (int64_t)k * d_in;
  hipLaunchKernelGGL(atoms_to_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, D,
                     ldd, d_in, total, out);
  return hipGetLastError();
}

}  // namespace dfs
