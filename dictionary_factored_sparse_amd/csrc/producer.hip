// producer.hip -- the steps that produce D_g and C_l, on the GPU:
//   * P = (D^T S D + lambda I)^-1, the fixed inverse of coefficient-space
//     pruning ("DictLLM: Shared Dictionaries for Post-Training Compression",
//     "Method II: prune in coefficient space", Eq. (6)-(7));
//   * fixed-inverse pruning of each coefficient column with compensation
//     (same section, Algorithm 1 and Eq. (7));
//   * the dictionary refit D (C C^T + lambda I) = W C^T (same review,
//     "Method III: refit the dictionary", Eq. (9)).
// These run once per group, offline, in fp32.  Every product here has the
// form C = A B^T with both operands row-major (K contiguous), so one VALU
// GEMM serves them all; the symmetric positive definite inverses use
// Gauss-Jordan elimination without pivoting (stable for such matrices), one
// launch per pivot.
#include "dfs_internal.hpp"

namespace dfs {
namespace {

// ------------------------------------------------------------------ GEMM
// C[m][n] = alpha * sum_k A[m][k] B[n][k] + beta * C[m][n] + (m == n ? diag : 0)
// 128 x 128 tiles, 256 threads, 8 x 8 outputs per thread, K in steps of 16
// through LDS (stored k-major, rows padded by 4 floats).
constexpr int kBM = 128, kBN = 128, kBK = 16, kGT = 256;

__global__ __launch_bounds__(kGT) void gemm_nt_kernel(const float* A, int64_t lda, const float* B,
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
      Bs[lk][r] = (gn < N && gk < K) ? B[(int64_t)gn * ldb + gk] : 0.0f;
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
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = m0 + (i < 4 ? tm * 4 + i : 64 + tm * 4 + i - 4);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = n0 + (j < 4 ? tn * 4 + j : 64 + tn * 4 + j - 4);
      if (n >= N) continue;
      float v = alpha * acc[i][j];
      if (beta != 0.0f) v += beta * C[(int64_t)m * ldc + n];
      if (m == n) v += diag;
      C[(int64_t)m * ldc + n] = v;
    }
  }
}

// ------------------------------------------------------------------ inverse
// In-place Gauss-Jordan inversion of an n x n symmetric positive definite
// matrix.  Pivot step p maps, from the old row p (rp) and column p (cp):
//   a_pp -> 1 / a_pp,  a_pj -> a_pj / a_pp,  a_ip -> -a_ip / a_pp,
//   a_ij -> a_ij - a_ip (a_pj / a_pp);
// after the n steps A holds its inverse.  Each step also saves the new row and
// column p + 1 for the next step.  A pivot that is not positive and finite
// sets *err (the matrix was not positive definite; the result is undefined).
__global__ __launch_bounds__(256) void gj_init_kernel(const float* A, int64_t lda, int n, float* rp,
                                                      float* cp) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    rp[i] = A[i];
    cp[i] = A[(int64_t)i * lda];
  }
}

__global__ __launch_bounds__(256) void gj_step_kernel(float* A, int64_t lda, int n, int p,
                                                      const float* rp, const float* cp, float* rn,
                                                      float* cn, uint32_t* err) {
  const int j = blockIdx.x * 64 + (threadIdx.x & 63);
  const int i = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (i >= n || j >= n) return;
  const float piv = rp[p];
  if (i == p && j == p && !(piv > 0.0f && piv < __builtin_inff())) atomicOr(err, 1u);
  float v;
  if (i == p)
    v = j == p ? 1.0f / piv : rp[j] / piv;
  else if (j == p)
    v = -cp[i] / piv;
  else
    v = A[(int64_t)i * lda + j] - cp[i] * (rp[j] / piv);
  A[(int64_t)i * lda + j] = v;
  if (i == p + 1) rn[j] = v;
  if (j == p + 1) cn[i] = v;
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

hipError_t launch_gemm_nt_f32(const float* A, int64_t lda, const float* B, int64_t ldb, float* C,
                              int64_t ldc, int M, int N, int K, float alpha, float beta, float diag,
                              hipStream_t s) {
  dim3 grid((N + kBN - 1) / kBN, (M + kBM - 1) / kBM);
  hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(kGT), 0, s, A, lda, B, ldb, C, ldc, M, N, K, alpha,
                     beta, diag);
  return hipGetLastError();
}

size_t spd_inverse_ws_bytes(int n) { return 256 + 4 * (((size_t)n * 4 + 255) / 256 * 256); }

hipError_t launch_spd_inverse(float* A, int64_t lda, int n, void* ws, hipStream_t s) {
  uint32_t* err = (uint32_t*)ws;
  const size_t vb = ((size_t)n * 4 + 255) / 256 * 256;
  float* buf[4];
  for (int q = 0; q < 4; ++q) buf[q] = (float*)((char*)ws + 256 + q * vb);
  hipError_t e = hipMemsetAsync(err, 0, 4, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gj_init_kernel, dim3((n + 255) / 256), dim3(256), 0, s, A, lda, n, buf[0],
                     buf[1]);
  dim3 grid((n + 63) / 64, (n + 3) / 4);
  for (int p = 0; p < n; ++p) {
    const int cur = (p & 1) * 2, nxt = 2 - cur;
    hipLaunchKernelGGL(gj_step_kernel, grid, dim3(256), 0, s, A, lda, n, p, buf[cur],
                       buf[cur + 1], buf[nxt], buf[nxt + 1], err);
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
