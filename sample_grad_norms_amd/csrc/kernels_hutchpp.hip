// Hutch++ kernels for gfx950: the per-sample orthonormal basis of the sketch
// and the projection of the tail columns onto its complement.
//
// Method ('Efficient DP-SGD for LLMs with Randomized Clipping', papernotes.org
// note, 关键设计 › Hutch++ 头-尾分解的低误差变体; gist.science/nl summary,
// Kernmechanisme item 2): with O = G^T A A^T G, the sketch X = O S spans the
// dominant directions; Q is an orthonormal basis of Col(X), the head
// ||A^T G Q||_F^2 is exact on span(Q) and the tail is a Hutchinson estimate
// on the complement, ||A^T G (I - Q Q^T) P||_F^2.
//
// The basis is built by Gram-Schmidt with each column projected against the
// kept basis twice, in fp64, one work group per sample. A column is kept when
// its residual norm exceeds tau times the largest column norm of X. The kept
// columns are written compacted, zero columns after them, into the first m_s
// columns of the stage-1 matrix W3 = [Q | P'] of the head/tail pass; the
// tail kernel writes P' = P - Q (Q^T P) into the next m_t columns.
#include "device_common.h"
#include "internal.h"

namespace dpn {

constexpr int kQrThreads = 256;
constexpr int kMaxCols = 32;

// Sum of `cnt` per-thread values over the work group; every thread gets the
// totals. `red` holds kQrThreads / 64 * kMaxCols doubles.
__device__ __forceinline__ void block_sum(double* v, int cnt, double* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int j = 0; j < cnt; ++j) {
    const double s = wave_sum(v[j]);
    if (lane == 0) red[wv * kMaxCols + j] = s;
  }
  __syncthreads();
  for (int j = 0; j < cnt; ++j) {
    double s = 0.0;
#pragma unroll
    for (int w = 0; w < kQrThreads / 64; ++w) s += red[w * kMaxCols + j];
    v[j] = s;
  }
  __syncthreads();
}

// X [B][p][ldx] fp32 (first m columns valid) -> basis Qd [B][m][p] fp64
// (scratch), vbuf [B][p] fp64 (scratch), W3 [B][p][ldw] fp32 columns 0..m-1,
// rank [B] int32 (optional).
__global__ void __launch_bounds__(kQrThreads) k_hpp_basis(const float* __restrict__ X, int ldx, int p, int m,
                                                          float tau, double* Qd, double* vbuf, float* W3, int ldw,
                                                          int32_t* rank) {
  __shared__ double red[kQrThreads / 64 * kMaxCols];
  const int i = blockIdx.x;
  const float* Xi = X + (int64_t)i * p * ldx;
  double* Q = Qd + (int64_t)i * m * p;
  double* v = vbuf + (int64_t)i * p;
  float* Wi = W3 + (int64_t)i * p * ldw;

  // largest column norm of X
  double nrm[kMaxCols];
  for (int j = 0; j < m; ++j) nrm[j] = 0.0;
  for (int r = threadIdx.x; r < p; r += kQrThreads)
    for (int j = 0; j < m; ++j) {
      const double x = (double)Xi[(int64_t)r * ldx + j];
      nrm[j] += x * x;
    }
  block_sum(nrm, m, red);
  double scale = 0.0;
  for (int j = 0; j < m; ++j) scale = fmax(scale, sqrt(nrm[j]));

  int kept = 0;
  double dots[kMaxCols];
  for (int j = 0; j < m; ++j) {
    for (int r = threadIdx.x; r < p; r += kQrThreads) v[r] = (double)Xi[(int64_t)r * ldx + j];
    for (int pass = 0; pass < 2; ++pass) {
      for (int q = 0; q < kept; ++q) dots[q] = 0.0;
      for (int r = threadIdx.x; r < p; r += kQrThreads) {
        const double x = v[r];
        for (int q = 0; q < kept; ++q) dots[q] += Q[(int64_t)q * p + r] * x;
      }
      block_sum(dots, kept, red);
      for (int r = threadIdx.x; r < p; r += kQrThreads) {
        double x = v[r];
        for (int q = 0; q < kept; ++q) x -= dots[q] * Q[(int64_t)q * p + r];
        v[r] = x;
      }
    }
    double nv = 0.0;
    for (int r = threadIdx.x; r < p; r += kQrThreads) nv += v[r] * v[r];
    block_sum(&nv, 1, red);
    nv = sqrt(nv);
    if (nv > (double)tau * scale && nv > 0.0) {
      const double inv = 1.0 / nv;
      for (int r = threadIdx.x; r < p; r += kQrThreads) Q[(int64_t)kept * p + r] = v[r] * inv;
      ++kept;
    }
    // every thread reads v and Q of its own rows only; the block_sum barriers
    // order the next column's reads after these writes
  }
  __syncthreads();
  for (int r = threadIdx.x; r < p; r += kQrThreads)
    for (int j = 0; j < m; ++j) Wi[(int64_t)r * ldw + j] = j < kept ? (float)Q[(int64_t)j * p + r] : 0.f;
  if (rank && threadIdx.x == 0) rank[i] = kept;
}

// Tail column tcol of sample i: P'[:, tcol] = P[:, tcol] - Q (Q^T P[:, tcol]),
// written to W3 column m + tcol. Grid (B, m_t).
__global__ void __launch_bounds__(kQrThreads) k_hpp_tail(const void* __restrict__ P, int ptype, int ldp, int p,
                                                         int m, const double* __restrict__ Qd,
                                                         const int32_t* __restrict__ rank_in, float* W3, int ldw) {
  __shared__ double red[kQrThreads / 64 * kMaxCols];
  const int i = blockIdx.x, tcol = blockIdx.y;
  const double* Q = Qd + (int64_t)i * m * p;
  float* Wi = W3 + (int64_t)i * p * ldw;
  const int kept = rank_in[i];
  auto pval = [&](int r) -> double {
    if (ptype == SRC_BF16) return (double)bf16_bits_to_f32(((const uint16_t*)P)[(int64_t)r * ldp + tcol]);
    return (double)((const float*)P)[(int64_t)r * ldp + tcol];
  };
  double dots[kMaxCols];
  for (int q = 0; q < kept; ++q) dots[q] = 0.0;
  for (int r = threadIdx.x; r < p; r += kQrThreads) {
    const double x = pval(r);
    for (int q = 0; q < kept; ++q) dots[q] += Q[(int64_t)q * p + r] * x;
  }
  block_sum(dots, kept, red);
  for (int r = threadIdx.x; r < p; r += kQrThreads) {
    double x = pval(r);
    for (int q = 0; q < kept; ++q) x -= dots[q] * Q[(int64_t)q * p + r];
    Wi[(int64_t)r * ldw + m + tcol] = (float)x;
  }
}

hipError_t launch_hpp_basis(const float* X, int ldx, int B, int p, int m, float tau, double* Qd, double* vbuf,
                            float* W3, int ldw, int32_t* rank, hipStream_t s) {
  hipLaunchKernelGGL(k_hpp_basis, dim3(B), dim3(kQrThreads), 0, s, X, ldx, p, m, tau, Qd, vbuf, W3, ldw, rank);
  return hipGetLastError();
}

hipError_t launch_hpp_tail(const void* P, int ptype, int ldp, int B, int p, int m, int mt, const double* Qd,
                           const int32_t* rank, float* W3, int ldw, hipStream_t s) {
  hipLaunchKernelGGL(k_hpp_tail, dim3(B, mt), dim3(kQrThreads), 0, s, P, ptype, ldp, p, m, Qd, rank, W3, ldw);
  return hipGetLastError();
}

}  // namespace dpn
