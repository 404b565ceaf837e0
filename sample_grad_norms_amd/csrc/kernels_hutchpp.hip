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
// Q is the Q factor of X with positive diagonal (unique for the kept
// columns), by Cholesky QR in fp64, in two kernels:
//   k_hpp_gram  : partial X^T X and X^T P over chunks of rows with fp64 MFMA
//                 (v_mfma_f64_16x16x4), many work groups per sample;
//   k_hpp_apply : every work group first sums its sample's partials in a
//                 fixed order and factors X^T X = R^T R in LDS (right-looking,
//                 one entry of the Schur complement per thread) with a rank
//                 rule: column j is kept when its residual after projecting
//                 out the kept columns before it (the Cholesky diagonal)
//                 exceeds tau times the largest column norm of X; the same
//                 eliminations on the identity give Ri = R^-1 on the kept
//                 columns (zero rows and columns elsewhere); M = Q^T P =
//                 Ri^T X^T P and N = Ri M; then
//                 Q = X Ri and P' = P - Q M = P - X N with fp64 MFMA.
// Columns keep their positions: a dropped column of X gives a zero column of
// Q, which adds nothing to the head. W3 = [Q (MP columns) | P' (m_t)].
// The rank rule bounds the condition number of the kept columns by about
// 1/tau, so Q is orthonormal to about (1/tau)^2 * 2^-53 ~ 1e-6 in fp64.
#include "device_common.h"
#include "internal.h"

namespace dpn {

typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kMaxTail = 32;
constexpr int kGramRows = 256;   // rows of X per k_hpp_gram work group
constexpr int kApplyRows = 64;   // rows of X per k_hpp_apply work group (4 waves x 16)

__device__ __forceinline__ f64x4_t mfma_f64(double a, double b, f64x4_t c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

template <int MP>
struct HppTiles {
  static constexpr int TA = MP / 16;            // 16-column tiles of X
  static constexpr int NG = TA * (TA + 1) / 2;  // Gram tiles (upper triangle)
  static constexpr int NT = NG + 2 * TA;        // + X^T P tiles (tail columns up to 32)
};

__device__ __forceinline__ double tail_val(const void* P, int ptype, int p, int mt, int row, int t) {
  if (row >= p || t >= mt) return 0.0;
  if (ptype == SRC_BF16) return (double)bf16_bits_to_f32(((const uint16_t*)P)[(int64_t)row * mt + t]);
  return (double)ldg_f32((const float*)P + (int64_t)row * mt + t);
}

// Partial tiles of X^T X (upper triangle) and X^T P for kGramRows rows:
// part [B][nparts][NT][4][64] (the accumulator registers of each tile).
// The contraction runs over rows: K slot l / 16 is row 4 ks + l / 16.
template <int MP>
__global__ void __launch_bounds__(256) k_hpp_gram(const float* __restrict__ X, int p, int mt,
                                                  const void* __restrict__ P, int ptype, double* part) {
  using H = HppTiles<MP>;
  constexpr int TA = H::TA, NG = H::NG, NT = H::NT;
  __shared__ double red[4][NT][4][64];
  const int s = blockIdx.x, i = blockIdx.y, nparts = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const float* Xi = X + (int64_t)i * p * MP;
  f64x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  constexpr int U = kGramRows / 4 / 4;  // K steps per wave, loads issued together
  double xa[U][TA], pv[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int row = s * kGramRows + 4 * (wv * U + u) + g;
#pragma unroll
    for (int a = 0; a < TA; ++a) xa[u][a] = row < p ? (double)ldg_f32(Xi + (int64_t)row * MP + 16 * a + n) : 0.0;
    pv[u][0] = tail_val(P, ptype, p, mt, row, n);
    pv[u][1] = tail_val(P, ptype, p, mt, row, 16 + n);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int a = 0, t = 0; a < TA; ++a)
#pragma unroll
      for (int b = a; b < TA; ++b, ++t) acc[t] = mfma_f64(xa[u][a], xa[u][b], acc[t]);
#pragma unroll
    for (int a = 0; a < TA; ++a)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) acc[NG + 2 * a + tt] = mfma_f64(xa[u][a], pv[u][tt], acc[NG + 2 * a + tt]);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wv][t][j][lane] = acc[t][j];
  __syncthreads();
  double* out = part + ((int64_t)i * nparts + s) * NT * 256;
  for (int e = tid; e < NT * 256; e += 256) {
    const int t = e >> 8, j = (e >> 6) & 3, l = e & 63;
    out[e] = (red[0][t][j][l] + red[1][t][j][l]) + (red[2][t][j][l] + red[3][t][j][l]);
  }
}

// The basis of one sample in LDS: the Gram tiles summed from their partials,
// R with the rank rule, Ri = R^-1 on the kept columns, M = Q^T P and N = Ri M.
template <int MP>
struct HppBasis {
  double G[MP][MP], XP[MP][kMaxTail], R[MP][MP], Ri[MP][MP], M[MP][kMaxTail], N[MP][kMaxTail];
  double sj[MP];   // 1 / R[j][j] of kept columns, 0 of dropped ones
};

// Run by all 256 threads of a work group (it holds barriers): sum of sample
// i's partial tiles in a fixed order (every lane's loads in flight at once),
// Cholesky with the rank rule, Ri, M and N. Every work group that runs it on
// the same partials gets bitwise the same basis. Returns the kept columns.
template <int MP>
__device__ uint32_t hpp_basis(const double* __restrict__ part, int nparts, float tau, int i, HppBasis<MP>& sb) {
  using H = HppTiles<MP>;
  constexpr int TA = H::TA, NG = H::NG, NT = H::NT;
  double (&G)[MP][MP] = sb.G;
  double (&XP)[MP][kMaxTail] = sb.XP;
  double (&R)[MP][MP] = sb.R;
  double (&Ri)[MP][MP] = sb.Ri;
  double (&M)[MP][kMaxTail] = sb.M;
  const int l = threadIdx.x;
  const double* pi = part + (int64_t)i * nparts * NT * 256;
  // fixed-order sum; lane q, element j of a v_mfma_f64_16x16x4 result is (row q/16 + 4 j, column q % 16)
  for (int e = l; e < NT * 256; e += 256) {
    double v = 0.0;
    for (int s0 = 0; s0 < nparts; s0 += 8) {  // eight loads in flight, summed in part order
      double w[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) w[u] = s0 + u < nparts ? pi[(int64_t)(s0 + u) * NT * 256 + e] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) v += w[u];
    }
    const int t = e >> 8, j = (e >> 6) & 3, q = e & 63;
    const int r = (q >> 4) + 4 * j, c = q & 15;
    if (t < NG) {
      int a = 0, b = 0;
      for (int aa = 0, k = 0; aa < TA; ++aa)
        for (int bb = aa; bb < TA; ++bb, ++k)
          if (k == t) {
            a = aa;
            b = bb;
          }
      G[16 * a + r][16 * b + c] = v;
      G[16 * b + c][16 * a + r] = v;
    } else {
      const int a = (t - NG) >> 1, tt = (t - NG) & 1;
      XP[16 * a + r][16 * tt + c] = v;
    }
  }
  __syncthreads();

  // Right-looking Cholesky on the Schur complement Sc (= G at the start), one
  // entry per thread: at step j, if column j is kept, row j of R (formed only
  // where needed) is row j of Sc times 1 / Sc[j][j]^(1/2) and every later entry (a, b) loses
  // R[j][a] R[j][b]; so the diagonal Sc[j][j] a step reads is G[j][j] minus
  // the squares of the kept rows above it, subtracted in row order. The same
  // row operations on the identity give E = R^-T: row j of E is scaled by the
  // same factor, which is kept in sj[] and applied once at the end (rows of
  // dropped columns get 0), so a step reads only row j, which it never writes,
  // and needs one barrier.
  double (&Sc)[MP][MP] = G;
  double (&E)[MP][MP] = Ri;
  double (&sj)[MP] = sb.sj;
  for (int e = l; e < MP * MP; e += 256) (&E[0][0])[e] = (e / MP == e % MP) ? 1.0 : 0.0;
  double dmax = 0.0;
  for (int j = 0; j < MP; ++j) dmax = fmax(dmax, Sc[j][j]);
  const double scale = sqrt(fmax(dmax, 0.0));
  __syncthreads();
  uint32_t keep = 0;
  for (int j = 0; j < MP; ++j) {
    const double nj = sqrt(fmax(Sc[j][j], 0.0));
    const bool kept = nj > (double)tau * scale && nj > 0.0;   // uniform
    const double inv = kept ? 1.0 / nj : 0.0;
    if (kept) keep |= 1u << j;
    if (l == 0) sj[j] = inv;
    if (kept) {
      for (int e = l; e < MP * MP; e += 256) {
        const int r = e / MP, c = e % MP;
        if (r > j) {
          const double rr = Sc[j][r] * inv;                   // R[j][r]
          if (c > j) Sc[r][c] -= rr * (Sc[j][c] * inv);
          E[r][c] -= rr * (E[j][c] * inv);
        }
      }
    }
    __syncthreads();
  }
  for (int e = l; e < MP * MP; e += 256) (&E[0][0])[e] *= sj[e / MP];
  __syncthreads();
  // Ri = E^T, back into Ri's storage (E aliases it): transpose via R (scratch)
  for (int e = l; e < MP * MP; e += 256) (&R[0][0])[e] = E[e % MP][e / MP];
  __syncthreads();
  for (int e = l; e < MP * MP; e += 256) (&Ri[0][0])[e] = (&R[0][0])[e];
  __syncthreads();
  // M[c][t] = sum_a Ri[a][c] XP[a][t]
  for (int e = l; e < MP * kMaxTail; e += 256) {
    const int c = e / kMaxTail, t = e % kMaxTail;
    double v = 0.0;
    for (int a = 0; a <= c; ++a) v += Ri[a][c] * XP[a][t];
    M[c][t] = v;
  }
  __syncthreads();
  // N[a][t] = sum_c Ri[a][c] M[c][t]
  for (int e = l; e < MP * kMaxTail; e += 256) {
    const int a = e / kMaxTail, t = e % kMaxTail;
    double v = 0.0;
    for (int c = a; c < MP; ++c) v += Ri[a][c] * M[c][t];
    sb.N[a][t] = v;
  }
  __syncthreads();
  return keep;
}

// Q = X Ri and P' = P - X N for kApplyRows rows (16 per wave); K slot l / 16
// is column 4 ks + l / 16 of X. Each work group first forms its sample's
// basis from the Gram partials itself (a few microseconds of LDS work), which
// costs less than a launch of its own between the two kernels.
template <int MP>
__global__ void __launch_bounds__(256) k_hpp_apply(const float* __restrict__ X, int p, int mt,
                                                   const void* __restrict__ P, int ptype,
                                                   const double* __restrict__ part, int nparts, float tau,
                                                   int32_t* rank_out, float* W3, int ldw) {
  constexpr int TA = MP / 16;
  __shared__ HppBasis<MP> sb;
  const int i = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const uint32_t keep = hpp_basis<MP>(part, nparts, tau, i, sb);
  if (blockIdx.x == 0 && tid == 0 && rank_out) rank_out[i] = __popc(keep);
  double (&Ri)[MP][MP] = sb.Ri;
  double (&N)[MP][kMaxTail] = sb.N;
  const float* Xi = X + (int64_t)i * p * MP;
  float* Wi = W3 + (int64_t)i * p * ldw;
  const int r0 = blockIdx.x * kApplyRows + 16 * wv;
  const int arow = r0 + n;
  double xa[MP / 4], pr[4][2];
#pragma unroll
  for (int ks = 0; ks < MP / 4; ++ks) xa[ks] = arow < p ? (double)ldg_f32(Xi + (int64_t)arow * MP + 4 * ks + g) : 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = r0 + g + 4 * j;
    pr[j][0] = tail_val(P, ptype, p, mt, row, n);
    pr[j][1] = tail_val(P, ptype, p, mt, row, 16 + n);
  }
  __syncthreads();
  f64x4_t q[TA], pn[2];
#pragma unroll
  for (int t = 0; t < TA; ++t) q[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  pn[0] = pn[1] = f64x4_t{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < MP / 4; ++ks) {
    const int col = 4 * ks + g;
#pragma unroll
    for (int t = 0; t < TA; ++t) q[t] = mfma_f64(xa[ks], Ri[col][16 * t + n], q[t]);
    pn[0] = mfma_f64(xa[ks], N[col][n], pn[0]);
    pn[1] = mfma_f64(xa[ks], N[col][16 + n], pn[1]);
  }
  // lane l, element j of a v_mfma_f64_16x16x4 result: row l/16 + 4 j, column l % 16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = r0 + g + 4 * j;
    if (row >= p) continue;
    float* wr = Wi + (int64_t)row * ldw;
#pragma unroll
    for (int t = 0; t < TA; ++t) stg_f32(wr + 16 * t + n, (float)q[t][j]);
    if (n < mt) stg_f32(wr + MP + n, (float)(pr[j][0] - pn[0][j]));
    if (16 + n < mt) stg_f32(wr + MP + 16 + n, (float)(pr[j][1] - pn[1][j]));
  }
}

size_t hpp_qr_scratch_bytes(int MP, int B, int p) {
  const int nparts = (p + kGramRows - 1) / kGramRows;
  const int NT = MP == 16 ? HppTiles<16>::NT : HppTiles<32>::NT;
  const size_t part = (size_t)B * nparts * NT * 256 * 8;
  return (part + 255) / 256 * 256;
}

template <int MP>
static hipError_t hpp_qr(const float* X, int B, int p, int mt, const void* P, int ptype, float tau, float* W3,
                         int ldw, int32_t* rank, char* scratch, hipStream_t s) {
  const int nparts = (p + kGramRows - 1) / kGramRows;
  double* part = (double*)scratch;
  hipLaunchKernelGGL(k_hpp_gram<MP>, dim3(nparts, B), dim3(256), 0, s, X, p, mt, P, ptype, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_hpp_apply<MP>, dim3((p + kApplyRows - 1) / kApplyRows, B), dim3(256), 0, s, X, p, mt, P,
                     ptype, (const double*)part, nparts, tau, rank, W3, ldw);
  return hipGetLastError();
}

hipError_t launch_hpp_qr(const float* X, int MP, int B, int p, int mt, const void* P, int ptype, float tau, float* W3,
                         int ldw, int32_t* rank, void* scratch, hipStream_t s) {
  if (MP == 16) return hpp_qr<16>(X, B, p, mt, P, ptype, tau, W3, ldw, rank, (char*)scratch, s);
  if (MP == 32) return hpp_qr<32>(X, B, p, mt, P, ptype, tau, W3, ldw, rank, (char*)scratch, s);
  return hipErrorInvalidValue;
}

}  // namespace dpn
