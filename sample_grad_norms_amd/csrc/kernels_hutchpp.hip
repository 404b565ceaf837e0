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
//                 (v_mfma_f64_16x16x4), many work groups per sample; when
//                 the sketch pass split T, k_hpp_ysum_gram first sums the
//                 chunk's rows of X over the split partials (and stores X),
//                 in place of that pass's own split-T sum;
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
// 1/tau, so Q is orthonormal to about (1/tau)^2 * 2^-53 ~ 1e-8 in fp64.
#include <cstring>

#include "device_common.h"
#include "internal.h"

namespace dpn {

typedef double f64x4_t __attribute__((ext_vector_type(4)));
constexpr int kMaxTail = 32;
constexpr int kGramRows = 128;   // rows of X per Gram work group (k_hpp_gram, k_hpp_ysum_gram)
constexpr int kApplyRows = 64;   // rows of X per k_hpp_apply work group (4 waves x 16)
constexpr int kMaxYCols = 32;    // columns of a stored sketch pass that k_hpp_ysum_pack takes

__device__ __forceinline__ f64x4_t mfma_f64(double a, double b, f64x4_t c) {
  return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

template <int MP>
struct HppTiles {
  static constexpr int TA = MP / 16;            // 16-column tiles of X
  static constexpr int NG = TA * (TA + 1) / 2;  // Gram tiles (upper triangle)
  static constexpr int NT = NG + 2 * TA;        // + X^T P tiles (tail columns up to 32)
};

// Loads in these kernels are issued unconditionally from indices clamped into
// range and the out-of-range values replaced afterwards: a load under a
// per-lane condition gets a wait of its own, which serialises them.

// Entry (row, t) of the tail projection P [p][mt], 0 outside it.
template <bool BF16>
__device__ __forceinline__ double tail_val(const void* P, int p, int mt, int row, int t) {
  const int64_t off = (int64_t)min(row, p - 1) * mt + min(t, mt - 1);
  const float v = BF16 ? bf16_bits_to_f32(((const uint16_t*)P)[off]) : ldg_f32((const float*)P + off);
  return row < p && t < mt ? (double)v : 0.0;
}

// Entry (row, c) of X [p][MP], 0 past p rows.
template <int MP>
__device__ __forceinline__ double x_val(const float* Xi, int p, int row, int c) {
  const float v = ldg_f32(Xi + (int64_t)min(row, p - 1) * MP + c);
  return row < p ? (double)v : 0.0;
}

// Partial tiles of X^T X (upper triangle) and X^T P for kGramRows rows:
// part [B][nparts][NT][4][64] (the accumulator registers of each tile).
// The contraction runs over rows: K slot l / 16 is row 4 ks + l / 16.
// xrow(row, c) gives entry (row, c) of X, 0 past p rows; pv holds the tail
// projection's entries (row0 + 4 u, 16 tt + n), loaded by the caller.
template <int MP, class XRow>
__device__ __forceinline__ void hpp_gram_tiles(const XRow& xrow, const double (&pv)[kGramRows / 16][2], int row0,
                                               double* part) {
  using H = HppTiles<MP>;
  constexpr int TA = H::TA, NG = H::NG, NT = H::NT;
  constexpr int U = kGramRows / 4 / 4;  // K steps per wave, loads issued together
  __shared__ double red[4][NT][4][64];
  const int s = blockIdx.x, i = blockIdx.y, nparts = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15;
  f64x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  double xa[U][TA];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int a = 0; a < TA; ++a) xa[u][a] = xrow(row0 + 4 * u, 16 * a + n);
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

// The tail projection's entries a lane of the Gram tiles uses.
__device__ __forceinline__ void hpp_tail_rows(const void* P, int ptype, int p, int mt, int row0,
                                              double (&pv)[kGramRows / 16][2]) {
  constexpr int U = kGramRows / 16;
  const int n = threadIdx.x & 15;
  if (ptype == SRC_BF16) {  // uniform
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) pv[u][tt] = tail_val<true>(P, p, mt, row0 + 4 * u, 16 * tt + n);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) pv[u][tt] = tail_val<false>(P, p, mt, row0 + 4 * u, 16 * tt + n);
  }
}

// Row of the first K step of this lane: wave wv takes rows 64 wv .. 64 wv + 63
// of the chunk, four per K step.
__device__ __forceinline__ int hpp_gram_row0() {
  return blockIdx.x * kGramRows + 4 * (threadIdx.x >> 6) * (kGramRows / 16) + ((threadIdx.x & 63) >> 4);
}

// Gram partials from the stored X [B][p][MP].
template <int MP>
__global__ void __launch_bounds__(256) k_hpp_gram(const float* __restrict__ X, int p, int mt,
                                                  const void* __restrict__ P, int ptype, double* part) {
  const float* Xi = X + (int64_t)blockIdx.y * p * MP;
  const int row0 = hpp_gram_row0();
  double pv[kGramRows / 16][2];
  hpp_tail_rows(P, ptype, p, mt, row0, pv);
  hpp_gram_tiles<MP>([&](int row, int c) { return x_val<MP>(Xi, p, row, c); }, pv, row0, part);
}

// The sketch pass's split-T sum fused with the Gram partials: the work group
// sums its kGramRows rows of X over the nsplit partial tiles of Ypart
// [nsplit][B][p][MP] (in split order, fp64, rounded to fp32), stores them to
// X as the pass's own split-T sum would, and forms the partial tiles from
// those fp32 values, so X and the tiles are bitwise what the split-T sum
// followed by k_hpp_gram give.
template <int MP>
__global__ void __launch_bounds__(256) k_hpp_ysum_gram(const float* __restrict__ Ypart, int nsplit, int B,
                                                       float* X, int p, int mt, const void* __restrict__ P,
                                                       int ptype, double* part) {
  __shared__ float tile[kGramRows * MP];
  const int i = blockIdx.y, rb = blockIdx.x * kGramRows;
  const int row0 = hpp_gram_row0();
  double pv[kGramRows / 16][2];
  hpp_tail_rows(P, ptype, p, mt, row0, pv);
  const int64_t stride = (int64_t)B * p * MP;
  const float* Y = Ypart + ((int64_t)i * p + rb) * MP;
  float* Xo = X + ((int64_t)i * p + rb) * MP;
  // every lane's loads of a split are issued together (J float4 groups, one
  // row each as MP is a multiple of 4), eight splits at a time
  constexpr int J = kGramRows * MP / 1024;
  bool ok[J];
  double y[J][4];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    ok[j] = rb + (1024 * j + 4 * (int)threadIdx.x) / MP < p;
#pragma unroll
    for (int q = 0; q < 4; ++q) y[j][q] = 0.0;
  }
#pragma unroll 8
  for (int ts = 0; ts < nsplit; ++ts) {
    float4 v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = 1024 * j + 4 * threadIdx.x;
      v[j] = ldg_f32x4(Y + ts * stride + (ok[j] ? e : 0));
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      y[j][0] += ok[j] ? (double)v[j].x : 0.0;
      y[j][1] += ok[j] ? (double)v[j].y : 0.0;
      y[j][2] += ok[j] ? (double)v[j].z : 0.0;
      y[j][3] += ok[j] ? (double)v[j].w : 0.0;
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = 1024 * j + 4 * threadIdx.x;
    const float4 f = make_float4((float)y[j][0], (float)y[j][1], (float)y[j][2], (float)y[j][3]);
    *(float4*)(tile + e) = f;
    if (ok[j]) stg16(Xo + e, make_uint4(__float_as_uint(f.x), __float_as_uint(f.y), __float_as_uint(f.z),
                                        __float_as_uint(f.w)));
  }
  __syncthreads();
  hpp_gram_tiles<MP>(
      [&](int row, int c) { return row < p ? (double)tile[(row - rb) * MP + c] : 0.0; }, pv, row0, part);
}

// The basis of one sample in LDS: the Gram tiles summed from their partials,
// R with the rank rule, Ri = R^-1 on the kept columns, M = Q^T P and N = Ri M.
template <int MP>
struct HppBasis {
  double G[MP][MP], XP[MP][kMaxTail], R[MP][MP], Ri[MP][MP], M[MP][kMaxTail], N[MP][kMaxTail];
  double xmax2;    // the largest squared column norm of X
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
  // fixed-order sum over the parts (sixteen or eight at a time, every tile's
  // loads in flight together); lane q, element j of a v_mfma_f64_16x16x4 result is
  // (row q/16 + 4 j, column q % 16); thread l holds element l of each tile
  constexpr int PR = NT <= 3 ? 16 : 8;   // parts whose loads are in flight together
  double v[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) v[t] = 0.0;
  for (int s0 = 0; s0 < nparts; s0 += PR) {
    double w[NT][PR];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < PR; ++u) w[t][u] = pi[(int64_t)min(s0 + u, nparts - 1) * NT * 256 + t * 256 + l];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < PR; ++u) v[t] += s0 + u < nparts ? w[t][u] : 0.0;
  }
  {
    const int j = l >> 6, q = l & 63;
    const int r = (q >> 4) + 4 * j, c = q & 15;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < NG) {
        int a = 0, b = 0;
        for (int aa = 0, k = 0; aa < TA; ++aa)
          for (int bb = aa; bb < TA; ++bb, ++k)
            if (k == t) {
              a = aa;
              b = bb;
            }
        G[16 * a + r][16 * b + c] = v[t];
        G[16 * b + c][16 * a + r] = v[t];
      } else {
        const int a = (t - NG) >> 1, tt = (t - NG) & 1;
        XP[16 * a + r][16 * tt + c] = v[t];
      }
    }
  }
  __syncthreads();

  // Right-looking Cholesky on the Schur complement Sc (= G at the start), one
  // entry per thread: at step j the pivot is d_j = Sc[j][j]; if column j is
  // kept, row j of R is row j of Sc over d_j^(1/2) and every later entry
  // (a, b) loses Sc[j][a] Sc[j][b] / d_j, so the d_j a step reads is G[j][j]
  // minus the squares of the kept rows above it, subtracted in row order.
  // The same row operations on the identity give E = R^-T with its rows left
  // unscaled: row j is scaled by d_j^(-1/2) once at the end (rows of dropped
  // columns by 0). The square roots wait until after the loop (Sc[j][j]
  // keeps d_j, since later steps change only entries below and right of it).
  // Column j is kept when d_j^(1/2) > tau max_a ||x_a||, compared as squares.
  // Steps go in pairs, one barrier each: every thread reads rows j and j + 1
  // and recomputes the entries of row j + 1 it needs after step j with the
  // same operations as their owners, then applies both steps to its own
  // entries, which it holds in registers; it stores those of rows read by
  // later pairs (rows past j + 1) before the barrier and the rest after the
  // loop, so no entry of rows j, j + 1 changes while the pair reads them.
  double (&Sc)[MP][MP] = G;
  double (&E)[MP][MP] = R;
  constexpr int EPT = MP * MP / 256;   // entries per thread
  static_assert(MP % 2 == 0, "steps go in pairs");
  for (int e = l; e < MP * MP; e += 256) (&E[0][0])[e] = (e / MP == e % MP) ? 1.0 : 0.0;
  double dmax = 0.0;
  for (int j = 0; j < MP; ++j) dmax = fmax(dmax, Sc[j][j]);
  const double thr = (double)tau * sqrt(fmax(dmax, 0.0));
  const double thr2 = thr * thr;
  if (l == 0) sb.xmax2 = dmax;
  double xs[EPT], xe[EPT];   // this thread's entries of Sc and E
#pragma unroll
  for (int u = 0; u < EPT; ++u) {
    const int e = l + 256 * u;
    xs[u] = (&Sc[0][0])[e];
    xe[u] = (e / MP == e % MP) ? 1.0 : 0.0;
  }
  __syncthreads();
  uint32_t keep = 0;
  for (int j = 0; j < MP; j += 2) {
    const int j1 = j + 1;
    const double dj = Sc[j][j], aj1 = Sc[j][j1];
    double d1 = Sc[j1][j1];
    double s0r[EPT], s0c[EPT], e0c[EPT], s1r[EPT], s1c[EPT], e1c[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = l + 256 * u, r = e / MP, c = e % MP;
      s0r[u] = Sc[j][r];
      s0c[u] = Sc[j][c];
      e0c[u] = E[j][c];
      s1r[u] = Sc[j1][r];
      s1c[u] = Sc[j1][c];
      e1c[u] = E[j1][c];
    }
    // step j
    const bool kept0 = dj > 0.0 && dj > thr2;   // uniform
    if (kept0) {
      keep |= 1u << j;
      const double inv = 1.0 / dj;
      // row j + 1 after step j, as its owners compute it (their factor is
      // Sc[j][j+1] / d_j)
      const double f1 = aj1 * inv;
      d1 -= f1 * aj1;
#pragma unroll
      for (int u = 0; u < EPT; ++u) {
        const int e = l + 256 * u, r = e / MP, c = e % MP;
        if (r > j) s1r[u] -= f1 * s0r[u];
        if (c > j) s1c[u] -= f1 * s0c[u];
        e1c[u] -= f1 * e0c[u];
        if (r > j) {
          const double f = s0r[u] * inv;
          if (c > j) xs[u] -= f * s0c[u];
          xe[u] -= f * e0c[u];
        }
      }
    }
    // step j + 1
    const bool kept1 = d1 > 0.0 && d1 > thr2;   // uniform
    if (kept1) {
      keep |= 1u << j1;
      const double inv = 1.0 / d1;
#pragma unroll
      for (int u = 0; u < EPT; ++u) {
        const int e = l + 256 * u, r = e / MP, c = e % MP;
        if (r > j1) {
          const double f = s1r[u] * inv;
          if (c > j1) xs[u] -= f * s1c[u];
          xe[u] -= f * e1c[u];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int e = l + 256 * u, r = e / MP;
      if (r > j1) {
        (&Sc[0][0])[e] = xs[u];
        (&E[0][0])[e] = xe[u];
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < EPT; ++u) {
    const int e = l + 256 * u;
    (&Sc[0][0])[e] = xs[u];
    (&E[0][0])[e] = xe[u];
  }
  __syncthreads();
  // Ri = E^T with row c of E (held in R) scaled by d_c^(-1/2), 0 for dropped
  // columns; every thread takes the square roots it needs itself
  for (int e = l; e < MP * MP; e += 256) {
    const int a = e / MP, c = e % MP;
    const double sc = (keep >> c) & 1u ? 1.0 / sqrt(Sc[c][c]) : 0.0;
    (&Ri[0][0])[e] = E[c][a] * sc;
  }
  __syncthreads();
  // M[c][t] = sum_a Ri[a][c] XP[a][t]
  // (both sums run over the triangle of Ri in index order; every operand is
  // read before the first product)
  for (int e = l; e < MP * kMaxTail; e += 256) {
    const int c = e / kMaxTail, t = e % kMaxTail;
    double ra[MP], xa[MP];
#pragma unroll
    for (int a = 0; a < MP; ++a) {
      ra[a] = Ri[a][c];
      xa[a] = XP[a][t];
    }
    double v = 0.0;
#pragma unroll
    for (int a = 0; a < MP; ++a)
      if (a <= c) v += ra[a] * xa[a];
    M[c][t] = v;
  }
  __syncthreads();
  // N[a][t] = sum_c Ri[a][c] M[c][t]
  for (int e = l; e < MP * kMaxTail; e += 256) {
    const int a = e / kMaxTail, t = e % kMaxTail;
    double ra[MP], mc[MP];
#pragma unroll
    for (int c = 0; c < MP; ++c) {
      ra[c] = Ri[a][c];
      mc[c] = M[c][t];
    }
    double v = 0.0;
#pragma unroll
    for (int c = 0; c < MP; ++c)
      if (c >= a) v += ra[c] * mc[c];
    sb.N[a][t] = v;
  }
  __syncthreads();
  return keep;
}

// ---------------------------------------------------------------------------
// The next pass's tables and packed projection, written by the kernel that
// produces the projection, so that pass needs no prepare launch.
// ---------------------------------------------------------------------------
// Record 0 and both work lists, as the prepare kernel writes them for a lone
// layer: items1 (0, sample, row block, 0), items2 (0, sample, column block,
// T split) with the split innermost.
// Every work group of the grid writes its own slice of the entries (work
// group 0 also the record), so no group carries all of them.
__device__ void hpp_write_tables(const HppNext& nx) {
  const int nb = gridDim.x * gridDim.y, b = blockIdx.y * gridDim.x + blockIdx.x;
  const int total = nx.n1 + nx.n2, per = (total + nb - 1) / nb;
  const int end = min(total, (b + 1) * per);
  for (int r = b * per + threadIdx.x; r < end; r += blockDim.x) {
    if (r < nx.n1) {
      const int i = r / nx.rbs;
      nx.items1[r] = make_int4(0, i, r - i * nx.rbs, 0);
    } else {
      const int r2 = r - nx.n1;
      const int ts = r2 % nx.nsplit, q = r2 / nx.nsplit;
      const int ub = q % nx.ubs, i = q / nx.ubs;
      nx.items2[r2] = make_int4(0, i, ub, ts);
    }
  }
  if (b == 0 && threadIdx.x == 0) nx.recs[0] = nx.rec;
}

// The packed units of rows r0 .. r0 + 63 (r0 a multiple of 64) of sample
// smp, from an fp32 tile in LDS (row-major, ldt floats a row): unit (ks, jb,
// h, lane) holds rows 32 ks + 8 (lane / 16) + 0..7 of column 16 jb + lane %
// 16, as bf16 (h = 0) or the bf16 residual (h = 1); rows past `rows` and
// columns past `ncols` are zero. The same units the prepare kernel packs.
__device__ void hpp_pack_tile(const float* tile, int ldt, int r0, int smp, const HppNext& nx) {
  const int units = 2 * nx.NCB * 2 * 64;  // two K steps of 32 rows
  for (int u = threadIdx.x; u < units; u += blockDim.x) {
    const int lane = u & 63;
    int q = u >> 6;
    const int h = q & 1;
    q >>= 1;
    const int jb = q % nx.NCB, ks = r0 / 32 + q / nx.NCB;
    const int c = 16 * jb + (lane & 15);
    uint32_t b[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int v = 32 * ks + 8 * (lane >> 4) + s;
      const float x = (v < nx.rows && c < nx.ncols) ? tile[(v - r0) * ldt + c] : 0.f;
      uint32_t hi, lo;
      split_bf16(x, hi, lo);
      b[s] = h ? lo : hi;
    }
    stg16(nx.W + smp * nx.w_stride_b + (int64_t)((ks * nx.NCB + jb) * 2 + h) * 64 + lane, pack8(b));
  }
}

// Split-T sum of a stored pass for 64 rows of one sample (in split order,
// fp64, rounded to fp32 as the stored Y would be), packed for the next pass.
__global__ void __launch_bounds__(256) k_hpp_ysum_pack(const float* __restrict__ Ypart, int nsplit, int B, int w,
                                                       int NC, HppNext nx) {
  __shared__ float tile[64 * kMaxYCols];
  const int i = blockIdx.y, r0 = blockIdx.x * 64;
  const int64_t stride = (int64_t)B * w * NC;
  const float* Y = Ypart + ((int64_t)i * w + r0) * NC;
  for (int e = 4 * threadIdx.x; e < 64 * NC; e += 1024) {  // NC is a multiple of 16: one row per float4
    double y[4] = {0.0, 0.0, 0.0, 0.0};
    if (r0 + e / NC < w) {
#pragma unroll 8
      for (int ts = 0; ts < nsplit; ++ts) {
        const float4 v = ldg_f32x4(Y + ts * stride + e);
        y[0] += (double)v.x;
        y[1] += (double)v.y;
        y[2] += (double)v.z;
        y[3] += (double)v.w;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[e + q] = (float)y[q];
  }
  __syncthreads();
  hpp_pack_tile(tile, NC, r0, i, nx);
  hpp_write_tables(nx);
}

// Q = X Ri and P' = P - X N for kApplyRows rows (16 per wave); K slot l / 16
// is column 4 ks + l / 16 of X. Each work group first forms its sample's
// basis from the Gram partials itself (a few microseconds of LDS work), which
// costs less than a launch of its own between the two kernels.
template <int MP>
__global__ void __launch_bounds__(256) k_hpp_apply(const float* __restrict__ X, int p, int mt,
                                                   const void* __restrict__ P, int ptype,
                                                   const double* __restrict__ part, int nparts, float tau,
                                                   int32_t* rank_out, float* resid_out, int ms, float* W3, int ldw,
                                                   int pack, HppNext nx) {
  constexpr int TA = MP / 16;
  __shared__ HppBasis<MP> sb;
  __shared__ float tile[kApplyRows * (MP + kMaxTail)];   // this group's rows of W3, when packing
  const int i = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  // this group's rows of X and P, loaded before the basis so their latency
  // overlaps it
  const float* Xi = X + (int64_t)i * p * MP;
  float* Wi = W3 + (int64_t)i * p * ldw;
  const int r0 = blockIdx.x * kApplyRows + 16 * wv;
  const int arow = r0 + n;
  double xa[MP / 4], pr[4][2];
#pragma unroll
  for (int ks = 0; ks < MP / 4; ++ks) xa[ks] = x_val<MP>(Xi, p, arow, 4 * ks + g);
  if (ptype == SRC_BF16) {  // uniform
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) pr[j][tt] = tail_val<true>(P, p, mt, r0 + g + 4 * j, 16 * tt + n);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) pr[j][tt] = tail_val<false>(P, p, mt, r0 + g + 4 * j, 16 * tt + n);
  }
  const uint32_t keep = hpp_basis<MP>(part, nparts, tau, i, sb);
  if (blockIdx.x == 0 && tid == 0 && rank_out) rank_out[i] = __popc(keep);
  // the residual each keep decision compared with tau: the Cholesky pivot
  // d_j (the squared residual of column j after the kept columns before it;
  // the diagonal of the Schur complement keeps it) over the largest squared
  // column norm, as a norm ratio
  if (blockIdx.x == 0 && tid < ms && resid_out) {
    const double m2 = sb.xmax2;
    resid_out[(int64_t)i * ms + tid] = m2 > 0.0 ? (float)sqrt(fmax(sb.G[tid][tid], 0.0) / m2) : 0.f;
  }
  double (&Ri)[MP][MP] = sb.Ri;
  double (&N)[MP][kMaxTail] = sb.N;
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
    if (pack) {  // for the next pass the rows go to LDS only (rows past p too; the packer zeroes them)
      float* tr = tile + (row - blockIdx.x * kApplyRows) * ldw;
#pragma unroll
      for (int t = 0; t < TA; ++t) tr[16 * t + n] = (float)q[t][j];
      if (n < mt) tr[MP + n] = (float)(pr[j][0] - pn[0][j]);
      if (16 + n < mt) tr[MP + 16 + n] = (float)(pr[j][1] - pn[1][j]);
      continue;
    }
    if (row >= p) continue;
    float* wr = Wi + (int64_t)row * ldw;
#pragma unroll
    for (int t = 0; t < TA; ++t) stg_f32(wr + 16 * t + n, (float)q[t][j]);
    if (n < mt) stg_f32(wr + MP + n, (float)(pr[j][0] - pn[0][j]));
    if (16 + n < mt) stg_f32(wr + MP + 16 + n, (float)(pr[j][1] - pn[1][j]));
  }
  if (pack) {  // uniform
    __syncthreads();
    hpp_pack_tile(tile, ldw, blockIdx.x * kApplyRows, i, nx);
    hpp_write_tables(nx);
  }
}

size_t hpp_qr_scratch_bytes(int MP, int B, int p) {
  const int nparts = (p + kGramRows - 1) / kGramRows;
  const int NT = MP == 16 ? HppTiles<16>::NT : HppTiles<32>::NT;
  const size_t part = (size_t)B * nparts * NT * 256 * 8;
  return (part + 255) / 256 * 256;
}

template <int MP>
static hipError_t hpp_qr(const float* Ypart, int nsplit, float* X, int B, int p, int mt, const void* P, int ptype,
                         float tau, float* W3, int ldw, int32_t* rank, float* resid, int ms, char* scratch,
                         const HppNext* next, hipStream_t s) {
  const int nparts = (p + kGramRows - 1) / kGramRows;
  double* part = (double*)scratch;
  if (Ypart)
    hipLaunchKernelGGL(k_hpp_ysum_gram<MP>, dim3(nparts, B), dim3(256), 0, s, Ypart, nsplit, B, X, p, mt, P, ptype,
                       part);
  else
    hipLaunchKernelGGL(k_hpp_gram<MP>, dim3(nparts, B), dim3(256), 0, s, X, p, mt, P, ptype, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  HppNext nx;
  std::memset(&nx, 0, sizeof(nx));
  if (next) nx = *next;
  hipLaunchKernelGGL(k_hpp_apply<MP>, dim3((p + kApplyRows - 1) / kApplyRows, B), dim3(256), 0, s, X, p, mt, P,
                     ptype, (const double*)part, nparts, tau, rank, resid, ms, W3, ldw, next ? 1 : 0, nx);
  return hipGetLastError();
}

hipError_t launch_hpp_qr(const float* Ypart, int nsplit, float* X, int MP, int B, int p, int mt, const void* P,
                         int ptype, float tau, float* W3, int ldw, int32_t* rank, float* resid, int ms, void* scratch,
                         const HppNext* next, hipStream_t s) {
  if (next && (ldw > MP + kMaxTail || next->ncols > ldw || next->NCB * 16 != ldw)) return hipErrorInvalidValue;
  if (ms < 0 || ms > MP || ms > 256) return hipErrorInvalidValue;
  if (Ypart && nsplit < 1) return hipErrorInvalidValue;
  if (MP == 16)
    return hpp_qr<16>(Ypart, nsplit, X, B, p, mt, P, ptype, tau, W3, ldw, rank, resid, ms, (char*)scratch, next, s);
  if (MP == 32)
    return hpp_qr<32>(Ypart, nsplit, X, B, p, mt, P, ptype, tau, W3, ldw, rank, resid, ms, (char*)scratch, next, s);
  return hipErrorInvalidValue;
}

hipError_t launch_hpp_ysum_pack(const float* Ypart, int nsplit, int B, int w, int NC, const HppNext& next,
                                hipStream_t s) {
  if (NC > kMaxYCols || next.ncols > NC || next.NCB * 16 != NC || next.rows != w) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_hpp_ysum_pack, dim3((w + 63) / 64, B), dim3(256), 0, s, Ypart, nsplit, B, w, NC, next);
  return hipGetLastError();
}

}  // namespace dpn
