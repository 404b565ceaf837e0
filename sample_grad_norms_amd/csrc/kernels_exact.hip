// Exact per-sample squared norm ||A_i^T G_i||_F^2, the comparator of the
// estimators ('Efficient DP-SGD for LLMs with Randomized Clipping',
// papernotes.org note, 研究背景与动机 and 相关工作: explicit per-sample
// gradients cost O(T d p), ghost clipping works on T x T Gram matrices;
// gist.science/nl summary, Complexiteitsreductie).
//
// Explicit route: W_i = A_i^T G_i is formed tile by tile in MFMA
// accumulators (contraction over T, both operands transposed in registers)
// and squared in place; nothing of size d x p is stored.
// Gram route: n_i = <A_i A_i^T, G_i G_i^T>_F; a work group forms matching
// tiles of both Gram matrices (contractions over d and p, operands read
// row-major as stored; 256 x 128 in bf16, 128 x 128 in fp32) and sums their
// elementwise product, each unordered pair of rows once with weight 2 off
// the diagonal; nothing of size T x T is stored.
// Both write one fp64 partial per tile; the per-sample finisher adds them in
// a fixed order.
#include "device_common.h"
#include "internal.h"

namespace dpn {

struct ExactArgs {
  const void* A;
  const void* G;
  int32_t B, T, d, p;
  int32_t tu, tv;       // explicit: tiles along d and p; gram: tu = tiles along T
  int32_t n_items;
  int32_t slots;        // partial slots per sample
  double2* partials;
};

// ---------------------------------------------------------------------------
// Explicit, bf16: one work group per 256 (d) x 256 (p) tile of W_i, each wave
// a 128 x 128 quarter (wave w: A columns 128 (w % 2), G columns 128 (w / 2)).
// Every 32-row chunk of the tile's A and G columns (2 x 16 KB) is streamed
// into LDS with direct global-to-LDS loads (four-slot ring, three chunks in
// flight), so each A and G fragment is read from memory once for two waves.
// The MFMA operands (16 columns x 32 rows, T along K) are read straight from
// the row-major chunk with transposing LDS reads; the 16-byte units of a row
// are XOR-swizzled by the row index so the four rows of one such read fall on
// different banks. Rows past T are loaded from a zero row; columns past d or
// p load the last valid column and the W entries they make are left out of
// the sum. Tiles are numbered with the A tile fastest, so the tiles one XCD
// takes (a contiguous range) cover all of A for a few G tiles, and G is
// fetched from HBM about once.
// With one wave per SIMD nothing hides a stall but the wave's own MFMAs, so
// each chunk's 64 MFMAs run in shells of growing max(e, f): the first needs
// two operands, not nine, and the eight loads of chunk c + 3 are spread over
// the shells instead of issued as one block ahead of them.
// ---------------------------------------------------------------------------
constexpr int kXTile = 256;                       // tile edge along d and along p
constexpr int kXRows = 32;                        // rows per chunk (one MFMA K step)
constexpr int kXOpBytes = kXRows * kXTile * 2;    // one operand's chunk (16 KB)
constexpr int kXBufs = 4;                         // LDS ring: three chunks in flight, one in use

__device__ __attribute__((aligned(16))) uint4 g_zero_row[kXTile / 8];  // 512 zero bytes (static storage)

// 16 x 32 operand of columns m0 .. m0 + 15 from a swizzled 32 x 256 chunk:
// K slot (g, s) is row slot_row(g, s), as in the other contractions.
__device__ __forceinline__ uint4 tr_operand(const unsigned char* chunk, int m0, int n, int g) {
  const int j = n >> 2, q = n & 3;
  const int u = (m0 >> 3) + (q >> 1), half = (q & 1) * 8;
  const int k1 = 4 * g + j, k2 = 16 + 4 * g + j;  // rows of K slots s = j and s = 4 + j
  const uint2 lo = lds_read_tr16(chunk + k1 * 512 + ((u ^ (k1 & 7)) << 4) + half);
  const uint2 hi = lds_read_tr16(chunk + k2 * 512 + ((u ^ (k2 & 7)) << 4) + half);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

__global__ void __launch_bounds__(256) k_exact_explicit_bf16(ExactArgs a) {
  constexpr int kStage = 2 * kXOpBytes;           // A chunk, then G chunk
  constexpr int kDma = kXOpBytes / 1024 / 4;      // 1 KB loads per wave per operand per chunk
  constexpr int kP = 2 * kDma;                    // loads per wave per chunk
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kXBufs * kStage];
  __shared__ double red[4];
  const int item = xcd_item(blockIdx.x, (uint32_t)a.n_items);
  const int per_i = a.tu * a.tv;
  const int i = item / per_i, rem = item - i * per_i;
  const int tv = rem / a.tu, tu = rem - tv * a.tu;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int T = a.T, d = a.d, p = a.p;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;

  // loads: instruction j of wave wv fills chunk row 8 wv + 2 j + lane / 32 at
  // unit position lane % 32, which holds the tile's column unit
  // (lane % 32) ^ (row % 8) (512 bytes per row)
  const int pos = lane & 31;
  const uint16_t* Ab = (const uint16_t*)a.A + (int64_t)i * T * d;
  const uint16_t* Gb = (const uint16_t*)a.G + (int64_t)i * T * p;
  const unsigned char* zero = (const unsigned char*)g_zero_row + pos * 16;
  int acol[kDma], gcol[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int unit = pos ^ ((2 * j + (lane >> 5)) & 7);
    acol[j] = min(kXTile * tu + 8 * unit, d - 8);
    gcol[j] = min(kXTile * tv + 8 * unit, p - 8);
  }
  const int nch = (T + kXRows - 1) / kXRows;
  // Load j (0..3) of one operand of chunk c; chunks past the end load the
  // zero row into a slot no later chunk uses, so every chunk issues the same
  // loads and the waits below are constant.
  auto dma = [&](int c, int j, int side) {
    const int t = kXRows * c + 8 * wv + 2 * j + (lane >> 5);
    const uint32_t buf = lds_base + (uint32_t)((c % kXBufs) * kStage + side * kXOpBytes + (4 * wv + j) * 1024);
    const void* src = side ? (const void*)(Gb + (int64_t)t * p + gcol[j]) : (const void*)(Ab + (int64_t)t * d + acol[j]);
    dma16(t < T ? src : (const void*)zero, buf);   // cached: four to eight work groups read each fragment
  };

  const int wa = wv & 1, wg = wv >> 1;
  f32x4_t acc[8][8];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int f = 0; f < 8; ++f) acc[e][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Each chunk's MFMAs run in shells s = max(e, f) = 0..7, so the first needs
  // two operands; the operands of shell s + 1 and one load of chunk c + 3 are
  // issued before shell s's MFMAs.
#pragma unroll
  for (int c = 0; c < kXBufs - 1; ++c)
#pragma unroll
    for (int j = 0; j < kDma; ++j) { dma(c, j, 0); dma(c, j, 1); }
  for (int c = 0; c < nch; ++c) {
    DPN_WAIT_VMCNT(2 * kP);   // chunk c landed (chunks c + 1 and c + 2 may be in flight)
    block_barrier();
    const unsigned char* buf = lds + (c % kXBufs) * kStage;
    uint4 oa[8], og[8];
    oa[0] = tr_operand(buf, 128 * wa, n, g);
    og[0] = tr_operand(buf + kXOpBytes, 128 * wg, n, g);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < 7) {
        oa[s + 1] = tr_operand(buf, 128 * wa + 16 * (s + 1), n, g);
        og[s + 1] = tr_operand(buf + kXOpBytes, 128 * wg + 16 * (s + 1), n, g);
      }
      dma(c + kXBufs - 1, s >> 1, s & 1);
#pragma unroll
      for (int t = 0; t < s; ++t) {
        acc[s][t] = mfma_bf16(oa[s], og[t], acc[s][t]);
        acc[t][s] = mfma_bf16(oa[t], og[s], acc[t][s]);
      }
      acc[s][s] = mfma_bf16(oa[s], og[s], acc[s][s]);
      __builtin_amdgcn_sched_barrier(0);   // keep the shells in order (hoisting all reads costs registers)
    }
  }
  DPN_WAIT_VMCNT(0);   // the trailing zero-row loads land before the work group ends
  // acc[e][f] lane (n, g), register r: W[u][v] with u = column 128 wa + 16 e + 4 g + r
  // of the tile's A columns and v = 128 wg + 16 f + n of its G columns
  const int u0 = kXTile * tu + 128 * wa, v0 = kXTile * tv + 128 * wg;
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double y = (double)acc[e][f][r];
        if (u0 + 16 * e + 4 * g + r < d && v0 + 16 * f + n < p) ss += y * y;
      }
  ss = wave_sum(ss);
  if (lane == 0) red[wv] = ss;
  __syncthreads();
  if (threadIdx.x == 0) a.partials[(int64_t)i * a.slots + rem] = make_double2((red[0] + red[1]) + (red[2] + red[3]), 0.0);
}

// ---------------------------------------------------------------------------
// Explicit, fp32: one wave per 64 x 64 tile; a lane's float4 of 4 consecutive
// columns of A (of G) at row 4 st + l/16 feeds the four MFMAs of its column
// offset, so no transpose is needed.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(64) k_exact_explicit_f32(ExactArgs a) {
  const int item = xcd_item(blockIdx.x, (uint32_t)a.n_items);
  const int per_i = a.tu * a.tv;
  const int i = item / per_i, rem = item - i * per_i;
  const int tu = rem / a.tv, tv = rem - tu * a.tv;
  const int lane = threadIdx.x, n = lane & 15, g = lane >> 4;
  const int T = a.T, d = a.d, p = a.p;
  const int ua = 64 * tu + 4 * n, vb = 64 * tv + 4 * n;
  const bool aok = ua < d, gok = vb < p;
  const float* Ap = (const float*)a.A + (int64_t)i * T * d + ua;
  const float* Gp = (const float*)a.G + (int64_t)i * T * p + vb;
  f32x4_t acc[4][4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[e][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int t0 = 0; t0 < T; t0 += 4) {
    const int t = t0 + g;
    const float4 x = (t < T && aok) ? ldg_f32x4(Ap + (int64_t)t * d) : z;
    const float4 y = (t < T && gok) ? ldg_f32x4(Gp + (int64_t)t * p) : z;
    const float xv[4] = {x.x, x.y, x.z, x.w}, yv[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[e][f] = mfma_f32(xv[e], yv[f], acc[e][f]);
  }
  double ss = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const double v = (double)acc[e][f][r];
        ss += v * v;
      }
  ss = wave_sum(ss);
  if (lane == 0) a.partials[(int64_t)i * a.slots + rem] = make_double2(ss, 0.0);
}

// Lower-triangular tile pair (bt >= bs) of linear index j.
__device__ __forceinline__ void tri_pair(int j, int& bt, int& bs) {
  int t = (int)((sqrt(8.0 * j + 1.0) - 1.0) * 0.5);
  while ((t + 1) * (t + 2) / 2 <= j) ++t;
  while (t * (t + 1) / 2 > j) --t;
  bt = t;
  bs = j - t * (t + 1) / 2;
}

// ---------------------------------------------------------------------------
// Gram, bf16: a work group takes rows t in [256 tb, 256 tb + 256) against
// rows s in [128 sb, 128 sb + 128) of one sample, for every s block that
// starts before the t block ends; entries weigh 2 (s < t), 1 (s = t) or 0
// (s > t), so every unordered pair of rows counts once. Wave (wy, wx) holds
// the 128 (t) x 64 (s) quarter of both Gram tiles, A A^T (K = d) then G G^T
// (K = p), in 2 x 128 accumulator registers: 12 operand reads per 32 MFMAs.
// K is streamed 32 columns at a time; a chunk is the pair's 384 rows x 64
// bytes (24 KB), stored as 24 one-kilobyte pieces of 16 rows in MFMA operand
// order (lane l holds row l % 16, columns 8 (l / 16) .. + 7), so an operand
// is one contiguous, conflict-free 16-byte read per lane. A six-slot ring
// keeps four chunks in flight; rows past T and columns past d (p) come from
// a zero row, and chunks past the end load zero rows into a slot no later
// chunk reads, so the waits are constant.
// ---------------------------------------------------------------------------
constexpr int kGT = 256, kGS = 128;            // t and s rows of a tile pair
constexpr int kGPieces = (kGT + kGS) / 16;     // 1 KB pieces per chunk (24)
constexpr int kGChunk = kGPieces * 1024;       // 24 KB
constexpr int kGBufs = 6;                      // 144 KB ring
constexpr int kGLoads = kGPieces / 4;          // loads per wave per chunk (6)

__device__ __forceinline__ void gram_pair(int j, int& tb, int& sb) {
  int t = (int)((sqrt(4.0 * j + 1.0) - 1.0) * 0.5);  // t (t + 1) <= j < (t + 1) (t + 2)
  while ((t + 1) * (t + 2) <= j) ++t;
  while (t * (t + 1) > j) --t;
  tb = t;
  sb = j - t * (t + 1);
}

__global__ void __launch_bounds__(256) k_exact_gram_bf16(ExactArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kGBufs * kGChunk];
  __shared__ double red[4];
  const int item = xcd_item(blockIdx.x, (uint32_t)a.n_items);
  const int i = item / a.slots, j = item - i * a.slots;
  int tb, sb;
  gram_pair(j, tb, sb);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
  const int T = a.T, d = a.d, p = a.p;
  const int nA = (d + 31) / 32, nst = nA + (p + 31) / 32;
  const uint16_t* Ab = (const uint16_t*)a.A + (int64_t)i * T * d;
  const uint16_t* Gb = (const uint16_t*)a.G + (int64_t)i * T * p;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
  const unsigned char* zero = (const unsigned char*)g_zero_row + (lane & 31) * 16;

  int row[kGLoads];
#pragma unroll
  for (int jj = 0; jj < kGLoads; ++jj) {
    const int pc = kGLoads * wv + jj;
    const int r = pc < kGT / 16 ? kGT * tb + 16 * pc + n : kGS * sb + 16 * (pc - kGT / 16) + n;
    row[jj] = r < T ? r : -1;
  }
  auto dma = [&](int st) {
    const bool onA = st < nA;
    const uint16_t* M = onA ? Ab : Gb;
    const int w = onA ? d : p;
    const int col = (onA ? st : st - nA) * 32 + 8 * g;
    const uint32_t buf = lds_base + (uint32_t)((st % kGBufs) * kGChunk);
#pragma unroll
    for (int jj = 0; jj < kGLoads; ++jj) {
      const bool ok = st < nst && row[jj] >= 0 && col < w;
      dma16(ok ? (const void*)(M + (int64_t)row[jj] * w + col) : (const void*)zero,
            buf + (uint32_t)((kGLoads * wv + jj) * 1024));
    }
  };
  const int wy = wv >> 1, wx = wv & 1;
  f32x4_t ka[8][4], kg[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ka[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      kg[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  auto chunk = [&](int st, f32x4_t (&acc)[8][4]) {
    const unsigned char* buf = lds + (st % kGBufs) * kGChunk + lane * 16;
    uint4 sv[4], tv[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) sv[q] = *(const uint4*)(buf + (kGT / 16 + 4 * wx + q) * 1024);
#pragma unroll
    for (int m = 0; m < 8; ++m) tv[m] = *(const uint4*)(buf + (8 * wy + m) * 1024);
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[m][q] = mfma_bf16(tv[m], sv[q], acc[m][q]);
  };
#pragma unroll
  for (int st = 0; st < kGBufs - 1; ++st) dma(st);
  for (int st = 0; st < nA; ++st) {
    DPN_WAIT_VMCNT((kGBufs - 2) * kGLoads);
    block_barrier();
    dma(st + kGBufs - 1);
    chunk(st, ka);
  }
  for (int st = nA; st < nst; ++st) {
    DPN_WAIT_VMCNT((kGBufs - 2) * kGLoads);
    block_barrier();
    dma(st + kGBufs - 1);
    chunk(st, kg);
  }
  DPN_WAIT_VMCNT(0);   // the trailing zero-row loads land before the work group ends
  // acc[m][q] lane (n, g), register r: Gram entry (t, s) with t = 256 tb +
  // 128 wy + 16 m + 4 g + r and s = 128 sb + 64 wx + 16 q + n
  double ss = 0.0;
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = kGT * tb + 128 * wy + 16 * m + 4 * g + r, u = kGS * sb + 64 * wx + 16 * q + n;
        const double wgt = (t >= T || u > t) ? 0.0 : (u < t ? 2.0 : 1.0);
        ss += wgt * ((double)ka[m][q][r] * (double)kg[m][q][r]);
      }
  ss = wave_sum(ss);
  if (lane == 0) red[wv] = ss;
  __syncthreads();
  if (threadIdx.x == 0)
    a.partials[(int64_t)i * a.slots + j] = make_double2((red[0] + red[1]) + (red[2] + red[3]), 0.0);
}

// ---------------------------------------------------------------------------
// Gram, fp32: same tiling with v_mfma_f32_16x16x4f32; a lane's float4 of 4
// consecutive columns feeds four MFMAs (K slot l / 16 is column 16 ks + 4 (l/16) + q).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void gram_tile_f32(const float* M, int T, int w, int trow0, int srow0,
                                              f32x4_t (&acc)[4][4], int n, int g) {
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  const int nks = (w + 15) >> 4;
  for (int ks = 0; ks < nks; ++ks) {
    const int col = 16 * ks + 4 * g;
    const bool cok = col < w;
    float4 ta[4], sb[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int tr = trow0 + 16 * m + n, sr = srow0 + 16 * m + n;
      ta[m] = (cok && tr < T) ? ldg_f32x4(M + (int64_t)tr * w + col) : z;
      sb[m] = (cok && sr < T) ? ldg_f32x4(M + (int64_t)sr * w + col) : z;
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[m][q] = mfma_f32(ta[m].x, sb[q].x, acc[m][q]);
        acc[m][q] = mfma_f32(ta[m].y, sb[q].y, acc[m][q]);
        acc[m][q] = mfma_f32(ta[m].z, sb[q].z, acc[m][q]);
        acc[m][q] = mfma_f32(ta[m].w, sb[q].w, acc[m][q]);
      }
  }
}

__global__ void __launch_bounds__(256) k_exact_gram_f32(ExactArgs a) {
  __shared__ double red[4];
  const int per_i = a.tu * (a.tu + 1) / 2;
  const int item = xcd_item(blockIdx.x, (uint32_t)a.n_items);
  const int i = item / per_i, j = item - i * per_i;
  int bt, bs;
  tri_pair(j, bt, bs);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, n = lane & 15, g = lane >> 4;
  const int trow0 = 128 * bt + 64 * (wv >> 1), srow0 = 128 * bs + 64 * (wv & 1);
  const int T = a.T;
  f32x4_t ka[4][4], kg[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ka[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      kg[m][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  gram_tile_f32((const float*)a.A + (int64_t)i * T * a.d, T, a.d, trow0, srow0, ka, n, g);
  gram_tile_f32((const float*)a.G + (int64_t)i * T * a.p, T, a.p, trow0, srow0, kg, n, g);
  double ss = 0.0;
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) ss += (double)ka[m][q][r] * (double)kg[m][q][r];
  ss = wave_sum(ss);
  if (lane == 0) red[wv] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double wgt = bs < bt ? 2.0 : 1.0;
    a.partials[(int64_t)i * a.slots + j] = make_double2(wgt * ((red[0] + red[1]) + (red[2] + red[3])), 0.0);
  }
}

// Work decomposition shared with the host: explicit tiles are 256 x 256
// (bf16) or 64 x 64 (fp32) of W_i; Gram work groups take 256 (t) x 128 (s)
// pairs, nT (nT + 1) of them for nT = ceil(T / 256) (bf16), or 128 x 128
// pairs with t >= s (fp32).
void exact_tiles(bool bf16, bool gram, int64_t T, int64_t d, int64_t p, int32_t& tu, int32_t& tv, int32_t& slots) {
  if (gram && bf16) {
    tu = (int32_t)((T + kGT - 1) / kGT);
    tv = tu;
    slots = tu * (tu + 1);
  } else if (gram) {
    tu = (int32_t)((T + 127) / 128);
    tv = tu;
    slots = tu * (tu + 1) / 2;
  } else {
    const int64_t e = bf16 ? kXTile : 64;
    tu = (int32_t)((d + e - 1) / e);
    tv = (int32_t)((p + e - 1) / e);
    slots = tu * tv;
  }
}

hipError_t launch_exact(const void* A, const void* G, bool bf16, bool gram, int32_t B, int32_t T, int32_t d,
                        int32_t p, double2* partials, hipStream_t s) {
  ExactArgs a;
  a.A = A;
  a.G = G;
  a.B = B;
  a.T = T;
  a.d = d;
  a.p = p;
  exact_tiles(bf16, gram, T, d, p, a.tu, a.tv, a.slots);
  a.n_items = B * a.slots;
  a.partials = partials;
  if (gram) {
    if (bf16) hipLaunchKernelGGL(k_exact_gram_bf16, dim3(a.n_items), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_exact_gram_f32, dim3(a.n_items), dim3(256), 0, s, a);
  } else {
    if (bf16) hipLaunchKernelGGL(k_exact_explicit_bf16, dim3(a.n_items), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(k_exact_explicit_f32, dim3(a.n_items), dim3(64), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace dpn
