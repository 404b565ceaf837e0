// Kernels of the projected-contraction path on gfx950: the prepare pass
// (layer records, work-item lists, MFMA-packed W where W is not read in
// place), the skinny row projection
// V = X1 W (stage 1), the T contraction Y = X2^T V with a fused squared
// Frobenius reduction (stage 2), the split-T reduction, the per-sample
// finisher and the clip factors.
//
// Method ('Efficient DP-SGD for LLMs with Randomized Clipping', papernotes.org
// note, 关键设计 › Hutchinson 随机投影估范数): the squared per-sample gradient
// norm of a linear layer is estimated by ||A_i^T (G_i P)||_F^2 with G P formed
// first; 方法详解 › 整体框架: estimates are summed over the layers of a sample
// and turned into the clip factor min(C / sqrt(n_i), 1).
//
// Both contractions are k wide (2k flops per element read, k = 32 on the
// pages), far below the bf16 MFMA ridge, so the kernels are bound by streaming
// X1 and X2 from HBM once each. The fp32 intermediate V is handed to the bf16
// MFMA of stage 2 as a hi + lo pair of bf16 values (error <= 2^-17 relative).
#include "device_common.h"
#include "internal.h"

namespace dpn {

// ---------------------------------------------------------------------------
// Prepare: one thread per unit. Units of a layer, in order: packed-W units,
// stage-1 item entries, stage-2 item entries, and one unit for the record.
// Each layer's units start on a work-group boundary, so a work group finds
// its layer with a uniform search (scalar loads from the argument table).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float load_src(const void* p, int64_t idx, int type) {
  if (type == SRC_BF16) return bf16_bits_to_f32(((const uint16_t*)p)[idx]);
  return ((const float*)p)[idx];
}

// Element (v, c) of sample smp's W source. Sign sources hold one bit per
// entry, 32 columns to a word (bit c % 32 of word c / 32 of row v): 0 is +1,
// 1 is -1; the 1/sqrt(k) scale is applied to the finished sums instead.
// The identity source projects a narrow side onto itself (exact norms).
__device__ __forceinline__ float w_value(const PrepLayer& P, int smp, int v, int c) {
  if (P.wsrc_type == SRC_IDENTITY) return v == c ? 1.f : 0.f;
  const int64_t row = smp * P.wsrc_stride_b + (int64_t)v * P.ld;
  if (P.wsrc_type == SRC_SIGN) {
    const uint32_t word = ((const uint32_t*)P.wsrc)[row + (c >> 5)];
    return ((word >> (c & 31)) & 1u) ? -1.f : 1.f;
  }
  return load_src(P.wsrc, row + c, P.wsrc_type);
}

// Rows v0 .. v0 + 7 of column c of sample smp's W source, zero past `rows`
// rows or P.ncols columns. The indices are clamped into range and every load
// is issued before any is used (a load under a per-lane condition gets a wait
// of its own), with the source type decided once for all eight.
__device__ __forceinline__ void w_values8(const PrepLayer& P, int smp, int v0, int c, int rows, float x[8]) {
  const int cc = min(c, P.ncols - 1);
  const int64_t base = smp * P.wsrc_stride_b;
  int vr[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) vr[s] = min(v0 + s, rows - 1);
  switch (P.wsrc_type) {
    case SRC_IDENTITY:
#pragma unroll
      for (int s = 0; s < 8; ++s) x[s] = v0 + s == c ? 1.f : 0.f;
      break;
    case SRC_SIGN: {
      uint32_t wd[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) wd[s] = ((const uint32_t*)P.wsrc)[base + (int64_t)vr[s] * P.ld + (cc >> 5)];
#pragma unroll
      for (int s = 0; s < 8; ++s) x[s] = ((wd[s] >> (cc & 31)) & 1u) ? -1.f : 1.f;
      break;
    }
    case SRC_BF16: {
      uint16_t hv[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) hv[s] = ((const uint16_t*)P.wsrc)[base + (int64_t)vr[s] * P.ld + cc];
#pragma unroll
      for (int s = 0; s < 8; ++s) x[s] = bf16_bits_to_f32(hv[s]);
      break;
    }
    default:
#pragma unroll
      for (int s = 0; s < 8; ++s) x[s] = ((const float*)P.wsrc)[base + (int64_t)vr[s] * P.ld + cc];
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) x[s] = (v0 + s < rows && c < P.ncols) ? x[s] : 0.f;
}

__global__ void __launch_bounds__(256) k_prepare(PrepArgs a) {
  const int first = blockIdx.x * 256;
  // the last layer whose first unit is <= first (binary search over the
  // kernel-argument table: a few dependent scalar loads, not one per layer)
  int l = 0, hi = a.nlayers - 1;
  while (l < hi) {
    const int mid = (l + hi + 1) >> 1;
    if (a.L[mid].unit_begin <= first) l = mid;
    else hi = mid - 1;
  }
  const PrepLayer& P = a.L[l];
  int r = first + threadIdx.x - P.unit_begin;
  if (r >= P.n_pack + P.n1 + P.n2 + 1) return;  // padding up to the next layer's first work group
  const int NCB = a.NCB, NC = 16 * NCB;

  if (r < P.n_pack) {
    const int rows = P.rec.w1;
    if (!a.f32_target) {
      // bf16 fragments for the B operand of stage 1: unit (smp, ks, jb, h,
      // lane) holds rows v = 32 ks + 8 (lane / 16) + s, s = 0..7, of column
      // 16 jb + lane % 16; h = 0 is the bf16 value (hi), h = 1 the residual.
      const int HL = a.HL;
      const int nks = (rows + 63) / 64 * 2;  // even number of K steps: stage 1 loads two per stage
      const int per_s = nks * NCB * HL * 64;
      const int smp = r / per_s;
      int q = r - smp * per_s;
      const int lane = q & 63;
      q >>= 6;
      const int h = q % HL;
      q /= HL;
      const int jb = q % NCB;
      const int ks = q / NCB;
      const int c = 16 * jb + (lane & 15);
      const int v0 = 32 * ks + 8 * (lane >> 4);
      float x[8];
      w_values8(P, smp, v0, c, rows, x);
      uint32_t b[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        uint32_t hi, lo;
        split_bf16(x[s], hi, lo);
        b[s] = h ? lo : hi;
      }
      uint4* dst = (uint4*)P.rec.W + smp * P.rec.w_stride_b;
      dst[(int64_t)((ks * NCB + jb) * HL + h) * 64 + lane] = pack8(b);
    } else {
      // fp32 rows [rows16][NC], zero padded.
      const int rows16 = (rows + 15) / 16 * 16;
      const int per_s = rows16 * NC;
      const int smp = r / per_s;
      const int q = r - smp * per_s;
      const int v = q / NC, c = q - v * NC;
      float x = 0.f;
      if (v < rows && c < P.ncols) x = w_value(P, smp, v, c);
      ((float*)P.rec.W)[smp * P.rec.w_stride_b + q] = x;
    }
    return;
  }
  r -= P.n_pack;
  if (r < P.n1) {
    const int i = r / a.rbs, rb = r - i * a.rbs;
    a.items1[P.k1_begin + r] = make_int4(P.layer, i, rb, 0);
    return;
  }
  r -= P.n1;
  if (r < P.n2) {
    // T split innermost: the split-T reduction finds item (i, ub) at a
    // multiple of nsplit.
    const int ts = r % a.nsplit, q = r / a.nsplit;
    const int ub = q % P.ubs, i = q / P.ubs;
    a.items2[P.k2_begin + r] = make_int4(P.layer, i, ub, ts);
    return;
  }
  a.recs[P.layer] = P.rec;
}

// ---------------------------------------------------------------------------
// Stage 1, bf16: V = X1 W for 128 rows of one sample.
//
// X1 and the packed W are streamed into LDS 64 columns (one 128-byte line per
// row) and two K steps at a time with direct global-to-LDS loads: every wave
// instruction moves 1 KB of whole lines without using registers (X1 with
// non-temporal loads, so the stream does not evict W from L2), and three
// stages are in flight while one is multiplied. The loads are issued from
// inline assembly so that the only waits on them are the ones placed here:
// before each barrier a wave waits for its own loads of the stage about to be
// read, and the later stages stay in flight.
// Wave w owns rows 32w..32w+31 (two 16-row MFMA tiles); the 16-byte units of
// an X1 row are XOR-swizzled by the row index so the A-operand reads spread
// over the LDS banks. After the last stage lane l of wave w holds rows
// slot_row(l / 16, s) of chunk w, so the hi/lo bf16 B-operand fragments of
// stage 2 are written straight from the accumulators.
// Each work group starts its pass over the columns at its own stage and wraps
// around: when every group reads the same column offset of rows whose length
// is a large power of two, the concurrent reads fall on few HBM channels.
// Groups are dealt to the XCDs round robin, so the eight neighbours of a
// group (one per XCD) share a start and the groups that share an XCD get
// starts 41 stages apart (modulo the stage count).
// V layout: [B][Tpad/32][NCB][2][64] uint4.
// ---------------------------------------------------------------------------
// Work items and the layer record: from the tables, or in implicit mode
// (one layer; StageArgs::rec0) derived from the item index.
template <bool IMPL>
__device__ __forceinline__ int4 stage1_item(const StageArgs& a, uint32_t b) {
  if (IMPL) {
    const int i = (int)b / a.rbs;
    return make_int4(0, i, (int)b - i * a.rbs, 0);
  }
  return a.items[b];
}
template <bool IMPL>
__device__ __forceinline__ int4 stage2_item(const StageArgs& a, int b) {
  if (IMPL) {
    const int ts = b % a.nsplit, q = b / a.nsplit;
    return make_int4(0, q / a.ubs, q % a.ubs, ts);
  }
  return a.items[b];
}
template <bool IMPL>
__device__ __forceinline__ const LayerRec* layer_rec(const StageArgs& a, int layer) {
  return IMPL ? &a.rec0 : a.recs + layer;
}

__device__ __attribute__((aligned(16))) uint4 g_zero16[1];   // 16 zero bytes (static storage)

constexpr int kK1Cols = 64;                          // columns of X1 per stage (one 128-byte line)
constexpr int kK1XDma = 32 * kK1Cols * 2 / 1024;     // 1 KB X1 instructions per wave per stage (its 32 rows)
constexpr int kK1Bufs = 4;                           // LDS ring: three stages in flight, one in use

// NW waves. KS = 1: wave w owns rows 32 w .. 32 w + 31 of a 32 NW-row item
// (128 rows normally, 64 when 128-row items would leave CUs idle). KS > 1
// (K split): the item has 32 NW / KS rows, wave w takes 32-row group w / KS
// of it, and stage st holds KS consecutive 64-column chunks, one per K slot
// (chunk KS st + w % KS, counted from the group's first chunk), each with
// its 64 rows of W; at the end the partial sums of K slots 1 .. KS - 1 are
// added to slot 0's through LDS in slot order, so the result does not depend
// on timing. KS = NW: one 32-row item for all waves (calls with few items);
// KS = 2 with four waves: 64-row items with two waves' loads per row group.
// RAW (HL = 1): W is the caller's bf16 [w1][NC] matrix. A chunk's 64 rows
// of it are one contiguous run, loaded as they are (rows past w1 from a zero
// row) and kept row-major in LDS; each B operand is two transposing reads
// (rows 32 kk + 8 g .. + 3 and + 4 .. + 7 of column 16 jb + n), so the call
// needs no packed copy of W. IMPL: implicit mode (items and record not in
// memory; always RAW).
template <int NCB, int HL, int NW, int KS>
constexpr int rowproj_lds_bytes() {   // the stage ring of one work group
  return kK1Bufs * (NW * 32 * kK1Cols * 2 + KS * 2 * NCB * HL * 1024);
}

// One stage-1 item it = (layer, sample, row block) on the work group's LDS
// ring lds (rowproj_lds_bytes, 1 KB aligned); key picks the first column
// chunk (work groups start at different chunks). Every wave of the group
// calls it; waves other than a K split's slot 0 return before the store.
template <int NCB, int HL, int NW, bool RAW, bool IMPL, int KS>
__device__ __forceinline__ void rowproj_bf16_item(const StageArgs& a, const int4 it, uint32_t key, unsigned char* lds) {
  static_assert(!RAW || HL == 1, "W read in place is bf16");
  static_assert(!IMPL || RAW, "implicit mode reads W in place");
  static_assert(NW % KS == 0, "the K split spreads each 32-row group over KS waves");
  constexpr int NC = 16 * NCB;
  constexpr int kRows = 32 * NW / KS;                    // rows per item
  constexpr int kK1XBytes = NW * 32 * kK1Cols * 2;       // X1 bytes per stage (16 KB for 4 waves)
  constexpr int kWBlocks = 2 * NCB * HL;                 // 1 KB W fragment blocks per chunk
  constexpr int kStage = kK1XBytes + KS * kWBlocks * 1024;
  constexpr int kPerWave = kK1XDma + KS * kWBlocks / NW; // loads every wave issues per stage (at least)
  static_assert(kK1Bufs * kStage == rowproj_lds_bytes<NCB, HL, NW, KS>(), "ring size");
  static_assert(kK1Bufs * kStage <= 160 * 1024, "the stage ring must fit the LDS of one work group");
  const LayerRec* L = layer_rec<IMPL>(a, it.x);
  const int i = it.y, rb = it.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int rg = KS == 1 ? wv : wv / KS;                 // this wave's 32-row group within the item
  const int kq = KS == 1 ? 0 : wv % KS;                  // this wave's chunk within a stage
  const int w = L->w1, T = a.T;
  const int r0 = rb * kRows;
  const uint16_t* X = (const uint16_t*)L->X1 + (int64_t)i * T * w;
  const uint4* Wp = (const uint4*)L->W + i * L->w_stride_b + lane;  // packed to an even number of K steps
  const uint16_t* Wr = (const uint16_t*)L->W;                       // RAW: [w][NC] as the caller holds it
  const int nch = (w + kK1Cols - 1) / kK1Cols;                      // 64-column chunks
  const int nst = (nch + KS - 1) / KS;
  const int rot = (int)((key >> 3) * 41u % (unsigned)nch);          // first chunk of this group
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;

  // X1 source of this lane: instruction j of wave wv fills LDS rows
  // 8 (4 wv + j) + lane / 8 at unit position lane % 8, which holds global
  // unit (lane % 8) ^ (row % 8) of row 32 rg + 8 j + lane / 8 of the item.
  // Rows past T and columns past w read the last valid row / unit instead:
  // those values only ever meet zero rows of A or zero rows of W, so they
  // contribute nothing.
  const int urow0 = 32 * wv + (lane >> 3);
  const int gunit = (lane & 7) ^ (urow0 & 7);  // row % 8 is the same for all j (rows step by 8)
  const int grow0 = r0 + 32 * rg + (lane >> 3);
  auto chunk_of = [&](int st, int q) {         // chunk read by slot q of stage st (nch or more: none)
    const int c = KS * st + q;
    if (c >= nch) return nch;
    return c + rot < nch ? c + rot : c + rot - nch;
  };
  auto dma = [&](int st) {
    if (st >= nst) return;
    const uint32_t buf = lds_base + (uint32_t)((st % kK1Bufs) * kStage);
    const int cx = chunk_of(st, kq);
    int col = min(cx, nch - 1) * kK1Cols + gunit * 8;
    col = col < w ? col : w - 8;
#pragma unroll
    for (int j = 0; j < kK1XDma; ++j) {
      int row = grow0 + 8 * j;
      row = row < T ? row : T - 1;
      dma16_stream(X + (int64_t)row * w + col, buf + (uint32_t)((wv * kK1XDma + j) * 1024));
    }
#pragma unroll
    for (int m0 = 0; m0 < (KS * kWBlocks + NW - 1) / NW; ++m0) {
      const int m = NW * m0 + wv;                // W block m: chunk slot m / kWBlocks, block m % kWBlocks
      if (m < KS * kWBlocks) {
        const int q = m / kWBlocks, mb = m % kWBlocks;
        const int cw = chunk_of(st, q);
        if (RAW) {  // block mb: rows 64 cw + (512 / NC) mb .., 2 NCB lanes of 16 bytes a row
          const int row = 64 * cw + mb * (512 / NC) + lane / (2 * NCB);
          const void* src =
              row < w ? (const void*)(Wr + (int64_t)row * NC + 8 * (lane % (2 * NCB))) : (const void*)g_zero16;
          dma16(src, buf + (uint32_t)(kK1XBytes + m * 1024));
        } else {
          dma16(Wp + ((int64_t)min(cw, nch - 1) * kWBlocks + mb) * 64, buf + (uint32_t)(kK1XBytes + m * 1024));
        }
      }
    }
  };

  f32x4_t acc[2][NCB];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb) acc[mt][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  dma(0);
  dma(1);
  dma(2);
  for (int st = 0; st < nst; ++st) {
    // this wave's loads of stage st have landed once at most the later
    // stages' loads are outstanding; the barrier then publishes every wave's
    // loads of stage st and frees the buffer of stage st - 1
    if (st + 2 < nst) DPN_WAIT_VMCNT(2 * kPerWave);
    else if (st + 1 < nst) DPN_WAIT_VMCNT(kPerWave);
    else DPN_WAIT_VMCNT(0);
    block_barrier();
    dma(st + 3);
    if (KS > 1 && KS * st + kq >= nch) continue;  // no chunk for this wave in the last stage (wave-uniform)
    const unsigned char* buf = lds + (st % kK1Bufs) * kStage;
    const uint4* wf = (const uint4*)(buf + kK1XBytes + kq * kWBlocks * 1024) + lane;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      uint4 f[NCB][HL];
      if (RAW) {
        const unsigned char* wr =
            buf + kK1XBytes + kq * kWBlocks * 1024 + (32 * kk + 8 * g + (n >> 2)) * (NC * 2) + (n & 3) * 8;
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb) {
          const uint2 lo = lds_read_tr16(wr + 32 * jb);
          const uint2 hi = lds_read_tr16(wr + 4 * (NC * 2) + 32 * jb);
          f[jb][0] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
      } else {
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
          for (int h = 0; h < HL; ++h) f[jb][h] = wf[((kk * NCB + jb) * HL + h) * 64];
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int row = 32 * wv + 16 * mt + n;
        const uint4 x = *(const uint4*)(buf + row * 128 + (((4 * kk + g) ^ (row & 7)) * 16));
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
          for (int h = 0; h < HL; ++h) acc[mt][jb] = mfma_bf16(x, f[jb][h], acc[mt][jb]);
      }
    }
  }

  if (KS > 1) {
    // partial sums of K slots 1 .. KS - 1 through LDS (every wave is past its
    // last LDS read once all have reached this barrier), added by the row
    // group's slot-0 wave in slot order
    block_barrier();
    float* red = (float*)lds + rg * (KS - 1) * (2 * NCB * 256);
    if (kq > 0) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
          for (int r = 0; r < 4; ++r) red[(((kq - 1) * 2 + mt) * NCB + jb) * 256 + r * 64 + lane] = acc[mt][jb][r];
    }
    __syncthreads();
    if (kq > 0) return;
#pragma unroll
    for (int q = 1; q < KS; ++q)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[mt][jb][r] += red[(((q - 1) * 2 + mt) * NCB + jb) * 256 + r * 64 + lane];
  }

  if (r0 + 32 * rg >= T) return;  // chunk past the sequence: stage 2 never reads it
  uint4* out = (uint4*)L->V + ((int64_t)i * (a.Tpad / 32) + r0 / 32 + rg) * L->vstride + lane;
#pragma unroll
  for (int jb = 0; jb < NCB; ++jb) {
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) split_bf16(acc[s >> 2][jb][s & 3], hi[s], lo[s]);
    stg16(out + (jb * 2 + 0) * 64, pack8(hi));
    stg16(out + (jb * 2 + 1) * 64, pack8(lo));
  }
}

template <int NCB, int HL, int NW, bool RAW, bool IMPL, int KS>
__global__ void __launch_bounds__(64 * NW) k_rowproj_bf16(StageArgs a) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[rowproj_lds_bytes<NCB, HL, NW, KS>()];
  rowproj_bf16_item<NCB, HL, NW, RAW, IMPL, KS>(a, stage1_item<IMPL>(a, blockIdx.x), blockIdx.x, lds);
}

// ---------------------------------------------------------------------------
// Stage 1, fp32: the same decomposition with v_mfma_f32_16x16x4f32. A lane
// loads 4 consecutive columns of its row and feeds them to four MFMAs (K slot
// l / 16 stands for column 16 ks + 4 (l / 16) + q of MFMA q).
// V layout: [B][Tpad][NC] float.
// ---------------------------------------------------------------------------
template <int NCB>
__global__ void __launch_bounds__(256) k_rowproj_f32(StageArgs a) {
  constexpr int NC = 16 * NCB;
  const int4 it = a.items[blockIdx.x];
  const LayerRec* L = a.recs + it.x;
  const int i = it.y, rb = it.z;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int w = L->w1, T = a.T;
  const int r0 = rb * kRowsK1 + 32 * wv;
  if (r0 >= T) return;
  const float* X = (const float*)L->X1 + (int64_t)i * T * w;
  const float* Wf = (const float*)L->W + i * L->w_stride_b;
  const int nks = (w + 15) >> 4;
  const bool ok0 = r0 + n < T, ok1 = r0 + 16 + n < T;
  const float* x0 = X + (int64_t)(r0 + n) * w + 4 * g;
  const float* x1 = X + (int64_t)(r0 + 16 + n) * w + 4 * g;

  f32x4_t acc[2][NCB];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb) acc[mt][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int ks = 0; ks < nks; ++ks) {
    const int v = 16 * ks + 4 * g;
    const bool vok = v < w;
    const float4 g0 = (vok && ok0) ? *(const float4*)(x0 + 16 * ks) : z;
    const float4 g1 = (vok && ok1) ? *(const float4*)(x1 + 16 * ks) : z;
    const float gv0[4] = {g0.x, g0.y, g0.z, g0.w};
    const float gv1[4] = {g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int jb = 0; jb < NCB; ++jb) {
        const float wq = Wf[(int64_t)(v + q) * NC + 16 * jb + n];
        acc[0][jb] = mfma_f32(gv0[q], wq, acc[0][jb]);
        acc[1][jb] = mfma_f32(gv1[q], wq, acc[1][jb]);
      }
  }

  const int vs = L->vstride;
  float* out = (float*)L->V + ((int64_t)i * a.Tpad + r0) * vs;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(16 * mt + 4 * g + r) * vs + 16 * jb + n] = acc[mt][jb][r];
}

// ---------------------------------------------------------------------------
// Stage-2 epilogues.
// direct: squared Frobenius sums of the tile, columns < split and the rest,
//         reduced over the work group in a fixed order into one partial slot.
// else:   the tile is stored to Ypart[ts][i][u][NC].
// Lane l's accumulator (e, jb, r) is Y[u0 + ustride (4 (l/16) + r) + e][16 jb + l%16].
// ---------------------------------------------------------------------------
template <int NCB, int NE, bool DIRECT, int NW = 4>
__device__ __forceinline__ void tcontract_epilogue(const StageArgs& a, const LayerRec* L, f32x4_t (&acc)[NE][NCB],
                                                   int i, int ub, int ts, int wave_u0, int ustride, int lane,
                                                   int wv) {
  static_assert(NW == 2 || NW == 4, "work groups of two or four waves");
  constexpr int NC = 16 * NCB;
  const int n = lane & 15, g = lane >> 4;
  if (DIRECT) {
    __shared__ double red[NW][2];
    const int split = L->split;
    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const double y = (double)acc[e][jb][r];
          if (16 * jb + n < split) s0 += y * y;
          else s1 += y * y;
        }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    if (lane == 0) {
      red[wv][0] = s0;
      red[wv][1] = s1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double r0 = red[0][0] + red[1][0], r1 = red[0][1] + red[1][1];
      if (NW == 4) {
        r0 += red[2][0] + red[3][0];
        r1 += red[2][1] + red[3][1];
      }
      a.partials[(int64_t)i * a.slots_per_sample + L->slot_base + ub] = make_double2(r0, r1);
    }
  } else {
    const int w = L->w2;
    float* Y = L->Ypart + ((int64_t)ts * a.B + i) * w * NC;
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = wave_u0 + ustride * (4 * g + r) + e;
        if (u < w) {
#pragma unroll
          for (int jb = 0; jb < NCB; ++jb) stg_f32(Y + (int64_t)u * NC + 16 * jb + n, acc[e][jb][r]);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Stage 2, bf16: Y = X2^T V over the chunks of one T split, for 128 NW
// columns of X2 (NW waves x 128: 512 columns normally, 256 on two waves for
// calls that split T, so that they need half the splits).
//
// Each 32-row chunk of X2 (32 rows x 1 KB) and its V fragments are streamed
// into LDS with direct global-to-LDS loads, as in stage 1 (wave w issues
// eight 1 KB loads of the chunk's rows, one row of 512 columns or two of 256
// each, and a share of the 1 KB V blocks), with two or three chunks in flight
// while one is multiplied. A lane then reads 8 rows (slot_row) of its
// 8 consecutive columns from LDS, transposes the 8 x 8 block in registers so
// the contraction index runs along the MFMA K slots, and multiplies it
// against the hi and lo fragments of V. Rows past T and columns past w load
// the last valid row / column and are zeroed after the LDS read.
//
// KT = 2 (two-wave column groups only, T split into partial tiles): two such
// pairs of waves take the first and the second half of the split's chunks,
// each stage holding one chunk of each half, and the second pair's
// accumulators are added to the first's through LDS at the end. A call then
// needs half the splits (and half the partial tiles) for as many work groups
// of four waves. When the split has an odd number of chunks, the second
// pair's last stage reloads the split's last chunk and zeroes it.
// ---------------------------------------------------------------------------
constexpr int kK2Rows = 32;                              // rows of X2 per stage (one MFMA K step)


template <int NCB, bool DIRECT, bool IMPL, int NW = 4, int KT = 1>
__global__ void __launch_bounds__(64 * NW * KT) k_tcontract_bf16(StageArgs a) {
  static_assert(NW == 2 || NW == 4, "work groups of two or four waves");
  static_assert(KT == 1 || (KT == 2 && NW == 2 && !DIRECT), "T halves only for two-wave groups that store tiles");
  constexpr int kCols = 128 * NW;                        // columns of X2 per item
  constexpr int kRowBytes = 2 * kCols;                   // one row of the item in LDS
  constexpr int kRowsPerDma = 1024 / kRowBytes;          // rows per 1 KB load (1 or 2)
  constexpr int kLanesPerRow = kRowBytes / 16;
  constexpr int kK2XBytes = kK2Rows * kRowBytes;         // X2 bytes per stage (32 or 16 KB)
  constexpr int kVBlocks = 2 * NCB;                      // 1 KB V fragment blocks per chunk
  constexpr int kHalf = kK2XBytes + kVBlocks * 1024;     // one chunk and its V blocks
  constexpr int kStage = KT * kHalf;
  constexpr int kBufs = NW * KT == 4 ? (NW == 4 ? (NCB <= 2 ? 4 : 3) : (4 * kStage <= 160 * 1024 ? 4 : 3))
                                     : (4 * kStage <= 80 * 1024 ? 4 : 3);  // LDS ring
  constexpr int kXDma = kK2XBytes / 1024 / NW;           // 1 KB X2 loads per wave per stage (8)
  constexpr int kP = kXDma + kVBlocks / NW;              // loads every wave issues per stage (at least)
  static_assert(KT == 1 || kBufs * kStage >= NW * 8 * NCB * 4 * 64 * 4, "the ring holds the accumulator exchange");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kBufs * kStage];
  const int4 it = stage2_item<IMPL>(a, xcd_item(blockIdx.x, (uint32_t)a.n_items));
  const LayerRec* L = layer_rec<IMPL>(a, it.x);
  const int i = it.y, ub = it.z, ts = it.w;
  const int w = L->w2, T = a.T;
  const int lane = threadIdx.x & 63;
  const int wv = KT == 1 ? (int)(threadIdx.x >> 6) : (int)(threadIdx.x >> 6) % NW;   // column wave
  const int wt = KT == 1 ? 0 : (int)(threadIdx.x >> 6) / NW;                         // T half
  const int n = lane & 15, g = lane >> 4;
  const int wave_u0 = ub * kCols + wv * 128;
  const bool uok = wave_u0 + 8 * n < w;
  // this lane's 16 bytes of each loaded row, and its row within a 1 KB load
  const int dcol = min(ub * kCols + 8 * (lane % kLanesPerRow), w - 8);
  const int drow = lane / kLanesPerRow;
  const uint16_t* X = (const uint16_t*)L->X2 + (int64_t)i * T * w + dcol;
  const uint4* V = (const uint4*)L->V + (int64_t)i * (a.Tpad / 32) * (NCB * 2 * 64) + lane;
  const int nch = (T + 31) >> 5;
  const int c0 = (int)((int64_t)ts * nch / a.nsplit), c1 = (int)((int64_t)(ts + 1) * nch / a.nsplit);
  const int ncs = (c1 - c0 + KT - 1) / KT;               // stages (chunks of the first half)
  // this pair's first chunk, and its number of chunks
  const int cw = c0 + wt * ncs, nw = KT == 1 ? ncs : (wt == 0 ? ncs : c1 - c0 - ncs);
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;

  auto dma = [&](int st) {
    if (st >= ncs) return;
    const uint32_t buf = lds_base + (uint32_t)((st % kBufs) * kStage + wt * kHalf);
    const int c = st < nw ? cw + st : c1 - 1;   // past this pair's chunks: reloaded, zeroed after the read
#pragma unroll
    for (int j = 0; j < kXDma; ++j) {
      int t = kK2Rows * c + (kXDma * wv + j) * kRowsPerDma + drow;
      t = t < T ? t : T - 1;
      dma16_stream(X + (int64_t)t * w, buf + (uint32_t)((kXDma * wv + j) * 1024));
    }
#pragma unroll
    for (int m0 = 0; m0 < (kVBlocks + NW - 1) / NW; ++m0) {
      const int m = NW * m0 + wv;
      if (m < kVBlocks) dma16(V + ((int64_t)c * kVBlocks + m) * 64, buf + (uint32_t)(kK2XBytes + m * 1024));
    }
  };

  f32x4_t acc[8][NCB];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb) acc[e][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int st = 0; st < kBufs - 1; ++st) dma(st);
  for (int st = 0; st < ncs; ++st) {
    // this wave's loads of stage st have landed once at most its loads of
    // the later stages are outstanding; the barrier publishes every wave's
    // loads and frees the buffer of stage st - 1
    wait_after<kP>(min(kBufs - 2, ncs - 1 - st));
    block_barrier();
    dma(st + kBufs - 1);
    const unsigned char* buf = lds + (st % kBufs) * kStage + wt * kHalf;
    const int t0 = kK2Rows * (cw + st);
    const bool cok = KT == 1 || st < nw;
    uint4 raw[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int r = slot_row(g, s);
      const uint4 x = *(const uint4*)(buf + r * kRowBytes + wv * 256 + n * 16);
      raw[s] = (uok && cok && t0 + r < T) ? x : z;
    }
    uint4 bv[NCB][2];
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 v = *(const uint4*)(buf + kK2XBytes + (jb * 2 + h) * 1024 + lane * 16);
        bv[jb][h] = cok ? v : z;
      }
    uint4 op[8];
    transpose8x8_bf16(raw, op);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb) acc[e][jb] = mfma_bf16(op[e], bv[jb][h], acc[e][jb]);
  }
  if constexpr (KT == 2) {
    // the second pair's sums are added to the first pair's (in that order)
    float* xch = (float*)lds + (int64_t)wv * (8 * NCB * 4 * 64) + lane;
    __syncthreads();   // every wave is done with the ring
    if (wt == 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
          for (int r = 0; r < 4; ++r) xch[((e * NCB + jb) * 4 + r) * 64] = acc[e][jb][r];
    }
    __syncthreads();
    if (wt == 1) return;
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[e][jb][r] += xch[((e * NCB + jb) * 4 + r) * 64];
  }
  tcontract_epilogue<NCB, 8, DIRECT, NW>(a, L, acc, i, ub, ts, wave_u0, 8, lane, wv);
}

// ---------------------------------------------------------------------------
// Stage 2, fp32: 4 rows per MFMA step; a lane's float4 of 4 consecutive
// columns feeds four MFMAs (one per column offset e), so no transpose is
// needed. 256 columns per work group (4 waves x 64).
// ---------------------------------------------------------------------------
template <int NCB, bool DIRECT>
__global__ void __launch_bounds__(256) k_tcontract_f32(StageArgs a) {
  constexpr int NC = 16 * NCB;
  const int4 it = a.items[xcd_item(blockIdx.x, (uint32_t)a.n_items)];
  const LayerRec* L = a.recs + it.x;
  const int i = it.y, ub = it.z, ts = it.w;
  const int w = L->w2, T = a.T;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int wave_u0 = ub * kColsK2F32 + wv * 64;
  const bool uok = wave_u0 + 4 * n < w;
  const float* X = (const float*)L->X2 + (int64_t)i * T * w + wave_u0 + 4 * n;
  const float* V = (const float*)L->V + (int64_t)i * a.Tpad * NC + n;
  const int nch = (T + 31) >> 5;
  const int c0 = (int)((int64_t)ts * nch / a.nsplit), c1 = (int)((int64_t)(ts + 1) * nch / a.nsplit);
  const int t_end = min(T, 32 * c1);

  f32x4_t acc[4][NCB];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb) acc[e][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (wave_u0 < w) {
    for (int t0 = 32 * c0; t0 < t_end; t0 += 4) {
      const int t = t0 + g;
      const float4 x = (uok && t < T) ? ldg_f32x4(X + (int64_t)t * w) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int jb = 0; jb < NCB; ++jb) {
        const float b = (t < T) ? ldg_f32(V + (int64_t)t * NC + 16 * jb) : 0.f;
        acc[0][jb] = mfma_f32(x.x, b, acc[0][jb]);
        acc[1][jb] = mfma_f32(x.y, b, acc[1][jb]);
        acc[2][jb] = mfma_f32(x.z, b, acc[2][jb]);
        acc[3][jb] = mfma_f32(x.w, b, acc[3][jb]);
      }
    }
  }
  tcontract_epilogue<NCB, 4, DIRECT>(a, L, acc, i, ub, ts, wave_u0, 4, lane, wv);
}

// ---------------------------------------------------------------------------
// Split-T reduction: one wave per kYsumChunk elements of the Y tile of a
// (layer, sample, column block). Each lane sums 4 consecutive elements over
// the nsplit partial tiles in split order (fp64; eight splits' loads are in
// flight at a time), then either squares and reduces into the wave's own
// partial slot (MODE_SQ) or stores Y (MODE_STORE).
// ---------------------------------------------------------------------------
template <int MODE, bool IMPL>
__global__ void __launch_bounds__(64) k_ysum(StageArgs a, int NC, int cols_per_block, int ychunks) {
  const int blk = blockIdx.x / ychunks, chunk = blockIdx.x - blk * ychunks;
  const int4 it = stage2_item<IMPL>(a, blk * a.nsplit);
  const LayerRec* L = layer_rec<IMPL>(a, it.x);
  const int i = it.y, ub = it.z;
  const int w = L->w2;
  const int u0 = ub * cols_per_block;
  const int nel = min(cols_per_block, w - u0) * NC;
  const int64_t tile = (int64_t)a.B * w * NC;
  const float* Yp = L->Ypart + ((int64_t)i * w + u0) * NC;
  const int e = chunk * kYsumChunk + 4 * (int)threadIdx.x;
  const int split = L->split;
  double s0 = 0.0, s1 = 0.0;
  if (e < nel) {  // nel is a multiple of 16, so all four elements are in the tile
    double y[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 8
    for (int ts = 0; ts < a.nsplit; ++ts) {
      const float4 v = ldg_f32x4(Yp + ts * tile + e);
      y[0] += (double)v.x;
      y[1] += (double)v.y;
      y[2] += (double)v.z;
      y[3] += (double)v.w;
    }
    if (MODE == MODE_SQ) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if ((e + q) % NC < split) s0 += y[q] * y[q];
        else s1 += y[q] * y[q];
      }
    } else {
      float* dst = L->Yout + ((int64_t)i * w + u0) * NC + e;
#pragma unroll
      for (int q = 0; q < 4; ++q) stg_f32(dst + q, (float)y[q]);
    }
  }
  if (MODE == MODE_SQ) {
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    if (threadIdx.x == 0)
      a.partials[(int64_t)i * a.slots_per_sample + L->slot_base + ub * ychunks + chunk] = make_double2(s0, s1);
  }
}

// ---------------------------------------------------------------------------
// Finisher: per sample, sum the partial slots in a fixed order (strided per
// thread, then a fixed tree), add to n when accumulating, and optionally emit
// the two column-group sums (head / tail) and the clip factor.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float clip_value(float n, float C) {
  if (n != n) return n;
  if (!(n > 0.f)) return 1.f;
  const double c = (double)C / sqrt((double)n);
  return (float)(c < 1.0 ? c : 1.0);
}

__global__ void __launch_bounds__(256) k_finish(const double2* __restrict__ partials, int32_t slots, float* n,
                                                int accumulate, float* head, float* tail, float* c, float C,
                                                int with_clip, double scale) {
  __shared__ double r0[256], r1[256];
  const int i = blockIdx.x, t = threadIdx.x;
  const double2* P = partials + (int64_t)i * slots;
  double s0 = 0.0, s1 = 0.0;
  for (int j = t; j < slots; j += 256) {
    const double2 v = P[j];
    s0 += v.x;
    s1 += v.y;
  }
  r0[t] = s0;
  r1[t] = s1;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (t < h) {
      r0[t] += r0[t + h];
      r1[t] += r1[t + h];
    }
    __syncthreads();
  }
  if (t == 0) {
    const double tot = (r0[0] + r1[0]) * scale;
    const float nv = (float)(accumulate ? (double)n[i] + tot : tot);
    n[i] = nv;
    if (head) head[i] = (float)(r0[0] * scale);
    if (tail) tail[i] = (float)(r1[0] * scale);
    if (with_clip) c[i] = clip_value(nv, C);
  }
}

__global__ void __launch_bounds__(256) k_clip(const float* n, int32_t B, float C, float* c) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < B) c[i] = clip_value(n[i], C);
}

// ---------------------------------------------------------------------------
// One-launch Hutchinson over one layer, samples assigned to XCDs.
//
// Coherence: the L2 of an XCD serves all of its CUs, and the vector L1 is
// write-through. A producer's V and item sums are plain stores; it waits
// until they are acknowledged (vmcnt 0) before it bumps its sample's counter
// with an agent-scope atomic. A consumer on the same XCD polls that counter
// with atomic read-modify-writes (adding 0), which are performed where the
// increments are, and then reads the data past its own L1 (sc0) from the
// shared L2. No work group waits on a work group of another XCD, so
// no L2 has to be written back. Tickets are taken in order, and a stage-2
// item waits only on stage-1 items of lower tickets, which running work
// groups hold and finish without waiting: the scheme cannot deadlock,
// whatever the dispatch; the waits are bounded all the same.
// ---------------------------------------------------------------------------

// 8 rows x 4 columns of bf16 (row s: columns 0, 1 in word x, 2, 3 in word y)
// to 4 operands of 8 rows each (column e's rows 0..7, row 0 in the low half of
// word 0).
__device__ __forceinline__ void transpose8x4_bf16(const uint2 in[8], uint4 out[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = (e < 2) ? in[2 * k].x : in[2 * k].y;
      const uint32_t b = (e < 2) ? in[2 * k + 1].x : in[2 * k + 1].y;
      w[k] = (e & 1) ? pack_hi16(a, b) : pack_lo16(a, b);
    }
    out[e] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Stage 2 of the one-launch call: the sum of squares of Y = X2^T V over the
// columns u0 .. u0 + 63 of one sample's X2 [T][w] and all of T. Wave q takes
// the q-th quarter of the 32-row chunks, streamed through an LDS ring as the
// stage kernels do (its chunk's rows of 128 bytes and its V blocks, read
// past L1); a lane reads 8 rows of its 4 consecutive columns and transposes
// them so T runs along the MFMA K slots. The quarters' accumulators are added
// to wave 0's in wave order through LDS. Returns the sum in thread 0.
template <int NCB>
__device__ double tcontract64_item(const uint16_t* X2, const uint4* Vs, int T, int w, int u0, unsigned char* lds) {
  constexpr int kXBytes = 32 * 128;               // one chunk of 64 columns
  constexpr int kVBlocks = 2 * NCB;               // 1 KB V blocks per chunk
  constexpr int kWave = kXBytes + kVBlocks * 1024;
  constexpr int kStage = kXcdWaves * kWave;
  constexpr int kBufs = 4;
  constexpr int kP = 4 + kVBlocks;                // loads every wave issues per stage
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int nch = (T + 31) >> 5;
  const int ncs = (nch + kXcdWaves - 1) / kXcdWaves;          // stages
  const int cw = wv * ncs, nw = max(0, min(ncs, nch - cw));   // this wave's first chunk, and its chunks
  const bool uok = u0 + 4 * n < w;                            // w is a multiple of 8
  const uint16_t* X = X2 + min(u0 + 8 * (lane & 7), w - 8);   // this lane's 16 bytes of a row
  const int drow = lane >> 3;                                 // and its row within a 1 KB load
  const uint4* V = Vs + lane;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;

  auto dma = [&](int st) {
    if (st >= ncs) return;
    const uint32_t buf = lds_base + (uint32_t)((st % kBufs) * kStage + wv * kWave);
    const int c = st < nw ? cw + st : nch - 1;   // past this quarter's chunks: reloaded, zeroed after the read
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = min(32 * c + 8 * j + drow, T - 1);
      dma16_stream(X + (int64_t)t * w, buf + (uint32_t)(j * 1024));
    }
#pragma unroll
    for (int m = 0; m < kVBlocks; ++m) dma16_l2(V + ((int64_t)c * kVBlocks + m) * 64, buf + (uint32_t)(kXBytes + m * 1024));
  };

  f32x4_t acc[4][NCB];
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb) acc[e][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint2 z2 = make_uint2(0, 0);
  const uint4 z = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int st = 0; st < kBufs - 1; ++st) dma(st);
  for (int st = 0; st < ncs; ++st) {
    wait_after<kP>(min(kBufs - 2, ncs - 1 - st));
    block_barrier();
    dma(st + kBufs - 1);
    const unsigned char* buf = lds + (st % kBufs) * kStage + wv * kWave;
    const int t0 = 32 * (cw + st);
    const bool cok = st < nw;
    uint2 raw[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int r = slot_row(g, s);
      const uint2 x = *(const uint2*)(buf + r * 128 + n * 8);
      raw[s] = (uok && cok && t0 + r < T) ? x : z2;
    }
    uint4 bv[NCB][2];
#pragma unroll
    for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 v = *(const uint4*)(buf + kXBytes + (jb * 2 + h) * 1024 + lane * 16);
        bv[jb][h] = cok ? v : z;
      }
    uint4 op[4];
    transpose8x4_bf16(raw, op);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb) acc[e][jb] = mfma_bf16(op[e], bv[jb][h], acc[e][jb]);
  }
  // quarters 1..3 added to quarter 0 in that order, then the squares
  __syncthreads();   // every wave is done with the ring
  float* xch = (float*)lds + lane;
  if (wv > 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) xch[((((wv - 1) * 4 + e) * NCB + jb) * 4 + r) * 64] = acc[e][jb][r];
  }
  __syncthreads();
  double sum = 0.0;
  if (wv == 0) {
#pragma unroll
    for (int q = 0; q < kXcdWaves - 1; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[e][jb][r] += xch[(((q * 4 + e) * NCB + jb) * 4 + r) * 64];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int jb = 0; jb < NCB; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const double y = (double)acc[e][jb][r];
          sum += y * y;
        }
    sum = wave_sum(sum);
  }
  return sum;
}

template <int NCB>
constexpr int xcd_lds_bytes() {
  constexpr int s1 = rowproj_lds_bytes<NCB, 1, kXcdWaves, kXcdWaves>();
  constexpr int s2 = 4 * kXcdWaves * (32 * 128 + 2 * NCB * 1024);
  return s1 > s2 ? s1 : s2;
}

__global__ void __launch_bounds__(256) k_xcd_reset(uint32_t* ctr, int32_t words) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < words) ctr[i] = 0u;
}

template <int NCB>
__global__ void __launch_bounds__(64 * kXcdWaves) k_hutch_xcd(XcdArgs x) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[xcd_lds_bytes<NCB>()];
  __shared__ int s_ticket, s_ok;
  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  xcc &= 7u;
  const int B = x.B, n1 = x.n1, n2 = x.n2, per = n1 + n2;
  const int mine = ((int)B - (int)xcc + 7) / 8;   // samples xcc, xcc + 8, ...
  uint32_t* ticket = x.ctr + xcc;
  uint32_t* done1 = x.ctr + 8;
  uint32_t* done2 = x.ctr + 8 + B;
  uint32_t* timeouts = x.ctr + 8 + 2 * B;
  const int T = x.st.T, Tpad = x.st.Tpad, d = x.d;
  for (;;) {
    if (threadIdx.x == 0) s_ticket = (int)__hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int t = s_ticket;
    __syncthreads();
    if (t >= mine * per) break;   // uniform
    const int s = (int)xcc + 8 * (t / per), r = t % per;
    if (r < n1) {
      rowproj_bf16_item<NCB, 1, kXcdWaves, true, true, kXcdWaves>(x.st, make_int4(0, s, r, 0), (uint32_t)t, lds);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's V stores have reached L2
      __syncthreads();
      if (threadIdx.x == 0) __hip_atomic_fetch_add(done1 + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      continue;
    }
    if (threadIdx.x == 0) {   // the sample's stage 1, with a bounded wait
      uint32_t polls = 0;
      int ok = 1;
      while (atomic_read_u32(done1 + s) < (uint32_t)n1) {
        if (++polls > x.spin_limit) {
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      s_ok = ok;
    }
    __syncthreads();
    if (!s_ok) {   // uniform: the sample's estimate is marked invalid and this work group stops
      if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        x.n[s] = __int_as_float(0x7fc00000);
        if (x.c) x.c[s] = __int_as_float(0x7fc00000);
      }
      break;
    }
    const int item = r - n1;
    const uint16_t* X2 = x.A + (int64_t)s * T * d;
    const uint4* Vs = (const uint4*)x.st.rec0.V + (int64_t)s * (Tpad / 32) * (NCB * 2 * 64);
    const double sum = tcontract64_item<NCB>(X2, Vs, T, d, 64 * item, lds);
    if (threadIdx.x == 0) {
      x.sums[(int64_t)s * n2 + item] = sum;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the sum has reached L2
      s_ticket = (int)__hip_atomic_fetch_add(done2 + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (s_ticket == n2 - 1 && threadIdx.x < 64) {   // the sample's last item: wave 0 sums the items' sums
      // (lane j the items j and j + 64, read past L1; then a fixed tree over the lanes)
      const double* sp = x.sums + (int64_t)s * n2;
      const int j0 = threadIdx.x, j1 = threadIdx.x + 64;
      double v0, v1;
      ldg2_f64_l2(sp + min(j0, n2 - 1), sp + min(j1, n2 - 1), v0, v1);
      double tot = (j0 < n2 ? v0 : 0.0) + (j1 < n2 ? v1 : 0.0);
      tot = wave_sum(tot);
      if (threadIdx.x == 0) {
        const float nv = (float)(x.accumulate ? (double)x.n[s] + tot : tot);
        x.n[s] = nv;
        if (x.c) x.c[s] = clip_value(nv, x.C);
      }
    }
    __syncthreads();   // the ring, the exchange area and s_ticket are free for the next item
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_prepare(const PrepArgs& a, hipStream_t s) {
  if (a.total_units <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_prepare, dim3((a.total_units + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

// The K split carries KS chunks of W per stage: only NCB HL <= 2 fits the LDS
// (the host takes 64-row items for wider W), so no other is instantiated.
template <int NCB, int HL, int NW, bool RAW, bool IMPL, int KS>
static void rowproj_bf16_one(const StageArgs& a, hipStream_t s) {
  // only the forms whose stage ring fits the LDS (the host asks for no other)
  if constexpr (rowproj_lds_bytes<NCB, HL, NW, KS>() <= 160 * 1024)
    hipLaunchKernelGGL((k_rowproj_bf16<NCB, HL, NW, RAW, IMPL, KS>), dim3(a.n_items), dim3(64 * NW), 0, s, a);
}

template <int NW, int HL, bool RAW, bool IMPL, int KS>
static void rowproj_bf16_ncb(const StageArgs& a, int NCB, hipStream_t s) {
  if (NCB == 1) rowproj_bf16_one<1, HL, NW, RAW, IMPL, KS>(a, s);
  else if (NCB == 2) rowproj_bf16_one<2, HL, NW, RAW, IMPL, KS>(a, s);
  else rowproj_bf16_one<4, HL, NW, RAW, IMPL, KS>(a, s);
}

template <int NW, int KS>
static void rowproj_bf16_nw(const StageArgs& a, int NCB, int HL, bool raw, bool implicit, hipStream_t s) {
  if (implicit) rowproj_bf16_ncb<NW, 1, true, true, KS>(a, NCB, s);
  else if (raw) rowproj_bf16_ncb<NW, 1, true, false, KS>(a, NCB, s);
  else if (HL == 1) rowproj_bf16_ncb<NW, 1, false, false, KS>(a, NCB, s);
  else rowproj_bf16_ncb<NW, 2, false, false, KS>(a, NCB, s);
}

hipError_t launch_rowproj(const StageArgs& a, bool bf16, int NCB, int HL, int rows1, bool raw, bool implicit,
                          hipStream_t s, int ks1) {
  if (a.n_items <= 0) return hipSuccess;
  if ((raw || implicit) && (!bf16 || HL != 1)) return hipErrorInvalidValue;
  if (implicit && a.rbs < 1) return hipErrorInvalidValue;
  const dim3 grid(a.n_items), blk(256);
  if (bf16) {
    if (ks1 != 1 && (ks1 != 2 || rows1 != kRowsK1Small || NCB * HL > 4)) return hipErrorInvalidValue;
    if (rows1 == kRowsK1) rowproj_bf16_nw<4, 1>(a, NCB, HL, raw, implicit, s);
    else if (rows1 == kRowsK1Small && ks1 == 2) rowproj_bf16_nw<4, 2>(a, NCB, HL, raw, implicit, s);
    else if (rows1 == kRowsK1Small) rowproj_bf16_nw<2, 1>(a, NCB, HL, raw, implicit, s);
    else if (rows1 == kRowsK1Tiny && NCB * HL <= 2) rowproj_bf16_nw<4, 4>(a, NCB, HL, raw, implicit, s);
    else return hipErrorInvalidValue;
  } else {
    if (rows1 != kRowsK1) return hipErrorInvalidValue;
    if (NCB == 1) hipLaunchKernelGGL((k_rowproj_f32<1>), grid, blk, 0, s, a);
    else if (NCB == 2) hipLaunchKernelGGL((k_rowproj_f32<2>), grid, blk, 0, s, a);
    else hipLaunchKernelGGL((k_rowproj_f32<4>), grid, blk, 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_tcontract(const StageArgs& a, bool bf16, int NCB, int cols, bool direct, bool implicit,
                            hipStream_t s, int halves) {
  if (a.n_items <= 0) return hipSuccess;
  if (implicit && (!bf16 || a.ubs < 1 || (NCB != 1 && NCB != 2 && NCB != 4))) return hipErrorInvalidValue;
  if (bf16 && cols != kColsK2Bf16 && cols != kColsK2Bf16Narrow) return hipErrorInvalidValue;
  if (halves != 1 && (halves != 2 || !bf16 || cols != kColsK2Bf16Narrow || direct || NCB > 2))
    return hipErrorInvalidValue;
  const dim3 grid(a.n_items), blk(256);
  if (halves == 2) {  // two pairs of waves over 256 columns, one half of the split each
#define DPN_TCH(N, I) hipLaunchKernelGGL((k_tcontract_bf16<N, false, I, 2, 2>), grid, blk, 0, s, a)
    if (implicit) {
      if (NCB == 1) DPN_TCH(1, true);
      else DPN_TCH(2, true);
    } else {
      if (NCB == 1) DPN_TCH(1, false);
      else DPN_TCH(2, false);
    }
#undef DPN_TCH
    return hipGetLastError();
  }
  if (bf16 && cols == kColsK2Bf16Narrow) {  // two-wave work groups of 256 columns
    const dim3 blk2(128);
#define DPN_TCN(N, I)                                                                           \
  do {                                                                                          \
    if (direct) hipLaunchKernelGGL((k_tcontract_bf16<N, true, I, 2>), grid, blk2, 0, s, a);     \
    else hipLaunchKernelGGL((k_tcontract_bf16<N, false, I, 2>), grid, blk2, 0, s, a);           \
  } while (0)
    if (implicit) {
      if (NCB == 1) DPN_TCN(1, true);
      else if (NCB == 2) DPN_TCN(2, true);
      else DPN_TCN(4, true);
    } else {
      if (NCB == 1) DPN_TCN(1, false);
      else if (NCB == 2) DPN_TCN(2, false);
      else if (NCB == 3) DPN_TCN(3, false);
      else if (NCB == 4) DPN_TCN(4, false);
      else DPN_TCN(6, false);
    }
#undef DPN_TCN
    return hipGetLastError();
  }
#define DPN_TC(KER, N)                                                          \
  do {                                                                          \
    if (direct) hipLaunchKernelGGL((KER<N, true>), grid, blk, 0, s, a);         \
    else hipLaunchKernelGGL((KER<N, false>), grid, blk, 0, s, a);               \
  } while (0)
#define DPN_TCB(N, I)                                                                         \
  do {                                                                                        \
    if (direct) hipLaunchKernelGGL((k_tcontract_bf16<N, true, I>), grid, blk, 0, s, a);       \
    else hipLaunchKernelGGL((k_tcontract_bf16<N, false, I>), grid, blk, 0, s, a);             \
  } while (0)
  if (bf16 && implicit) {
    if (NCB == 1) DPN_TCB(1, true);
    else if (NCB == 2) DPN_TCB(2, true);
    else DPN_TCB(4, true);
  } else if (bf16) {
    if (NCB == 1) DPN_TCB(1, false);
    else if (NCB == 2) DPN_TCB(2, false);
    else if (NCB == 3) DPN_TCB(3, false);
    else if (NCB == 4) DPN_TCB(4, false);
    else DPN_TCB(6, false);
  } else {
    if (NCB == 1) DPN_TC(k_tcontract_f32, 1);
    else if (NCB == 2) DPN_TC(k_tcontract_f32, 2);
    else if (NCB == 3) DPN_TC(k_tcontract_f32, 3);
    else if (NCB == 6) DPN_TC(k_tcontract_f32, 6);
    else DPN_TC(k_tcontract_f32, 4);
  }
#undef DPN_TC
#undef DPN_TCB
  return hipGetLastError();
}

hipError_t launch_ysum(const StageArgs& a, int NCB, int cols_per_block, int mode, bool implicit, hipStream_t s) {
  const int blocks = a.n_items / a.nsplit;
  const int ychunks = ysum_chunks(cols_per_block, NCB);
  if (blocks <= 0) return hipSuccess;
  if (implicit && a.ubs < 1) return hipErrorInvalidValue;
  const dim3 grid(blocks * ychunks);
  if (mode == MODE_SQ && implicit)
    hipLaunchKernelGGL((k_ysum<MODE_SQ, true>), grid, dim3(64), 0, s, a, 16 * NCB, cols_per_block, ychunks);
  else if (mode == MODE_SQ)
    hipLaunchKernelGGL((k_ysum<MODE_SQ, false>), grid, dim3(64), 0, s, a, 16 * NCB, cols_per_block, ychunks);
  else if (implicit)
    hipLaunchKernelGGL((k_ysum<MODE_STORE, true>), grid, dim3(64), 0, s, a, 16 * NCB, cols_per_block, ychunks);
  else
    hipLaunchKernelGGL((k_ysum<MODE_STORE, false>), grid, dim3(64), 0, s, a, 16 * NCB, cols_per_block, ychunks);
  return hipGetLastError();
}

hipError_t launch_finish(const double2* partials, int32_t B, int32_t slots, float* n, int accumulate, float* head,
                         float* tail, float* c, float C, int with_clip, double scale, hipStream_t s) {
  hipLaunchKernelGGL(k_finish, dim3(B), dim3(256), 0, s, partials, slots, n, accumulate, head, tail, c, C,
                     with_clip, scale);
  return hipGetLastError();
}

hipError_t launch_hutch_xcd(const XcdArgs& x, int NCB, hipStream_t s) {
  if (x.B < 1 || x.n1 < 1 || x.n2 < 1 || (NCB != 1 && NCB != 2)) return hipErrorInvalidValue;
  const int words = (int)xcd_counters(x.B);
  hipLaunchKernelGGL(k_xcd_reset, dim3((words + 255) / 256), dim3(256), 0, s, x.ctr, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one work group per CU of each XCD (a multiple of 8 keeps the dispatch even)
  const dim3 grid(256), blk(64 * kXcdWaves);
  if (NCB == 1) hipLaunchKernelGGL(k_hutch_xcd<1>, grid, blk, 0, s, x);
  else hipLaunchKernelGGL(k_hutch_xcd<2>, grid, blk, 0, s, x);
  return hipGetLastError();
}

hipError_t launch_clip(const float* n, int32_t B, float C, float* c, hipStream_t s) {
  hipLaunchKernelGGL(k_clip, dim3((B + 255) / 256), dim3(256), 0, s, n, B, C, c);
  return hipGetLastError();
}

}  // namespace dpn
