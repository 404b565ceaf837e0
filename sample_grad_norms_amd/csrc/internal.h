// Internal launch interface between the C-ABI host layer and the kernels.
//
// Every projected contraction in the library has the same two-stage shape:
//   stage 1 (row projection):  V_i = X1_i W      X1_i [T][w1], W [w1][NC]
//   stage 2 (T contraction):   Y_i = X2_i^T V_i  X2_i [T][w2], Y_i [w2][NC]
// followed either by the squared Frobenius norm of Y_i (split into two column
// groups, so Hutch++ gets its head and tail from one pass) or by storing Y_i.
// For the Hutchinson estimate X1 = G, W = P, X2 = A. The host describes each
// layer of a call once; a prepare kernel writes those descriptions, the work
// item lists and (unless stage 1 reads W in place) the MFMA-packed W into the
// workspace, so one launch of each stage covers every layer of a call. A call
// over one layer whose W is read in place needs no prepare launch at all
// (StageArgs' implicit mode).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dpn {

constexpr int kRowsK1 = 128;      // rows of X1 per stage-1 work item (4 waves x 32)
constexpr int kRowsK1Small = 64;  // same with 2 waves (bf16)
constexpr int kRowsK1Tiny = 32;   // bf16, 4 waves splitting the columns of 32 rows (when 128-row items leave CUs idle)
constexpr int kColsK2Bf16 = 512;  // columns of X2 per stage-2 work item, bf16 (4 waves x 128)
constexpr int kColsK2Bf16Narrow = 256;  // same on 2 waves, for calls that split T
constexpr int kColsK2F32 = 256;   // same, fp32 (4 waves x 64)
constexpr int kYsumChunk = 256;   // elements of a Y tile per split-T reduction work group (one wave)
constexpr int kPrepChunk = 160;   // layers described per prepare launch (a ~24 KB kernel-argument table; one launch covers a 1B-class model)

// SIGN: bit-packed +-1, ld in 32-bit words; IDENTITY: W = I (no source array)
enum SrcType : int32_t { SRC_F32 = 0, SRC_BF16 = 1, SRC_SIGN = 2, SRC_IDENTITY = 3 };

// Device-side description of one layer (written by the prepare kernel).
struct LayerRec {
  const void* X1;      // [B][T][w1]
  const void* W;       // packed W (see PrepLayer)
  void* V;             // stage-1 output: bf16 hi/lo fragments or fp32 rows
  const void* X2;      // [B][T][w2]
  float* Ypart;        // split-T partial tiles [nsplit][B][w2][NC] (NULL if nsplit == 1 and no store)
  float* Yout;         // stored Y [B][w2][NC] (store mode only)
  int64_t w_stride_b;  // packed-W units between samples (0: W shared by the batch)
  int32_t w1, w2;
  int32_t slot_base;   // first partial slot of this layer within a sample (per column block, or
                       // per column block and tile chunk when T is split)
  int32_t split;       // columns < split go to the first sum, the rest to the second
  int32_t vstride;     // V units between consecutive 32-row chunks (bf16: uint4 fragments) or rows (fp32:
                       // floats); several projections that share X2 write side by side into one V
  int32_t pad_;
};

// Host-filled description used by the prepare kernel.
struct PrepLayer {
  LayerRec rec;
  const void* wsrc;        // W source, row-major [rows][ld] (per sample: + smp * wsrc_stride_b)
  int64_t wsrc_stride_b;   // source elements between samples (0: shared)
  int32_t wsrc_type;       // SrcType
  int32_t ld, ncols;       // source row stride and valid columns (< NC pads with zeros)
  int32_t nsamples;        // 1 (shared W) or B
  int32_t layer;           // index of this layer in the record table
  int32_t unit_begin;      // first prepare unit of this layer within the launch (a multiple of 256)
  int32_t n_pack;          // packing units
  int32_t k1_begin, n1;    // stage-1 items: global range and count
  int32_t k2_begin, n2;    // stage-2 items: global range and count
  int32_t ubs;             // stage-2 column blocks of X2 per sample
  int32_t pad_;
};
// An entry of the prepare table describes a stage-1 projection (packed W and
// stage-1 items), a stage-2 group (stage-2 items), or both; n_pack, n1 or n2
// is zero for the parts an entry does not have.

struct PrepArgs {
  PrepLayer L[kPrepChunk];
  LayerRec* recs;
  int4* items1;            // (layer, sample, row block, 0)
  int4* items2;            // (layer, sample, column block, T split)
  int32_t nlayers, total_units;
  int32_t NCB, HL;         // packed W: column blocks of 16, hi/lo halves (bf16 target)
  int32_t f32_target;      // pack W as fp32 rows [rows16][NC] instead of bf16 fragments
  int32_t rbs;             // stage-1 row blocks per sample (Tpad / rows per item)
  int32_t nsplit;          // stage-2 T splits
};

struct StageArgs {
  const LayerRec* recs;
  const int4* items;
  int32_t n_items;
  int32_t B, T, Tpad, nsplit;
  int32_t slots_per_sample;
  double2* partials;       // [B][slots] (sum of squares below / above split)
  // Implicit mode (a call over one layer, bf16, with a [w1][16 NCB] bf16 W
  // read as it is): no record or item table in memory; the layer is rec0
  // (rec0.W the caller's W) and item b is derived from b: stage 1
  // (0, b / rbs, b % rbs, 0), stage 2 (0, sample, column block, split) with
  // the split innermost and ubs column blocks per sample.
  LayerRec rec0;
  int32_t rbs, ubs;
};

// mode for stage 2 and the split-T reduction
enum Mode : int32_t { MODE_SQ = 0, MODE_STORE = 1 };

hipError_t launch_prepare(const PrepArgs& a, hipStream_t s);
// raw: every record's W is the caller's bf16 [w1][16 NCB] matrix, read in
// place (bf16, HL == 1 only); implicit: the stages run in implicit mode
// (which reads W in place too).
// ks1 = 2 (bf16, rows1 == kRowsK1Small, NCB HL <= 4): the 64-row items on
// four waves, two per 32-row group, each streaming every other column chunk.
hipError_t launch_rowproj(const StageArgs& a, bool bf16, int NCB, int HL, int rows1, bool raw, bool implicit,
                          hipStream_t s, int ks1 = 1);
// direct = 1: nsplit == 1 and mode SQ, partial sums are written by the stage
// itself; otherwise Y partial tiles go to Ypart and launch_ysum finishes them.
// NCB in {1, 2, 3, 4, 6}: the column blocks of V (those of every projection of a group).
// cols: columns of X2 per item (kColsK2Bf16 or kColsK2Bf16Narrow for bf16; kColsK2F32).
// halves = 2: bf16, kColsK2Bf16Narrow, not direct, NCB <= 2: four waves per
// item, two on each half of the item's T split.
hipError_t launch_tcontract(const StageArgs& a, bool bf16, int NCB, int cols, bool direct, bool implicit,
                            hipStream_t s, int halves = 1);
hipError_t launch_ysum(const StageArgs& a, int NCB, int cols_per_block, int mode, bool implicit, hipStream_t s);
// work groups of the split-T reduction per (layer, sample, column block)
inline int ysum_chunks(int cols_per_block, int NCB) { return (cols_per_block * 16 * NCB + kYsumChunk - 1) / kYsumChunk; }
// n (+)= scale * (sum of both partial sums); head / tail get the scaled sums.
hipError_t launch_finish(const double2* partials, int32_t B, int32_t slots, float* n, int accumulate,
                         float* head, float* tail, float* c, float C, int with_clip, double scale, hipStream_t s);
hipError_t launch_clip(const float* n, int32_t B, float C, float* c, hipStream_t s);

// One-launch Hutchinson call over one bf16 layer whose P is read in place
// (k = 16 or 32), for calls too small to fill the GPU with separate stage
// launches. Sample i belongs to XCD i % 8: that XCD's work groups take
// tickets in order from its counter, first the sample's stage-1 items (32
// rows of G each, the four-wave K split of stage 1), then its stage-2 items
// (64 columns of A over all of T, four waves on the quarters of T, squares
// summed in the item). The stage-2 items of a sample wait (bounded) until
// its stage-1 items are done; V and the items' sums pass between the work
// groups of one XCD through that XCD's L2; the last stage-2 item of a sample
// sums the items' sums in item order and writes n (and c).
struct XcdArgs {
  StageArgs st;            // stage 1 in implicit mode: rec0 = (G, P in place, V), T, Tpad
  const uint16_t* A;       // [B][T][d]
  double* sums;            // [B][n2] stage-2 item sums
  uint32_t* ctr;           // [8] tickets, [B] stage-1 items done, [B] stage-2 items done, [1] timeouts
  float* n;                // [B]
  float* c;                // [B] or null
  float C;
  int32_t accumulate;
  int32_t B, d, n1, n2;    // n1 = ceil(T / 32), n2 = ceil(d / 64)
  uint32_t spin_limit;     // polls of a stage-2 item's wait before it gives up (n = NaN)
};
constexpr int kXcdWaves = 4;
// counters of one call: 8 + 2 B + 1 words
inline int64_t xcd_counters(int64_t B) { return 8 + 2 * B + 1; }
// Two launches: a small kernel that zeroes the counters (no memset, so a
// caller may capture the call in a graph), then the call's kernel.
hipError_t launch_hutch_xcd(const XcdArgs& x, int NCB, hipStream_t s);

// Hutch++: orthonormal basis Q of the sketch X [B][p][MP] (MP = 16 or 32
// columns, zero past m_s; dropped columns give zero columns of Q) and
// P' = P - Q (Q^T P), written as W3 [B][p][ldw] = [Q (MP columns) | P' (mt
// columns)], rank per sample into rank [B]. `scratch` holds
// hpp_qr_scratch_bytes(MP, B, p) bytes (256-byte aligned).
size_t hpp_qr_scratch_bytes(int MP, int B, int p);

// The tables of a single-layer bf16 pass (record 0, both work lists) and its
// packed projection, for a kernel that produces the projection to write in
// place of that pass's prepare launch: W (the record's packed W) holds the
// hi/lo bf16 fragments of an fp32 matrix with `rows` rows and `ncols` valid
// columns, in NCB 16-column blocks, w_stride_b units per sample, as the
// prepare kernel packs them.
struct HppNext {
  LayerRec rec;
  LayerRec* recs;
  int4* items1;
  int4* items2;
  uint4* W;
  int64_t w_stride_b;
  int32_t n1, rbs, n2, ubs, nsplit;
  int32_t rows, ncols, NCB;
};

// next == nullptr: W3 is written; else next's packed W (from the same values) and
// tables are written in its place, and W3 is not. Ypart == nullptr: X holds
// the sketch; else X is first written as the split-T sum of Ypart
// [nsplit][B][p][MP] (in split order, fp64, rounded to fp32), in place of
// the sketch pass's own split-T sum.
hipError_t launch_hpp_qr(const float* Ypart, int nsplit, float* X, int MP, int B, int p, int mt, const void* P,
                         int ptype, float tau, float* W3, int ldw, int32_t* rank, float* resid, int ms, void* scratch,
                         const HppNext* next, hipStream_t s);
// The split-T sum of a stored pass, Ypart [nsplit][B][w][NC] fp32 summed in
// split order (fp64), packed straight into `next`'s projection (the stored
// Y of that pass is not written), with next's tables.
hipError_t launch_hpp_ysum_pack(const float* Ypart, int nsplit, int B, int w, int NC, const HppNext& next,
                                hipStream_t s);

// Exact squared norms: one fp64 partial per tile into partials [B][slots].
void exact_tiles(bool bf16, bool gram, int64_t T, int64_t d, int64_t p, int32_t& tu, int32_t& tv, int32_t& slots);
hipError_t launch_exact(const void* A, const void* G, bool bf16, bool gram, int32_t B, int32_t T, int32_t d,
                        int32_t p, double2* partials, hipStream_t s);

// Read-only stream of `bytes` (a positive multiple of 16384) from buf.
hipError_t launch_read_probe(const void* buf, int64_t bytes, hipStream_t s);

}  // namespace dpn
