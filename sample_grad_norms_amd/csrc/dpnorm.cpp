// libdpnorm host layer: argument checks, workspace layout and launches.
//
// Every estimate in the library is one or more two-stage passes
// (V = X1 W, then Y = X2^T V with the squared Frobenius norm of Y or Y
// itself as the result; see internal.h). The host describes the layers of a
// pass, lays out the caller's workspace with a bump allocator (the same code
// answers the *_workspace queries, so a query and a call always agree), and
// enqueues: prepare launches (records, work lists, packed W), one stage-1
// launch, one stage-2 launch, the split-T reduction when T is split, and the
// per-sample finisher.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <numeric>
#include <vector>

#include "dpnorm.h"
#include "internal.h"

using namespace dpn;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kTargetItems = 1024;   // stage-2 work items wanted before T is split
constexpr int kMinChunksPerSplit = 16;   // >= 512 rows per T split
constexpr int64_t kMinItems = 256;       // below this many items (one per CU), splits may be shorter
constexpr int kMinChunksPerSplitSmall = 8;  // ... down to 256 rows
constexpr int kMaxK = 64;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Bump {
  size_t off = 0;
  size_t take(size_t bytes) {
    off = align_up(off);
    const size_t o = off;
    off += bytes;
    return o;
  }
};

// One layer of a two-stage pass.
struct PassLayer {
  const void* X1 = nullptr;
  const void* X2 = nullptr;
  int64_t w1 = 0, w2 = 0;
  const void* wsrc = nullptr;   // W source, row-major [w1][ld]
  int wsrc_type = SRC_BF16;
  int64_t ld = 0;
  int ncols = 0;                // valid columns of W
  int nsamples = 1;             // 1: W shared by the batch; B: one W per sample
  int64_t wsrc_stride_b = 0;    // source elements between samples
  int split = 1 << 30;          // head/tail column split of the squared sums
  float* Yout = nullptr;        // store mode destination [B][w2][NC]
};

// Layers that read the same X2 (same pointer and width) form one stage-2
// group: their V blocks sit side by side in one V, so X2 is streamed once
// for all of them and the squared norm of the wide Y is the sum of theirs.
struct PassGroup {
  std::vector<int> members;     // layer indices, in call order
  int ncb = 0;                  // column blocks of the group's V (members x NCB)
  int ubs = 0;                  // stage-2 column blocks of X2 per sample
  int k2_begin = 0, n2 = 0;     // stage-2 items
  int slot_base = 0;
  size_t off_V = 0, off_Yp = 0;
};

struct PassPlan {
  bool bf16 = true;
  int NCB = 2, HL = 1;
  int64_t B = 0, T = 0, Tpad = 0;
  int nch = 0, nsplit = 1, cols2 = kColsK2Bf16, rbs = 0;
  int halves2 = 1;  // 2: stage-2 items of 256 columns on two pairs of waves, one per half of the T split
  int rows1 = kRowsK1;  // rows per stage-1 item
  int ks1 = 1;          // 2: 64-row items on four waves that split the columns in two
  bool store = false;
  bool fuse = false;            // group layers that share X2
  size_t off_recs = 0, off_items1 = 0, off_items2 = 0, off_partials = 0;
  std::vector<size_t> off_W;
  std::vector<int> k1_begin, n1, n_pack, group_of, jb0;  // per layer
  // prepare-table entries: (layer, group) pairs; a layer alone in its group
  // carries the group too, a group of several layers has an entry of its own
  std::vector<std::pair<int, int>> entries;
  std::vector<PassGroup> groups;
  std::vector<int> class_ncb, class_begin, class_end;    // stage-2 item ranges, one per group width
  int64_t total1 = 0, total2 = 0;
  int slots = 0;
  bool direct() const { return !store && nsplit == 1; }
  bool needs_ysum() const { return nsplit > 1; }
};

int ncb_of(int64_t ncols) { return ncols <= 16 ? 1 : (ncols <= 32 ? 2 : 4); }

// Group widths (in 16-column blocks) that stage 2 is built for.
bool ncb_supported(int ncb) { return ncb == 1 || ncb == 2 || ncb == 3 || ncb == 4 || ncb == 6; }

size_t packed_units(const PassPlan& pl, int64_t rows) {
  if (pl.bf16) return (size_t)((rows + 63) / 64 * 2) * pl.NCB * pl.HL * 64;  // uint4 units, even K steps
  return (size_t)((rows + 15) / 16 * 16) * 16 * pl.NCB;                   // floats
}

// Stage-2 groups: with pl.fuse, layers with the same (X2, w2) are grouped in
// call order, each group as wide as the supported widths allow; otherwise
// every layer is its own group.
void form_groups(PassPlan& pl, const std::vector<PassLayer>& L) {
  const int nl = (int)L.size();
  pl.groups.clear();
  // layers reading one X2, in order of their first layer, each in call order
  // (one pass with a map, so a call over many layers plans in O(L log L))
  std::vector<std::vector<int>> lists;
  std::map<std::pair<uintptr_t, int64_t>, int> list_of;
  for (int l = 0; l < nl; ++l) {
    if (pl.fuse && L[l].X2) {
      const auto key = std::make_pair((uintptr_t)L[l].X2, L[l].w2);
      const auto it = list_of.find(key);
      if (it != list_of.end()) {
        lists[it->second].push_back(l);
        continue;
      }
      list_of.emplace(key, (int)lists.size());
    }
    lists.push_back({l});
  }
  for (const std::vector<int>& same : lists) {
    size_t at = 0;
    while (at < same.size()) {
      int take = (int)std::min<size_t>(same.size() - at, 6 / pl.NCB > 0 ? 6 / pl.NCB : 1);
      while (take > 1 && !ncb_supported(take * pl.NCB)) --take;
      PassGroup g;
      g.members.assign(same.begin() + at, same.begin() + at + take);
      g.ncb = take * pl.NCB;
      pl.groups.push_back(g);
      at += take;
    }
  }
}

// Lay out one pass over `L` in the workspace. Only sizes are used.
void plan_pass(PassPlan& pl, const std::vector<PassLayer>& L, Bump& bump) {
  const int nl = (int)L.size();
  pl.Tpad = (pl.T + kRowsK1 - 1) / kRowsK1 * kRowsK1;
  pl.nch = (int)((pl.T + 31) / 32);
  // bf16 stage 1 takes smaller items when 128-row items would leave CUs
  // idle: 64 rows on two waves; 32 rows over four waves that split the
  // columns when even those leave CUs idle and the LDS holds four chunks of W
  // per stage (NCB HL <= 2). (Four-wave K-split groups take one CU each, so
  // where 64-row items already fill the CUs they would run in two rounds.)
  const int64_t items128 = (int64_t)nl * pl.B * (pl.Tpad / kRowsK1);
  pl.rows1 = kRowsK1;
  if (pl.bf16 && items128 < kMinItems)
    pl.rows1 = 2 * items128 < kMinItems && pl.NCB * pl.HL <= 2 ? kRowsK1Tiny : kRowsK1Small;
  // 64-row items that fit the CUs in one round, one work group each, take
  // four waves: two per 32-row group, each streaming every other column
  // chunk (where two-wave groups could run two to a CU, they keep two waves)
  if (pl.bf16 && pl.rows1 == kRowsK1Small && pl.NCB * pl.HL <= 4 && 2 * items128 <= kMinItems) pl.ks1 = 2;
  pl.rbs = (int)(pl.Tpad / pl.rows1);
  pl.cols2 = pl.bf16 ? kColsK2Bf16 : kColsK2F32;
  form_groups(pl, L);
  const int ng = (int)pl.groups.size();
  pl.group_of.assign(nl, 0);
  pl.jb0.assign(nl, 0);
  int64_t base_items = 0;
  for (int gi = 0; gi < ng; ++gi) {
    PassGroup& g = pl.groups[gi];
    for (size_t j = 0; j < g.members.size(); ++j) {
      pl.group_of[g.members[j]] = gi;
      pl.jb0[g.members[j]] = (int)j * pl.NCB;
    }
    base_items += pl.B * ((L[g.members[0]].w2 + pl.cols2 - 1) / pl.cols2);
  }
  // A bf16 call whose 512-column items, split into pieces of at least 512
  // rows, would leave CUs idle takes items of 256 columns on two waves: twice
  // the items per split, so fewer and longer splits (and fewer partial tiles)
  // for as many work groups.
  if (pl.bf16 && base_items < kTargetItems &&
      base_items * std::min<int64_t>((kTargetItems + base_items - 1) / base_items,
                                     std::max(1, pl.nch / kMinChunksPerSplit)) < kMinItems) {
    pl.cols2 = kColsK2Bf16Narrow;
    base_items = 0;
    for (const PassGroup& g : pl.groups) base_items += pl.B * ((L[g.members[0]].w2 + pl.cols2 - 1) / pl.cols2);
  }
  for (PassGroup& g : pl.groups) g.ubs = (int)((L[g.members[0]].w2 + pl.cols2 - 1) / pl.cols2);
  // Split T when there are few (layer, sample, column block) items: more
  // splits fill the CUs but write and re-read more partial tiles, so splits
  // keep at least 512 rows, or 256 while the launch would leave CUs idle.
  pl.nsplit = 1;
  if (base_items < kTargetItems) {
    const int max_split = std::max(1, pl.nch / kMinChunksPerSplit);
    const int64_t want = (kTargetItems + base_items - 1) / base_items;
    pl.nsplit = (int)std::min<int64_t>(want, max_split);
    if (base_items * pl.nsplit < kMinItems) {
      const int max_small = std::max(1, pl.nch / kMinChunksPerSplitSmall);
      const int64_t fill = (kMinItems + base_items - 1) / base_items;
      pl.nsplit = std::max(pl.nsplit, (int)std::min<int64_t>(fill, max_small));
    }
  }
  // A bf16 call that splits T under 512-column items takes 256-column items
  // on two pairs of waves, each pair on one half of a split twice as long:
  // as many work groups of four waves, half the partial tiles to write and
  // sum. (Only where every group is at most 32 columns wide: the pairs'
  // stages fill the LDS at that width.)
  if (pl.bf16 && pl.cols2 == kColsK2Bf16 && pl.nsplit > 1 &&
      std::all_of(pl.groups.begin(), pl.groups.end(), [](const PassGroup& g) { return g.ncb <= 2; })) {
    pl.cols2 = kColsK2Bf16Narrow;
    pl.halves2 = 2;
    pl.nsplit = (pl.nsplit + 1) / 2;
    for (PassGroup& g : pl.groups) g.ubs = (int)((L[g.members[0]].w2 + pl.cols2 - 1) / pl.cols2);
  } else if (pl.bf16 && pl.cols2 == kColsK2Bf16Narrow && pl.nsplit > 1 && pl.nch / pl.nsplit >= kMinChunksPerSplit &&
             std::all_of(pl.groups.begin(), pl.groups.end(), [](const PassGroup& g) { return g.ncb <= 2; })) {
    // 256-column items whose splits keep at least 512 rows take the two
    // pairs of waves too, with the same splits: each pair streams half of
    // the item's rows (Hutch++ B=4, T=4096, d=p=2048: 130.4-132.4 us ->
    // 129.8-131.4 us; with 256-row splits the halves were slower)
    pl.halves2 = 2;
  }
  // stage-1 items, largest rows first so the launch ends on short items
  std::vector<int> order(nl);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return L[a].w1 > L[b].w1; });
  pl.k1_begin.assign(nl, 0);
  pl.n1.assign(nl, 0);
  pl.n_pack.assign(nl, 0);
  pl.total1 = 0;
  for (int l : order) {
    pl.k1_begin[l] = (int)pl.total1;
    pl.n1[l] = (int)(pl.B * pl.rbs);
    pl.total1 += pl.n1[l];
  }
  for (int l = 0; l < nl; ++l) pl.n_pack[l] = (int)(L[l].nsamples * packed_units(pl, L[l].w1));
  // stage-2 items, one contiguous range per group width
  pl.class_ncb.clear();
  pl.class_begin.clear();
  pl.class_end.clear();
  pl.total2 = 0;
  pl.slots = 0;
  for (int ncb : {1, 2, 3, 4, 6}) {
    const int64_t begin = pl.total2;
    for (PassGroup& g : pl.groups) {
      if (g.ncb != ncb) continue;
      g.k2_begin = (int)pl.total2;
      g.n2 = (int)(pl.B * g.ubs * pl.nsplit);
      pl.total2 += g.n2;
      g.slot_base = pl.slots;
      pl.slots += g.ubs * (pl.nsplit > 1 ? ysum_chunks(pl.cols2, g.ncb) : 1);
    }
    if (pl.total2 > begin) {
      pl.class_ncb.push_back(ncb);
      pl.class_begin.push_back((int)begin);
      pl.class_end.push_back((int)pl.total2);
    }
  }
  pl.entries.clear();
  for (int l = 0; l < nl; ++l) {
    const int gi = pl.group_of[l];
    pl.entries.push_back({l, pl.groups[gi].members.size() == 1 ? gi : -1});
  }
  for (int gi = 0; gi < ng; ++gi)
    if (pl.groups[gi].members.size() > 1) pl.entries.push_back({-1, gi});
  pl.off_recs = bump.take(sizeof(LayerRec) * pl.entries.size());
  pl.off_items1 = bump.take(sizeof(int4) * pl.total1);
  pl.off_items2 = bump.take(sizeof(int4) * pl.total2);
  pl.off_partials = bump.take(sizeof(double2) * pl.B * pl.slots);
  pl.off_W.assign(nl, 0);
  const size_t unit = pl.bf16 ? 16 : 4;
  for (int l = 0; l < nl; ++l) pl.off_W[l] = bump.take(unit * (size_t)pl.n_pack[l]);
  for (PassGroup& g : pl.groups) {
    g.off_V = bump.take((size_t)pl.B * pl.Tpad * 16 * g.ncb * 4);
    g.off_Yp = pl.nsplit > 1 ? bump.take((size_t)pl.nsplit * pl.B * L[g.members[0]].w2 * 16 * g.ncb * 4) : 0;
  }
}

// Launches of a pass at most (a pass that reads W in place may skip its prepare).
int pass_launches(const PassPlan& pl) {
  const int entries = (int)pl.entries.size();
  const int classes = (int)pl.class_ncb.size();
  return (entries + kPrepChunk - 1) / kPrepChunk + 1 + classes * (pl.needs_ysum() ? 2 : 1);
}

// Optional event trace around each launch.
struct Tracer {
  dpnorm_trace* t = nullptr;
  hipStream_t s = nullptr;
  hipError_t begin() {
    if (!t) return hipSuccess;
    t->count = 1;
    return hipEventRecord(t->events[0], s);
  }
  hipError_t mark(int kind) {
    if (!t) return hipSuccess;
    t->kinds[t->count - 1] = kind;
    return hipEventRecord(t->events[t->count++], s);
  }
};

#define DPN_TRY(expr)                              \
  do {                                             \
    const hipError_t e_ = (expr);                  \
    if (e_ != hipSuccess) return e_;               \
  } while (0)

// Prepare-table entry e of a pass (pl.entries): its record and what the
// prepare kernel derives from it. The record of entry e is recs[e]. raw:
// stage 1 reads the layer's W in place (no packing units).
void fill_entry(const PassPlan& pl, const std::vector<PassLayer>& L, char* base, int e, PrepLayer& P,
                bool raw = false) {
  std::memset(&P, 0, sizeof(P));
  LayerRec& R = P.rec;
  R.split = 1 << 30;
  const int le = pl.entries[e].first, ge = pl.entries[e].second;
  if (le >= 0) {  // stage-1 projection
    const PassLayer& in = L[le];
    const PassGroup& g = pl.groups[pl.group_of[le]];
    R.X1 = in.X1;
    R.W = raw ? in.wsrc : base + pl.off_W[le];
    R.w_stride_b = in.nsamples > 1 ? (int64_t)packed_units(pl, in.w1) : 0;
    R.w1 = (int32_t)in.w1;
    if (pl.bf16) {
      R.V = (uint4*)(base + g.off_V) + (size_t)pl.jb0[le] * 2 * 64;
      R.vstride = g.ncb * 2 * 64;
    } else {
      R.V = (float*)(base + g.off_V) + (size_t)pl.jb0[le] * 16;
      R.vstride = 16 * g.ncb;
    }
    P.wsrc = in.wsrc;
    P.wsrc_stride_b = in.wsrc_stride_b;
    P.wsrc_type = in.wsrc_type;
    P.ld = (int32_t)in.ld;
    P.ncols = in.ncols;
    P.nsamples = in.nsamples;
    P.n_pack = raw ? 0 : pl.n_pack[le];
    P.k1_begin = pl.k1_begin[le];
    P.n1 = pl.n1[le];
  }
  if (ge >= 0) {  // stage-2 group (V is the group's whole V, at offset 0 for a lone layer)
    const PassGroup& g = pl.groups[ge];
    const PassLayer& in = L[g.members[0]];
    R.X2 = in.X2;
    R.V = base + g.off_V;
    R.vstride = pl.bf16 ? g.ncb * 2 * 64 : 16 * g.ncb;
    R.Ypart = pl.nsplit > 1 ? (float*)(base + g.off_Yp) : (pl.store ? in.Yout : nullptr);
    R.Yout = in.Yout;
    R.w2 = (int32_t)in.w2;
    R.slot_base = g.slot_base;
    R.split = in.split;
    P.k2_begin = g.k2_begin;
    P.n2 = g.n2;
    P.ubs = g.ubs;
  }
  P.layer = e;
}

bool aligned(const void* p, size_t a);

// Stage 1 reads every layer's W in place when each is the caller's bf16
// [w1][16 NCB] matrix, 16-byte aligned and shared by the batch: the prepare
// kernel then only writes the records and item lists.
bool raw_pass(const PassPlan& pl, const std::vector<PassLayer>& L) {
  if (!pl.bf16 || pl.HL != 1 || L.empty()) return false;
  for (const PassLayer& in : L)
    if (in.wsrc_type != SRC_BF16 || in.nsamples != 1 || in.ld != 16 * pl.NCB || in.ncols != 16 * pl.NCB ||
        in.wsrc == nullptr || !aligned(in.wsrc, 16))
      return false;
  return true;
}

// Such a pass over one layer runs its stages in implicit mode: the layer's
// record travels in the launch arguments and the work items are derived from
// their indices, so the pass launches no prepare kernel at all.
bool implicit_pass(const PassPlan& pl, const std::vector<PassLayer>& L) {
  return L.size() == 1 && pl.entries.size() == 1 && pl.groups.size() == 1 && pl.class_ncb.size() == 1 &&
         pl.groups[0].ncb == pl.NCB && raw_pass(pl, L);
}

// prepare = false: the tables and packed W are already in place (written by
// the kernel that produced W); ysum = false: the split-T partial tiles are
// left for the caller to reduce.
hipError_t run_pass(const PassPlan& pl, const std::vector<PassLayer>& L, char* base, hipStream_t s, Tracer& tr,
                    bool prepare = true, bool ysum = true) {
  const int entries = (int)pl.entries.size();
  LayerRec* recs = (LayerRec*)(base + pl.off_recs);
  int4* items1 = (int4*)(base + pl.off_items1);
  int4* items2 = (int4*)(base + pl.off_items2);
  const bool raw = prepare && raw_pass(pl, L);
  const bool impl = raw && implicit_pass(pl, L);
  for (int c0 = 0; prepare && !impl && c0 < entries; c0 += kPrepChunk) {
    PrepArgs a;
    std::memset(&a, 0, sizeof(a));
    a.recs = recs;
    a.items1 = items1;
    a.items2 = items2;
    a.NCB = pl.NCB;
    a.HL = pl.HL;
    a.f32_target = pl.bf16 ? 0 : 1;
    a.rbs = pl.rbs;
    a.nsplit = pl.nsplit;
    int units = 0;
    const int cn = std::min(kPrepChunk, entries - c0);
    for (int j = 0; j < cn; ++j) {
      PrepLayer& P = a.L[j];
      fill_entry(pl, L, base, c0 + j, P, raw);
      P.unit_begin = units;
      units += (P.n_pack + P.n1 + P.n2 + 1 + 255) / 256 * 256;  // next entry starts a work group
    }
    a.nlayers = cn;
    a.total_units = units;
    DPN_TRY(launch_prepare(a, s));
    DPN_TRY(tr.mark(DPNORM_KERNEL_PREPARE));
  }
  StageArgs st;
  std::memset(&st, 0, sizeof(st));
  st.recs = recs;
  st.B = (int32_t)pl.B;
  st.T = (int32_t)pl.T;
  st.Tpad = (int32_t)pl.Tpad;
  st.nsplit = pl.nsplit;
  st.slots_per_sample = pl.slots;
  st.partials = (double2*)(base + pl.off_partials);

  if (impl) {
    PrepLayer P;
    fill_entry(pl, L, base, 0, P, true);
    st.rec0 = P.rec;
    st.rbs = pl.rbs;
    st.ubs = pl.groups[0].ubs;
  }

  st.items = items1;
  st.n_items = (int32_t)pl.total1;
  DPN_TRY(launch_rowproj(st, pl.bf16, pl.NCB, pl.HL, pl.rows1, raw, impl, s, pl.ks1));
  DPN_TRY(tr.mark(DPNORM_KERNEL_ROWPROJ));

  for (size_t c = 0; c < pl.class_ncb.size(); ++c) {
    st.items = items2 + pl.class_begin[c];
    st.n_items = pl.class_end[c] - pl.class_begin[c];
    DPN_TRY(launch_tcontract(st, pl.bf16, pl.class_ncb[c], pl.cols2, pl.direct(), impl, s,
                             pl.class_ncb[c] <= 2 ? pl.halves2 : 1));
    DPN_TRY(tr.mark(DPNORM_KERNEL_TCONTRACT));
    if (pl.needs_ysum() && ysum) {
      DPN_TRY(launch_ysum(st, pl.class_ncb[c], pl.cols2, pl.store ? MODE_STORE : MODE_SQ, impl, s));
      DPN_TRY(tr.mark(DPNORM_KERNEL_YSUM));
    }
  }
  return hipSuccess;
}

// The tables and packed W of a pass over one layer whose W is per-sample fp32
// with bf16 hi/lo packing, for a kernel that writes them in place of that
// pass's prepare launch; false when the pass is not of that form.
bool next_tables(const PassPlan& pl, const std::vector<PassLayer>& L, char* base, HppNext& nx) {
  if (!pl.bf16 || pl.HL != 2 || L.size() != 1 || pl.entries.size() != 1 || L[0].wsrc_type != SRC_F32) return false;
  PrepLayer P;
  fill_entry(pl, L, base, 0, P);
  if (P.k1_begin != 0 || P.k2_begin != 0 || P.rec.w_stride_b == 0) return false;
  std::memset(&nx, 0, sizeof(nx));
  nx.rec = P.rec;
  nx.recs = (LayerRec*)(base + pl.off_recs);
  nx.items1 = (int4*)(base + pl.off_items1);
  nx.items2 = (int4*)(base + pl.off_items2);
  nx.W = (uint4*)P.rec.W;
  nx.w_stride_b = P.rec.w_stride_b;
  nx.n1 = P.n1;
  nx.rbs = pl.rbs;
  nx.n2 = P.n2;
  nx.ubs = P.ubs;
  nx.nsplit = pl.nsplit;
  nx.rows = (int32_t)L[0].w1;
  nx.ncols = P.ncols;
  nx.NCB = pl.NCB;
  return true;
}

// ---------------------------------------------------------------------------
// Argument checks
// ---------------------------------------------------------------------------
size_t esize(dpnorm_dtype dt) { return dt == DPNORM_BF16 ? 2 : 4; }

bool dtype_ok(int dt) { return dt == DPNORM_F32 || dt == DPNORM_BF16; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Shape limits shared by the estimators: sizes >= 1, widths multiples of the
// 16-byte row granule, every index used on the device fits its type.
dpnorm_status check_dims(dpnorm_dtype dt, int64_t B, int64_t T, int64_t d, int64_t p) {
  if (B < 1 || T < 1 || d < 1 || p < 1) return DPNORM_ERR_SIZE;
  const int64_t g = dt == DPNORM_BF16 ? 8 : 4;
  if (d % g != 0 || p % g != 0) return DPNORM_ERR_SIZE;
  const int64_t lim = (int64_t)1 << 30;
  if (T > lim || d > lim || p > lim || B > lim) return DPNORM_ERR_SIZE;
  const int64_t Tpad = (T + kRowsK1 - 1) / kRowsK1 * kRowsK1;
  if (B > ((int64_t)1 << 31) / Tpad) return DPNORM_ERR_SIZE;   // B * Tpad < 2^31
  const int64_t w = std::max(d, p);
  if (T > INT64_MAX / w / B / 4) return DPNORM_ERR_SIZE;       // byte sizes fit int64
  return DPNORM_OK;
}

dpnorm_status check_C(float C) {
  if (!(C > 0.f) || !std::isfinite(C)) return DPNORM_ERR_VALUE;
  return DPNORM_OK;
}

dpnorm_status hip_status(hipError_t e) { return e == hipSuccess ? DPNORM_OK : DPNORM_ERR_HIP; }

// ---------------------------------------------------------------------------
// Hutchinson (grouped; a single layer is a group of one)
// ---------------------------------------------------------------------------
struct HutchCall {
  PassPlan plan;
  std::vector<PassLayer> layers;
  size_t bytes = 0;
};

// Kinds of Hutchinson call:
//  HUTCH_DENSE : each layer's P is [p][k] of the call's element type;
//  HUTCH_SIGN  : each layer's P is bit-packed +-1 ([p][ceil(k/32)] 32-bit
//                words); the 1/sqrt(k) of the entries is applied as 1/k on
//                the finished sums;
//  HUTCH_ROUTED: as DENSE, except that a layer whose narrow side min(d, p) is
//                at most k gets its exact norm: that side is projected by the
//                identity, so the two stages contract W = A^T G over it (A and
//                G swap roles when d is the narrow side); P is not read there.
enum HutchKind { HUTCH_DENSE = 0, HUTCH_SIGN = 1, HUTCH_ROUTED = 2 };

bool routed_exact(int64_t d, int64_t p, int64_t k) { return std::min(d, p) <= k; }

// fuse: layers that share their streamed input (same pointer and width)
// share one stage-2 pass.
dpnorm_status build_hutch(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B, int64_t T, int64_t k,
                          bool need_ptrs, bool fuse, HutchKind kind, HutchCall& hc) {
  const bool sign = kind == HUTCH_SIGN;
  if (!layers) return DPNORM_ERR_NULL;
  if (!dtype_ok(dt)) return DPNORM_ERR_DTYPE;
  if (L < 1 || L > (1 << 20)) return DPNORM_ERR_SIZE;
  if (k < 1 || k > kMaxK) return DPNORM_ERR_SIZE;
  hc.layers.resize(L);
  int64_t items1 = 0, items2 = 0;
  for (int64_t l = 0; l < L; ++l) {
    const dpnorm_layer& y = layers[l];
    const dpnorm_status st = check_dims(dt, B, T, y.d, y.p);
    if (st != DPNORM_OK) return st;
    const bool exact = kind == HUTCH_ROUTED && routed_exact(y.d, y.p, k);
    if (need_ptrs) {
      if (!y.A || !y.G || (!exact && !y.P)) return DPNORM_ERR_NULL;
      if (!aligned(y.A, 16) || !aligned(y.G, 16)) return DPNORM_ERR_ALIGN;
      if (!exact && !aligned(y.P, sign ? 4 : esize(dt))) return DPNORM_ERR_ALIGN;
    }
    PassLayer& pl = hc.layers[l];
    if (exact) {
      const bool swap = y.d < y.p;  // project the narrow side
      pl.X1 = swap ? y.A : y.G;
      pl.X2 = swap ? y.G : y.A;
      pl.w1 = swap ? y.d : y.p;
      pl.w2 = swap ? y.p : y.d;
      pl.wsrc = nullptr;
      pl.wsrc_type = SRC_IDENTITY;
      pl.ld = 0;
      pl.ncols = (int)pl.w1;
    } else {
      pl.X1 = y.G;
      pl.X2 = y.A;
      pl.w1 = y.p;
      pl.w2 = y.d;
      pl.wsrc = y.P;
      pl.wsrc_type = sign ? SRC_SIGN : (dt == DPNORM_BF16 ? SRC_BF16 : SRC_F32);
      pl.ld = sign ? (k + 31) / 32 : k;
      pl.ncols = (int)k;
    }
    items1 += B * ((T + kRowsK1Tiny - 1) / kRowsK1Tiny);
    items2 += B * ((pl.w2 + kColsK2F32 - 1) / kColsK2F32) * 64;
  }
  if (items1 >= ((int64_t)1 << 31) || items2 >= ((int64_t)1 << 31)) return DPNORM_ERR_SIZE;
  PassPlan& p = hc.plan;
  p.bf16 = dt == DPNORM_BF16;
  p.NCB = ncb_of(k);
  p.HL = 1;  // P is an input of the call's own element type: exact in bf16
  p.B = B;
  p.T = T;
  p.store = false;
  p.fuse = fuse;
  Bump bump;
  plan_pass(p, hc.layers, bump);
  hc.bytes = align_up(bump.off);
  return DPNORM_OK;
}

// The one-launch path (launch_hutch_xcd): one bf16 layer, P read in place
// (16-byte aligned; P == NULL in a workspace query counts as such), k = 16 or
// 32, B a multiple of 8 (every XCD takes as many samples) and a call small
// enough that separate stage launches, each with its fixed cost, would
// dominate it, with d <= 8192 (at most 128 stage-2 items a sample, whose
// sums the finisher wave reads two a lane). Workspace: V, the stage-2 item
// sums, the counters.
constexpr double kXcdMaxBytes = 160e6;   // B T (d + p) 2 at most
constexpr int64_t kXcdMaxT = 2048;
constexpr uint32_t kXcdSpinLimit = 1u << 16;   // polls (each an atomic and a short sleep) of a stage-2 wait: some ms,
                                              // far beyond any stage 1 of these sizes (tens of us)

struct XcdPlan {
  bool use = false;
  int NCB = 0;
  int32_t n1 = 0, n2 = 0;
  int64_t Tpad = 0;
  size_t off_V = 0, off_sums = 0, off_ctr = 0, bytes = 0;
};

// Switched off: its first GPU runs (B=8, T=1024, d=p=2048, k=32) did not
// finish within 120 s, twice, the second time with the stage-2 wait polling
// through a returning atomic; the cause is not established, so no call takes
// this path.
constexpr bool kXcdEnabled = false;

XcdPlan xcd_plan(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B, int64_t T, int64_t k,
                 HutchKind kind) {
  XcdPlan x;
  if (!kXcdEnabled || kind != HUTCH_DENSE || L != 1 || dt != DPNORM_BF16 || (k != 16 && k != 32) || B < 8 || B % 8 != 0) return x;
  const dpnorm_layer& y = layers[0];
  if (y.P && !aligned(y.P, 16)) return x;
  if (T > kXcdMaxT || y.d > 8192 || (double)B * (double)T * (double)(y.d + y.p) * 2.0 > kXcdMaxBytes) return x;
  x.NCB = (int)(k / 16);
  x.Tpad = (T + kRowsK1 - 1) / kRowsK1 * kRowsK1;
  x.n1 = (int32_t)((T + 31) / 32);
  x.n2 = (int32_t)((y.d + 63) / 64);
  Bump bump;
  x.off_V = bump.take((size_t)B * x.Tpad * 16 * x.NCB * 4);   // 32-row chunks of NCB x 2 KB (hi and lo)
  x.off_sums = bump.take((size_t)B * x.n2 * 8);
  x.off_ctr = bump.take((size_t)xcd_counters(B) * 4);
  x.bytes = align_up(bump.off);
  x.use = true;
  return x;
}

dpnorm_status hutch_impl(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B, int64_t T, int64_t k,
                         float* n, int accumulate, float* c, float C, void* ws, size_t ws_bytes, hipStream_t stream,
                         dpnorm_trace* trace, HutchKind kind = HUTCH_DENSE, int32_t* routes = nullptr) {
  const bool sign = kind == HUTCH_SIGN;
  HutchCall hc;
  dpnorm_status st = build_hutch(layers, L, dt, B, T, k, true, true, kind, hc);
  if (st != DPNORM_OK) return st;
  // A workspace sized without knowing which layers share A (a query with
  // NULL pointers) may be too small for the fused plan: run unfused then.
  if (ws_bytes < hc.bytes) {
    HutchCall plain;
    if (build_hutch(layers, L, dt, B, T, k, true, false, kind, plain) == DPNORM_OK && ws_bytes >= plain.bytes)
      hc = std::move(plain);
  }
  if (!n) return DPNORM_ERR_NULL;
  if (accumulate != 0 && accumulate != 1) return DPNORM_ERR_VALUE;
  if (!aligned(n, 4) || (c && !aligned(c, 4))) return DPNORM_ERR_ALIGN;
  if (c) {
    st = check_C(C);
    if (st != DPNORM_OK) return st;
  }
  if (hc.bytes > 0 && !ws) return DPNORM_ERR_NULL;
  if (ws_bytes < hc.bytes) return DPNORM_ERR_WORKSPACE;
  if (ws && !aligned(ws, kAlign)) return DPNORM_ERR_ALIGN;
  // outputs must not overlap any input or the workspace
  const size_t nb = (size_t)B * 4;
  const size_t e = esize(dt);
  for (int64_t l = 0; l < L; ++l) {
    const dpnorm_layer& y = layers[l];
    const size_t sa = (size_t)B * T * y.d * e, sg = (size_t)B * T * y.p * e;
    const size_t sp = sign ? (size_t)y.p * ((k + 31) / 32) * 4 : (size_t)y.p * k * e;
    const bool reads_P = !(kind == HUTCH_ROUTED && routed_exact(y.d, y.p, k));
    for (const float* o : {(const float*)n, (const float*)c}) {
      if (!o) continue;
      if (overlaps(o, nb, y.A, sa) || overlaps(o, nb, y.G, sg) || (reads_P && overlaps(o, nb, y.P, sp)))
        return DPNORM_ERR_VALUE;
    }
  }
  if (overlaps(n, nb, ws, hc.bytes) || (c && overlaps(c, nb, ws, hc.bytes))) return DPNORM_ERR_VALUE;
  if (c && c != n && overlaps(c, nb, n, nb)) return DPNORM_ERR_VALUE;
  if (trace) {
    if (!trace->events || !trace->kinds) return DPNORM_ERR_NULL;
    const int need = pass_launches(hc.plan) + 1;
    if (trace->capacity < need + 1) return DPNORM_ERR_SIZE;
  }

  if (routes)
    for (int64_t l = 0; l < L; ++l) routes[l] = kind == HUTCH_ROUTED && routed_exact(layers[l].d, layers[l].p, k) ? 1 : 0;
  const XcdPlan xp = trace ? XcdPlan() : xcd_plan(layers, L, dt, B, T, k, kind);
  if (xp.use && ws_bytes >= xp.bytes && !overlaps(n, nb, ws, xp.bytes) && !(c && overlaps(c, nb, ws, xp.bytes))) {
    const dpnorm_layer& y = layers[0];
    char* base = (char*)ws;
    XcdArgs a;
    std::memset(&a, 0, sizeof(a));
    a.st.B = (int32_t)B;
    a.st.T = (int32_t)T;
    a.st.Tpad = (int32_t)xp.Tpad;
    a.st.nsplit = 1;
    a.st.rec0.X1 = y.G;
    a.st.rec0.W = y.P;
    a.st.rec0.V = base + xp.off_V;
    a.st.rec0.w1 = (int32_t)y.p;
    a.st.rec0.w2 = (int32_t)y.d;
    a.st.rec0.vstride = xp.NCB * 2 * 64;
    a.st.rec0.split = 1 << 30;
    a.A = (const uint16_t*)y.A;
    a.sums = (double*)(base + xp.off_sums);
    a.ctr = (uint32_t*)(base + xp.off_ctr);
    a.n = n;
    a.c = c;
    a.C = c ? C : 1.f;
    a.accumulate = accumulate;
    a.B = (int32_t)B;
    a.d = (int32_t)y.d;
    a.n1 = xp.n1;
    a.n2 = xp.n2;
    a.spin_limit = kXcdSpinLimit;
    if (const char* sl = std::getenv("DPNORM_XCD_SPIN_LIMIT")) a.spin_limit = (uint32_t)std::strtoul(sl, nullptr, 10);
    return hip_status(launch_hutch_xcd(a, xp.NCB, stream));
  }
  Tracer tr;
  tr.t = trace;
  tr.s = stream;
  hipError_t he = tr.begin();
  if (he == hipSuccess) he = run_pass(hc.plan, hc.layers, (char*)ws, stream, tr);
  if (he == hipSuccess)
    he = launch_finish((const double2*)((char*)ws + hc.plan.off_partials), (int32_t)B, hc.plan.slots, n, accumulate,
                       nullptr, nullptr, c, c ? C : 1.f, c ? 1 : 0, sign ? 1.0 / (double)k : 1.0, stream);
  if (he == hipSuccess) he = tr.mark(DPNORM_KERNEL_FINISH);
  return hip_status(he);
}

// ---------------------------------------------------------------------------
// Hutch++ (three passes, basis and tail in between)
// ---------------------------------------------------------------------------
constexpr float kRankTau = 1e-4f;  // column kept when residual > tau * largest sketch column norm (the sketch's
                                    // own rounding, about 1e-5 of it, stays well below)
constexpr int kMaxSketch = 32;      // sketch columns handled by the basis kernel

struct HppCall {
  int64_t ms = 0, mt = 0;
  PassPlan p1, p2, p3;
  std::vector<PassLayer> l1, l2, l3;
  size_t off_ys = 0, off_x = 0, off_w3 = 0, off_rank = 0, off_qr = 0;
  int NC1 = 0, NC3 = 0;
  size_t bytes = 0;
};

dpnorm_status build_hutchpp(const void* A, const void* G, const void* S, const void* P, dpnorm_dtype dt, int64_t B,
                            int64_t T, int64_t d, int64_t p, int64_t k, bool need_ptrs, HppCall& hc) {
  if (!dtype_ok(dt)) return DPNORM_ERR_DTYPE;
  dpnorm_status st = check_dims(dt, B, T, d, p);
  if (st != DPNORM_OK) return st;
  if (k < 3 || k > 96) return DPNORM_ERR_SIZE;
  hc.ms = (k + 2) / 3;
  hc.mt = k - 2 * hc.ms;
  if (hc.mt < 1 || hc.ms > kMaxSketch || hc.mt > kMaxSketch || 16 * ncb_of(hc.ms) + hc.mt > kMaxK)
    return DPNORM_ERR_SIZE;
  if (need_ptrs) {
    if (!A || !G || !S || !P) return DPNORM_ERR_NULL;
    if (!aligned(A, 16) || !aligned(G, 16) || !aligned(S, esize(dt)) || !aligned(P, esize(dt))) return DPNORM_ERR_ALIGN;
  }
  const bool bf16 = dt == DPNORM_BF16;
  const int src = bf16 ? SRC_BF16 : SRC_F32;
  const int ncb1 = ncb_of(hc.ms), ncb3 = ncb_of(16 * ncb1 + hc.mt);  // W3 = [Q (16 ncb1 columns) | P']
  hc.NC1 = 16 * ncb1;
  hc.NC3 = 16 * ncb3;
  Bump bump;
  // pass 1: Y_S = A^T (G S)   [B][d][NC1]
  hc.l1.resize(1);
  hc.l1[0].X1 = G; hc.l1[0].w1 = p; hc.l1[0].X2 = A; hc.l1[0].w2 = d;
  hc.l1[0].wsrc = S; hc.l1[0].wsrc_type = src; hc.l1[0].ld = hc.ms; hc.l1[0].ncols = (int)hc.ms;
  hc.p1.bf16 = bf16; hc.p1.NCB = ncb1; hc.p1.HL = 1; hc.p1.B = B; hc.p1.T = T; hc.p1.store = true;
  plan_pass(hc.p1, hc.l1, bump);
  hc.off_ys = bump.take((size_t)B * d * hc.NC1 * 4);
  // pass 2: X = G^T (A Y_S) = O S   [B][p][NC1]
  hc.l2.resize(1);
  hc.l2[0].X1 = A; hc.l2[0].w1 = d; hc.l2[0].X2 = G; hc.l2[0].w2 = p;
  hc.l2[0].wsrc_type = SRC_F32; hc.l2[0].ld = hc.NC1; hc.l2[0].ncols = (int)hc.ms;
  hc.l2[0].nsamples = (int)B; hc.l2[0].wsrc_stride_b = d * hc.NC1;
  hc.p2.bf16 = bf16; hc.p2.NCB = ncb1; hc.p2.HL = 2; hc.p2.B = B; hc.p2.T = T; hc.p2.store = true;
  plan_pass(hc.p2, hc.l2, bump);
  hc.off_x = bump.take((size_t)B * p * hc.NC1 * 4);
  // the head/tail matrix W3 = [Q | P']   [B][p][NC3]
  hc.off_w3 = bump.take((size_t)B * p * hc.NC3 * 4);
  hc.off_rank = bump.take((size_t)B * 4);
  hc.off_qr = bump.take(hpp_qr_scratch_bytes(hc.NC1, (int)B, (int)p));
  // pass 3: head = ||A^T G Q||^2, tail = ||A^T G P'||^2
  hc.l3.resize(1);
  hc.l3[0].X1 = G; hc.l3[0].w1 = p; hc.l3[0].X2 = A; hc.l3[0].w2 = d;
  hc.l3[0].wsrc_type = SRC_F32; hc.l3[0].ld = hc.NC3; hc.l3[0].ncols = (int)(hc.NC1 + hc.mt);
  hc.l3[0].nsamples = (int)B; hc.l3[0].wsrc_stride_b = p * hc.NC3; hc.l3[0].split = hc.NC1;
  hc.p3.bf16 = bf16; hc.p3.NCB = ncb3; hc.p3.HL = 2; hc.p3.B = B; hc.p3.T = T; hc.p3.store = false;
  plan_pass(hc.p3, hc.l3, bump);
  hc.bytes = align_up(bump.off);
  return DPNORM_OK;
}

// ---------------------------------------------------------------------------
// Exact
// ---------------------------------------------------------------------------
dpnorm_status exact_plan(dpnorm_dtype dt, int64_t B, int64_t T, int64_t d, int64_t p, dpnorm_route route, bool& gram,
                         int32_t& slots, size_t& bytes) {
  if (!dtype_ok(dt)) return DPNORM_ERR_DTYPE;
  if (route != DPNORM_EXACT_AUTO && route != DPNORM_EXACT_EXPLICIT && route != DPNORM_EXACT_GRAM)
    return DPNORM_ERR_DTYPE;
  const dpnorm_status st = check_dims(dt, B, T, d, p);
  if (st != DPNORM_OK) return st;
  gram = route == DPNORM_EXACT_GRAM || (route == DPNORM_EXACT_AUTO && (double)d * (double)p > (double)T * (double)T);
  int32_t tu = 0, tv = 0;
  // work groups per sample, as exact_tiles counts them (in 64 bits first)
  const bool bf16 = dt == DPNORM_BF16;
  const int64_t e = bf16 ? 256 : 64, nt = (T + 255) / 256, mt = (T + 127) / 128;
  const int64_t tiles = gram ? (bf16 ? nt * (nt + 1) : mt * (mt + 1) / 2) : ((d + e - 1) / e) * ((p + e - 1) / e);
  if (tiles * B >= ((int64_t)1 << 31)) return DPNORM_ERR_SIZE;
  exact_tiles(dt == DPNORM_BF16, gram, T, d, p, tu, tv, slots);
  bytes = align_up(sizeof(double2) * (size_t)B * slots);
  return DPNORM_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (dpnorm_hutch_grouped_noalloc)
// ---------------------------------------------------------------------------
// One array per GPU, held from the module's load on that GPU until the process
// ends. In host code `scratch` names a host-side stand-in, never the device
// memory: its device address is fetched once per device with
// hipGetSymbolAddress and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[DPNORM_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch array; the stream must
// belong to that device.
dpnorm_status static_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DPNORM_ERR_HIP;
  if (stream) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return DPNORM_ERR_HIP;
    if (sd != dev) return DPNORM_ERR_VALUE;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return DPNORM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DPNORM_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int dpnorm_version(void) { return 100; }

const char* dpnorm_status_string(int status) {
  switch (status) {
    case DPNORM_OK: return "DPNORM_OK";
    case DPNORM_ERR_NULL: return "DPNORM_ERR_NULL: a required pointer is NULL";
    case DPNORM_ERR_SIZE: return "DPNORM_ERR_SIZE: a size is out of range or misaligned";
    case DPNORM_ERR_DTYPE: return "DPNORM_ERR_DTYPE: unknown element type or route";
    case DPNORM_ERR_VALUE: return "DPNORM_ERR_VALUE: invalid value or overlapping output";
    case DPNORM_ERR_WORKSPACE: return "DPNORM_ERR_WORKSPACE: workspace smaller than the query";
    case DPNORM_ERR_ALIGN: return "DPNORM_ERR_ALIGN: pointer not aligned";
    case DPNORM_ERR_HIP: return "DPNORM_ERR_HIP: a HIP launch or call failed";
    default: return "unknown dpnorm status";
  }
}

dpnorm_status dpnorm_read_probe(const void* buf, int64_t bytes, hipStream_t stream) {
  if (!buf) return DPNORM_ERR_NULL;
  if (bytes <= 0 || bytes % 16384 != 0 || bytes > ((int64_t)1 << 44)) return DPNORM_ERR_SIZE;
  if (!aligned(buf, 16)) return DPNORM_ERR_ALIGN;
  return hip_status(launch_read_probe(buf, bytes, stream));
}

dpnorm_status dpnorm_hutchpp_split(int64_t k, int64_t* m_s, int64_t* m_t) {
  if (!m_s || !m_t) return DPNORM_ERR_NULL;
  if (k < 3 || k > 96) return DPNORM_ERR_SIZE;
  *m_s = (k + 2) / 3;
  *m_t = k - 2 * *m_s;
  if (*m_t < 1) return DPNORM_ERR_SIZE;
  return DPNORM_OK;
}

dpnorm_status dpnorm_hutch_workspace(dpnorm_dtype dt, int64_t B, int64_t T, int64_t d, int64_t p, int64_t k,
                                     size_t* bytes) {
  if (!bytes) return DPNORM_ERR_NULL;
  dpnorm_layer y;
  y.A = y.G = y.P = nullptr;
  y.d = d;
  y.p = p;
  HutchCall hc;
  const dpnorm_status st = build_hutch(&y, 1, dt, B, T, k, false, true, HUTCH_DENSE, hc);
  if (st != DPNORM_OK) return st;
  *bytes = std::max(hc.bytes, xcd_plan(&y, 1, dt, B, T, k, HUTCH_DENSE).bytes);
  return DPNORM_OK;
}

dpnorm_status dpnorm_hutch_grouped_workspace(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B,
                                             int64_t T, int64_t k, size_t* bytes) {
  if (!bytes) return DPNORM_ERR_NULL;
  HutchCall hc;
  const dpnorm_status st = build_hutch(layers, L, dt, B, T, k, false, true, HUTCH_DENSE, hc);
  if (st != DPNORM_OK) return st;
  *bytes = std::max(hc.bytes, xcd_plan(layers, L, dt, B, T, k, HUTCH_DENSE).bytes);
  return DPNORM_OK;
}

dpnorm_status dpnorm_hutch(const void* A, const void* G, const void* P, dpnorm_dtype dt, int64_t B, int64_t T,
                           int64_t d, int64_t p, int64_t k, float* n, int accumulate, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  dpnorm_layer y;
  y.A = A;
  y.G = G;
  y.P = P;
  y.d = d;
  y.p = p;
  return hutch_impl(&y, 1, dt, B, T, k, n, accumulate, nullptr, 1.f, ws, ws_bytes, stream, nullptr);
}

dpnorm_status dpnorm_hutch_grouped(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B, int64_t T,
                                   int64_t k, float* n, int accumulate, float* c, float C, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  return hutch_impl(layers, L, dt, B, T, k, n, accumulate, c, C, ws, ws_bytes, stream, nullptr);
}

dpnorm_status dpnorm_hutch_grouped_traced(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B,
                                          int64_t T, int64_t k, float* n, int accumulate, float* c, float C,
                                          void* ws, size_t ws_bytes, hipStream_t stream, dpnorm_trace* trace) {
  if (!trace) return DPNORM_ERR_NULL;
  return hutch_impl(layers, L, dt, B, T, k, n, accumulate, c, C, ws, ws_bytes, stream, trace);
}

dpnorm_status dpnorm_hutch_grouped_noalloc(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B,
                                           int64_t T, int64_t k, float* n, int accumulate, float* c, float C,
                                           hipStream_t stream) {
  // the plan must fit the static scratch (sharing A if that fits, else not)
  // before the device is touched
  HutchCall hc;
  const dpnorm_status st = build_hutch(layers, L, dt, B, T, k, true, true, HUTCH_DENSE, hc);
  if (st != DPNORM_OK) return st;
  if (hc.bytes > DPNORM_STATIC_SCRATCH_BYTES) {
    HutchCall plain;
    if (build_hutch(layers, L, dt, B, T, k, true, false, HUTCH_DENSE, plain) != DPNORM_OK ||
        plain.bytes > DPNORM_STATIC_SCRATCH_BYTES)
      return DPNORM_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  const dpnorm_status sst = static_scratch(stream, &ws);
  if (sst != DPNORM_OK) return sst;
  return hutch_impl(layers, L, dt, B, T, k, n, accumulate, c, C, ws, DPNORM_STATIC_SCRATCH_BYTES, stream, nullptr);
}

dpnorm_status dpnorm_hutch_sign(const void* A, const void* G, const uint32_t* S_bits, dpnorm_dtype dt, int64_t B,
                                int64_t T, int64_t d, int64_t p, int64_t k, float* n, int accumulate, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  dpnorm_layer y;
  y.A = A;
  y.G = G;
  y.P = S_bits;
  y.d = d;
  y.p = p;
  return hutch_impl(&y, 1, dt, B, T, k, n, accumulate, nullptr, 1.f, ws, ws_bytes, stream, nullptr, HUTCH_SIGN);
}

dpnorm_status dpnorm_hutch_sign_grouped(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B, int64_t T,
                                        int64_t k, float* n, int accumulate, float* c, float C, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  return hutch_impl(layers, L, dt, B, T, k, n, accumulate, c, C, ws, ws_bytes, stream, nullptr, HUTCH_SIGN);
}

dpnorm_status dpnorm_norms_routed_workspace(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B,
                                            int64_t T, int64_t k, size_t* bytes) {
  if (!bytes) return DPNORM_ERR_NULL;
  HutchCall hc;
  const dpnorm_status st = build_hutch(layers, L, dt, B, T, k, false, true, HUTCH_ROUTED, hc);
  if (st != DPNORM_OK) return st;
  *bytes = hc.bytes;
  return DPNORM_OK;
}

dpnorm_status dpnorm_norms_routed(const dpnorm_layer* layers, int64_t L, dpnorm_dtype dt, int64_t B, int64_t T,
                                  int64_t k, float* n, int accumulate, float* c, float C, int32_t* routes, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  return hutch_impl(layers, L, dt, B, T, k, n, accumulate, c, C, ws, ws_bytes, stream, nullptr, HUTCH_ROUTED, routes);
}

dpnorm_status dpnorm_hutchpp_workspace(dpnorm_dtype dt, int64_t B, int64_t T, int64_t d, int64_t p, int64_t k,
                                       size_t* bytes) {
  if (!bytes) return DPNORM_ERR_NULL;
  HppCall hc;
  const dpnorm_status st = build_hutchpp(nullptr, nullptr, nullptr, nullptr, dt, B, T, d, p, k, false, hc);
  if (st != DPNORM_OK) return st;
  *bytes = hc.bytes;
  return DPNORM_OK;
}

dpnorm_status dpnorm_hutchpp(const void* A, const void* G, const void* S, const void* P, dpnorm_dtype dt, int64_t B,
                             int64_t T, int64_t d, int64_t p, int64_t k, float* n, int accumulate, float* head,
                             float* tail, int32_t* rank, float* resid, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  HppCall hc;
  dpnorm_status st = build_hutchpp(A, G, S, P, dt, B, T, d, p, k, true, hc);
  if (st != DPNORM_OK) return st;
  if (!n) return DPNORM_ERR_NULL;
  if (accumulate != 0 && accumulate != 1) return DPNORM_ERR_VALUE;
  if (!aligned(n, 4) || (head && !aligned(head, 4)) || (tail && !aligned(tail, 4)) || (rank && !aligned(rank, 4)) ||
      (resid && !aligned(resid, 4)))
    return DPNORM_ERR_ALIGN;
  if (!ws) return DPNORM_ERR_NULL;
  if (ws_bytes < hc.bytes) return DPNORM_ERR_WORKSPACE;
  if (!aligned(ws, kAlign)) return DPNORM_ERR_ALIGN;
  const size_t nb = (size_t)B * 4, e = esize(dt);
  const size_t sa = (size_t)B * T * d * e, sg = (size_t)B * T * p * e;
  const size_t ss = (size_t)p * hc.ms * e, sp = (size_t)p * hc.mt * e;
  const void* outs[5] = {n, head, tail, rank, resid};
  const size_t ob[5] = {nb, nb, nb, nb, nb * (size_t)hc.ms};
  for (int j = 0; j < 5; ++j) {
    const void* o = outs[j];
    if (!o) continue;
    if (overlaps(o, ob[j], A, sa) || overlaps(o, ob[j], G, sg) || overlaps(o, ob[j], S, ss) ||
        overlaps(o, ob[j], P, sp) || overlaps(o, ob[j], ws, hc.bytes))
      return DPNORM_ERR_VALUE;
    for (int q = j + 1; q < 5; ++q)
      if (outs[q] && overlaps(o, ob[j], outs[q], ob[q])) return DPNORM_ERR_VALUE;
  }
  char* base = (char*)ws;
  hc.l1[0].Yout = (float*)(base + hc.off_ys);
  hc.l2[0].wsrc = base + hc.off_ys;
  hc.l2[0].Yout = (float*)(base + hc.off_x);
  hc.l3[0].wsrc = base + hc.off_w3;
  float* W3 = (float*)(base + hc.off_w3);
  int32_t* rk = (int32_t*)(base + hc.off_rank);
  Tracer tr;
  // In bf16, the kernels that produce pass 2's and pass 3's projections (the
  // split-T sum of pass 1, the basis kernel) also pack them and write those
  // passes' tables, so neither pass launches its prepare kernel.
  HppNext nx2, nx3;
  const bool fuse2 = hc.p1.needs_ysum() && hc.p1.groups.size() == 1 && next_tables(hc.p2, hc.l2, base, nx2);
  const bool fuse3 = next_tables(hc.p3, hc.l3, base, nx3);
  hipError_t he = run_pass(hc.p1, hc.l1, base, stream, tr, true, !fuse2);
  if (he == hipSuccess && fuse2)
    he = launch_hpp_ysum_pack((const float*)(base + hc.p1.groups[0].off_Yp), hc.p1.nsplit, (int)B, (int)d, hc.NC1,
                              nx2, stream);
  // The sketch pass's split-T sum runs inside the first basis kernel, which
  // needs the same rows of X for its Gram partials.
  const bool sum2 = hc.p2.needs_ysum() && hc.p2.groups.size() == 1;
  if (he == hipSuccess) he = run_pass(hc.p2, hc.l2, base, stream, tr, !fuse2, !sum2);
  if (he == hipSuccess)
    he = launch_hpp_qr(sum2 ? (const float*)(base + hc.p2.groups[0].off_Yp) : nullptr, hc.p2.nsplit,
                       (float*)(base + hc.off_x), hc.NC1, (int)B, (int)p, (int)hc.mt, P,
                       dt == DPNORM_BF16 ? SRC_BF16 : SRC_F32, kRankTau, W3, hc.NC3, rk, resid, (int)hc.ms,
                       base + hc.off_qr,
                       fuse3 ? &nx3 : nullptr, stream);
  if (he == hipSuccess) he = run_pass(hc.p3, hc.l3, base, stream, tr, !fuse3);
  if (he == hipSuccess)
    he = launch_finish((const double2*)(base + hc.p3.off_partials), (int32_t)B, hc.p3.slots, n, accumulate, head,
                       tail, nullptr, 1.f, 0, 1.0, stream);
  if (he == hipSuccess && rank) he = hipMemcpyAsync(rank, rk, nb, hipMemcpyDeviceToDevice, stream);
  return hip_status(he);
}

dpnorm_status dpnorm_exact_workspace(dpnorm_dtype dt, int64_t B, int64_t T, int64_t d, int64_t p, dpnorm_route route,
                                     size_t* bytes) {
  if (!bytes) return DPNORM_ERR_NULL;
  bool gram = false;
  int32_t slots = 0;
  return exact_plan(dt, B, T, d, p, route, gram, slots, *bytes);
}

dpnorm_status dpnorm_exact(const void* A, const void* G, dpnorm_dtype dt, int64_t B, int64_t T, int64_t d, int64_t p,
                           dpnorm_route route, float* n, int accumulate, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  bool gram = false;
  int32_t slots = 0;
  size_t bytes = 0;
  dpnorm_status st = exact_plan(dt, B, T, d, p, route, gram, slots, bytes);
  if (st != DPNORM_OK) return st;
  if (!A || !G || !n || !ws) return DPNORM_ERR_NULL;
  if (!aligned(A, 16) || !aligned(G, 16) || !aligned(n, 4) || !aligned(ws, kAlign)) return DPNORM_ERR_ALIGN;
  if (accumulate != 0 && accumulate != 1) return DPNORM_ERR_VALUE;
  if (ws_bytes < bytes) return DPNORM_ERR_WORKSPACE;
  const size_t nb = (size_t)B * 4, e = esize(dt);
  if (overlaps(n, nb, A, (size_t)B * T * d * e) || overlaps(n, nb, G, (size_t)B * T * p * e) ||
      overlaps(n, nb, ws, bytes))
    return DPNORM_ERR_VALUE;
  hipError_t he = launch_exact(A, G, dt == DPNORM_BF16, gram, (int32_t)B, (int32_t)T, (int32_t)d, (int32_t)p,
                               (double2*)ws, stream);
  if (he == hipSuccess)
    he = launch_finish((const double2*)ws, (int32_t)B, slots, n, accumulate, nullptr, nullptr, nullptr, 1.f, 0, 1.0,
                       stream);
  return hip_status(he);
}

dpnorm_status dpnorm_clip_factors(const float* n, int64_t B, float C, float* c, hipStream_t stream) {
  if (!n || !c) return DPNORM_ERR_NULL;
  if (B < 1 || B > ((int64_t)1 << 30)) return DPNORM_ERR_SIZE;
  const dpnorm_status st = check_C(C);
  if (st != DPNORM_OK) return st;
  if (!aligned(n, 4) || !aligned(c, 4)) return DPNORM_ERR_ALIGN;
  if (c != n && overlaps(c, (size_t)B * 4, n, (size_t)B * 4)) return DPNORM_ERR_VALUE;
  return hip_status(launch_clip(n, (int32_t)B, C, c, stream));
}

dpnorm_status dpnorm_event_create(hipEvent_t* ev) {
  if (!ev) return DPNORM_ERR_NULL;
  return hip_status(hipEventCreate(ev));
}
dpnorm_status dpnorm_event_destroy(hipEvent_t ev) {
  if (!ev) return DPNORM_ERR_NULL;
  return hip_status(hipEventDestroy(ev));
}
dpnorm_status dpnorm_event_elapsed_ms(hipEvent_t start, hipEvent_t stop, float* ms) {
  if (!start || !stop || !ms) return DPNORM_ERR_NULL;
  return hip_status(hipEventElapsedTime(ms, start, stop));
}
dpnorm_status dpnorm_event_record(hipEvent_t ev, hipStream_t stream) {
  if (!ev) return DPNORM_ERR_NULL;
  return hip_status(hipEventRecord(ev, stream));
}
dpnorm_status dpnorm_event_synchronize(hipEvent_t ev) {
  if (!ev) return DPNORM_ERR_NULL;
  return hip_status(hipEventSynchronize(ev));
}

}  // extern "C"
