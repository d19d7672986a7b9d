// C ABI of libfa_relayout.so: argument validation (pure host code, run before
// any HIP call), per-device launch geometry, and the exported entry points
// declared in include/fa_relayout.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/fa_relayout.h"
#include "../../include/fa_instrument.h"
#include "fa_fwd_kernel.h"
#include "fa_relayout_kernel.h"

namespace {

constexpr int kQTile = 128;
constexpr int kMaxDevices = 64;
// uint32 words of timestamps per unit of an instrumented launch: one record
// of 8 words for each of the 8 waves.
constexpr int kStampWordsPerUnit = 64;
constexpr float kMaxScale = 65536.0f;   // 2^16

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shared checks of both layouts.  P == 1 for the plain layout.
int validate(const void* q, const void* k, const void* v, const void* out, int B, int H, int S,
             int D, int P, float scale, const uint64_t* mask) {
  if (!q || !k || !v || !out) return FA_EINVAL;
  if (B <= 0 || H <= 0 || S <= 0 || P <= 0) return FA_EINVAL;
  // The kernel takes each weight as exp2(fma(s, c, -m)), c = scale * log2(e),
  // m = the rounded product of the row's largest score: the row's weights
  // share the factor exp2(rounding error of m), which cancels in the
  // normalisation while |s * c| < 2^24 (the factor stays within [1/2, 2]);
  // |scale| <= 2^16 keeps that for every score up to 2^7.5 in magnitude, and
  // larger scales are rejected.  (Far beyond, at |s * c| near 2^31 and up,
  // the factor would leave fp32's range.)
  if (!std::isfinite(scale) || std::fabs(scale) > kMaxScale) return FA_EINVAL;
  if (D != 64 && D != 128) return FA_EUNSUPPORTED;
  if (S % P != 0) return FA_EDIV;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
    return FA_EALIGN;
  if (mask && !aligned(mask, 8)) return FA_EALIGN;
  // Per-head slices are addressed with 32-bit byte offsets, which run up to
  // one 256-query tile past the last row.
  if (((int64_t)S + 256) * D * 2 > (int64_t)INT32_MAX) return FA_ERANGE;
  const int64_t nqt = (S + kQTile - 1) / kQTile;
  if ((int64_t)B * H * nqt > (int64_t)INT32_MAX) return FA_ERANGE;
  if ((int64_t)H * nqt * ((nqt + 63) / 64) > ((int64_t)1 << 40)) return FA_ERANGE;
  return FA_OK;
}

struct DeviceGeom {
  int cus = 0;
  int occ[2][2][3] = {};   // [D == 128][mode][variant]
};

std::mutex g_geom_mutex;
DeviceGeom g_geom[kMaxDevices];

// Persistent grid size for (D, mode, var) on the current device: every
// resident workgroup slot of the chip, or -1 if the device cannot be queried.
int grid_cap_for(int D, fa::StoreMode mode, fa::Variant var) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lock(g_geom_mutex);
  DeviceGeom& gm = g_geom[dev];
  if (gm.cus == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      return -1;
    gm.cus = cus;
  }
  int& occ = gm.occ[D == 128][(int)mode][(int)var];
  if (occ == 0) {
    int blocks = 0;
    if (fa::kernel_occupancy(D, mode, var, &blocks) != 0 || blocks <= 0) return -1;
    occ = blocks;
  }
  return gm.cus * occ;
}

// Extra checks for slab-layout inputs: a stage of 64 keys may cross at most
// one slab boundary, and a whole input tensor is addressed with 32-bit byte
// offsets.
int validate_slab_in(int B, int H, int S, int D, int P) {
  if (S / P < 64) return FA_EUNSUPPORTED;
  if ((int64_t)B * H * S * D * 2 > (int64_t)INT32_MAX) return FA_ERANGE;
  return FA_OK;
}

// Constants for n / d with (umulhi(n, magic) + n) >> shift, exact for
// n < 2^31 and 1 <= d < 2^31 (Granlund and Montgomery, "Division by
// invariant integers using multiplication", 1994): shift = ceil(log2 d),
// magic = floor(2^32 (2^shift - d) / d) + 1.
void div_magic(uint32_t d, uint32_t* magic, int* shift) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  *shift = l;
  *magic = (uint32_t)((((uint64_t)1 << 32) * ((1ull << l) - d)) / d + 1);
}

// How one dense call splits into launches: `whole` units of whole 256-query
// tiles on up to `cap` workgroups, then either (split_units > 0) the last
// round's tiles as 2 x tail half tiles in a second launch on up to
// `split_cap`, or (tail > 0, with a workspace) the last round's `tail`
// tiles shared by the `cap` workgroups of the first launch -- tile i's
// first tail_len stages on workgroup i, the tiles' remaining stages in
// slices of tail_hlen on the others -- their partial results merged by a
// second, small launch -- or (dyn_pieces > 0, with a workspace) a dynamic
// schedule: the first whole_units tiles, then the `tail` last tiles in
// dyn_pieces key pieces of falling length, the full rounds of whole tiles
// round-robin and everything after them handed to the workgroups of one
// launch from a counter in the workspace as they free up, the pieces merged
// by the second launch.
struct DensePlan {
  int whole_units = 0, split_units = 0, cap = 0, split_cap = 0;
  int tail = 0, tail_len = 0, tail_hlen = 0;
  int dyn_pieces = 0;
  int split_pieces = 0;    // > 1: each half tile cut into that many key pieces
  // Tiles of the split launch (two half tiles each, in split_pieces pieces).
  int tail_tiles() const { return split_units / (2 * (split_pieces > 1 ? split_pieces : 1)); }
  int64_t ws_bytes = 0;    // workspace the tail round needs
  int64_t queue_offset = 0; // dynamic schedule: the counter's byte offset in it
};

// The shortest slice (in 64-key stages) for which the tail round is spread
// over the workgroups: each slice writes a ~136 KiB partial that the merge
// reads back, which a slice of 64 stages (~0.1 ms) hides and a slice of a
// dozen does not (the Image share's 12-stage slices measured 7% slower than
// the split half tiles); shorter slices keep the schedule without a
// workspace.
constexpr int kTailMinSlice = 64;
// The shortest piece (in 64-key stages, both groups together) a half tile
// is cut into when the split launch is spread over a workspace.
constexpr int kMinPieceStages = 16;
// Dynamic schedule: the most key pieces per tail tile, the most partial
// slots per workgroup of the grid, and the fewest 64-key stages of a tile it
// cuts.  Workgroups run at unequal speeds (the chiplets of one device differ
// by up to ~15% under load, by more on some devices), so a fixed partition
// of the last round leaves the fast ones idle at the end; handing the last
// round's tiles out in pieces of falling length as workgroups free up
// evens out the finish.
constexpr int kDynMaxPieces = 6;
constexpr int kDynSlotsPerWorkgroup = 4;
constexpr int kDynMinStages = 256;

// Launch geometry of a call with params p (units = every tile): the number
// of units per launch and the persistent grid caps, or FA_EDEVICE.
// use_ws: the caller brings a workspace, so the tail round may be spread.
int plan_call(int D, fa::StoreMode mode, bool masked, const fa::FwdParams& p, DensePlan* plan,
              bool use_ws = false, int64_t ws_limit = INT64_MAX) {
  const fa::Variant var = masked ? fa::Variant::Masked : fa::Variant::Whole;
  const int cap = grid_cap_for(D, mode, var);
  if (cap <= 0) return FA_EDEVICE;
  *plan = DensePlan{};
  plan->cap = cap;
  plan->whole_units = p.units;
  if (masked) return FA_OK;
  // Dense: whole 256-query tiles fill `cap` CUs per round.  When the last
  // round would keep at most half of the CUs busy, its R tiles run instead as
  // 2R half-tiles with the keys split inside each workgroup (about half the
  // time of a whole tile), in a second launch on the same stream.
  const int tail = p.units % cap;
  const int stages = (p.S + 63) / 64;
  // The dynamic schedule, for calls of at least one full round and a last
  // round at least half full (t tail tiles in P = min(6, 4 cap / t) >= 4
  // pieces each).  Workspace: one partial slot per piece, then the counter.
  const int dyn_pieces = tail > 0 ? std::min(kDynMaxPieces, kDynSlotsPerWorkgroup * cap / tail) : 0;
  const int64_t dyn_ws = (int64_t)tail * dyn_pieces * fa::seg_floats(D) * 4 + 256;
  if (use_ws && p.units >= cap + tail && 2 * tail >= cap && stages >= kDynMinStages &&
      dyn_ws <= ws_limit) {
    plan->whole_units = p.units - tail;
    plan->tail = tail;
    plan->dyn_pieces = dyn_pieces;
    plan->queue_offset = dyn_ws - 256;
    plan->ws_bytes = dyn_ws;
    return FA_OK;
  }
  const int64_t span = (int64_t)tail * stages;
  const int64_t slice = (span + cap - 1) / cap;
  if (use_ws && tail > 0 && slice >= kTailMinSlice && slice < stages) {
    // Each of the cap slots runs about slice stages: tile i's first slice
    // on slot i, the t (stages - slice) stages of the tiles' ends in equal
    // slices (no longer than slice) on the cap - t others.  Workspace: one
    // slot per lead and one per (helper, tile end) piece, tail + cap - 1.
    const int64_t ends = (int64_t)tail * (stages - slice);
    plan->whole_units = p.units - tail;
    plan->tail = tail;
    plan->tail_len = (int)slice;
    plan->tail_hlen = (int)((ends + (cap - tail) - 1) / (cap - tail));
    plan->ws_bytes = (int64_t)(tail + cap) * fa::seg_floats(D) * 4;
    return FA_OK;
  }
  if (tail == 0 || 2 * tail > cap || stages < 2) return FA_OK;
  const int split_cap = grid_cap_for(D, mode, fa::Variant::Split);
  if (split_cap <= 0) return FA_EDEVICE;
  plan->whole_units = p.units - tail;
  plan->split_units = 2 * tail;
  plan->split_cap = split_cap;
  // With a workspace, half tiles that leave most workgroups idle are cut
  // into pieces of at least kMinPieceStages key stages, one per workgroup,
  // merged by a second launch.
  const int pieces = std::min(split_cap / (2 * tail), stages / kMinPieceStages);
  if (use_ws && pieces >= 2) {
    plan->split_pieces = pieces;
    plan->split_units = 2 * tail * pieces;
    plan->ws_bytes = (int64_t)plan->split_units * fa::seg_floats(D) * 4;
  }
  return FA_OK;
}

// Validated call -> kernel parameters (every tile as one launch's units).
int make_params(fa::StoreMode mode, const void* q, const void* k, const void* v, void* out,
                int B, int H, int S, int D, int P, float scale, const uint64_t* mask, bool slab_in,
                fa::FwdParams* pp) {
  int st = validate(q, k, v, out, B, H, S, D, P, scale, mask);
  if (st == FA_OK && slab_in) st = validate_slab_in(B, H, S, D, P);
  if (st != FA_OK) return st;
  fa::FwdParams& p = *pp;
  p = fa::FwdParams{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.out = static_cast<uint16_t*>(out);
  p.mask = mask;
  p.B = B;
  p.H = H;
  p.S = S;
  p.P = P;
  p.Sp = S / P;
  div_magic((uint32_t)p.Sp, &p.sp_magic, &p.sp_shift);
  // Dense attention runs on 256-query tiles; a block mask gives each
  // 128-query tile its own key set, so masked calls run on 128-query tiles
  // with the keys split between the two wave groups.
  const int rows = fa::tile_rows(mask ? fa::Variant::Masked : fa::Variant::Whole);
  p.nqt = (S + rows - 1) / rows;
  p.units = B * H * p.nqt;
  p.unit_base = 0;
  p.nmt = (S + kQTile - 1) / kQTile;
  p.mw = (p.nmt + 63) / 64;
  p.c = (float)((double)scale * 1.4426950408889634073599246810019);
  // With c == 0 every score weighs exp2(0) = 1; any positive c small enough
  // that |s| * c rounds away against 1 gives the same weights bit for bit,
  // and keeps (-inf) * c = -inf for the keys past S.
  if (p.c == 0.0f) p.c = 1e-30f;
  p.stamps = nullptr;
  return FA_OK;
}

// Enqueue the launches of a call.  instr != 0: timestamped instances, the
// records of the split launch following those of the whole-tile launch.
int launch_call(int D, fa::StoreMode mode, const fa::FwdParams& p, const DensePlan& plan,
                hipStream_t stream, bool slab_in, int instr) {
  const bool masked = p.mask != nullptr;
  const fa::Variant var = masked ? fa::Variant::Masked : fa::Variant::Whole;
  if (plan.tail > 0) {
    if (!p.ws || instr) return FA_ELAUNCH;
    fa::FwdParams whole = p;
    whole.units = plan.whole_units;
    whole.tail = plan.tail;
    whole.tail_len = plan.tail_len;
    whole.tail_hlen = plan.tail_hlen;
    if (plan.dyn_pieces > 0) {
      whole.dyn_pieces = plan.dyn_pieces;
      whole.queue = reinterpret_cast<int*>(reinterpret_cast<char*>(p.ws) + plan.queue_offset);
      if (fa::launch_queue_reset(whole.queue, stream) != 0) return FA_ELAUNCH;
    }
    if (fa::launch_fwd(D, mode, var, whole, plan.cap, stream, slab_in, 0) != 0) return FA_ELAUNCH;
    return fa::launch_merge(D, mode, whole, stream) == 0 ? FA_OK : FA_ELAUNCH;
  }
  if (plan.whole_units > 0) {
    fa::FwdParams whole = p;
    whole.units = plan.whole_units;
    if (fa::launch_fwd(D, mode, var, whole, plan.cap, stream, slab_in, instr) != 0)
      return FA_ELAUNCH;
  }
  if (plan.split_units > 0) {
    fa::FwdParams half = p;
    half.units = plan.split_units;
    half.unit_base = p.units - plan.tail_tiles();
    if (instr) half.stamps = p.stamps + (size_t)plan.whole_units * kStampWordsPerUnit;
    if (plan.split_pieces > 1) {
      if (!p.ws || instr) return FA_ELAUNCH;
      half.split_pieces = plan.split_pieces;
    }
    if (fa::launch_fwd(D, mode, fa::Variant::Split, half, plan.split_cap, stream, slab_in,
                       instr) != 0)
      return FA_ELAUNCH;
    if (plan.split_pieces > 1 && fa::launch_merge_split(D, mode, half, stream) != 0)
      return FA_ELAUNCH;
  }
  return FA_OK;
}

int run(fa::StoreMode mode, const void* q, const void* k, const void* v, void* out, int B, int H,
        int S, int D, int P, float scale, const uint64_t* mask, hipStream_t stream,
        bool slab_in = false) {
  fa::FwdParams p;
  int st = make_params(mode, q, k, v, out, B, H, S, D, P, scale, mask, slab_in, &p);
  if (st != FA_OK) return st;
  DensePlan plan;
  st = plan_call(D, mode, mask != nullptr, p, &plan);
  if (st != FA_OK) return st;
  return launch_call(D, mode, p, plan, stream, slab_in, 0);
}

// A workspace argument: null only when the call needs none (ws_bytes == 0 is
// then allowed too), else 16-byte aligned and at least `need` bytes.
int check_workspace(const void* ws, int64_t ws_bytes, int64_t need) {
  if (need == 0) return FA_OK;
  if (!ws) return FA_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 15) return FA_EALIGN;
  if (ws_bytes < need) return FA_ERANGE;
  return FA_OK;
}

// Dense calls with a workspace: the tail round spread over every workgroup.
// Masked calls need no workspace and run as without one.
int run_ws(fa::StoreMode mode, const void* q, const void* k, const void* v, void* out, int B,
           int H, int S, int D, int P, float scale, const uint64_t* mask, void* ws,
           int64_t ws_bytes, hipStream_t stream, bool slab_in = false) {
  fa::FwdParams p;
  int st = make_params(mode, q, k, v, out, B, H, S, D, P, scale, mask, slab_in, &p);
  if (st != FA_OK) return st;
  if (ws_bytes < 0) return FA_EINVAL;
  DensePlan plan;
  st = plan_call(D, mode, mask != nullptr, p, &plan, true);
  if (st != FA_OK) return st;
  st = check_workspace(ws, ws_bytes, plan.ws_bytes);
  if (st != FA_OK) return st;
  p.ws = static_cast<float*>(ws);
  return launch_call(D, mode, p, plan, stream, slab_in, 0);
}

int validate_relayout(const void* plain, const void* out, int B, int H, int S, int D, int P) {
  if (!plain || !out) return FA_EINVAL;
  if (B <= 0 || H <= 0 || S <= 0 || P <= 0) return FA_EINVAL;
  if (D != 64 && D != 128) return FA_EUNSUPPORTED;
  if (S % P != 0) return FA_EDIV;
  if (!aligned(plain, 16) || !aligned(out, 16)) return FA_EALIGN;
  // 32-bit chunk indices inside the kernel.
  if ((int64_t)B * H * S * (D / 8) >= ((int64_t)1 << 31)) return FA_ERANGE;
  return FA_OK;
}

int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

int run_relayout(const void* plain, void* out, int B, int H, int S, int D, int P,
                 hipStream_t stream) {
  const int st = validate_relayout(plain, out, B, H, S, D, P);
  if (st != FA_OK) return st;
  const int cus = cu_count();
  if (cus <= 0) return FA_EDEVICE;
  fa::RelayoutParams rp;
  rp.B = (uint32_t)B;
  rp.H = (uint32_t)H;
  rp.S = (uint32_t)S;
  rp.Sp = (uint32_t)(S / P);
  rp.rows = (uint32_t)B * (uint32_t)H * (uint32_t)S;
  const int grid = fa::relayout_grid(D, rp.rows, cus);
  return fa::launch_relayout(D, plain, out, rp, grid, stream) == 0 ? FA_OK : FA_ELAUNCH;
}

// Scratch of the allocation-free entry point: the partial results of a
// dense call's last round, 1024 slots of seg_floats(128) floats (the dynamic
// schedule's t < G tail tiles in P <= 4 G / t pieces use at most 4 G slots
// and its counter 256 bytes after them; a round of t tiles spread over G
// workgroups uses t + G - 1 < 2 G slots, a round cut into half-tile pieces
// at most G), in a static device array so that the entry point allocates
// nothing.  Each GPU the library runs on holds its own copy (136 MiB) until
// the process ends.  Host code never uses the array's name as an address:
// scratch_address() takes the device address once per device.
constexpr size_t kScratchFloats = 4 * 256 * (size_t)fa::seg_floats(128) + 64;
static __device__ __align__(256) float scratch[kScratchFloats];

std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, taken with hipGetSymbolAddress
// on the first call on that device (the device current), or nullptr.
float* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = static_cast<float*>(ptr);
  }
  return g_scratch_ptr[dev];
}

// attn_fwd_relayout_ws_async with `scratch` as the workspace.
int run_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H, int S,
                int D, int P, float scale, const uint64_t* mask, hipStream_t stream) {
  fa::FwdParams p;
  int st = make_params(fa::StoreMode::Slab, q, k, v, out, B, H, S, D, P, scale, mask, false, &p);
  if (st != FA_OK) return st;
  DensePlan plan;
  // A plan within the scratch array: the dynamic schedule only where its
  // partial slots fit, else the spread tail round (at most 2 cap - 1 slots).
  st = plan_call(D, fa::StoreMode::Slab, mask != nullptr, p, &plan, true,
                 (int64_t)sizeof(scratch));
  if (st != FA_OK) return st;
  if (plan.ws_bytes > (int64_t)sizeof(scratch)) return FA_ERANGE;
  if (plan.ws_bytes > 0) {
    p.ws = scratch_address();
    if (!p.ws) return FA_EDEVICE;
  }
  return launch_call(D, fa::StoreMode::Slab, p, plan, stream, false, 0);
}

int finish_blocking(int st) {
  if (st != FA_OK) return st;
  return hipStreamSynchronize(nullptr) == hipSuccess ? FA_OK : FA_EEXEC;
}

}  // namespace

extern "C" {

int attn_fwd_relayout_async(const void* q, const void* k, const void* v, void* out_slabs, int B,
                            int H, int S, int D, int P, float scale, const uint64_t* mask,
                            void* stream) {
  return run(fa::StoreMode::Slab, q, k, v, out_slabs, B, H, S, D, P, scale, mask,
             static_cast<hipStream_t>(stream));
}

int attn_fwd_relayout(const void* q, const void* k, const void* v, void* out_slabs, int B, int H,
                      int S, int D, int P, float scale, const uint64_t* mask) {
  return finish_blocking(
      run(fa::StoreMode::Slab, q, k, v, out_slabs, B, H, S, D, P, scale, mask, nullptr));
}

int attn_fwd_slab_to_slab_async(const void* q_slabs, const void* k_slabs, const void* v_slabs,
                                void* out_slabs, int B, int H, int S, int D, int P, float scale,
                                const uint64_t* mask, void* stream) {
  return run(fa::StoreMode::Slab, q_slabs, k_slabs, v_slabs, out_slabs, B, H, S, D, P, scale,
             mask, static_cast<hipStream_t>(stream), true);
}

int attn_fwd_slab_to_slab(const void* q_slabs, const void* k_slabs, const void* v_slabs,
                          void* out_slabs, int B, int H, int S, int D, int P, float scale,
                          const uint64_t* mask) {
  return finish_blocking(run(fa::StoreMode::Slab, q_slabs, k_slabs, v_slabs, out_slabs, B, H, S,
                             D, P, scale, mask, nullptr, true));
}

int attn_fwd_plain_async(const void* q, const void* k, const void* v, void* out, int B, int H,
                         int S, int D, float scale, const uint64_t* mask, void* stream) {
  return run(fa::StoreMode::Plain, q, k, v, out, B, H, S, D, 1, scale, mask,
             static_cast<hipStream_t>(stream));
}

int attn_fwd_plain(const void* q, const void* k, const void* v, void* out, int B, int H, int S,
                   int D, float scale, const uint64_t* mask) {
  return finish_blocking(
      run(fa::StoreMode::Plain, q, k, v, out, B, H, S, D, 1, scale, mask, nullptr));
}

int relayout_to_slabs_async(const void* plain, void* out_slabs, int B, int H, int S, int D,
                            int P, void* stream) {
  return run_relayout(plain, out_slabs, B, H, S, D, P, static_cast<hipStream_t>(stream));
}

int relayout_to_slabs(const void* plain, void* out_slabs, int B, int H, int S, int D, int P) {
  return finish_blocking(run_relayout(plain, out_slabs, B, H, S, D, P, nullptr));
}

int attn_fwd_relayout_ws_async(const void* q, const void* k, const void* v, void* out_slabs,
                               int B, int H, int S, int D, int P, float scale,
                               const uint64_t* mask, void* workspace, int64_t workspace_bytes,
                               void* stream) {
  return run_ws(fa::StoreMode::Slab, q, k, v, out_slabs, B, H, S, D, P, scale, mask, workspace,
                workspace_bytes, static_cast<hipStream_t>(stream));
}

int attn_fwd_relayout_noalloc_async(const void* q, const void* k, const void* v, void* out_slabs,
                                    int B, int H, int S, int D, int P, float scale,
                                    const uint64_t* mask, void* stream) {
  return run_noalloc(q, k, v, out_slabs, B, H, S, D, P, scale, mask,
                     static_cast<hipStream_t>(stream));
}

int attn_fwd_slab_to_slab_ws_async(const void* q_slabs, const void* k_slabs, const void* v_slabs,
                                   void* out_slabs, int B, int H, int S, int D, int P,
                                   float scale, const uint64_t* mask, void* workspace,
                                   int64_t workspace_bytes, void* stream) {
  return run_ws(fa::StoreMode::Slab, q_slabs, k_slabs, v_slabs, out_slabs, B, H, S, D, P, scale,
                mask, workspace, workspace_bytes, static_cast<hipStream_t>(stream), true);
}

int attn_fwd_plain_ws_async(const void* q, const void* k, const void* v, void* out, int B, int H,
                            int S, int D, float scale, const uint64_t* mask, void* workspace,
                            int64_t workspace_bytes, void* stream) {
  return run_ws(fa::StoreMode::Plain, q, k, v, out, B, H, S, D, 1, scale, mask, workspace,
                workspace_bytes, static_cast<hipStream_t>(stream));
}

int64_t attn_fwd_workspace_bytes(int B, int H, int S, int D) {
  if (B <= 0 || H <= 0 || S <= 0) return FA_EINVAL;
  if (D != 64 && D != 128) return FA_EUNSUPPORTED;
  if (((int64_t)S + 256) * D * 2 > (int64_t)INT32_MAX) return FA_ERANGE;
  const int64_t tiles = (int64_t)B * H * ((S + 255) / 256);
  if (tiles > (int64_t)INT32_MAX) return FA_ERANGE;
  fa::FwdParams p{};
  p.S = S;
  p.units = (int)tiles;
  DensePlan plan;
  const int st = plan_call(D, fa::StoreMode::Slab, false, p, &plan, true);
  if (st != FA_OK) return st;
  return plan.ws_bytes;
}

int attn_fwd_relayout_instrumented_async(const void* q, const void* k, const void* v,
                                         void* out_slabs, int B, int H, int S, int D, int P,
                                         float scale, const uint64_t* mask, int boundary,
                                         uint32_t* stamps, int64_t stamp_words,
                                         int* launch_units, void* stream) {
  fa::FwdParams p;
  int st = make_params(fa::StoreMode::Slab, q, k, v, out_slabs, B, H, S, D, P, scale, mask, false,
                       &p);
  if (st != FA_OK) return st;
  if (boundary < 0 || boundary > 2) return FA_EINVAL;
  if (!stamps) return FA_EINVAL;
  if (D != 128 || !(scale > 0.0f)) return FA_EUNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(stamps) & 15) return FA_EALIGN;
  if (stamp_words < attn_instrumented_stamp_words(B, H, S)) return FA_ERANGE;
  DensePlan plan;
  st = plan_call(D, fa::StoreMode::Slab, mask != nullptr, p, &plan);
  if (st != FA_OK) return st;
  p.stamps = stamps;
  if (launch_units) {
    launch_units[0] = plan.whole_units;
    launch_units[1] = plan.split_units;
  }
  return launch_call(D, fa::StoreMode::Slab, p, plan, static_cast<hipStream_t>(stream), false,
                     boundary + 1);
}

int64_t attn_instrumented_stamp_words(int B, int H, int S) {
  if (B <= 0 || H <= 0 || S <= 0) return 0;
  return (int64_t)kStampWordsPerUnit * B * H * ((S + kQTile - 1) / kQTile + 1);
}

const char* attn_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_EINVAL:
      return "invalid argument (null tensor, non-positive size, or scale not finite or beyond 2^16)";
    case FA_EDIV: return "S is not a multiple of the slab count P";
    case FA_EUNSUPPORTED:
      return "unsupported shape (D must be 64 or 128; slab inputs need S/P >= 64)";
    case FA_EALIGN: return "misaligned pointer (tensors need 16 bytes, the mask 8)";
    case FA_ERANGE: return "sizes exceed the kernel's index range";
    case FA_ELAUNCH: return "kernel launch failed";
    case FA_EDEVICE: return "no usable HIP device";
    case FA_EEXEC: return "kernel execution failed";
    default: return "unknown status";
  }
}

int attn_abi_version(void) { return FA_ABI_VERSION; }

}  // extern "C"
