// Internal interface between the C ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum class StoreMode : int { Slab = 0, Plain = 1 };

// Forms of the kernel (8 waves, one workgroup per CU).  Whole: 256-query
// tiles, the two wave groups holding 128 queries each and sharing one K/V
// stream (dense attention).  Split: one 128-query half of a 256-query tile,
// its keys split between the two groups (the last, partial round of a dense
// launch).  Masked: the split form on 128-query tiles, one mask row each,
// each group streaming half of the row's kept 128-key tiles.
enum class Variant : int { Whole = 0, Split = 1, Masked = 2 };
constexpr int tile_rows(Variant v) { return v == Variant::Masked ? 128 : 256; }

// Kernel arguments, passed by value.  Every tensor is bf16 stored as uint16_t.
struct FwdParams {
  const uint16_t* q;     // [B][H][S][D]
  const uint16_t* k;     // [B][H][S][D]
  const uint16_t* v;     // [B][H][S][D]
  uint16_t* out;         // slabs [P][B][S/P][H][D] or plain [B][H][S][D]
  const uint64_t* mask;  // [H][nmt][mw] keep bits, or nullptr
  int B, H, S, P, Sp;    // Sp = S / P
  int nqt;               // output tiles (tile_rows queries) per (b, h)
  int units;             // work units of this launch (see unit_base)
  int unit_base;         // Split: unit u is half u % 2 of tile unit_base + u / 2
                         // (Whole, Masked: unit u is tile u)
  int nmt;               // 128-key mask tiles per row (= nqt)
  int mw;                // 64-bit words per mask row
  float c;               // scale * log2(e)
  // Slab-layout inputs only: n / Sp = (umulhi(n, sp_magic) + n) >> sp_shift
  // for n < 2^31.
  uint32_t sp_magic;
  int sp_shift;
  // Instrumented launches only: per-unit timestamp records (8 uint32 per
  // unit and wave), else nullptr.
  uint32_t* stamps;
  // Whole form only: the tail round, the next `tail` tiles after the
  // launch's `units` whole units, each split at stage tail_len < ns (ns =
  // ceil(S / 64)): workgroup slot i < tail runs tile i's stages [0,
  // tail_len), the other slots equal slices of tail_hlen stages of the tiles'
  // ends taken one after another.  Partial results go to ws (seg_floats(D)
  // floats per slot, tail + grid - 1 slots) and fa_merge_kernel stores those
  // tiles.  tail = 0: no tail round.
  int tail, tail_len, tail_hlen;
  float* ws;
  // Split form only: when > 1, each half tile is cut into split_pieces
  // pieces of its key stages, unit u being piece u % split_pieces of half
  // unit_base * 2 + u / split_pieces; the pieces' partial results go to ws
  // slot u and fa_merge_split_kernel stores the half tiles.
  int split_pieces;
  // Whole form only: a dynamic schedule when queue != nullptr -- items 0 ..
  // units - 1 are whole units and items units + i the pieces of the `tail`
  // tiles after them, each cut into P = dyn_pieces pieces, piece j holding
  // the share (P - j) / (P (P + 1) / 2) of the key stages (piece i / tail of
  // tile units + i % tail, partial result to ws slot (i % tail) P + i /
  // tail); on a grid of G, workgroup slot s runs
  // items s, s + G, ... below R = (units / G) G, then items R + q, q the old
  // values of the counter *queue (zero at launch), one atomic add per item.
  // fa_merge_kernel stores the tail tiles.
  int* queue;
  int dyn_pieces;
};

// Workspace slot of one tail segment, in floats: per wave (8) and lane (64)
// the O^T accumulator divided by the row sum, as D / 8 quads of floats
// ([wave][quad][lane][4]), then per wave and lane {running max, row sum, 0,
// 0} from seg_ml_offset(D) on.
constexpr int seg_ml_offset(int D) { return 8 * (D / 8) * 64 * 4; }
constexpr int seg_floats(int D) { return seg_ml_offset(D) + 8 * 64 * 4; }

// Launch with at most `grid_cap` persistent workgroups; 0 on success.
// slab_in: q, k, v are [P][B][S/P][H][D] (sequence-sharded) instead of
// [B][H][S][D]; only with StoreMode::Slab.  instr: 0 for the product
// kernels; for the timestamped instances (D = 128, slab output, c > 0,
// [B][H][S][D] inputs, p.stamps set) the tile boundary: 1 piggybacked (as
// the product kernels), 2 completion-coupled, 3 stores then prologue with
// one wait for both.
int launch_fwd(int D, StoreMode mode, Variant var, const FwdParams& p, int grid_cap,
               hipStream_t stream, bool slab_in = false, int instr = 0);
// The merge kernel of a call's tail round (p.tail tiles, p.ws), on the
// stream after the whole-form launch that wrote the partials; 0 on success.
int launch_merge(int D, StoreMode mode, const FwdParams& p, hipStream_t stream);
// The merge of a split launch cut into pieces (p.split_pieces > 1, p.units
// pieces, p.ws), on the stream after that launch; 0 on success.
int launch_merge_split(int D, StoreMode mode, const FwdParams& p, hipStream_t stream);
// Zeroes a dynamic schedule's counter, on the stream before its launch.
int launch_queue_reset(int* queue, hipStream_t stream);
// Resident workgroups per CU for the instance (D, mode, var); 0 on success.
int kernel_occupancy(int D, StoreMode mode, Variant var, int* blocks_per_cu);

}  // namespace fa
