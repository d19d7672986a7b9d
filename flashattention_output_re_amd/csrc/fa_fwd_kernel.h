// Internal interface between the C ABI layer and the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum class StoreMode : int { Slab = 0, Plain = 1 };

// Kernel arguments, passed by value.  Every tensor is bf16 stored as uint16_t.
struct FwdParams {
  const uint16_t* q;     // [B][H][S][D]
  const uint16_t* k;     // [B][H][S][D]
  const uint16_t* v;     // [B][H][S][D]
  uint16_t* out;         // slabs [P][B][S/P][H][D] or plain [B][H][S][D]
  const uint64_t* mask;  // [H][nmt][mw] keep bits, or nullptr
  int B, H, S, P, Sp;    // Sp = S / P
  int nqt;               // 128-query output tiles per (b, h)
  int units;             // B * H * nqt output tiles
  int nmt;               // 128-key mask tiles per row (= nqt)
  int mw;                // 64-bit words per mask row
  float c;               // scale * log2(e)
};

// Launch with at most `grid_cap` persistent workgroups; 0 on success.
int launch_fwd(int D, StoreMode mode, const FwdParams& p, int grid_cap, hipStream_t stream);
// Resident workgroups per CU for the instance (D, mode); 0 on success.
int kernel_occupancy(int D, StoreMode mode, int* blocks_per_cu);

}  // namespace fa
