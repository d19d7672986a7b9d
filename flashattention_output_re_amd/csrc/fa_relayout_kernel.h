// Internal interface of the standalone re-layout kernel.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct RelayoutParams {
  uint32_t B, H, S, Sp;   // Sp = S / P
  uint32_t rows;          // B * H * S output rows
};

// Enqueue the copy plain [B][H][S][D] -> slabs [P][B][S/P][H][D]; 0 on success.
int launch_relayout(int D, const void* plain, void* out, const RelayoutParams& p, int grid,
                    hipStream_t stream);
// Grid size for `rows` rows of D elements on a device with `cus` CUs.
int relayout_grid(int D, uint32_t rows, int cus);

}  // namespace fa
