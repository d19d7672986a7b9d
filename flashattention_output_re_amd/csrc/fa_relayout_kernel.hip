// Standalone head-to-sequence re-layout (the exchange half of the serial
// baseline): out_slabs[p][b][t][h][d] = plain[b][h][p * (S/P) + t][d].
//
// Pure data movement, HBM-bound: every element is read once and written
// once.  A row of D bf16 is 2D bytes contiguous in both layouts, so each
// lane moves one 16-byte chunk and a wave covers 64 / (D/8) whole rows; the
// output is walked in order (rows of consecutive heads are adjacent there),
// the input side reads whole rows at a stride of S rows per head.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_relayout_kernel.h"

namespace fa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRelayoutThreads = 256;
constexpr int kRelayoutUnroll = 4;   // chunks per thread per iteration

template <int CHUNKS>   // 16-byte chunks per row (D / 8)
__global__ __launch_bounds__(kRelayoutThreads)
void relayout_kernel(const u32x4* __restrict__ in, u32x4* __restrict__ out, RelayoutParams p) {
  const uint32_t total = p.rows * CHUNKS;   // output chunks
  const uint32_t stride = gridDim.x * kRelayoutThreads * kRelayoutUnroll;
  for (uint32_t base = blockIdx.x * kRelayoutThreads * kRelayoutUnroll + threadIdx.x; base < total;
       base += stride) {
    u32x4 v[kRelayoutUnroll];
    uint32_t dst[kRelayoutUnroll];
    bool ok[kRelayoutUnroll];
#pragma unroll
    for (int u = 0; u < kRelayoutUnroll; ++u) {
      const uint32_t i = base + u * kRelayoutThreads;
      ok[u] = i < total;
      dst[u] = i;
      if (ok[u]) {
        const uint32_t row = i / CHUNKS, c = i % CHUNKS;
        // Output row (((p * B + b) * Sp + t) * H + h).
        const uint32_t h = row % p.H;
        uint32_t r = row / p.H;
        const uint32_t t = r % p.Sp;
        r /= p.Sp;
        const uint32_t b = r % p.B;
        const uint32_t slab = r / p.B;
        const uint32_t s = slab * p.Sp + t;
        v[u] = in[((b * p.H + h) * p.S + s) * CHUNKS + c];
      }
    }
#pragma unroll
    for (int u = 0; u < kRelayoutUnroll; ++u)
      if (ok[u]) out[dst[u]] = v[u];
  }
}

int launch_relayout(int D, const void* plain, void* out, const RelayoutParams& p, int grid,
                    hipStream_t stream) {
  const u32x4* in = static_cast<const u32x4*>(plain);
  u32x4* o = static_cast<u32x4*>(out);
  if (D == 128)
    hipLaunchKernelGGL(relayout_kernel<16>, dim3(grid), dim3(kRelayoutThreads), 0, stream, in, o, p);
  else if (D == 64)
    hipLaunchKernelGGL(relayout_kernel<8>, dim3(grid), dim3(kRelayoutThreads), 0, stream, in, o, p);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int relayout_grid(int D, uint32_t rows, int cus) {
  const uint64_t chunks = (uint64_t)rows * (D / 8);
  const uint64_t per_block = (uint64_t)kRelayoutThreads * kRelayoutUnroll;
  uint64_t blocks = (chunks + per_block - 1) / per_block;
  const uint64_t cap = (uint64_t)cus * 8;   // enough resident waves to keep HBM busy
  if (blocks > cap) blocks = cap;
  return blocks < 1 ? 1 : (int)blocks;
}

}  // namespace fa
