// Store-burst microbenchmark for the Burst-Gap model (see include/fa_burst_gap.h).
//
// Each producer is one workgroup of four waves pinned to its own CU by its
// LDS request.  A burst is a sweep of 16-byte stores over the producer's
// share of the burst; the issue time is taken after a workgroup barrier that
// does not wait for the stores to complete (no release fence), so it is the
// sender-visible time the pages model: stores are accepted and drain while
// the producer moves on.  The gap is a dependent FMA chain whose length the
// caller sets.  Stores complete (vmcnt) only at the very end -- unless the
// caller asks for the completion-coupled form, where every wave makes its
// burst's stores visible device-wide (a release fence at device scope: L2
// write-back, then the wait for completion) before the barrier that takes
// the issue time, so a burst is only over once it has drained.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fa_relayout.h"
#include "../../include/fa_burst_gap.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kLdsBytes = 96 * 1024;   // one producer per CU
constexpr uint32_t kMagic = 0x9E3779B9u;

struct BurstGapParams {
  int producers, chunks, bursts, gap_iters, nontemporal, coupled;
};

__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(kThreads) void burst_gap_kernel(u32x4* dst, uint64_t* times,
                                                             BurstGapParams p) {
  // Unused beyond one word: its size keeps every other producer off this CU.
  __shared__ uint32_t lds_pin[kLdsBytes / 4];
  const int k = blockIdx.x, tid = threadIdx.x;
  if (tid == 0) *(volatile uint32_t*)&lds_pin[k & 1023] = (uint32_t)k;
  uint64_t* tail = times + 3ull * p.producers * p.bursts + 4ull * k;
  if (tid == 0) {
    tail[0] = __builtin_amdgcn_s_memtime();
    tail[1] = __builtin_amdgcn_s_memrealtime();
  }
  float acc = (float)tid * 1e-3f;
  for (int i = 0; i < p.bursts; ++i) {
    barrier_no_fence();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    u32x4* base = dst + ((size_t)i * p.producers + k) * p.chunks;
    if (p.nontemporal) {
      for (int c = tid; c < p.chunks; c += kThreads)
        __builtin_nontemporal_store(u32x4{(uint32_t)i, (uint32_t)k, (uint32_t)c, kMagic}, base + c);
    } else {
      for (int c = tid; c < p.chunks; c += kThreads)
        base[c] = u32x4{(uint32_t)i, (uint32_t)k, (uint32_t)c, kMagic};
    }
    // Coupled: a device-scope release -- write back the L2 and wait until
    // this wave's stores are complete, visible beyond this XCD.
    if (p.coupled) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    barrier_no_fence();   // every wave has issued (coupled: completed) its stores
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    for (int g = 0; g < p.gap_iters; ++g) {
      acc = __builtin_fmaf(acc, 0.999999f, 1e-6f);
      asm volatile("" : "+v"(acc));   // one real FMA per iteration, kept in order
    }
    barrier_no_fence();
    const uint64_t t2 = __builtin_amdgcn_s_memtime();
    if (tid == 0) {
      uint64_t* t = times + 3ull * ((size_t)k * p.bursts + i);
      t[0] = t0;
      t[1] = t1;
      t[2] = t2;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's stores completed
  __syncthreads();
  if (tid == 0) {
    tail[2] = __builtin_amdgcn_s_memtime();
    tail[3] = __builtin_amdgcn_s_memrealtime();
  }
}

}  // namespace

extern "C" int burst_gap_run_async(void* dst, uint64_t* times, int producers,
                                   int bytes_per_producer, int bursts, int gap_iters,
                                   int nontemporal, int coupled, void* stream) {
  if (!dst || !times) return FA_EINVAL;
  if (producers < 1 || producers > 4096 || bursts < 1 || bursts > 4096 || gap_iters < 0 ||
      bytes_per_producer <= 0 || bytes_per_producer % 4096 != 0 ||
      (nontemporal != 0 && nontemporal != 1) || (coupled != 0 && coupled != 1))
    return FA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(dst) & 15) || (reinterpret_cast<uintptr_t>(times) & 7))
    return FA_EALIGN;
  if ((uint64_t)bursts * producers * bytes_per_producer > (1ull << 40)) return FA_ERANGE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_EDEVICE;
  BurstGapParams p{producers, bytes_per_producer / 16, bursts, gap_iters, nontemporal, coupled};
  hipLaunchKernelGGL(burst_gap_kernel, dim3(producers), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4*>(dst), times, p);
  return hipGetLastError() == hipSuccess ? FA_OK : FA_ELAUNCH;
}
