// Fused FlashAttention forward + Ulysses slab store for gfx950 (MI355X).
//
// One persistent workgroup of 4 wavefronts owns a 128-query output tile of one
// (batch, head): it streams the K/V tiles of the whole sequence through LDS,
// runs QK^T and PV on the bf16 MFMA units with an fp32 online softmax, and in
// the epilogue stores the finished tile straight into the P destination slabs
// of the head-to-sequence re-layout, then moves on to its next output tile
// without waiting for those stores ("Technical Summary: X-Stage in DiT
// Inference", Key Contributions 3: the output-tile owner issues the stores and
// resumes the next tile's Q-loop; no dedicated communication wavefront).  The
// same kernel body with StoreMode::Plain writes [B][H][S][D] instead.
//
// Layout choices (all per wavefront, 32 queries):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims of K from
//   LDS, B = 16 dims x 32 queries of Q kept in VGPRs.  The accumulator puts one
//   query per lane (lane % 32) and 16 keys per lane, so a row's max and sum are
//   lane-local except for one exchange between the two wave halves
//   (v_permlane32_swap).
//   O^T = V^T P^T: the S^T accumulator, rounded to bf16, is directly the B
//   operand (same query per lane, keys as the contraction index).  The A
//   operand needs V transposed; V is written to LDS as V^T with the keys of
//   each 16-key group permuted so that one ds_read_b128 yields exactly the 8
//   keys a lane's half of the wave contributes to the contraction.
//   The O^T accumulator again holds one query per lane; one permlane32 swap
//   turns its 4-wide d runs into 8 consecutive d, so the epilogue issues
//   128-bit stores.
//
// Softmax runs in the log2 domain (c = scale * log2 e, p = exp2(s c - m)).
// The running max is only raised when a row's new max exceeds it by more than
// kTau (2^8 headroom for p); the final division by the row sum makes the
// result independent of which max was used.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_kernel.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int BM = 128;          // queries per output tile (= mask tile)
constexpr int BN = 64;           // keys per LDS stage
constexpr float kTau = 8.0f;     // lazy-rescale threshold, log2 units
constexpr uint32_t kBufFlags = 0x00020000u;  // raw buffer, 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           (int)kBufFlags);
}

// 16 bytes at byte offset `off`; offsets past the resource's size read as 0.
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// Exchange between the two halves of the wavefront.  With inputs a, b the
// results are lo = [a_lanes0-31, b_lanes0-31], hi = [a_lanes32-63, b_lanes32-63].
struct Pair { uint32_t lo, hi; };
__device__ __forceinline__ Pair swap_halves(uint32_t a, uint32_t b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  return Pair{(uint32_t)r[0], (uint32_t)r[1]};
}
__device__ __forceinline__ float halves_max(float x) {
  Pair p = swap_halves(f2u(x), f2u(x));
  return fmaxf(u2f(p.lo), u2f(p.hi));
}
__device__ __forceinline__ float halves_min(float x) {
  Pair p = swap_halves(f2u(x), f2u(x));
  return fminf(u2f(p.lo), u2f(p.hi));
}
__device__ __forceinline__ float halves_sum(float x) {
  Pair p = swap_halves(f2u(x), f2u(x));
  return u2f(p.lo) + u2f(p.hi);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Position of key j (0..15 within its 16-key group) in the V^T LDS row: the
// middle two 4-key blocks trade places, so that positions 8g..8g+7 hold the
// keys {0-3, 8-11} (g = 0) and {4-7, 12-15} (g = 1) the MFMA B operand uses.
__device__ __forceinline__ int vt_pos_of_quad(int quad16) {   // quad16 = (j % 16) / 4
  return (quad16 == 1) ? 2 : (quad16 == 2) ? 1 : quad16;
}
// XOR swizzle of the 16-byte chunks of a V^T row (8 chunks per 64-key row).
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 3) ^ d) & 7; }

template <int D>
struct Smem {
  static constexpr int KROW = D + 8;                 // padded K row, elements
  static constexpr int K_ELEMS = BN * KROW;
  static constexpr int V_ELEMS = D * BN;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int BYTES = 2 * STAGE * 2;        // double buffered, bf16
};

template <int D>
struct Stage {
  static constexpr int KCH = D / 8;                                  // 16 B chunks per row
  static constexpr int K_PER_T = BN * KCH / kThreads;                // K chunks per thread
  static constexpr int V_GROUPS = (BN / 4) * KCH;                    // 4 rows x 16 B groups
  u32x4 k[K_PER_T];
  u32x4 v[4];
};

template <int D>
__device__ __forceinline__ void stage_load(Stage<D>& st, __amdgpu_buffer_rsrc_t rk,
                                           __amdgpu_buffer_rsrc_t rv, int key0, int tid) {
  constexpr int KCH = Stage<D>::KCH;
#pragma unroll
  for (int i = 0; i < Stage<D>::K_PER_T; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / KCH, ch = idx % KCH;
    st.k[i] = load16(rk, (uint32_t)((key0 + row) * D * 2 + ch * 16));
  }
  if (Stage<D>::V_GROUPS >= kThreads || tid < Stage<D>::V_GROUPS) {
    const int ch = tid % KCH, quad = tid / KCH;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      st.v[r] = load16(rv, (uint32_t)((key0 + 4 * quad + r) * D * 2 + ch * 16));
  }
}

template <int D>
__device__ __forceinline__ void stage_store(const Stage<D>& st, uint16_t* ks, uint16_t* vt,
                                            int tid) {
  constexpr int KCH = Stage<D>::KCH;
  constexpr int KROW = Smem<D>::KROW;
#pragma unroll
  for (int i = 0; i < Stage<D>::K_PER_T; ++i) {
    const int idx = tid + kThreads * i;
    const int row = idx / KCH, ch = idx % KCH;
    *reinterpret_cast<u32x4*>(ks + row * KROW + ch * 8) = st.k[i];
  }
  if (Stage<D>::V_GROUPS >= kThreads || tid < Stage<D>::V_GROUPS) {
    const int ch = tid % KCH, quad = tid / KCH;
    const int pos = 16 * (quad >> 2) + 4 * vt_pos_of_quad(quad & 3);   // key position of row 4*quad
    const int chunk = pos >> 3, half = pos & 7;                        // 16 B chunk, element offset
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int par = 0; par < 2; ++par) {
        const int d = 8 * ch + 2 * w + par;
        const uint32_t e0 = par ? (st.v[0][w] >> 16) : (st.v[0][w] & 0xffffu);
        const uint32_t e1 = par ? (st.v[1][w] >> 16) : (st.v[1][w] & 0xffffu);
        const uint32_t e2 = par ? (st.v[2][w] >> 16) : (st.v[2][w] & 0xffffu);
        const uint32_t e3 = par ? (st.v[3][w] >> 16) : (st.v[3][w] & 0xffffu);
        u32x2 val = {e0 | (e1 << 16), e2 | (e3 << 16)};
        uint16_t* row = vt + d * BN;
        *reinterpret_cast<u32x2*>(row + ((chunk ^ vt_swz(d)) << 3) + half) = val;
      }
    }
  }
}

// Iterates the K/V stages (BN keys each) a query tile attends to: all stages
// for dense attention, or the stages of the kept 128-key mask tiles.
struct StageIter {
  const uint64_t* row;   // mask row (nullptr = dense)
  int S, nmt, mw;
  __device__ int first() const {
    if (!row) return 0;
    return next_tile(0);
  }
  __device__ int next_tile(int mt) const {             // first kept mask tile >= mt, as a stage
    if (mt >= nmt) return -1;
    int w = mt >> 6;
    uint64_t bits = row[w] & (~0ull << (mt & 63));
    while (bits == 0) {
      if (++w >= mw) return -1;
      bits = row[w];
    }
    const int t = (w << 6) + __builtin_ctzll(bits);
    return t < nmt ? 2 * t : -1;
  }
  __device__ int next(int st) const {
    const int nx = st + 1;
    if (nx * BN >= S) return -1;
    if (!row || (nx & 1)) return nx;                   // dense, or the second half of a mask tile
    return next_tile(nx >> 1);
  }
};

template <int D, StoreMode MODE>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(FwdParams p) {
  constexpr int NKS = D / 16;     // QK^T contraction steps
  constexpr int NDB = D / 32;     // 32-dim blocks of O^T
  constexpr int KROW = Smem<D>::KROW;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * Smem<D>::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const float c = p.c;
  const uint32_t head_bytes = (uint32_t)p.S * D * 2;

  for (int unit = blockIdx.x; unit < p.units; unit += gridDim.x) {
    const int bh = unit / p.nqt, qt = unit - bh * p.nqt;
    const int b = bh / p.H, h = bh - b * p.H;
    const size_t head_off = (size_t)bh * p.S * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + head_off, head_bytes);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + head_off, head_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + head_off, head_bytes);

    // This lane's query and its B operand of S^T = K Q^T (8 dims per step).
    const int qrow = qt * BM + wave * 32 + l32;
    bf16x8 qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, load16(rq, (uint32_t)(qrow * D * 2 + ks * 32 + g * 16)));

    f32x16 acc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
    float m_run = -__builtin_inff();
    float l_run = 0.0f;

    StageIter it{p.mask ? p.mask + ((size_t)h * p.nmt + qt) * p.mw : nullptr, p.S, p.nmt, p.mw};
    int st = it.first();
    Stage<D> regs;
    if (st >= 0) {
      stage_load<D>(regs, rk, rv, st * BN, tid);
      stage_store<D>(regs, smem, smem + Smem<D>::K_ELEMS, tid);
    }
    __syncthreads();
    int buf = 0;
    while (st >= 0) {
      const int nx = it.next(st);
      if (nx >= 0) stage_load<D>(regs, rk, rv, nx * BN, tid);
      const uint16_t* ks_lds = smem + buf * Smem<D>::STAGE;
      const uint16_t* vt_lds = ks_lds + Smem<D>::K_ELEMS;

      // ---- S^T = K Q^T: two 32-key blocks.
      f32x16 s[2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        s[mb] = f32x16{};
        const uint16_t* krow = ks_lds + (32 * mb + l32) * KROW + g * 8;
#pragma unroll
        for (int kk = 0; kk < NKS; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + kk * 16);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], s[mb], 0, 0, 0);
        }
      }

      // ---- online softmax for this lane's query over its 32 keys of the stage.
      const bool tail = (st + 1) * BN > p.S;
      const int key0 = st * BN + 4 * g;
      if (tail) {
        const float fill = (c >= 0.0f) ? -__builtin_inff() : __builtin_inff();
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key0 + 32 * mb + 8 * (r >> 2) + (r & 3) >= p.S) s[mb][r] = fill;
      }
      float ext;
      if (c >= 0.0f) {
        ext = fmaxf(s[0][0], s[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) ext = fmaxf(ext, fmaxf(s[0][r], s[1][r]));
        ext = halves_max(ext);
      } else {
        ext = fminf(s[0][0], s[1][0]);
#pragma unroll
        for (int r = 1; r < 16; ++r) ext = fminf(ext, fminf(s[0][r], s[1][r]));
        ext = halves_min(ext);
      }
      const float m_new = fmaxf(m_run, ext * c);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run + kTau) != 0) {
        const float alpha = exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
      }
      bf16x8 pb[4];
      float lsum = 0.0f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = exp2f(__builtin_fmaf(s[mb][r], c, -m_run));
          if (tail && key0 + 32 * mb + 8 * (r >> 2) + (r & 3) >= p.S) x = 0.0f;
          lsum += x;
          pb[2 * mb + (r >> 3)][r & 7] = (__bf16)x;
        }
      }
      l_run += lsum;

      // ---- O^T += V^T P^T: four 16-key steps per 32-dim block.
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = 32 * db + l32;
        const uint16_t* vrow = vt_lds + d * BN;
        const int sw = vt_swz(d);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + (((2 * kk + g) ^ sw) << 3));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk], acc[db], 0, 0, 0);
        }
      }

      if (nx >= 0)
        stage_store<D>(regs, smem + (buf ^ 1) * Smem<D>::STAGE,
                       smem + (buf ^ 1) * Smem<D>::STAGE + Smem<D>::K_ELEMS, tid);
      __syncthreads();
      buf ^= 1;
      st = nx;
    }

    // ---- epilogue: normalise, round to bf16, store 8 consecutive dims per lane.
    const float l_tot = halves_sum(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (qrow < p.S) {
      size_t row_off;
      if (MODE == StoreMode::Slab) {
        const int slab = qrow / p.Sp, t = qrow - slab * p.Sp;
        row_off = (((size_t)slab * p.B + b) * p.Sp + t) * p.H + h;
      } else {
        row_off = (size_t)bh * p.S + qrow;
      }
      uint16_t* dst = p.out + row_off * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int r0 = 8 * hf;
          const uint32_t a0 = pack_bf16(acc[db][r0 + 0] * inv, acc[db][r0 + 1] * inv);
          const uint32_t a1 = pack_bf16(acc[db][r0 + 2] * inv, acc[db][r0 + 3] * inv);
          const uint32_t b0 = pack_bf16(acc[db][r0 + 4] * inv, acc[db][r0 + 5] * inv);
          const uint32_t b1 = pack_bf16(acc[db][r0 + 6] * inv, acc[db][r0 + 7] * inv);
          const Pair x = swap_halves(a0, b0);
          const Pair y = swap_halves(a1, b1);
          const u32x4 val = {x.lo, y.lo, x.hi, y.hi};
          *reinterpret_cast<u32x4*>(dst + 32 * db + 16 * hf + 8 * g) = val;
        }
      }
    }
  }
}

template <int D, StoreMode MODE>
static int launch_one(const FwdParams& p, int grid_cap, hipStream_t stream) {
  const int grid = p.units < grid_cap ? p.units : grid_cap;
  hipLaunchKernelGGL((fa_fwd_kernel<D, MODE>), dim3(grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int D, StoreMode MODE>
static int occupancy_one(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, fa_fwd_kernel<D, MODE>, kThreads, 0)
                 == hipSuccess ? 0 : -1;
}

int kernel_occupancy(int D, StoreMode mode, int* blocks_per_cu) {
  if (D == 128) return mode == StoreMode::Slab ? occupancy_one<128, StoreMode::Slab>(blocks_per_cu)
                                               : occupancy_one<128, StoreMode::Plain>(blocks_per_cu);
  if (D == 64) return mode == StoreMode::Slab ? occupancy_one<64, StoreMode::Slab>(blocks_per_cu)
                                              : occupancy_one<64, StoreMode::Plain>(blocks_per_cu);
  return -1;
}

int launch_fwd(int D, StoreMode mode, const FwdParams& p, int grid_cap, hipStream_t stream) {
  if (D == 128) return mode == StoreMode::Slab ? launch_one<128, StoreMode::Slab>(p, grid_cap, stream)
                                               : launch_one<128, StoreMode::Plain>(p, grid_cap, stream);
  if (D == 64) return mode == StoreMode::Slab ? launch_one<64, StoreMode::Slab>(p, grid_cap, stream)
                                              : launch_one<64, StoreMode::Plain>(p, grid_cap, stream);
  return -1;
}

}  // namespace fa
