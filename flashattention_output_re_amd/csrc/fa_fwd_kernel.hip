// Fused FlashAttention forward + Ulysses slab store for gfx950 (MI355X).
//
// Persistent workgroups own output tiles of one (batch, head) at a time: they
// stream the K/V tiles of the whole sequence through LDS, run QK^T and PV on
// the bf16 MFMA units with an fp32 online softmax, and in the epilogue issue
// the next tile's first loads, then store the finished tile straight into the
// P destination slabs of the head-to-sequence re-layout, and start the next
// tile's Q-loop while those stores drain: the wait before it covers only the
// loads ("Technical Summary: X-Stage in DiT Inference", Key Contributions 3:
// the output-tile owner issues the stores and resumes the next tile's Q-loop;
// no dedicated communication wavefront).  The kernel's header comment below
// ("Tile boundary") gives the counter argument.
// StoreMode::Plain runs the same body but writes [B][H][S][D].
//
// One kernel, fa_fwd_pp_kernel: 8 waves, one workgroup per CU, softmax and
// MFMA work in separate regions run by two wave groups in alternation (its
// own header comment below has the schedule), in three forms: whole
// 256-query tiles (dense), split-key 128-query half tiles (the last, partial
// round of a dense launch, whole or in pieces of their keys) and split-key
// 128-query tiles over the kept tiles of one mask row (block-sparse).
//
// Layout choices (per wavefront, 32 queries):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims of K from
//   LDS, B = 16 dims x 32 queries of Q held in VGPRs.  The accumulator puts one
//   query per lane (lane % 32) and 16 keys per lane, so a row's max and sum are
//   lane-local apart from one exchange between the wave halves
//   (v_permlane32_swap).
//   O^T = V^T P^T: the S^T accumulator, rounded to bf16, is directly the B
//   operand (same query per lane, keys as the contraction index).  V stays
//   row-major in LDS; the A operand comes from two ds_read_b64_tr_b16 per MFMA
//   whose row addresses put the keys in the accumulator's order.
//   The O^T accumulator again holds one query per lane; one permlane32 swap
//   turns its 4-wide runs of d into 8 consecutive d, so the epilogue issues
//   128-bit stores.
//   K/V stages reach LDS by buffer_load ... lds DMA with XOR-swizzled 16-byte
//   chunks (conflict-free operand reads).
//
// Softmax runs in the log2 domain (c = scale * log2 e, p = exp2(s c - m)).
// The probabilities are first taken against the running max as it stands; it
// is only raised, and the stage recomputed, when some lane's sum over the
// stage passes kRaise = 2^8.  So no probability exceeds 2^8, and a key that
// comes to dominate its row is re-centred to weigh 1: exactly 2^e with e the
// rounding error of its product s c (the max is that rounded product, the
// probability an fma), which rounds to 1 in bf16 while |s c| < 2^16.  The
// final division by the row sum makes the result independent of which max
// was used, the factor 2^e included.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_fwd_kernel.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128;          // rows of a mask tile (queries and keys); masked unit size
constexpr int BN = 64;           // keys per LDS stage
// Rounds of a masked launch's schedule a workgroup can hold (plain order
// beyond).
constexpr int kPlanMaxRounds = 256;
constexpr float kRaise = 256.0f;   // a lane's stage sum that raises the running max

// Tuning knob, overridable at build time (-D): operand reads issued ahead of
// their MFMA in the MFMA region.
#ifndef FA_MLEAD
#define FA_MLEAD 3
#endif
constexpr uint32_t kBufFlags = 0x00020000u;  // raw buffer, 32-bit data format

// Lambdas of the kernel body are always inlined: one that became a call
// would take its captures by address, and the unit's buffer resources would
// then be reloaded from private memory into vector registers.
#define FA_INL __attribute__((always_inline))


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

// K and V stages live in LDS row-major (one key per row, D bf16 = D/8 16-byte
// chunks), filled straight from global memory by buffer_load ... lds (lane l
// of a wave instruction writes the 16 bytes at M0 + 16 l).  Chunk c of row r
// sits at chunk position c ^ swz(r), which keeps the MFMA operand reads free
// of bank conflicts.
template <int D> struct Tile {
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int ELEMS = BN * D;               // bf16 per stage
};
// LDS: 64 banks of 4 bytes; a ds_read_b128 serves 16 lanes per pass, a
// ds_read_b64(_tr) 32.  A row of D = 128 (256 bytes) starts at bank 0, one of
// D = 64 (128 bytes) at bank 0 or 32 by the row's parity.
// K rows are read 16 at a time (lanes 0-15: rows r0 .. r0 + 15) at one
// logical chunk: D = 128 XORs the chunk with r % 16, giving 16 distinct
// 16-byte positions; D = 64 with (r / 2) % 8, distinct within each parity
// (which picks the half of the banks).
template <int D> __device__ __forceinline__ int k_swz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
// V is read by ds_read_b64_tr_b16: per 32 lanes, rows r0 .. r0 + 3 (r0 a
// multiple of 4) at 4 consecutive logical chunks each; the 4 rows' 64-byte
// runs must cover all 64 banks.  D = 128: XOR the chunk with 4 (r % 4);
// D = 64: rows of one parity share a bank half, so XOR with 4 ((r / 2) % 2).
template <int D> __device__ __forceinline__ int v_swz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}

// LDS-DMA instructions (1 KiB each) that each of four waves issues to move
// one K or V stage of BN keys.
template <int D> struct Dma {
  static constexpr int PER_WAVE4 = BN * Tile<D>::CH / (4 * 64);
};

// N consecutive 1 KB blocks of a K or V stage into LDS from `dst` on:
// instruction i moves 16 bytes per lane from byte offset base + off[i] of r
// into dst + 1024 i + 16 lane (the instruction offset, 1024 i, adds to both
// addresses, so it is taken out of the global one).  Written as inline
// assembly so that the compiler, which cannot see that it writes LDS, does
// not guard later LDS reads with waits of its own: the caller waits for the
// data (vmcnt) and synchronises the workgroup before any wave reads it.
// M0 is named as clobbered on purpose: the sequence writes it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int N>
__device__ __forceinline__ void dma_blocks(uint16_t* dst, __amdgpu_buffer_rsrc_t r, uint32_t base,
                                           const uint32_t* off) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)dst);
  static_assert(N == 1 || N == 2 || N == 4, "block count");
  if constexpr (N == 4) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
        "buffer_load_dwordx4 %2, %5, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds"
        :
        : "s"(lds), "v"(base + off[0]), "v"(base - 1024 + off[1]), "v"(base - 2048 + off[2]),
          "v"(base - 3072 + off[3]), "s"(r)
        : "memory", "m0");
  } else if constexpr (N == 2) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen lds\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen offset:1024 lds"
        :
        : "s"(lds), "v"(base + off[0]), "v"(base - 1024 + off[1]), "s"(r)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds), "v"(base + off[0]), "s"(r)
        : "memory", "m0");
  }
}
// One such instruction on its own: 16 bytes per lane from byte offset `addr`
// of r into LDS byte address lds + 16 lane.
__device__ __forceinline__ void dma_one(uint32_t lds, __amdgpu_buffer_rsrc_t r, uint32_t addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds), "v"(addr), "s"(r)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// A wave's share of one K or V stage as N single instructions that can be
// issued apart: instruction i moves the 1 KB block at LDS byte address
// lds + 1024 i from the lane offsets addr[i].
template <int N>
struct DmaPlan {
  uint32_t lds;
  __amdgpu_buffer_rsrc_t r;
  uint32_t addr[N];
  __device__ __forceinline__ void issue(int i) const { dma_one(lds + 1024u * i, r, addr[i]); }
};

// Byte offset, from the stage's first key, that lane `lane` of wave `wave`
// (of four) reads in DMA instruction q of a K (SWZ_V = false) or V stage.
template <int D, bool SWZ_V>
__device__ __forceinline__ uint32_t dma_lane_off(int wave, int lane, int q) {
  constexpr int CH = Tile<D>::CH;
  const int blk = Dma<D>::PER_WAVE4 * wave + q;
  const int pos = 64 * blk + lane;
  const int row = pos / CH, pc = pos % CH;
  const int lc = pc ^ (SWZ_V ? v_swz<D>(row) : k_swz<D>(row));
  return (uint32_t)(row * D * 2 + lc * 16);
}

__device__ __forceinline__ void wait_dma() {
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's LDS DMA has landed
}

// Wait until every LDS read and write of this wave has completed (lgkmcnt(0);
// vmcnt and expcnt not waited for).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Wait until at most N of this wave's vector memory operations are in flight
// (vmcnt(N); expcnt and lgkmcnt not waited for).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier without the release/acquire fence of __syncthreads(): the
// fence would wait for every LDS DMA still in flight.  Every LDS read issued
// before it has been consumed by then (the MFMAs that use them precede it);
// the empty asm statements keep the compiler from moving memory operations
// across it.
__device__ __forceinline__ void barrier_keep_dma() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// XCD-aware order of a persistent grid of G workgroups.  Workgroups are dealt
// to the 8 XCDs round-robin by id, so with this slot number XCD x takes, in
// each round of G units, the G / 8 consecutive units from x * G / 8 on (tiles
// of one head, whose K/V stream its L2 then fetches once) rather than every
// 8th unit.  A bijection on [0, G); the identity when G is not a multiple of 8.
__device__ __forceinline__ int xcd_slot(int block, int G) {
  return (G % 8 == 0) ? (block % 8) * (G / 8) + block / 8 : block;
}

// The 64-key stages of one mask row's kept 128-key tiles, in key order (two
// stages per tile), as one of two streams: stream 0 takes the first half of
// the row's 2K stages, stream 1 the second.  next() gives the first key of
// the stream's next stage, or S once the stream's K stages are used up.  Bits
// for tiles past the row's end are ignored.  All state is wave-uniform.
// The mask words are read through the constant address space, which makes
// them scalar loads: their wait (lgkmcnt) leaves the stream's K/V DMA in
// flight, where a vector load's vmcnt(0) would wait for all of it.
typedef const __attribute__((address_space(4))) uint64_t* mask_row_t;
struct KeptStages {
  mask_row_t row;
  int mw, w, half, left, S;
  uint64_t bits, last_mask;

  __device__ uint64_t word(int i) const { return i == mw - 1 ? row[i] & last_mask : row[i]; }

  // Positions the stream; returns K, the number of kept tiles in the row.
  __device__ int init(const uint64_t* r, int nmt, int words, int seq, int stream) {
    row = (mask_row_t)r;
    mw = words;
    S = seq;
    last_mask = (nmt & 63) ? (1ull << (nmt & 63)) - 1 : ~0ull;
    int kept = 0;
    for (int i = 0; i < mw; ++i) kept += __builtin_popcountll(word(i));
    // Stream 1 starts at stage K: skip K / 2 tiles and, for odd K, the first
    // half of the next one.
    int skip = stream ? kept >> 1 : 0;
    w = 0;
    bits = word(0);
    while (skip >= __builtin_popcountll(bits) && skip > 0) {
      skip -= __builtin_popcountll(bits);
      bits = word(++w);
    }
    for (; skip > 0; --skip) bits &= bits - 1;
    half = stream ? (kept & 1) : 0;
    left = kept;
    return kept;
  }

  __device__ int next() {
    if (left <= 0) return S;
    --left;
    while (bits == 0) bits = word(++w);
    const int key = ((w << 6) + __builtin_ctzll(bits)) * BM + half * BN;
    if (half) bits &= bits - 1;
    half ^= 1;
    return key;
  }
};

// A operand of S^T = K Q^T: keys 32 mb + (lane % 32), dims 16 kk + 8 (lane / 32) + [0, 8).
template <int D>
__device__ __forceinline__ bf16x8 k_operand(const uint16_t* kbuf, int mb, int kk, int l32, int g) {
  // Row 32 mb + l32 has the swizzle of row l32 (the swizzle masks fewer than 5 bits).
  const int r = 32 * mb + l32;
  return *reinterpret_cast<const bf16x8*>(kbuf + r * D + 8 * ((2 * kk + g) ^ k_swz<D>(l32)));
}

// A operand of O^T = V^T P^T for 16-key step kk and 32-dim block db: lane l
// holds dim 32 db + l % 32 at the keys 16 kk + {0-3, 8-11} (l < 32) or
// {4-7, 12-15} (l >= 32), the key order of the S^T accumulator.  Each
// transposing read gives a lane 4 keys of one dim; within 16 lanes, lane j
// points at key 4 (j / 16...)-relative row j / 4 and dims 4 (j % 4) + [0, 4).
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const uint16_t* vbuf, int kk, int db, int lane) {
  const int j = lane & 15, grp = lane >> 4;
  // Rows 16 kk + 8 half + lrow; every term but lrow is a multiple of 4, so the
  // row's swizzle is that of lrow.  The dims 32 db + 16 (grp & 1) + 4 (j & 3)
  // sit in chunk 4 db + c0 (c0 < 4) at element 4 (j & 1); the swizzle flips
  // only the db bits of the chunk, so each db has one per-lane offset and
  // kk and half add constants.
  const int lrow = 4 * (grp >> 1) + (j >> 2);
  const int c0 = 2 * (grp & 1) + ((j & 3) >> 1);
  const int col = 8 * ((4 * db + c0) ^ v_swz<D>(lrow)) + 4 * (j & 1);
  s16x4 h[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
    h[half] = lds_read_tr(vbuf + (16 * kk + 8 * half) * D + lrow * D + col);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
  return __builtin_bit_cast(bf16x8, v);
}

// S^T (two 32-key blocks x 32 queries) = K_stage Q^T.
template <int D>
__device__ __forceinline__ void qk_mfma(f32x16 (&s)[2], const uint16_t* ks,
                                        const bf16x8 (&qf)[D / 16], int l32, int g) {
  constexpr int NKS = D / 16;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    s[mb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk)
      s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand<D>(ks, mb, kk, l32, g), qf[kk],
                                                      s[mb], 0, 0, 0);
  }
}

// Online softmax of one K/V stage as one block of VALU work, run in a region
// of its own beside another wave's MFMAs.  This lane holds 32 scores of its
// query (two 32-key blocks x 16).  All 32 probabilities exp2(s c - m) as
// bf16 pairs (the B operand of the PV MFMAs) and their sum over four partial
// chains, against the running max m as it stands: no row extreme stands
// between the scores and the exponentials.  Only when some lane's sum passes
// kRaise (or is infinite, as at the first stage) does the wave take the
// row extreme (max for c > 0, min for c < 0), raise m to it and recompute
// the stage from the scores, which stay in sc.
template <bool NEG>
struct StageProbs {
  float alpha = 1.0f;
  bool rescale = false;
  uint32_t pk[16];

  // With SPREAD, issue(j), j = 0..3, issues this wave's share of the
  // region's LDS DMA at four points spread over the VALU work, so that the
  // waves of a group do not all queue their DMA instructions at the region's
  // start (split-key units, which move two stages per region).
  template <bool SPREAD, class Issue>
  __device__ __forceinline__ void compute(f32x16 (&sc)[2], float c, float& m_run, float& l_run,
                                          const Issue& issue) {
    auto point = [&](int j) {
      if constexpr (SPREAD) {
        __builtin_amdgcn_sched_barrier(0);
        issue(j);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    point(0);
    // The probabilities of the stage against a max m, as bf16 pairs in pk,
    // and their sum over four partial chains.
    auto probs = [&](float m, bool points) {
      const float neg_m = -m;
      float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int pi = 0; pi < 8; ++pi) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mb][2 * pi], c, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[mb][2 * pi + 1], c, neg_m));
          ls[(2 * pi) & 3] += p0;
          ls[(2 * pi + 1) & 3] += p1;
          pk[8 * mb + pi] = pack_bf16(p0, p1);
          if (points && mb == 0 && pi == 3) point(1);
        }
        if (points) point(2 + mb);
      }
      return (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };
    // First against the running max as it stands; only when some lane's sum
    // passes kRaise (or overflows) is the max raised to the row's extreme and
    // the stage recomputed (the scores are still in sc).
    float l_stage = probs(m_run, true);
    rescale = __builtin_amdgcn_ballot_w64(l_stage > kRaise) != 0;
    // Rare: laid out of line, so the common path takes no branch.
    if (__builtin_expect(rescale, 0)) {
      float e[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int mb = k >> 1, r0 = 8 * (k & 1);
        float x = sc[mb][r0];
#pragma unroll
        for (int r = 1; r < 8; ++r) x = NEG ? fminf(x, sc[mb][r0 + r]) : fmaxf(x, sc[mb][r0 + r]);
        e[k] = x;
      }
      float ex = NEG ? fminf(fminf(e[0], e[1]), fminf(e[2], e[3]))
                     : fmaxf(fmaxf(e[0], e[1]), fmaxf(e[2], e[3]));
      ex = NEG ? halves_min(ex) : halves_max(ex);
      const float m_new = fmaxf(m_run, ex * c);
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_stage = probs(m_new, false);
      l_run = l_run * alpha + l_stage;
    } else {
      l_run += l_stage;
    }
    // Keep all of it in the softmax region: without these uses the compiler
    // sinks the exponentials past the barrier into the MFMA region.
#pragma unroll
    for (int pi = 0; pi < 16; ++pi) asm volatile("" ::"v"(pk[pi]));
    asm volatile("" ::"v"(l_run), "v"(alpha));
  }

  // B operand of the PV MFMA over 16-key step kk.
  __device__ __forceinline__ bf16x8 p_operand(int kk) const {
    return __builtin_bit_cast(bf16x8, u32x4{pk[4 * kk], pk[4 * kk + 1], pk[4 * kk + 2], pk[4 * kk + 3]});
  }
};

// Keys >= S of a ragged last stage do not exist: their scores become fill
// (fill * c = -inf).  Lane (l32, g) holds keys 32 mb + 8 (r / 4) + 4 g + r % 4.
__device__ __forceinline__ void mask_tail(f32x16 (&sc)[2], int stage_key0, int S, int g, float fill) {
  // The common case first: the tail code is laid out of line, so a full
  // stage takes no branch here.
  if (__builtin_expect(stage_key0 + BN <= S, 1)) return;
  const int key0 = stage_key0 + 4 * g;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key0 + 32 * mb + 8 * (r >> 2) + (r & 3) >= S) sc[mb][r] = fill;
}

// Destination of the stores of lanes whose query row lies past the sequence
// (rows of a ragged last tile) and of the unused lanes of an instrumented
// build's timestamp store: written, never read.  Every lane of a storing
// wave issues every store of the epilogue, so that the wave issues a fixed
// number of store instructions per unit with no branch around them (the
// wait at the tile boundary counts them).  64 lanes x D <= 128 bf16.
__device__ __attribute__((aligned(256))) uint16_t fa_store_sink[64 * 128];

// Epilogue of one wave's 32 queries: scale by inv (1 / the row sum, or 0 for
// a row whose every key was masked out), round to bf16 and store 8
// consecutive dims per lane with 128-bit stores, into the slab of the query's
// destination (Slab) or the [B][H][S][D] output (Plain).  The NDBS 32-dim
// blocks of o cover dims [d0, d0 + 32 NDBS).  Exactly 2 NDBS store
// instructions per wave whatever the rows: a lane whose row is >= S stores
// into fa_store_sink.
template <int D, StoreMode MODE, int NDBS>
__device__ __forceinline__ void store_rows(const FwdParams& p, const f32x16 (&o)[NDBS], float inv,
                                           int qrow, int d0, int b, int h, int bh, int g,
                                           int lane) {
  const int row = qrow < p.S ? qrow : p.S - 1;
  size_t row_off;
  if (MODE == StoreMode::Slab) {
    const int slab = row / p.Sp, t = row - slab * p.Sp;
    row_off = (((size_t)slab * p.B + b) * p.Sp + t) * p.H + h;
  } else {
    row_off = (size_t)bh * p.S + row;
  }
  uint16_t* const dst = qrow < p.S ? p.out + row_off * D + d0 : fa_store_sink + lane * D;
#pragma unroll
  for (int db = 0; db < NDBS; ++db) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r0 = 8 * hf;
      const uint32_t a0 = pack_bf16(o[db][r0 + 0] * inv, o[db][r0 + 1] * inv);
      const uint32_t a1 = pack_bf16(o[db][r0 + 2] * inv, o[db][r0 + 3] * inv);
      const uint32_t b0 = pack_bf16(o[db][r0 + 4] * inv, o[db][r0 + 5] * inv);
      const uint32_t b1 = pack_bf16(o[db][r0 + 6] * inv, o[db][r0 + 7] * inv);
      const Pair x = swap_halves(a0, b0);
      const Pair y = swap_halves(a1, b1);
      *reinterpret_cast<u32x4*>(dst + 32 * db + 16 * hf + 8 * g) = u32x4{x.lo, y.lo, x.hi, y.hi};
    }
  }
}

// Low 32 bits of the shader clock counter.
__device__ __forceinline__ uint32_t clock_lo() { return (uint32_t)__builtin_amdgcn_s_memtime(); }

// Ping-pong kernel: 8 waves, one workgroup per CU.
// Waves 0-3 form group 0 and waves 4-7 group 1; the SIMD that runs wave w
// also runs wave w + 4.  Each K/V stage n of a wave is split into two regions
// separated by workgroup barriers: region S(n), the online softmax of the
// stage's scores (VALU only), and region M(n), all of the stage's MFMAs (the
// scores of stage n + 1, QK^T, and the PV product of stage n).  Group 1 runs
// one region behind group 0, so that on every SIMD the softmax of one wave
// issues beside the MFMAs of the other and the matrix core never waits for
// the softmax.  Only one score tile is live per wave: M(n) writes the scores
// that S(n + 1) consumes.
//
// Phases t are separated by barriers: group 0 runs S(n) in t = 2n and M(n) in
// 2n + 1, group 1 runs S(n) in 2n + 1 and M(n) in 2n + 2.  K stage j is read in
// M(j - 1) (phases 2j - 1 and 2j), V stage j in M(j) (phases 2j + 1 and
// 2j + 2).  DMA is issued in region S, into a slot whose last
// readers finished before the barrier that opened the region (every wave of
// a group reads all of a stage, so a slot may only be refilled once all of
// them are past it), and waited for at the end of a later region S of the
// same wave, before the barrier that precedes its readers.
//
// Whole units (SPLIT = false) are 256-query tiles: group 0 holds queries
// [0, 128), group 1 queries [128, 256), and both read the same K/V stages, so
// each stage crosses the L2 -> LDS path once per 256 queries.  Four buffers
// per tensor: group 0 loads K stage n + 3 in S(n) into the slot of K stage
// n - 1 (last read in phase 2n - 2), first read in phase 2n + 5; group 1 loads
// V stage n + 3 in S(n) into the slot of V stage n - 1 (last read in phase
// 2n), first read in phase 2n + 7.  Each waits for a stage two S regions
// after issuing it.
//
// Split units (SPLIT = true) fill the last, partial round of a launch: one
// 128-query half of a 256-query tile, with the keys split between the groups
// (group 0 the first ceil(ns / 2) stages, group 1 the rest).  Both groups
// hold the same queries and each computes on, and loads, its own K/V stream
// with two buffers per tensor: in S(n), K stage n + 2 into the slot of K
// stage n and V stage n + 1 into the slot of V stage n - 1 (both last read in
// M(n - 1)), both first read in M(n + 1).  At the end group 1 hands its
// partial (max, sum, O) to group 0 through LDS, and group 0 merges and stores
// the half tile.  With a workspace (p.split_pieces > 1) a split unit is one
// piece of a half tile's stages, split between the groups the same way, and
// group 0 writes the merged piece to the workspace for fa_merge_split_kernel
// instead of storing it.
//
// Masked units (MASKED = true, split-key) are the 128-query tiles of a block
// mask: the row's K kept 128-key tiles give 2K stages in key order, group 0
// takes the first K and group 1 the rest (KeptStages), with the split
// schedule above; tiles the mask drops are never loaded.
//
// SLAB_IN (any form, slab output only): q, k and v arrive sequence-sharded,
// [P][B][S/P][H][D], as before Ulysses' pre-attention exchange, and the loads
// read the tile's head straight from the slabs (slab_row, slab_dma); the
// arithmetic is unchanged, so the result equals that of [B][H][S][D] inputs
// bit for bit.
//
// Tile boundary (the piggyback).  When a unit's Q-loop is over, each wave
// first issues the next unit's prologue -- its Q fragments (as soon as the
// last stage's scores are formed, ahead of the epilogue's merge and
// normalisation) and the first K/V stages of its stream -- then the
// finished unit's slab stores, and then
// waits for the prologue only.  gfx950 counts vector loads and stores on one
// counter, vmcnt, which retires in issue order: vmcnt(N), N = the vector
// memory instructions issued after the prologue (the stores), completes every
// older load and leaves the stores in flight.  So the next unit's Q-loop
// starts while the stores drain.  Its first stages need no DMA wait at all
// (their data came with the prologue): none in S(0) and S(1) of a whole unit
// and in S(0) of a split unit.  The first wait that covers the stores is the
// one for the first refill issued after them, at the end of S(2) (whole) or
// S(1) (split), two or one stages into the next Q-loop.  Every wave issues the
// same number of stores per unit (2 NDB whole; NDB split, the two groups
// storing half of the dims each) with no branch around them, rows >= S going
// to fa_store_sink, so the count is exact.
//
// INSTR (instrumented instances, slab output, D = 128): 1 runs the kernel as
// above and writes one record of eight uint32 per unit and wave to p.stamps
// (index (unit * 8 + wave) * 8): the low 32 bits of the shader clock when the
// wait before the unit's Q-loop returned, after the barrier that starts it,
// when its last stage was done, when its last store instruction was issued,
// when those stores were complete (INSTR 2 only, else 0), then the unit, the
// workgroup and the high 32 bits of the clock at the store issue.  2 is the
// completion-coupled counterfactual the pages contrast with piggybacking:
// the owner issues its stores, waits until they are complete and visible
// beyond its XCD (a device-scope release: L2 write-back, vmcnt(0)), and only
// then issues the next unit's prologue.  3 keeps the order in which the
// stores come first and the next unit's prologue second, with one wait for
// both (so the next Q-loop waits for the stores as well, though their drain
// overlaps the prologue's loads).
template <int D, StoreMode MODE, bool NEG, bool SPLIT, bool MASKED = false, bool SLAB_IN = false,
          int INSTR = 0>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512),
                          amdgpu_waves_per_eu(2, 2)))
void fa_fwd_pp_kernel(FwdParams p) {
  static_assert(!MASKED || SPLIT, "masked units are split-key units");
  static_assert(INSTR == 0 || (MODE == StoreMode::Slab && D == 128), "instrumented instances");
  constexpr int NKS = D / 16;     // QK^T contraction steps
  constexpr int NDB = D / 32;     // 32-dim blocks of O^T
  constexpr int NA = 2 * NKS;     // QK^T MFMAs per stage
  constexpr int NB = 4 * NDB;     // PV MFMAs per stage
  constexpr int E = Tile<D>::ELEMS;
  constexpr int NG = SPLIT ? 2 : 1;          // K/V streams
  constexpr int NBUF = SPLIT ? 2 : 4;        // buffers per tensor and stream
  constexpr int PW = Dma<D>::PER_WAVE4;      // DMA instructions per wave, tensor and stage
  // DMA instructions a wave may leave in flight at the end of region S: its
  // last two regions' worth (whole units issue PW per region, split units
  // 2 PW, and wait for the older of two regions or for the previous one).
  constexpr int NDMA = 2 * PW;
  constexpr bool COUPLED = INSTR == 2;
  constexpr bool LATE = INSTR == 3;   // stores, then the next prologue, one wait for both
  // Buffer [i][e] of stream i; one object per (tensor, slot) so that the
  // compiler can tell a DMA into one buffer from reads of another.
  __shared__ __attribute__((aligned(16))) uint16_t kb0[NG][E];
  __shared__ __attribute__((aligned(16))) uint16_t kb1[NG][E];
  __shared__ __attribute__((aligned(16))) uint16_t kb2[NBUF == 4 ? NG : 1][NBUF == 4 ? E : 8];
  __shared__ __attribute__((aligned(16))) uint16_t kb3[NBUF == 4 ? NG : 1][NBUF == 4 ? E : 8];
  __shared__ __attribute__((aligned(16))) uint16_t vb0[NG][E];
  __shared__ __attribute__((aligned(16))) uint16_t vb1[NG][E];
  __shared__ __attribute__((aligned(16))) uint16_t vb2[NBUF == 4 ? NG : 1][NBUF == 4 ? E : 8];
  __shared__ __attribute__((aligned(16))) uint16_t vb3[NBUF == 4 ? NG : 1][NBUF == 4 ? E : 8];
  // Group 1's running (max, sum) hand-over (split units only).
  __shared__ float ml[SPLIT ? 4 * 256 : 1];
  // Masked launches: this workgroup's unit in each round of the schedule.
  __shared__ int plan_col[MASKED ? kPlanMaxRounds : 1];
  // Dynamic schedule: the next item's counter value, from wave 0 to all.
  __shared__ int dyn_next_lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wq = wave & 3;
  const int l32 = lane & 31, g = lane >> 5;
  const float c = p.c;
  const float fill = NEG ? __builtin_inff() : -__builtin_inff();   // fill * c = -inf
  const uint32_t head_bytes = (uint32_t)p.S * D * 2;
  const int ns = (p.S + BN - 1) / BN;                               // K/V stages (dense)
  const int nsh = (ns + 1) / 2;                                     // stages per stream (SPLIT)
  const int own = SPLIT ? grp : 0;   // the stream this wave computes on and (SPLIT) loads
  // Stage j of the stream sits in kbuf(j % NBUF) / vbuf(j % NBUF).
  auto kbuf = [&](int slot) FA_INL -> uint16_t* {
    if (NBUF == 4 && slot == 2) return kb2[own];
    if (NBUF == 4 && slot == 3) return kb3[own];
    return slot ? kb1[own] : kb0[own];
  };
  auto vbuf = [&](int slot) FA_INL -> uint16_t* {
    if (NBUF == 4 && slot == 2) return vb2[own];
    if (NBUF == 4 && slot == 3) return vb3[own];
    return slot ? vb1[own] : vb0[own];
  };
  // Per-lane offsets of this wave's share of a K and of a V stage.
  // Whole units: a wave only ever loads its group's tensor (group 0 K, group
  // 1 V), so one set of offsets serves both calls below.
  uint32_t koff[PW], voff[SPLIT ? PW : 1];
#pragma unroll
  for (int q = 0; q < PW; ++q) {
    if (SPLIT) {
      koff[q] = dma_lane_off<D, false>(wq, lane, q);
      voff[q] = dma_lane_off<D, true>(wq, lane, q);
    } else {
      koff[q] = grp == 0 ? dma_lane_off<D, false>(wq, lane, q) : dma_lane_off<D, true>(wq, lane, q);
    }
  }
  // Slab-layout inputs: key rows of one (b, h) are H D 2 bytes apart within a
  // slab, so a lane's offset within a stage becomes row * rowstride + chunk.
  // row0 is the lane's row in its first DMA instruction; instruction q moves
  // rows row0 + q * (64 / CH).
  constexpr int SH = D == 128 ? 8 : 7;                 // log2(D * 2)
  const uint32_t rowstride = (uint32_t)p.H * D * 2;
  const uint32_t in_bytes = (uint32_t)p.B * p.H * p.S * D * 2;   // < 2^31 for slab inputs
  const int row0 = (int)(koff[0] >> SH);
  if (SLAB_IN) {
#pragma unroll
    for (int q = 0; q < PW; ++q) {
      koff[q] = (koff[q] >> SH) * rowstride + (koff[q] & (2 * D - 1));
      if (SPLIT) voff[q] = (voff[q] >> SH) * rowstride + (voff[q] & (2 * D - 1));
    }
  }

  // A work unit: dense, 256-query tile `tile` (split units: its half
  // unit & 1); masked, 128-query tile qt of head bh, which is mask row qt;
  // a segment (whole form, tail round): stages [s0, s0 + nst) of a
  // 256-query tile, whose partial result goes to workspace slot seg.
  // [B][H][S][D] inputs: one buffer resource per head slice.  Slab inputs:
  // one per tensor, with the head's columns at head_col of every row.
  // Stage j of this wave's stream starts at key s0 + j (j < nst, in stages);
  // nloop stages are run (split units: as many for both groups, the stages
  // past the stream's end reading zeros).
  struct Unit {
    int uidx, bh, qt, b, h, qrow;
    int s0, nst, nloop, seg;
    uint32_t head_col;
    __amdgpu_buffer_rsrc_t rq, rk, rv;
  };
  auto make_tile = [&](int tile, Unit& u) FA_INL {
    u.bh = tile / p.nqt;
    u.qt = tile - u.bh * p.nqt;
    u.b = u.bh / p.H;
    u.h = u.bh - u.b * p.H;
    const size_t head_off = SLAB_IN ? 0 : (size_t)u.bh * p.S * D;
    const uint32_t in_size = SLAB_IN ? in_bytes : head_bytes;
    u.rq = make_rsrc(p.q + head_off, in_size);
    u.rk = make_rsrc(p.k + head_off, in_size);
    u.rv = make_rsrc(p.v + head_off, in_size);
    u.head_col = (uint32_t)u.h * D * 2;
  };
  auto make_unit = [&](int unit) FA_INL {
    Unit u;
    if (SPLIT && !MASKED && p.split_pieces > 1) {
      // Piece j of half tile hf: stages [a, b) of its ns, the first half
      // (rounded up) on group 0, the rest on group 1; its partial result
      // goes to workspace slot `unit`.
      const int hf = unit / p.split_pieces, j = unit - hf * p.split_pieces;
      make_tile(p.unit_base + (hf >> 1), u);
      u.uidx = unit;
      u.qrow = u.qt * 256 + (hf & 1) * 128 + wq * 32 + l32;
      const int ps = (ns + p.split_pieces - 1) / p.split_pieces;
      const int a = j * ps, b = a + ps < ns ? a + ps : ns;
      const int hs = (b - a + 1) / 2;
      u.s0 = a + own * hs;
      u.nst = own == 0 ? hs : (b - a) - hs;
      u.nloop = hs;
      u.seg = unit;
      return u;
    }
    make_tile(MASKED ? unit : SPLIT ? p.unit_base + (unit >> 1) : unit, u);
    u.uidx = unit;
    u.qrow = MASKED  ? u.qt * BM + wq * 32 + l32
             : SPLIT ? u.qt * 256 + (unit & 1) * 128 + wq * 32 + l32
                     : u.qt * 256 + wave * 32 + l32;
    u.s0 = own * nsh;
    u.nst = SPLIT ? (ns - u.s0 < nsh ? ns - u.s0 : nsh) : ns;
    u.nloop = SPLIT ? nsh : ns;
    u.seg = -1;
    return u;
  };
  // Tail segments (whole form): the tail round's t tiles, after the launch's
  // whole units, each split at stage L = p.tail_len < ns.  The lead segment
  // [0, L) of tile i runs on slot i: slots 0 .. t - 1 start together and
  // stream their tiles' K/V in step, as whole units do (tiles of one head,
  // an XCD's slots being consecutive).  The ends [L, ns) of the t tiles, one
  // span of t e stages (e = ns - L) tile by tile, are cut into slices of
  // Lh = p.tail_hlen <= L stages for the other slots: helper hh = sid - t
  // runs [hh Lh, (hh + 1) Lh) of the span, one segment per tile end it
  // meets.  Workspace slots: the lead of tile i writes slot i, helper hh's
  // piece of tile i slot t + i + hh (distinct, as the helpers' tiles never
  // go back; below t + G - 1).
  auto tail_segments = [&](int sid) FA_INL {
    if (SPLIT || MASKED || p.tail <= 0 || p.queue) return 0;
    if (sid < p.tail) return 1;
    const int e = ns - p.tail_len;
    if (e <= 0) return 0;
    const int a = (sid - p.tail) * p.tail_hlen;
    const int b = a + p.tail_hlen < p.tail * e ? a + p.tail_hlen : p.tail * e;
    if (a >= b) return 0;
    return (b - 1) / e - a / e + 1;
  };
  auto make_segment = [&](int sid, int j) FA_INL {
    Unit u;
    int ti, st0, st1, seg;
    if (sid < p.tail) {
      ti = sid;
      st0 = 0;
      st1 = p.tail_len;
      seg = sid;
    } else {
      const int e = ns - p.tail_len;
      const int hh = sid - p.tail;
      const int a = hh * p.tail_hlen;
      const int b = a + p.tail_hlen < p.tail * e ? a + p.tail_hlen : p.tail * e;
      ti = a / e + j;
      st0 = p.tail_len + (j == 0 ? a - ti * e : 0);
      st1 = p.tail_len + (b < (ti + 1) * e ? b : (ti + 1) * e) - ti * e;
      seg = p.tail + ti + hh;
    }
    make_tile(p.units + ti, u);
    u.uidx = -1;
    u.qrow = u.qt * 256 + wave * 32 + l32;
    u.s0 = st0;
    u.nst = st1 - st0;
    u.nloop = st1 - st0;
    u.seg = seg;
    return u;
  };
  // First key of stage j of unit u's stream; a stage past the end is read
  // at key S, which the buffer returns as zeros.
  auto key_of = [&](const Unit& u, int j) FA_INL { return j < u.nst ? (u.s0 + j) * BN : p.S; };
  // Slab inputs: byte offset of the row of token s < S of unit u's (b, h).
  auto slab_row = [&](const Unit& u, uint32_t s) FA_INL {
    const uint32_t ps = (__umulhi(s, p.sp_magic) + s) >> p.sp_shift;
    return ((ps * p.B + u.b) * p.Sp + (s - ps * p.Sp)) * rowstride + u.head_col;
  };
  // Slab inputs: this wave's share of the stage that starts at key `key`
  // into `dst`, lane offsets `lo` within the stage's first slab.  A stage
  // that runs past the end of a slab continues in the next slab, (B - 1) Sp
  // rows further on (Sp >= 64, so at most one boundary); keys >= S land
  // past the tensor and read as zeros.
  // The stage's address, scalar work that the stage loop does in the MFMA
  // region before the softmax region that issues the DMA (the softmax wave
  // is the one whose instruction stream bounds a stage).
  struct SlabAt {
    uint32_t base;   // byte offset of the stage's first row
    int left;        // rows before the slab boundary (>= BN: none in the stage)
  };
  auto slab_at = [&](const Unit& u, int key) FA_INL {
    if (key >= p.S) return SlabAt{in_bytes, BN};
    const uint32_t ps = (__umulhi((uint32_t)key, p.sp_magic) + key) >> p.sp_shift;
    return SlabAt{((ps * p.B + u.b) * p.Sp + (key - ps * p.Sp)) * rowstride + u.head_col,
                  (int)((ps + 1) * p.Sp) - key};
  };
  auto slab_dma_at = [&](uint16_t* dst, __amdgpu_buffer_rsrc_t r, const uint32_t* lo,
                         SlabAt a) FA_INL {
    if (a.left >= BN) {
      dma_blocks<PW>(dst, r, a.base, lo);
      return;
    }
    const uint32_t delta = (uint32_t)(p.B - 1) * p.Sp * rowstride;
    uint32_t o[PW];
#pragma unroll
    for (int q = 0; q < PW; ++q)
      o[q] = lo[q] + (row0 + q * (64 / Tile<D>::CH) >= a.left ? delta : 0u);
    dma_blocks<PW>(dst, r, a.base, o);
  };
  auto slab_dma = [&](const Unit& u, uint16_t* dst, __amdgpu_buffer_rsrc_t r, const uint32_t* lo,
                      int key) FA_INL { slab_dma_at(dst, r, lo, slab_at(u, key)); };
  // Slab inputs: the addresses of the stages the next softmax region loads
  // (whole units: K or V stage n + 3, one key for both; split units: K stage
  // n + 2 and V stage n + 1).
  SlabAt sl_k{0u, BN}, sl_v{0u, BN};
  // The same share as a DmaPlan ([B][H][S][D] inputs): instruction q reads
  // the byte offsets dma_blocks would use.
  auto plan_of = [&](uint16_t* dst, __amdgpu_buffer_rsrc_t r, const uint32_t* lo, int key) FA_INL {
    DmaPlan<PW> pl;
    pl.lds = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)dst);
    pl.r = r;
#pragma unroll
    for (int q = 0; q < PW; ++q) pl.addr[q] = (uint32_t)key * (D * 2) + lo[q];
    return pl;
  };
  // Masked units: this group's stream of kept stages, and the first keys of
  // stages n, n + 1 and n + 2 of the stream (key_n[0..2]), advanced after
  // each stage; the unit's nloop is the stream's number of stages.
  KeptStages kept;
  int key_n[3] = {0, 0, 0};
  auto start_stream = [&](Unit& u) FA_INL {
    if constexpr (MASKED) {
      u.nloop = kept.init(p.mask + ((size_t)u.h * p.nmt + u.qt) * p.mw, p.nmt, p.mw, p.S, own);
      key_n[0] = kept.next();
      key_n[1] = kept.next();
      key_n[2] = kept.next();
    }
  };
  // First key of stage j of this wave's stream.
  auto stage_key = [&](const Unit& u, int j) FA_INL { return MASKED ? key_n[j] : key_of(u, j); };
  // This wave's share of unit u's K or V stage that starts at key `key`
  // into slot `slot`.
  auto dma_k = [&](const Unit& u, int slot, int key) FA_INL {
    if constexpr (SLAB_IN) {
      slab_dma(u, kbuf(slot) + 64 * 8 * PW * wq, u.rk, koff, key);
    } else {
      dma_blocks<PW>(kbuf(slot) + 64 * 8 * PW * wq, u.rk, (uint32_t)key * (D * 2), koff);
    }
  };
  auto dma_v = [&](const Unit& u, int slot, int key) FA_INL {
    if constexpr (SLAB_IN) {
      slab_dma(u, vbuf(slot) + 64 * 8 * PW * wq, u.rv, SPLIT ? voff : koff, key);
    } else {
      dma_blocks<PW>(vbuf(slot) + 64 * 8 * PW * wq, u.rv, (uint32_t)key * (D * 2),
                     SPLIT ? voff : koff);
    }
  };

  Unit cur;                 // the unit whose Q-loop runs
  bf16x8 qf[NKS];           // its Q fragments
  f32x16 s[2];              // the score tile of the current stage
  f32x16 acc[NDB];          // O^T accumulator
  float m_run = 0.0f, l_run = 0.0f;

  // Prologue of unit u: the Q fragments (prologue_q) and the first K/V
  // stages of this wave's stream (prologue_kv) -- K stages 0 and 1 and V
  // stage 0 (SPLIT: each group, its own stream) or K stages 0-2 (group 0)
  // and V stages 0-2 (group 1).
  auto prologue_q = [&](const Unit& u) FA_INL {
    const uint32_t qbase = !SLAB_IN ? (uint32_t)(u.qrow * D * 2)
                           : u.qrow < p.S ? slab_row(u, (uint32_t)u.qrow) : in_bytes;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, load16(u.rq, qbase + ks * 32 + g * 16));
  };
  auto prologue_kv = [&](const Unit& u) FA_INL {
    if (SPLIT || grp == 0) {
      dma_k(u, 0, stage_key(u, 0));
      dma_k(u, 1, stage_key(u, 1));
    }
    if (!SPLIT && grp == 0) dma_k(u, 2, key_of(u, 2));
    if (SPLIT) {
      dma_v(u, 0, stage_key(u, 0));
    } else if (grp == 1) {
      dma_v(u, 0, stage_key(u, 0));
      dma_v(u, 1, stage_key(u, 1));
      dma_v(u, 2, key_of(u, 2));
    }
  };

  // The DMA issued in region S(n) (SLOT = n % NBUF), after the barrier
  // that ends every wave's reads of the slots it refills: at the region's
  // start, except that split units with [B][H][S][D] inputs spread theirs
  // over four points of the softmax (split_plans; measured faster there,
  // slower for whole units and for slab inputs, whose per-lane slab
  // addresses would then stay live through the softmax).
  // Whole units: K stage n + 3 (group 0) or V stage n + 3 (group 1) into
  // the slot that stage n - 1 freed.  Split units, each group on its own
  // stream: K stage n + 2 into the slot of K stage n (read in M(n - 1)) and
  // V stage n + 1 into the slot of V stage n - 1 (read in M(n - 1)).
  auto stage_dma = [&](auto SLOT, int n) FA_INL {
    constexpr int slot = decltype(SLOT)::value;
    if constexpr (SPLIT && SLAB_IN) {
      slab_dma_at(kbuf(slot) + 64 * 8 * PW * wq, cur.rk, koff, sl_k);
      slab_dma_at(vbuf((slot + 1) % NBUF) + 64 * 8 * PW * wq, cur.rv, voff, sl_v);
    } else if (SPLIT) {
      dma_k(cur, slot, MASKED ? key_n[2] : key_of(cur, n + 2));
      dma_v(cur, (slot + 1) % NBUF, MASKED ? key_n[1] : key_of(cur, n + 1));
    } else if constexpr (!SLAB_IN) {
      // One code path for both groups (the tensor and slot selected, not
      // branched on): the softmax wave takes no branch to issue its DMA.
      constexpr int sl = (slot + 3) % NBUF;
      uint16_t* const dst = (grp == 0 ? kbuf(sl) : vbuf(sl)) + 64 * 8 * PW * wq;
      dma_blocks<PW>(dst, grp == 0 ? cur.rk : cur.rv, (uint32_t)key_of(cur, n + 3) * (D * 2), koff);
    } else if (grp == 0) {
      slab_dma_at(kbuf((slot + 3) % NBUF) + 64 * 8 * PW * wq, cur.rk, koff, sl_k);
    } else {
      slab_dma_at(vbuf((slot + 3) % NBUF) + 64 * 8 * PW * wq, cur.rv, koff, sl_k);
    }
  };
  // Slab inputs: the addresses for the softmax region of stage n.
  auto slab_plan = [&](int n) FA_INL {
    if constexpr (SLAB_IN) {
      if constexpr (SPLIT) {
        sl_k = slab_at(cur, MASKED ? key_n[2] : key_of(cur, n + 2));
        sl_v = slab_at(cur, MASKED ? key_n[1] : key_of(cur, n + 1));
      } else {
        sl_k = slab_at(cur, key_of(cur, n + 3));
      }
    }
  };
  // Split units, [B][H][S][D] inputs: the same stages as DmaPlans, issued
  // during the softmax.
  struct SplitPlans { DmaPlan<PW> k, v; };
  auto split_plans = [&](auto SLOT, int n) FA_INL {
    constexpr int slot = decltype(SLOT)::value;
    const int wofs = 64 * 8 * PW * wq;
    return SplitPlans{plan_of(kbuf(slot) + wofs, cur.rk, koff,
                              MASKED ? key_n[2] : key_of(cur, n + 2)),
                      plan_of(vbuf((slot + 1) % NBUF) + wofs, cur.rv, voff,
                              MASKED ? key_n[1] : key_of(cur, n + 1))};
  };

  // Region S(n), SLOT = n % NBUF: this wave's DMA, the softmax of stage n,
  // then the wait that completes this wave's DMA from S(n - 2) (split
  // units: S(n - 1)) before the barrier that precedes its first readers.
  // The first stages of a unit need no wait (their stages came with the
  // prologue, which the tile boundary waited for): S(0) and S(1) of a whole
  // unit, S(0) of a split unit.
  auto region_s = [&](auto SLOT, int n, StageProbs<NEG>& sm) FA_INL {
    const int key0 = MASKED ? key_n[0] : key_of(cur, n);
    if constexpr (SPLIT && !SLAB_IN) {
      const SplitPlans pl = split_plans(SLOT, n);
      mask_tail(s, key0, p.S, g, fill);
      sm.template compute<true>(s, c, m_run, l_run, [&](int j) {
        constexpr int STEP = 4 / PW;
        if (j % STEP == 0) {
          pl.k.issue(j / STEP);
          pl.v.issue(j / STEP);
        }
      });
    } else {
      stage_dma(SLOT, n);
      mask_tail(s, key0, p.S, g, fill);
      sm.template compute<false>(s, c, m_run, l_run, [](int) {});
    }
    if (n >= (SPLIT ? 1 : 2)) wait_vm<NDMA>();
  };
  // Region M(n): the scores of stage n + 1 (K stage n + 1) and PV of stage
  // n (V stage n).  After the last stage the QK^T MFMAs read a buffer of
  // zeros and their result is unused.
  auto region_m = [&](auto SLOT, const StageProbs<NEG>& sm) FA_INL {
    constexpr int slot = decltype(SLOT)::value;
    // Raised wave priority while this wave issues MFMAs: when both waves
    // of a SIMD have an instruction ready, the matrix core's feeder goes
    // first and the softmax wave's VALU work fills the gaps.
    __builtin_amdgcn_s_setprio(2);
    const uint16_t* const kn = kbuf((slot + 1) % NBUF);
    const uint16_t* const vt = vbuf(slot);
    if (__builtin_expect(sm.rescale, 0)) {   // rare: out of line
#pragma unroll
      for (int i = 0; i < NDB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= sm.alpha;
    }
    static_assert(NA == NB, "one QK^T MFMA per PV MFMA");
    constexpr int LEAD = FA_MLEAD;
    auto ka_read = [&](int i) FA_INL { return k_operand<D>(kn, i & 1, i >> 1, l32, g); };
    auto va_read = [&](int j) FA_INL { return v_operand<D>(vt, j / NDB, j % NDB, lane); };
    // Whole units interleave the two products, QK^T MFMA i before PV MFMA
    // i; split units issue all of QK^T first, then PV.  Each accumulator
    // sees the same operands in the same order either way (the results
    // are bit-identical); these orders measured fastest for each form.
    auto qk = [&](int i, const bf16x8& a) FA_INL {
      s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i >> 1],
                                                         i < 2 ? f32x16{} : s[i & 1], 0, 0, 0);
    };
    auto pv = [&](int j, const bf16x8& a) FA_INL {
      acc[j % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sm.p_operand(j / NDB),
                                                             acc[j % NDB], 0, 0, 0);
    };
    if constexpr (!SPLIT) {
      bf16x8 ka[NA], va[NB];
#pragma unroll
      for (int i = 0; i < LEAD; ++i) {
        va[i] = va_read(i);
        ka[i] = ka_read(i);
      }
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (i + LEAD < NA) {
          va[i + LEAD] = va_read(i + LEAD);
          ka[i + LEAD] = ka_read(i + LEAD);
        }
        qk(i, ka[i]);
        pv(i, va[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Operand t: QK^T MFMA t (t < NA) or PV MFMA t - NA, read 2 LEAD ahead.
      bf16x8 op[NA + NB];
      auto rd = [&](int t) FA_INL { op[t] = t < NA ? ka_read(t) : va_read(t - NA); };
#pragma unroll
      for (int t = 0; t < 2 * LEAD; ++t) rd(t);
#pragma unroll
      for (int t = 0; t < NA + NB; ++t) {
        if (t + 2 * LEAD < NA + NB) rd(t + 2 * LEAD);
        if (t < NA)
          qk(t, op[t]);
        else
          pv(t - NA, op[t]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // One stage: S, barrier, M, barrier.
  auto stage = [&](auto SLOT, int n) FA_INL {
    StageProbs<NEG> sm;
    region_s(SLOT, n, sm);
    barrier_keep_dma();
    region_m(SLOT, sm);
    // Masked units advance their stream's stage keys here, at the end of
    // the MFMA region, rather than at the start of the next softmax region:
    // the scalar mask walk then costs the MFMA wave (whose operand reads
    // are all consumed by now) instead of the softmax wave.
    if (MASKED) {
      key_n[0] = key_n[1];
      key_n[1] = key_n[2];
      key_n[2] = kept.next();
    }
    slab_plan(n + 1);
    barrier_keep_dma();
  };
  // A unit's stages.
  auto stages = [&]() FA_INL {
    const int nloop = cur.nloop;
    for (int n = 0; n < nloop; n += NBUF) {
      stage(std::integral_constant<int, 0>{}, n);
      if (n + 1 >= nloop) break;
      stage(std::integral_constant<int, 1>{}, n + 1);
      if constexpr (NBUF == 4) {
        if (n + 2 >= nloop) break;
        stage(std::integral_constant<int, 2>{}, n + 2);
        if (n + 3 >= nloop) break;
        stage(std::integral_constant<int, 3>{}, n + 3);
      }
    }
  };

  // This workgroup's work items: the launch's units slot, slot + G, ... and
  // then (whole form) its tail segments, slots in XCD-aware order.  Masked
  // units run on the schedule below (plain order beyond its limits), which
  // deals each round's units by kept-tile count to consecutive slots: an
  // XCD's workgroups then hold units of about the same count, which walk
  // their rows' kept tiles at about the same pace, so the tiles that several
  // of them keep meet in its L2 close together in time (1.6% faster on a
  // 30%-dense mask than slots dealt round-robin over the XCDs).
  const int G = (int)gridDim.x;
  const int slot = xcd_slot(blockIdx.x, G);
  int n_units = slot < p.units ? (p.units - slot + G - 1) / G : 0;
  // Masked schedule.  A masked unit's Q-loop time is close to linear in K,
  // its row's kept tiles, so the plain order -- G units per round -- leaves
  // the workgroups that drew costly units running after the others.  The
  // rounds keep the plain order's units (round r holds units r G .. r G +
  // G - 1, so a round's workgroups still share heads and their K/V), and
  // within each the units are dealt in decreasing K (ties by index) in snake
  // order: in even rounds workgroup w takes the w-th costliest, in odd
  // rounds the (G - 1 - w)-th, so the costly units of one round pair with
  // the cheap ones of the next.  Every workgroup derives its own column
  // from the mask alone -- the kept tiles of every mask row (LDS atomics
  // into kb0, which no DMA has touched yet), then per round a search over K
  // with wave ballots -- so all agree without any exchange.
  constexpr int kPlanRows = NG * E / 2;    // int row counts that fit in kb0
  const int rounds = (p.units + G - 1) / G;
  const int plan_hn = p.H * p.nmt;          // mask rows
  const bool planned = MASKED && G <= 256 && rounds <= kPlanMaxRounds && plan_hn <= kPlanRows &&
                       plan_hn * p.mw < (1 << 24);
  if constexpr (MASKED) {
    if (planned) {
      int* const kept_of = reinterpret_cast<int*>(&kb0[0][0]);   // [mask row]
      for (int i = tid; i < plan_hn; i += 512) kept_of[i] = 0;
      __syncthreads();
      // Word i of row r is item f = i * rows + r, so a wave's lanes add
      // into distinct rows' counters.
      const int nw = plan_hn * p.mw;
      const float inv_hn = 1.0f / (float)plan_hn;
      const uint64_t last_mask = (p.nmt & 63) ? (1ull << (p.nmt & 63)) - 1 : ~0ull;
      for (int f0 = 0; f0 < nw; f0 += 512 * 8) {
        uint64_t wd[8];
        int row[8], wi[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int f = f0 + 512 * j + tid;
          // f / rows, exact after one correction (f < 2^24).
          int i = (int)((float)f * inv_hn);
          i -= i * plan_hn > f;
          i += (i + 1) * plan_hn <= f;
          wi[j] = i;
          row[j] = f - i * plan_hn;
          wd[j] = f < nw ? p.mask[(size_t)row[j] * p.mw + i] : 0ull;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint64_t x = wi[j] == p.mw - 1 ? wd[j] & last_mask : wd[j];
          if (x) atomicAdd(&kept_of[row[j]], __builtin_popcountll(x));
        }
      }
      __syncthreads();
      // Wave v finds this workgroup's unit in rounds v, v + 8, ...: the rank
      // k it takes, the K value c* of that rank (the largest c with more
      // than k units of K >= c, by bisection), and the unit among those of
      // K = c*, in index order.
      for (int r = wave; r < rounds; r += 8) {
        const int base = r * G;
        const int nr = p.units - base < G ? p.units - base : G;
        const int k = (r & 1) ? G - 1 - slot : slot;
        int unit = -1;
        if (k < nr) {
          int kc[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 64 * e + lane;
            kc[e] = j < nr ? kept_of[(base + j) % plan_hn] : -1;
          }
          auto count_ge = [&](int c) FA_INL {
            int n = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) n += __builtin_popcountll(__ballot(kc[e] >= c));
            return n;
          };
          int lo = 0, hi = p.nmt;   // count_ge(lo) = nr > k
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (count_ge(mid) > k) lo = mid; else hi = mid - 1;
          }
          int off = k - count_ge(lo + 1);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint64_t bits = __ballot(kc[e] == lo);
            const int n = __builtin_popcountll(bits);
            if (unit < 0 && off < n) {
              for (int t = 0; t < off; ++t) bits &= bits - 1;
              unit = base + 64 * e + __builtin_ctzll(bits);
            }
            off -= n;
          }
        }
        if (lane == 0) plan_col[r] = unit;
      }
      __syncthreads();
      n_units = rounds - (plan_col[rounds - 1] < 0 ? 1 : 0);
    }
  }
  // Dynamic schedule (whole form, p.queue set): the item index is the
  // position in the launch's item list (whole units, then the tail tiles'
  // pieces, piece by piece); the full rounds of whole units run round-robin
  // (item slot + i G, so that the 32 workgroups of a chiplet start their
  // tiles together and share each K/V stage in its L2), every later item
  // is dyn_static + the queue counter's old value, fetched by lane 0 of
  // wave 0 once the item's last stage is in (one atomic add per item, its
  // return awaited with no DMA left in flight; fetched earlier, the value
  // would hold a register through the stage loop) and passed to the other
  // waves through LDS at the barrier that ends the Q-loop.
  const bool dyn = !SPLIT && !MASKED && INSTR == 0 && p.queue != nullptr;
  const int dyn_n = dyn ? p.units + p.tail * p.dyn_pieces : 0;
  const int dyn_static = dyn ? p.units / G * G : 0;
  auto make_dyn = [&](int i) FA_INL {
    if (i < p.units) return make_unit(i);
    Unit u;
    const int pi = i - p.units, j = pi / p.tail, ti = pi - j * p.tail;
    make_tile(p.units + ti, u);
    u.uidx = -1;
    u.qrow = u.qt * 256 + wave * 32 + l32;
    // Piece j of P holds the share (P - j) / (P (P + 1) / 2) of the keys:
    // the pieces handed out last are the shortest, so that the workgroups
    // finish close together.
    const int P = p.dyn_pieces, tot = P * (P + 1) / 2;
    const int c0 = j * P - j * (j - 1) / 2, c1 = c0 + P - j;
    u.s0 = ns * c0 / tot;
    u.nst = ns * c1 / tot - u.s0;
    u.nloop = u.nst;
    u.seg = ti * p.dyn_pieces + j;
    return u;
  };
  const int n_items = dyn ? (slot < dyn_n ? 1 : 0) : n_units + tail_segments(slot);
  auto make_item = [&](int i) FA_INL {
    if (dyn) return make_dyn(i);
    if (planned) return make_unit(__builtin_amdgcn_readfirstlane(plan_col[i]));
    return i < n_units ? make_unit(slot + i * G) : make_segment(slot, i - n_units);
  };
  if (n_items == 0) return;
  int item = dyn ? slot : 0;
  cur = make_item(item);
  start_stream(cur);
  prologue_q(cur);
  prologue_kv(cur);
  wait_vm<0>();
  uint32_t t_ready = INSTR ? clock_lo() : 0u;
  for (;;) {
    // Every wave's prologue DMA has landed; every wave computes the scores of
    // its stream's first stage.
    barrier_keep_dma();
    const uint32_t t_start = INSTR ? clock_lo() : 0u;
    qk_mfma<D>(s, kbuf(0), qf, l32, g);
    // Every read of K stage 0 has returned before the barrier (split units
    // refill its slot in S(0)).
    wait_lds();
    barrier_keep_dma();
    if (grp == 1) barrier_keep_dma();   // group 1 starts one region behind
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
    // A finite starting max: the first stage's probabilities overflow against
    // it and raise it to the row's extreme (the rescale factor is then 0),
    // while keys past the end (fill, -inf after scaling) and a masked stream's
    // stage with no key at all (the second half of a kept last tile shorter
    // than 64 keys) weigh exp2(-inf) = 0 rather than NaN.
    m_run = -3.0e38f;
    l_run = 0.0f;
    slab_plan(0);

    stages();

    wait_dma();   // DMA of stages past the end, before the buffers are reused
    const uint32_t t_epi = INSTR ? clock_lo() : 0u;
    // Group 0's trailing region ends with the barrier that ends group 1's
    // last M: every wave's reads of the K/V buffers are over.  Dynamic
    // schedule: wave 0 fetches the next item's counter value and posts it
    // before that barrier.
    if (dyn && wave == 0) {
      if (lane == 0 && item + G >= dyn_static) dyn_next_lds = atomicAdd(p.queue, 1);
      wait_lds();
    }
    if (grp == 0) barrier_keep_dma();

    // The next item, and its Q fragments: the registers are free once the
    // last stage's scores are formed, and the loads, issued ahead of the
    // epilogue's merge and normalisation, leave the vector memory path to
    // the K/V DMA at the boundary (the CU issues the next unit's ~160 KiB of
    // loads and this unit's stores through one path, and the next Q-loop
    // starts only when they are in).  COUPLED and LATE keep all of the
    // prologue after the stores.
    const int next_item = !dyn ? item + 1
                          : item + G < dyn_static
                              ? item + G
                              : dyn_static + __builtin_amdgcn_readfirstlane(dyn_next_lds);
    const bool more = dyn ? next_item < dyn_n : next_item < n_items;
    constexpr bool kEarlyQ = !COUPLED && !LATE;
    Unit nxt = cur;
    if (kEarlyQ && more) {
      nxt = make_item(next_item);
      prologue_q(nxt);
    }

    // Split units: the two groups hold the same queries over different keys
    // and exchange half of their state through stream 0's four K/V buffers,
    // idle by now: wave wq of group 1 hands over its O^T accumulator's dims
    // [0, D/2), wave wq of group 0 its dims [D/2, D) (NDB/2 x 16 floats per
    // lane each, at float (db * 16 + r) * 64 + lane of buffer wq, the halves
    // disjoint), both their running max and sum (ml, by group); then each
    // merges the half it kept -- with x group 0's state and y group 1's,
    // O = O_x 2^(m_x - m) + O_y 2^(m_y - m), m = max(m_x, m_y), l alike --
    // and stores it (group 0 dims [0, D/2), group 1 dims [D/2, D)).
    constexpr int H2 = NDB / 2;
    if constexpr (SPLIT) {
      static_assert(NDB * 16 * 64 * 4 == E * 2, "one buffer per wave");
      float* const area = reinterpret_cast<float*>(wq == 0 ? kb0[0] : wq == 1 ? kb1[0]
                                                   : wq == 2 ? vb0[0] : vb1[0]);
      auto hand_over = [&](auto OFF) FA_INL {
        constexpr int off = decltype(OFF)::value;
#pragma unroll
        for (int db = off; db < off + H2; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) area[(db * 16 + r) * 64 + lane] = acc[db][r];
      };
      if (grp == 0)
        hand_over(std::integral_constant<int, H2>{});
      else
        hand_over(std::integral_constant<int, 0>{});
      ml[grp * 512 + wq * 64 + lane] = m_run;
      ml[grp * 512 + 256 + wq * 64 + lane] = l_run;
      __syncthreads();
      const float m_o = ml[(1 - grp) * 512 + wq * 64 + lane];
      const float l_o = ml[(1 - grp) * 512 + 256 + wq * 64 + lane];
      const float m_x = grp == 0 ? m_run : m_o, m_y = grp == 0 ? m_o : m_run;
      const float l_x = grp == 0 ? l_run : l_o, l_y = grp == 0 ? l_o : l_run;
      const float m = fmaxf(m_x, m_y);
      const float ax = __builtin_amdgcn_exp2f(m_x - m);
      const float ay = __builtin_amdgcn_exp2f(m_y - m);
      auto merge_kept = [&](auto OFF) FA_INL {
        constexpr int off = decltype(OFF)::value;
#pragma unroll
        for (int db = off; db < off + H2; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float other = area[(db * 16 + r) * 64 + lane];
            acc[db][r] = off == 0 ? acc[db][r] * ax + other * ay : other * ax + acc[db][r] * ay;
          }
      };
      if (grp == 0)
        merge_kept(std::integral_constant<int, 0>{});
      else
        merge_kept(std::integral_constant<int, H2>{});
      l_run = l_x * ax + l_y * ay;
      m_run = m;
      // Both groups have read the hand-over area before the next unit's
      // prologue refills stream 0's buffers.
      __syncthreads();
    }
    const float l_tot = halves_sum(l_run);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;

    // The tile boundary: the rest of the next unit's prologue, then this
    // unit's stores (COUPLED: the stores, their completion, then the
    // prologue).
    auto next_prologue = [&]() FA_INL {
      if (more) {
        if (!kEarlyQ) {
          nxt = make_item(next_item);
          prologue_q(nxt);
        }
        start_stream(nxt);
        prologue_kv(nxt);
      }
    };
    if (!COUPLED && !LATE) next_prologue();
    // Keep the stores after the prologue's loads.
    asm volatile("" ::: "memory");
    // After a wave's NS stores: the timestamps (INSTR), then the wait for
    // the prologue only, the NS stores (and the record store) staying in
    // flight; COUPLED: the wait for the stores, the prologue, and the wait
    // for everything.
    auto finish = [&](auto NS) FA_INL {
      constexpr int nst = decltype(NS)::value + (INSTR ? 1 : 0);
      if constexpr (INSTR) {
        const uint64_t t = __builtin_amdgcn_s_memtime();
        uint32_t t_complete = 0;
        if constexpr (COUPLED) {
          // The stores are complete and visible beyond this XCD (device-scope
          // release: L2 write-back, then the wait for completion).
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
          t_complete = clock_lo();
          next_prologue();
        }
        if constexpr (LATE) next_prologue();
        // Lanes 0 and 1 write the record; the others write the sink.
        // (Instrumented launches have no tail segments: cur.uidx >= 0.)
        uint32_t* const rec = p.stamps + ((size_t)cur.uidx * 8 + wave) * 8;
        const u32x4 val = lane == 0 ? u32x4{t_ready, t_start, t_epi, (uint32_t)t}
                                    : u32x4{t_complete, (uint32_t)cur.uidx, (uint32_t)blockIdx.x,
                                            (uint32_t)(t >> 32)};
        u32x4* const to = lane < 2 ? reinterpret_cast<u32x4*>(rec) + lane
                                   : reinterpret_cast<u32x4*>(fa_store_sink) + lane;
        *to = val;
      }
      if constexpr (COUPLED || LATE)
        wait_vm<0>();
      else
        wait_vm<nst>();
    };
    // Whole units: every wave stores its 32 queries.  Split units: each
    // group its half of the dims of the merged tile.  Tail segments and the
    // pieces of a split launch cut into pieces: every storing wave writes
    // its partial result -- the O^T accumulator normalised by its own row sum
    // (the same products store_rows forms, so the accumulator is not kept
    // twice), its running max and that row sum -- to workspace slot cur.seg
    // for the merge kernel (layout: seg_floats, wave w's part at w; split
    // units: the group-0 wave wq's part, its dims from both groups, max and
    // sum from group 0).
    auto write_partial = [&](auto OFF, auto N, int w) FA_INL {
      constexpr int off = decltype(OFF)::value, n = decltype(N)::value;
      float* const ws = p.ws + (size_t)cur.seg * seg_floats(D);
      typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int db = off; db < off + n; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<f32x4*>(ws + ((w * 4 * NDB + db * 4 + rr) * 64 + lane) * 4) =
              f32x4{acc[db][4 * rr] * inv, acc[db][4 * rr + 1] * inv, acc[db][4 * rr + 2] * inv,
                    acc[db][4 * rr + 3] * inv};
      if (off == 0)
        *reinterpret_cast<f32x4*>(ws + seg_ml_offset(D) + (w * 64 + lane) * 4) =
            f32x4{m_run, l_tot, 0.0f, 0.0f};
    };
    if constexpr (SPLIT) {
      auto store_half = [&](auto OFF) FA_INL {
        constexpr int off = decltype(OFF)::value;
        if (!MASKED && cur.seg >= 0) {
          write_partial(OFF, std::integral_constant<int, H2>{}, wq);
          finish(std::integral_constant<int, 4 * H2 + (off == 0 ? 1 : 0)>{});
        } else {
          const f32x16(&o)[H2] = *reinterpret_cast<const f32x16(*)[H2]>(&acc[off]);
          store_rows<D, MODE, H2>(p, o, inv, cur.qrow, 32 * off, cur.b, cur.h, cur.bh, g, lane);
          finish(std::integral_constant<int, 2 * H2>{});
        }
      };
      if (grp == 0)
        store_half(std::integral_constant<int, 0>{});
      else
        store_half(std::integral_constant<int, H2>{});
    } else if (cur.seg >= 0) {
      write_partial(std::integral_constant<int, 0>{}, std::integral_constant<int, NDB>{}, wave);
      finish(std::integral_constant<int, 4 * NDB + 1>{});
    } else {
      store_rows<D, MODE, NDB>(p, acc, inv, cur.qrow, 0, cur.b, cur.h, cur.bh, g, lane);
      finish(std::integral_constant<int, 2 * NDB>{});
    }
    if constexpr (INSTR) t_ready = clock_lo();
    if (!more) break;
    cur = nxt;
    item = next_item;
  }
}

// One wave's share (32 queries x D dims) of np partial results, workspace
// slots slot(0) .. slot(np - 1), combined into acc (unnormalised) and l:
// online over chunks of up to four partials, each chunk's loads all issued
// before any is used.  With m the largest running max so far, partial k
// weighs 2^(m_k - m) l_k, and what is summed is rescaled when m grows.
// Dim block db (32 dims) of the merge of np partial results for the rows of
// fused-kernel wave `wave`, each lane standing where that wave's lane stood:
// with m* the largest running max and weights w = 2^(m - m*) l, acc =
// sum w O_part and l = sum w, taken online over chunks of kMergeChunk
// partials, all of a chunk's loads issued before any is used.
constexpr int kMergeChunk = 8;
template <int D, class Slot>
__device__ __forceinline__ void merge_partials(const float* ws, int np, const Slot& slot, int wave,
                                               int db, int lane, f32x16& acc, float& l) {
  constexpr int NDB = D / 32, NQ = 4 * NDB, C = kMergeChunk;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  acc = f32x16{};
  l = 0.0f;
  float m = -3.0e38f;
  for (int k0 = 0; k0 < np; k0 += C) {
    f32x4 ml[C], o[C][4];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      // Past np, partial np - 1 again, weighed 0.
      const float* const w = ws + (size_t)slot(k0 + j < np ? k0 + j : np - 1) * seg_floats(D);
      ml[j] = reinterpret_cast<const f32x4*>(w + seg_ml_offset(D))[wave * 64 + lane];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        o[j][rr] = reinterpret_cast<const f32x4*>(w)[(wave * NQ + db * 4 + rr) * 64 + lane];
    }
    float mc = m;
#pragma unroll
    for (int j = 0; j < C; ++j)
      if (k0 + j < np) mc = fmaxf(mc, ml[j][0]);
    const float sc = __builtin_amdgcn_exp2f(m - mc);
    l *= sc;
    acc *= sc;
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const float a = k0 + j < np ? __builtin_amdgcn_exp2f(ml[j][0] - mc) * ml[j][1] : 0.0f;
      l += a;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[4 * rr + c] = __builtin_fmaf(a, o[j][rr][c], acc[4 * rr + c]);
    }
    m = mc;
  }
}

// Merge of a dense call's tail round: one workgroup of one wave per tail
// tile and wave of the fused kernel (blockIdx.y), each lane standing where
// the fused kernel's lane with the same query and dims stood.  Tile ti's
// partial results: its lead segment's (workspace slot ti) and those of the
// helpers hh whose slice [hh Lh, (hh + 1) Lh) of the tile-end span meets
// [ti e, (ti + 1) e) (slot t + ti + hh).  Each partial holds its output
// normalised by its own row sum l, taken against its own running max m
// (log2 domain); with m* the largest m and weights w = 2^(m - m*) l,
// O = sum w O_part / sum w, the partials taken lead first, then by helper,
// and the tile is rounded and stored like a whole unit's (merge_partials).
template <int D, StoreMode MODE>
__global__ __launch_bounds__(64) void fa_merge_kernel(FwdParams p) {
  const int lane = threadIdx.x;
  const int wave = blockIdx.y;
  const int l32 = lane & 31, g = lane >> 5;
  const int ns = (p.S + BN - 1) / BN;
  const int ti = blockIdx.x;
  const int tile = p.units + ti;
  const int bh = tile / p.nqt, qt = tile - bh * p.nqt;
  const int b = bh / p.H, h = bh - b * p.H;
  // Dynamic schedule: the tile's dyn_pieces pieces, slots ti * pieces + k.
  // Otherwise its lead and the helpers that met its end.
  const bool dyn = p.queue != nullptr;
  const int e = ns - p.tail_len, Lh = p.tail_hlen;
  const int h0 = !dyn && e > 0 ? ti * e / Lh : 0;
  const int np = dyn ? p.dyn_pieces : e > 0 ? ((ti + 1) * e - 1) / Lh - h0 + 2 : 1;
  auto slot = [&](int k) {
    return dyn ? ti * p.dyn_pieces + k : k == 0 ? ti : p.tail + ti + h0 + k - 1;
  };
  const int db = blockIdx.z;
  f32x16 acc[1];
  float l;
  merge_partials<D>(p.ws, np, slot, wave, db, lane, acc[0], l);
  // l is already the whole row's (each partial's sum covers both wave halves).
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  store_rows<D, MODE, 1>(p, acc, inv, qt * 256 + wave * 32 + l32, 32 * db, b, h, bh, g, lane);
}

// Merge of a split launch cut into pieces: one workgroup of one wave per half
// tile and group-0 wave (blockIdx.y), each lane where that wave's lane stood.
// Half tile hf's pieces are the workspace slots hf * pieces + j; they are
// combined as in fa_merge_kernel and the half tile is stored like a split
// unit's.
template <int D, StoreMode MODE>
__global__ __launch_bounds__(64) void fa_merge_split_kernel(FwdParams p) {
  const int lane = threadIdx.x;
  const int wave = blockIdx.y;
  const int l32 = lane & 31, g = lane >> 5;
  const int hf = blockIdx.x;
  const int tile = p.unit_base + (hf >> 1);
  const int bh = tile / p.nqt, qt = tile - bh * p.nqt;
  const int b = bh / p.H, h = bh - b * p.H;
  const int np = p.split_pieces;
  auto slot = [&](int k) { return hf * np + k; };
  const int db = blockIdx.z;
  f32x16 acc[1];
  float l;
  merge_partials<D>(p.ws, np, slot, wave, db, lane, acc[0], l);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  store_rows<D, MODE, 1>(p, acc, inv, qt * 256 + (hf & 1) * 128 + wave * 32 + l32, 32 * db, b, h,
                         bh, g, lane);
}

__global__ void fa_queue_reset_kernel(int* queue) { *queue = 0; }

int launch_queue_reset(int* queue, hipStream_t stream) {
  if (!queue) return -1;
  hipLaunchKernelGGL(fa_queue_reset_kernel, dim3(1), dim3(1), 0, stream, queue);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Kernel form of each variant: split-key units, masked units.
template <Variant VAR> constexpr bool kSplit = VAR != Variant::Whole;
template <Variant VAR> constexpr bool kMasked = VAR == Variant::Masked;

template <Variant VAR, int D, StoreMode MODE, bool NEG, bool SLAB_IN, int INSTR = 0>
static int launch_one(const FwdParams& p, int grid_cap, hipStream_t stream) {
  // A tail round spreads over every slot of the grid.
  const int grid = p.tail > 0 || p.units >= grid_cap ? grid_cap : p.units;
  hipLaunchKernelGGL((fa_fwd_pp_kernel<D, MODE, NEG, kSplit<VAR>, kMasked<VAR>, SLAB_IN, INSTR>),
                     dim3(grid), dim3(512), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <Variant VAR, int D, StoreMode MODE>
static int occupancy_one(int* blocks) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(
             blocks, fa_fwd_pp_kernel<D, MODE, false, kSplit<VAR>, kMasked<VAR>>, 512, 0) ==
                 hipSuccess
             ? 0
             : -1;
}

template <Variant VAR, int D>
static int occupancy_d(StoreMode mode, int* blocks) {
  return mode == StoreMode::Slab ? occupancy_one<VAR, D, StoreMode::Slab>(blocks)
                                 : occupancy_one<VAR, D, StoreMode::Plain>(blocks);
}

template <Variant VAR>
static int occupancy_v(int D, StoreMode mode, int* blocks) {
  return D == 128 ? occupancy_d<VAR, 128>(mode, blocks) : occupancy_d<VAR, 64>(mode, blocks);
}

int kernel_occupancy(int D, StoreMode mode, Variant var, int* blocks_per_cu) {
  if (D != 64 && D != 128) return -1;
  switch (var) {
    case Variant::Whole: return occupancy_v<Variant::Whole>(D, mode, blocks_per_cu);
    case Variant::Split: return occupancy_v<Variant::Split>(D, mode, blocks_per_cu);
    case Variant::Masked: return occupancy_v<Variant::Masked>(D, mode, blocks_per_cu);
  }
  return -1;
}

template <Variant VAR, int D, StoreMode MODE, bool SLAB_IN>
static int launch_sign(const FwdParams& p, int grid_cap, hipStream_t stream) {
  return p.c < 0.0f ? launch_one<VAR, D, MODE, true, SLAB_IN>(p, grid_cap, stream)
                    : launch_one<VAR, D, MODE, false, SLAB_IN>(p, grid_cap, stream);
}

// Slab-layout inputs are instantiated with slab outputs only.
template <Variant VAR, int D>
static int launch_d(StoreMode mode, const FwdParams& p, int grid_cap, hipStream_t stream,
                    bool slab_in) {
  if (slab_in)
    return mode == StoreMode::Slab ? launch_sign<VAR, D, StoreMode::Slab, true>(p, grid_cap, stream)
                                   : -1;
  return mode == StoreMode::Slab ? launch_sign<VAR, D, StoreMode::Slab, false>(p, grid_cap, stream)
                                 : launch_sign<VAR, D, StoreMode::Plain, false>(p, grid_cap, stream);
}

template <Variant VAR>
static int launch_v(int D, StoreMode mode, const FwdParams& p, int grid_cap, hipStream_t stream,
                    bool slab_in) {
  return D == 128 ? launch_d<VAR, 128>(mode, p, grid_cap, stream, slab_in)
                  : launch_d<VAR, 64>(mode, p, grid_cap, stream, slab_in);
}

// Instrumented instances: D = 128, slab output, c > 0, [B][H][S][D] inputs.
template <Variant VAR>
static int launch_instr(int instr, const FwdParams& p, int grid_cap, hipStream_t stream) {
  switch (instr) {
    case 1: return launch_one<VAR, 128, StoreMode::Slab, false, false, 1>(p, grid_cap, stream);
    case 2: return launch_one<VAR, 128, StoreMode::Slab, false, false, 2>(p, grid_cap, stream);
    case 3: return launch_one<VAR, 128, StoreMode::Slab, false, false, 3>(p, grid_cap, stream);
  }
  return -1;
}

template <int D, StoreMode MODE>
static int launch_merge_dm(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((fa_merge_kernel<D, MODE>), dim3(p.tail, 8, D / 32), dim3(64), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <int D, StoreMode MODE>
static int launch_merge_split_dm(const FwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((fa_merge_split_kernel<D, MODE>), dim3(p.units / p.split_pieces, 4, D / 32),
                     dim3(64), 0, stream, p);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_merge_split(int D, StoreMode mode, const FwdParams& p, hipStream_t stream) {
  if (p.split_pieces <= 1 || !p.ws || p.units % p.split_pieces != 0) return -1;
  if (D == 128)
    return mode == StoreMode::Slab ? launch_merge_split_dm<128, StoreMode::Slab>(p, stream)
                                   : launch_merge_split_dm<128, StoreMode::Plain>(p, stream);
  if (D == 64)
    return mode == StoreMode::Slab ? launch_merge_split_dm<64, StoreMode::Slab>(p, stream)
                                   : launch_merge_split_dm<64, StoreMode::Plain>(p, stream);
  return -1;
}

int launch_merge(int D, StoreMode mode, const FwdParams& p, hipStream_t stream) {
  if (p.tail <= 0 || !p.ws) return -1;
  if (D == 128)
    return mode == StoreMode::Slab ? launch_merge_dm<128, StoreMode::Slab>(p, stream)
                                   : launch_merge_dm<128, StoreMode::Plain>(p, stream);
  if (D == 64)
    return mode == StoreMode::Slab ? launch_merge_dm<64, StoreMode::Slab>(p, stream)
                                   : launch_merge_dm<64, StoreMode::Plain>(p, stream);
  return -1;
}

int launch_fwd(int D, StoreMode mode, Variant var, const FwdParams& p, int grid_cap,
               hipStream_t stream, bool slab_in, int instr) {
  if (D != 64 && D != 128) return -1;
  if (instr != 0) {
    if (D != 128 || mode != StoreMode::Slab || slab_in || !(p.c > 0.0f) || !p.stamps ||
        instr < 1 || instr > 3)
      return -1;
    switch (var) {
      case Variant::Whole: return launch_instr<Variant::Whole>(instr, p, grid_cap, stream);
      case Variant::Split: return launch_instr<Variant::Split>(instr, p, grid_cap, stream);
      case Variant::Masked: return launch_instr<Variant::Masked>(instr, p, grid_cap, stream);
    }
    return -1;
  }
  switch (var) {
    case Variant::Whole: return launch_v<Variant::Whole>(D, mode, p, grid_cap, stream, slab_in);
    case Variant::Split: return launch_v<Variant::Split>(D, mode, p, grid_cap, stream, slab_in);
    case Variant::Masked: return launch_v<Variant::Masked>(D, mode, p, grid_cap, stream, slab_in);
  }
  return -1;
}

}  // namespace fa
