/*
 * fa_instrument.h -- per-tile instrumentation of the fused attention kernel,
 * C ABI of libfa_relayout.so (same library as fa_relayout.h).
 *
 * The pages instrument each output tile of their fused kernels and report
 * the distribution of the spans over which a tile's remote stores are issued
 * and drained, and they contrast the piggybacked tile boundary (the owner
 * issues its tile's stores and resumes the next tile's Q-loop at once) with a
 * completion-coupled one (the owner waits for its stores to complete before
 * it resumes) ("Technical Summary: X-Stage in DiT Inference", Key
 * Contributions 3 and 4, Results: MegaMoE mechanism and FlashAttention-A2A
 * validation).  This entry point runs the same fused attention + slab store
 * as attn_fwd_relayout_async, in either form of the tile boundary, and
 * records shader-clock timestamps around every tile boundary.
 *
 * attn_fwd_relayout_instrumented_async: arguments q ... mask and stream as
 * for attn_fwd_relayout_async (the output is the same, bit for bit), plus
 *   boundary     0: the product kernel's piggybacked boundary -- the next
 *                unit's Q loads and first K/V stages are issued, then this
 *                unit's stores, and only the loads are waited for;
 *                1: the completion-coupled boundary -- the stores are issued
 *                and made visible device-wide (a device-scope release fence:
 *                L2 write-back, wait for completion), then the next unit's
 *                loads are issued;
 *                2: the stores, then the next unit's loads, with one wait
 *                for both (the stores drain while the loads are in flight,
 *                but the next Q-loop starts only once they are complete).
 *   stamps       device buffer of uint32, 16-byte aligned, at least
 *                attn_instrumented_stamp_words(B, H, S) words.  Units of the
 *                first launch (whole 256-query tiles, or masked 128-query
 *                tiles) come first, those of the second launch (split-key
 *                half tiles of a dense call's last round, if any) after
 *                them.  Record (unit u, wave w) = 8 words at
 *                ((u_offset + u) * 8 + w) * 8, u_offset = 0 for the first
 *                launch and launch_units[0] for the second:
 *                  [0] when the wait before unit u's Q-loop returned
 *                  [1] after the workgroup barrier that starts its Q-loop
 *                  [2] when its last K/V stage was done
 *                  [3] when its last store instruction was issued
 *                  [4] boundary 1 only: when its stores had completed (else 0)
 *                  [5] u   [6] the workgroup (blockIdx.x)
 *                  [7] high 32 bits of the clock at [3]
 *                [0]-[4] are the low 32 bits of the shader clock counter
 *                (s_memtime), which advances at the shader clock; differences
 *                are taken modulo 2^32.  The next unit a workgroup runs after
 *                unit u of a launch is u + (that launch's grid size); its
 *                record [0] minus u's [3] is the time the owner spent between
 *                issuing u's stores and being able to start the next Q-loop.
 *   launch_units host int[2] or NULL: receives the unit counts of the two
 *                launches (the second 0 when there is none).
 * Only D = 128 and scale > 0 are instrumented (FA_EUNSUPPORTED otherwise);
 * slab output, [B][H][S][D] inputs.  Status codes as attn_fwd_relayout_async,
 * plus FA_EINVAL (boundary not 0, 1 or 2, stamps NULL), FA_EALIGN (stamps not
 * 16-byte aligned) and FA_ERANGE (stamp_words too small), all checked before
 * any HIP call.  The timestamp stores add one store per wave and unit, so
 * timings differ slightly from the product kernel's.
 *
 * attn_instrumented_stamp_words: 64 * B * H * (ceil(S / 128) + 1), an upper
 * bound of the words a call needs (0 for non-positive sizes).
 */
#ifndef FA_INSTRUMENT_H
#define FA_INSTRUMENT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int attn_fwd_relayout_instrumented_async(const void* q, const void* k, const void* v,
                                         void* out_slabs, int B, int H, int S, int D, int P,
                                         float scale, const uint64_t* mask, int boundary,
                                         uint32_t* stamps, int64_t stamp_words,
                                         int* launch_units, void* stream);

int64_t attn_instrumented_stamp_words(int B, int H, int S);

#ifdef __cplusplus
}
#endif

#endif /* FA_INSTRUMENT_H */
