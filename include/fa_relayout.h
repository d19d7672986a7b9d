/*
 * fa_relayout.h -- fused FlashAttention forward + Ulysses head-to-sequence
 * re-layout for MI355X (gfx950).  C ABI of libfa_relayout.so.
 *
 * What it computes.  One GPU's share of Ulysses sequence-parallel attention
 * in diffusion-transformer inference (X-Stage abstract, CatalyzeX and fugumt
 * pages): for its H local heads over the whole sequence of S tokens, each
 * output tile of queries runs a non-causal FlashAttention forward pass (online
 * softmax over K/V tiles), and its owner stores the finished tile straight
 * into the sequence-sharded layout before resuming the next tile's Q-loop,
 * with no separate communication wavefront ("Technical Summary: X-Stage in
 * DiT Inference", Key Contributions 3, FlashAttention-A2A piggybacking).  On
 * one GPU the P destinations of the post-attention All-to-All are P local
 * slabs.  An optional per-head bitmask skips 128x128 tiles (bit-wise
 * block-sparse attention, ScalingAttention abstract on the CatalyzeX page).
 *
 *   O[b][h][s] = sum_j softmax_j(scale * <Q[b][h][s], K[b][h][j]>) V[b][h][j]
 *   slab p = s / (S/P), t = s % (S/P):
 *   out_slabs[p][b][t][h][d] = O[b][h][s][d]       (rounded to bf16, RNE)
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing, keeps no pointer after return and holds no
 *     state between calls other than a per-device cache of the CU count and
 *     occupancy; calls on different streams may run concurrently.
 *   - q, k, v: bf16 [B][H][S][D], contiguous, 16-byte aligned.
 *   - scale: multiplies Q K^T before the softmax; any finite value with
 *     |scale| <= 2^16 (0 gives the mean of V; negative values are allowed).
 *     The kernel forms scale * log2(e) * (q . k) in fp32; results meet the
 *     error bound of bf16 attention while that product stays below 2^24 in
 *     magnitude for every score (|q . k| < 2^7.5 at |scale| = 2^16, any
 *     score of unit-variance bf16 inputs at the usual 1/sqrt(D)).  Larger
 *     products are outside the contract, like NaN or Inf inputs.
 *   - mask: NULL for dense attention, else a device array of uint64 words
 *     [H][nT][W] with nT = ceil(S/128), W = ceil(nT/64), 8-byte aligned.
 *     Tile (i, j) of head h -- queries [128 i, 128 i + 128) against keys
 *     [128 j, 128 j + 128) -- takes part iff bit (j % 64) of word j / 64 of
 *     row (h, i) is set.  The same mask applies to every batch index.
 *     Masked tiles contribute nothing to the softmax; a query row whose
 *     tiles are all masked gets an output row of zeros.  Each 128-query
 *     tile is one work unit whose time grows with its row's kept tiles;
 *     each round of units is dealt in decreasing order of kept tiles, in
 *     alternating directions from round to round (a schedule every
 *     workgroup derives from the mask), which decides only where a tile is
 *     computed, never its result.
 *   - Keys at positions >= S do not exist (the ragged last tile is handled);
 *     rows >= S are never written.
 *   - Validation happens before any HIP call: on an error nothing is
 *     launched and nothing is written.
 *   - The _async entry points enqueue on `stream` (a hipStream_t; NULL is the
 *     null stream) and return; faults inside the kernel surface at the
 *     caller's next synchronisation.  The entry points without _async enqueue
 *     on the null stream and wait for completion, so they also report
 *     execution errors.
 *   - Outputs must not overlap the inputs (undefined behaviour otherwise).
 *
 * Return value: FA_OK (0) or one of the negative status codes below.
 */
#ifndef FA_RELAYOUT_H
#define FA_RELAYOUT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_OK 0
#define FA_EINVAL (-1)        /* null q/k/v/out; B, H, S or P <= 0; scale not finite or > 2^16 */
#define FA_EDIV (-2)          /* S is not a multiple of P */
#define FA_EUNSUPPORTED (-3)  /* D is not 64 or 128 (slab inputs: S/P < 64) */
#define FA_EALIGN (-4)        /* a tensor pointer not 16-byte aligned, mask not 8 */
#define FA_ERANGE (-5)        /* (S+256)*D*2 bytes per head >= 2^31, or too many tiles */
#define FA_ELAUNCH (-6)       /* the kernel launch was rejected */
#define FA_EDEVICE (-7)       /* no usable HIP device, or device query failed */
#define FA_EEXEC (-8)         /* (blocking entry points) execution failed */

#define FA_ABI_VERSION 1

/* Fused attention + slab store (the hot path).
 * out_slabs: bf16 [P][B][S/P][H][D], contiguous, 16-byte aligned; slab p is
 * the P-th contiguous block of B*(S/P)*H*D elements.  Enqueues on `stream`. */
int attn_fwd_relayout_async(const void* q, const void* k, const void* v,
                            void* out_slabs, int B, int H, int S, int D, int P,
                            float scale, const uint64_t* mask, void* stream);

/* As attn_fwd_relayout_async on the null stream, then waits for completion. */
int attn_fwd_relayout(const void* q, const void* k, const void* v,
                      void* out_slabs, int B, int H, int S, int D, int P,
                      float scale, const uint64_t* mask);

/* The whole Ulysses attention step on one GPU: both exchanges fused into the
 * attention kernel.  Ulysses sequence parallelism (named in the X-Stage
 * abstract, CatalyzeX and fugumt pages) exchanges twice around attention:
 * sequence -> head before it, head -> sequence after it.  The pages describe
 * fusing the second into FlashAttention; this entry point also fuses the
 * first into the Q/K/V loads (an extension the pages do not describe): the
 * inputs arrive sequence-sharded, q_slabs[p][b][t][h][d] = Q[b][h][p*(S/P) +
 * t][d] (the layout of out_slabs), and each tile's owner reads its head's
 * rows straight from the P slabs.  The result equals attn_fwd_relayout on the
 * same Q, K, V in [B][H][S][D] bit for bit.
 * q_slabs, k_slabs, v_slabs, out_slabs: bf16 [P][B][S/P][H][D], contiguous,
 * 16-byte aligned; outputs must not overlap inputs.  Same validation and
 * status codes as attn_fwd_relayout, plus FA_EUNSUPPORTED when S/P < 64 and
 * FA_ERANGE when one input tensor holds 2^31 bytes or more. */
int attn_fwd_slab_to_slab_async(const void* q_slabs, const void* k_slabs, const void* v_slabs,
                                void* out_slabs, int B, int H, int S, int D, int P, float scale,
                                const uint64_t* mask, void* stream);

int attn_fwd_slab_to_slab(const void* q_slabs, const void* k_slabs, const void* v_slabs,
                          void* out_slabs, int B, int H, int S, int D, int P, float scale,
                          const uint64_t* mask);

/* The same attention kernel writing the plain layout out[b][h][s][d]
 * (bf16 [B][H][S][D]) instead of the slabs: the measurement twin that the
 * fused store's overhead is taken against ("FlashAttention alone").  Same
 * arithmetic, so its values equal the slab output bit for bit. */
int attn_fwd_plain_async(const void* q, const void* k, const void* v, void* out,
                         int B, int H, int S, int D, float scale,
                         const uint64_t* mask, void* stream);

int attn_fwd_plain(const void* q, const void* k, const void* v, void* out,
                   int B, int H, int S, int D, float scale, const uint64_t* mask);

/* Standalone head-to-sequence re-layout: out_slabs[p][b][t][h][d] =
 * plain[b][h][p*(S/P) + t][d], a bit-exact copy of bf16 (or any 16-bit)
 * elements.  With attn_fwd_plain it forms the serial baseline the fused
 * kernel is measured against: attention first, then a separate exchange of
 * its output ("Technical Summary: X-Stage in DiT Inference", Results, the
 * serial FlashAttention-then-All-to-All execution the speedups are quoted
 * over; on one GPU the exchange is this local copy into P slabs).
 * plain: [B][H][S][D]; out_slabs: [P][B][S/P][H][D]; both contiguous, 16-byte
 * aligned, not overlapping.  Same validation and status codes as
 * attn_fwd_relayout (D must be 64 or 128; FA_ERANGE when B*H*S*D/8 >= 2^31).
 * HBM-bound: reads and writes B*H*S*D*2 bytes each. */
int relayout_to_slabs_async(const void* plain, void* out_slabs, int B, int H, int S, int D,
                            int P, void* stream);

int relayout_to_slabs(const void* plain, void* out_slabs, int B, int H, int S, int D, int P);

/* The dense calls above run the last, partial round of whole 256-query tiles
 * (when at most half as many tiles remain as the GPU has resident
 * workgroups; a fuller last round runs as whole tiles) as half tiles, the
 * keys split between a workgroup's two wave groups, which needs no memory
 * beyond the caller's tensors.  The _ws_ forms instead share that round among the workgroups.
 * A call of at least one full round whose last round holds t >= G/2 tiles
 * of at least 256 key stages runs a dynamic schedule: the full rounds
 * round-robin, then every later tile -- and the last t tiles cut into P =
 * min(6, 4 G / t) key pieces of falling length (piece j of P holding the
 * share (P - j) / (P (P + 1) / 2) of the keys), all first pieces before any
 * second -- handed to the workgroups one at a time, from a counter in the
 * workspace (zeroed by a launch of the call itself), as they free up: the
 * workgroups of one GPU do not all run at one speed, and the pieces let the
 * faster ones take more of the end.  Otherwise the round is spread over
 * every workgroup:
 * each of its t tiles is split at the same key stage L (about t/G of the
 * tile for G workgroups); workgroup i runs tile i's first L stages -- the t
 * leads start together and stream each tile's K/V in step, as full rounds
 * do -- and the other G - t workgroups run equal slices of the tiles'
 * remaining stages taken one tile after another.  Each piece writes its
 * partial result -- output normalised by its own row sum, running max, row
 * sum -- to the workspace, and a small second launch on the same stream
 * merges the partials of each tile and stores it like the fused kernel
 * does.  When that share L would be under 64 stages, the round runs as half
 * tiles as above, each cut into key pieces of at least 16 stages, one per
 * workgroup, merged the same way.  This balances the persistent owner
 * loop's last round (the schedule the pages'
 * fused kernels run their tiles in: "Technical Summary: X-Stage in DiT
 * Inference", Key Contributions 3) instead of leaving CUs idle; the result
 * equals the other form's within rounding (not bit for bit: the tail tiles'
 * sums are taken in another order).
 *   workspace: device memory owned by the caller, 16-byte aligned, at least
 *   attn_fwd_workspace_bytes(B, H, S, D) bytes for the current device (NULL
 *   and 0 are accepted when that is 0: masked calls and calls whose tiles
 *   fill whole rounds need none).  Its contents need no
 *   initialisation and are not meaningful afterwards; calls that may run
 *   concurrently need separate workspaces.
 * Status codes as attn_fwd_relayout_async / attn_fwd_plain_async, plus
 * FA_EINVAL (workspace NULL when one is needed, or workspace_bytes < 0),
 * FA_EALIGN (workspace not 16-byte aligned) and FA_ERANGE (workspace_bytes
 * too small), all checked before any kernel is launched. */
int attn_fwd_relayout_ws_async(const void* q, const void* k, const void* v, void* out_slabs,
                               int B, int H, int S, int D, int P, float scale,
                               const uint64_t* mask, void* workspace, int64_t workspace_bytes,
                               void* stream);

int attn_fwd_plain_ws_async(const void* q, const void* k, const void* v, void* out, int B, int H,
                            int S, int D, float scale, const uint64_t* mask, void* workspace,
                            int64_t workspace_bytes, void* stream);

/* attn_fwd_slab_to_slab_async with the last round spread as above: inputs
 * and output in the slab layout, workspace as for attn_fwd_relayout_ws_async
 * (attn_fwd_workspace_bytes gives the size).  Its result equals
 * attn_fwd_relayout_ws_async on the same Q, K, V in [B][H][S][D] bit for
 * bit.  Status codes as attn_fwd_slab_to_slab plus the workspace's. */
int attn_fwd_slab_to_slab_ws_async(const void* q_slabs, const void* k_slabs, const void* v_slabs,
                                   void* out_slabs, int B, int H, int S, int D, int P,
                                   float scale, const uint64_t* mask, void* workspace,
                                   int64_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the call of
 * attn_fwd_relayout_ws_async with the library's own workspace, a static
 * device array of 136 MiB that every GPU the library runs on holds until the
 * process ends, so a call needs no memory beyond q, k, v, out_slabs (and the
 * mask).  Same arguments (no workspace), status codes and result as
 * attn_fwd_relayout_ws_async; FA_ERANGE when a call would need more than the
 * array holds (only on GPUs with more than 512 resident workgroups; above
 * 256, where the dynamic schedule's pieces may not fit, a call whose pieces
 * do not runs the spread round instead, equal within rounding),
 * FA_EDEVICE when the array's device address cannot be obtained.  Every call
 * on one GPU shares that GPU's array: calls that may overlap on one GPU
 * (concurrent streams) race and must not be made; calls ordered on one
 * stream are safe.  Nothing carries over between calls (each call writes
 * every workspace slot it reads, and zeroes the dynamic schedule's counter
 * with a launch of its own before the kernel that counts), so nothing needs
 * clearing. */
int attn_fwd_relayout_noalloc_async(const void* q, const void* k, const void* v, void* out_slabs,
                                    int B, int H, int S, int D, int P, float scale,
                                    const uint64_t* mask, void* stream);

/* Bytes of workspace a dense _ws_ call of these sizes needs on the current
 * device (0 if none), or a negative status: FA_EINVAL (non-positive sizes),
 * FA_EUNSUPPORTED (D not 64 or 128), FA_ERANGE (sizes beyond the kernel's
 * index range), FA_EDEVICE (no usable device). */
int64_t attn_fwd_workspace_bytes(int B, int H, int S, int D);

/* Human-readable text of a status code (static storage, never NULL). */
const char* attn_status_string(int status);

/* FA_ABI_VERSION of the loaded library. */
int attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_RELAYOUT_H */
