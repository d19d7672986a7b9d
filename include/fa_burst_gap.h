/*
 * fa_burst_gap.h -- store-burst microbenchmark for the Burst-Gap model, C ABI
 * of libfa_relayout.so (same library as fa_relayout.h).
 *
 * The pages model the sender-visible time to issue a burst of stores as
 * T_iss(G; K, V) = max(T0_iss(K, V), V / R - G): K producers issue a burst of
 * aggregate volume V, then compute for a gap G before the next burst; T0_iss is
 * the backpressure-free issue time, R the effective drain rate and Q the
 * outstanding capacity that sustained injection exhausts ("X-Stage" summary
 * page, Methodology: the X-Stage abstraction and the Burst-Gap model).  This
 * kernel measures those quantities for plain (or non-temporal) 128-bit stores
 * into local HBM on one MI355X: the local analogue of the pages' remote-store
 * microbenchmarks.
 *
 * burst_gap_run_async: `producers` workgroups of 256 threads, one per CU
 * (each asks for 96 KiB of LDS so no two share a CU), run `bursts` rounds:
 *   issue bytes_per_producer bytes of 16-byte stores (no wait for completion;
 *   coupled = 1: every wave then makes its stores visible device-wide -- a
 *   release fence at device scope, which writes the L2 back and waits for
 *   completion -- the completion-coupled issuer the pages contrast with the
 *   X-Stage view, remote visibility being visibility beyond the issuing
 *   XCD's L2 on one GPU),
 *   workgroup barrier, then `gap_iters` iterations of a dependent FMA chain
 *   (the compute gap), workgroup barrier.
 * Chunk c (16 bytes) of producer k in burst i lands at byte offset
 *   ((i * producers + k) * (bytes_per_producer / 16) + c) * 16 of dst
 * and holds the four uint32 {i, k, c, 0x9E3779B9}.
 * times (device, uint64, 3 * producers * bursts + 4 * producers entries):
 *   times[3 * (k * bursts + i) + 0..2] = shader-clock stamps (s_memtime) at
 *   the start of burst i, after its last store was issued by every wave of
 *   producer k, and after its gap; then, per producer k, at
 *   times[3 * producers * bursts + 4 * k + 0..3]: s_memtime and s_memrealtime
 *   (a constant 100 MHz clock) at kernel start, and both again after the
 *   producer waited for all of its stores to complete.
 * dst (device) needs bursts * producers * bytes_per_producer bytes, 16-byte
 * aligned; bytes_per_producer is a positive multiple of 4096; producers in
 * [1, 4096]; bursts in [1, 4096]; gap_iters >= 0; nontemporal 0 or 1 selects
 * plain or non-temporal stores; coupled 0 or 1.  Returns FA_OK or FA_EINVAL / FA_EALIGN /
 * FA_ERANGE (dst larger than 2^40 bytes) / FA_ELAUNCH / FA_EDEVICE, checked
 * before any HIP call.  Caller owns both buffers.
 */
#ifndef FA_BURST_GAP_H
#define FA_BURST_GAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int burst_gap_run_async(void* dst, uint64_t* times, int producers, int bytes_per_producer,
                        int bursts, int gap_iters, int nontemporal, int coupled, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_BURST_GAP_H */
