/*
 * fp4q_membench.h -- C ABI of libfp4q_membench.so: K0, the hand-written HBM
 * probes that the quantizer's throughput is measured against on MI355X
 * (gfx950).  They are measurement kernels, not part of the quantizer.
 *
 * Every probe moves data in the quantizer's pattern: each wavefront owns
 * 4 KiB of consecutive units (64 lanes x 4 units; 16-byte units except for
 * the narrower reads), and every load or store instruction covers one
 * contiguous stretch of 64 units.  Pointers are DEVICE pointers; calls are
 * asynchronous on `stream` (a hipStream_t, NULL for the null stream) and
 * validate their arguments on the host first, returning the fp4q_status
 * codes of fp4q.h; a rejected call launches nothing.
 */
#ifndef FP4Q_MEMBENCH_H
#define FP4Q_MEMBENCH_H

#include <stdint.h>

#include "fp4q.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fp4q_k0_copy -- copy `bytes` bytes from src to dst (the copy ceiling).
 *   src, dst     16-byte aligned, non-overlapping; bytes a multiple of 16,
 *                at most 2^40.
 *   nontemporal  0: ordinary loads and stores; 1: non-temporal ones (nt);
 *                2: non-temporal loads and stores with nt and sc1, as the
 *                quantizer's input and BF16 dequant streams.  Other values:
 *                FP4Q_ERROR_INVALID_ARGUMENT.
 */
FP4Q_API fp4q_status fp4q_k0_copy(const void* src, void* dst, int64_t bytes, int nontemporal,
                                  void* stream);

/*
 * fp4q_k0_copy_stream -- the same copy by a fixed grid of `workgroups`
 * workgroups (1 to 2^20) of 256 lanes, whose wavefronts walk the 4 KiB
 * chunks with the grid's stride and load the next chunk before storing the
 * current one (a persistent, software-pipelined copy).
 */
FP4Q_API fp4q_status fp4q_k0_copy_stream(const void* src, void* dst, int64_t bytes,
                                         int nontemporal, int workgroups, void* stream);

/*
 * fp4q_k0_read -- read `bytes` bytes of src with loads of `width` bytes per
 * lane (1, 2, 4, 8 or 16; other widths: FP4Q_ERROR_INVALID_ARGUMENT),
 * non-temporal when `nontemporal` is nonzero,
 * writing nothing in practice: the XOR of everything read goes to sink[0]
 * only if it equals 0xFFFFFFFF.  The reference kernel for the HBM read
 * counters at each load width.
 *   src          width-aligned; bytes a multiple of width, at most 2^40.
 *   sink         uint32 [1], 4-byte aligned, device memory.
 */
FP4Q_API fp4q_status fp4q_k0_read(const void* src, int64_t bytes, int width, int nontemporal,
                                  uint32_t* sink, void* stream);

/*
 * fp4q_k0_mix -- read `bytes` bytes of src and write bytes / divisor bytes
 * to dst: each wavefront reads its 4 KiB and writes 4 KiB / divisor, the
 * XOR of `divisor` of its 16-byte units, contiguously (divisor 4 is the
 * routed-token quantizer's mix: 4 KiB of input and 1 KiB of codes per
 * wavefront; 1 is the copy).
 *   src, dst     16-byte aligned, non-overlapping; dst holds bytes / divisor.
 *   bytes        a multiple of 4096 (whole wavefront chunks), at most 2^40.
 *   divisor      1, 2 or 4 (else FP4Q_ERROR_INVALID_ARGUMENT).
 *   nontemporal  store mode as for fp4q_k0_copy (0, 1 or 2).
 */
FP4Q_API fp4q_status fp4q_k0_mix(const void* src, void* dst, int64_t bytes, int divisor,
                                 int nontemporal, void* stream);

/*
 * fp4q_k0_write -- write `bytes` bytes of an index-derived pattern to dst
 * (the write ceiling, and the reference kernel for the HBM write counter).
 *   dst          16-byte aligned; bytes a multiple of 16, at most 2^40.
 *   nontemporal  store mode as for fp4q_k0_copy (0, 1 or 2).
 */
FP4Q_API fp4q_status fp4q_k0_write(void* dst, int64_t bytes, int nontemporal, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* FP4Q_MEMBENCH_H */
