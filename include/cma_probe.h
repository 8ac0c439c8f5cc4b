/*
 * cma_probe.h -- microbenchmarks of the ceilings the library's kernels are
 * measured against (not part of the method's path). Each call validates its
 * arguments, enqueues one kernel on `stream` (a hipStream_t, NULL = default) and
 * returns CMA_OK, CMA_EINVAL (bad arguments, nothing launched) or CMA_EHIP; the
 * caller times the launch (HIP events) and owns every buffer.
 *
 * cma_probe_read:  n_wg workgroups of 512 threads stream `bytes` (device, 16-byte
 *                  aligned) once with 16-byte loads, four in flight per thread:
 *                  HBM read bandwidth for bytes >> the 256 MB last-level cache.
 *                  mode 0: a grid-stride loop; 1: each workgroup reads one
 *                  contiguous share in 8 KB runs. sink: device, n_wg * 512
 *                  uint32 (written only in a case that does not occur).
 * cma_probe_copy:  the same grid copies `bytes` from src to dst (16-byte aligned):
 *                  read + write bandwidth.
 * cma_probe_write: the same grid writes `bytes` to dst (16-byte aligned) with
 *                  16-byte stores: HBM write bandwidth. mode bit 0: non-temporal
 *                  stores (else plain); bit 1: each workgroup writes one
 *                  contiguous share in 8 KB runs (else a grid-stride loop).
 * cma_probe_valu:  n_wg workgroups of 256 threads; every lane runs `iters` rounds
 *                  of 8 independent chains of one vector operation (kind 0: the
 *                  hardware exp2, kind 1: fused multiply-add); out: device,
 *                  n_wg * 256 floats. Lane-operations per clock per SIMD give the
 *                  operation's issue rate.
 * cma_probe_mfma:  n_wg workgroups of 4 waves; every wave runs `iters` rounds of 8
 *                  independent 32x32x16 bf16 matrix products (2 * 32 * 32 * 16
 *                  flops each); out: device, n_wg * 256 floats.
 * cma_probe_lds:   n_wg workgroups of 512 threads (one per CU at a time) read a
 *                  64 KB LDS buffer `iters` times per lane in 16-byte reads, 8 in
 *                  flight, each wave instruction one conflict-free 1 KB run: the
 *                  LDS read bandwidth of a CU. sink: device, n_wg * 512 uint32.
 * cma_probe_l2:    n_wg workgroups of 8 waves each read the same `bytes` (a
 *                  multiple of 64 KB, small enough to stay in an XCD's 4 MB L2)
 *                  `iters` times with 1 KB-per-wave buffer loads, 8 in flight per
 *                  wave: the bandwidth from L2 into the compute units. sink as
 *                  for cma_probe_read (n_wg * 512 uint32).
 */
#ifndef CMA_PROBE_H
#define CMA_PROBE_H

#include <stdint.h>

#include "cma.h"

#ifdef __cplusplus
extern "C" {
#endif

int cma_probe_read(const void* src, int64_t bytes, int32_t n_wg, int32_t mode, void* sink, void* stream);
int cma_probe_copy(const void* src, void* dst, int64_t bytes, int32_t n_wg, void* stream);
int cma_probe_write(void* dst, int64_t bytes, int32_t n_wg, int32_t mode, void* stream);
int cma_probe_valu(int32_t kind, int32_t n_wg, int32_t iters, float* out, void* stream);
int cma_probe_mfma(int32_t n_wg, int32_t iters, float* out, void* stream);
int cma_probe_lds(int32_t n_wg, int32_t iters, void* sink, void* stream);
int cma_probe_l2(const void* buf, int32_t bytes, int32_t iters, int32_t n_wg, void* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* CMA_PROBE_H */
