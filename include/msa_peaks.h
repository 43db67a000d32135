/* msa_peaks.h -- libmsa_peaks.so, the benchmark's measuring instrument.
 *
 * Not part of the attention library (libmsa.so, include/msa.h): this small
 * library measures the rate the GPU's matrix cores sustain for the
 * instruction the chunked-prefill kernel is built on, so that the bench can
 * report it beside the published dense bf16 peak.  Built by the same build
 * step as libmsa.so, for gfx950.
 */
#ifndef MSA_PEAKS_H
#define MSA_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Launch `workgroups` workgroups of 256 threads (four wavefronts) on `stream`
 * (a hipStream_t; NULL for the default stream).  Every wavefront issues
 * iters x 8 independent v_mfma_f32_32x32x16_bf16 on register operands -- no
 * memory traffic -- so one call performs workgroups * 4 * iters * 8 * 32768
 * floating-point operations; the caller times the call on the stream.
 *
 * sink: DEVICE buffer of at least workgroups * 256 floats, owned by the
 *       caller; each thread writes one sum of its accumulators there (this
 *       keeps the results live).  Its contents carry no meaning.
 *
 * Returns 0 when the launch was accepted (asynchronous: the kernel may still
 * be running), -1 without touching the GPU when workgroups or iters lies
 * outside [1, 2^20] or sink is NULL, otherwise the HIP error code of the
 * launch. */
int msa_peaks_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MSA_PEAKS_H */
