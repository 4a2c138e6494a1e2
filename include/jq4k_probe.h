/*
 * jq4k_probe.h -- measurement kernels of libjq4k: the ceilings this GPU
 * reaches, reported beside the published peaks (8 TB/s HBM, 2.5 PFLOP/s
 * dense bf16) that the matmul roofline fractions are taken against.  Not part
 * of the matmul path.
 */
#ifndef JQ4K_PROBE_H
#define JQ4K_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

/* Streaming read of `bytes` (a multiple of 16) at device pointer p (16-byte
 * aligned): `workgroups` workgroups of 256 threads stride over the buffer,
 * 16 bytes per load, eight loads in flight per thread.  sink: device, one
 * uint32 per thread (workgroups * 256), written with the XOR of what the
 * thread read.  Returns 0, -1 for a bad argument (nothing launched), or the
 * launch's hipError_t. */
int jq4k_probe_read(const void *p, size_t bytes, uint32_t *sink, int workgroups,
                    hipStream_t stream);

/* Streaming read of `bytes` (a multiple of 16) at device pointer p (16-byte
 * aligned) in the pattern that reads HBM fastest here: one workgroup of 256
 * threads per 36 KB, each thread nine non-temporal 16-byte loads in flight,
 * every wave instruction 1 KB of consecutive bytes.  sink: device, at least
 * 256 uint32, written only when the XOR of a thread's bytes has one magic
 * value (it keeps the loads live).  Returns 0, -1 for a bad argument
 * (nothing launched), or the launch's hipError_t. */
int jq4k_probe_stream(const void *p, size_t bytes, uint32_t *sink, hipStream_t stream);

/* `iters` rounds of eight independent v_mfma_f32_32x32x16_bf16 (2 * 32 * 32 *
 * 16 flops each) per wave, register operands, `workgroups` workgroups of four
 * waves.  sink: device, one float per thread.  Returns 0, -1 for a bad
 * argument, or the launch's hipError_t. */
int jq4k_probe_mfma(long iters, float *sink, int workgroups, hipStream_t stream);

/* The inner loop of an int8-activation Q4_K matmul, from registers: per
 * sub-block of 32 k, the sixteen v_mfma_i32_16x16x32_i8 of a wave's 64 x 64
 * output tile (2 * 64 * 64 * 32 ops) and the fp32 rescale of each int32 sum
 * by the sub-block's weight scale and min and the activation block's scale,
 * `iters` sub-blocks, `workgroups` workgroups of four waves.  No loads, no
 * code unpacking, no activation quantisation: an upper bound on the rate
 * such a kernel reaches.  sink: device, one float per thread.  Returns 0,
 * -1 for a bad argument, or the launch's hipError_t. */
int jq4k_probe_mmq(long iters, float *sink, int workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* JQ4K_PROBE_H */
