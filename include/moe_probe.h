/* libmoe measurement probes -- not part of the MoE layer.
 *
 * Two kernels that show what the card reaches, in the same run as a benchmark of the layer, on the
 * two resources the layer's stages are bound by: a streaming device copy (HBM bandwidth) and a loop
 * of bf16 matrix instructions on register operands (MFMA throughput). Their results put the
 * layer's fractions of the published peaks (8 TB/s, 2.5 PFLOP/s dense bf16) beside what this
 * machine achieves at that moment, clock and power limits included.
 *
 * Both only enqueue work on `stream` (a hipStream_t, NULL = null stream) and return 0, -1 for an
 * invalid argument (checked on the host before any HIP call) or -4 for a failed launch.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst[0..bytes) = src[0..bytes): `blocks` blocks of 256 threads, 16 bytes per thread per step,
 * grid-stride. Device pointers, 16-byte aligned; bytes a positive multiple of 16; no overlap.
 * Bytes moved = 2 * bytes (read + write). */
int moe_probe_copy(const void* src, void* dst, int64_t bytes, int blocks, void* stream);

/* `blocks` blocks of 4 waves; each wave issues iters x 8 independent v_mfma_f32_32x32x16_bf16 on
 * register operands and writes one float per lane to out[blocks * 256] (device, 4-byte aligned).
 * Floating-point work = moe_probe_mfma_flops(blocks, iters). */
int moe_probe_mfma(int blocks, int iters, float* out, void* stream);
double moe_probe_mfma_flops(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
