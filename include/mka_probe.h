/*
 * mka_probe.h -- on-device peak probes that the FastMKA measurements are read
 * against, beside the published MI355X peaks.  They compute nothing of the
 * layer.
 *
 * Under sustained matrix-core load the shader clock of an MI355X drops well
 * below its 2.4 GHz peak, so the published dense bf16 MFMA figure (2.5
 * PFLOP/s) is not reachable by any kernel; a kernel's fraction of the
 * measured MFMA rate shows how much of what the chip sustains it uses.  The
 * same holds for HBM: the stream probe reads a buffer once.
 *
 * Conventions as in mka.h: device pointers, asynchronous on ``stream``
 * (a hipStream_t, NULL = default), MKA_OK or a negative MKA_ERR_* code,
 * arguments checked before anything is launched.
 */
#ifndef MKA_PROBE_H
#define MKA_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Dense bf16 MFMA loop: ``workgroups`` workgroups of four waves; each wave
 * issues ``iters`` rounds of four independent 32x32x16 bf16 MFMAs (fp32
 * accumulate), so one call performs workgroups * 4 * iters * 4 * 32768 flops.
 * One float per workgroup is written to ``sink`` (its value has no meaning; it
 * keeps the products live).  workgroups in [1, 65536], iters in [1, 2^24];
 * ``sink`` holds >= workgroups floats. */
int mka_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* sink, void* stream);

/* Streaming read of ``bytes`` bytes at ``src`` (16-byte aligned, bytes a
 * multiple of 16) with 16-byte loads, every byte read once; one float per
 * workgroup of the fixed grid (2048 workgroups of 256 threads) is written to
 * ``sink`` (>= 2048 floats). */
int mka_probe_stream_read(const void* src, size_t bytes, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MKA_PROBE_H */
