/*
 * fa_probe.h - measurement probes of libfa_probe_mi355x.so (not on the
 * attention path; the attention ABI is fa.h).
 *
 * The benchmark reports, beside each attention throughput, the shader clock
 * the chip held during the timed launches and the bf16 matrix-core rate it
 * attains in a register-only loop, so that a result can be read against what
 * the hardware delivered and not only against its published peak (ZimaSpace,
 * "Wie reduziert Flash Attention den Speicherverkehr während der lokalen
 * Inferenz?", section "Hardware- und Formunterstützung entscheiden über die
 * Verwendung des schnellen Pfads").
 *
 * All pointers are device pointers the caller owns; nothing is allocated.
 * Return codes: 0 success, -1 invalid argument, -2 HIP error (launch failed,
 * or no current device).  Work is enqueued on `stream` (NULL: null stream).
 */
#ifndef FA_MI355X_FA_PROBE_H
#define FA_MI355X_FA_PROBE_H

#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Clock stamp on many compute units: FA_PROBE_STAMP_BLOCKS one-wave
 * workgroups, spread over the chip by the dispatcher, each storing
 * {s_memtime (the 64-bit shader-clock counter, which differs in offset between
 * compute units), s_memrealtime (the 64-bit constant-rate counter), a tag of
 * its compute unit ((XCC id << 8) | HW_ID bits 8-15)} at out[3 b .. 3 b + 2].
 * Two stamps around a region give its mean shader clock on every compute unit
 * both reached: d(memtime) / d(realtime) times the constant rate
 * (fa_probe_wallclock_khz), matched by tag.  out: 3 x FA_PROBE_STAMP_BLOCKS
 * uint64, 8-byte aligned. */
#define FA_PROBE_STAMP_BLOCKS 2048
int fa_probe_stamp(uint64_t* out, fa_stream_t stream);

/* Grid size and bf16 FLOPs of fa_probe_mfma(iters): one workgroup of 4 waves
 * per half compute unit of the current device, each wave issuing iters x 4
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each).  Pure host code. */
int fa_probe_mfma_query(int iters, int* blocks, double* flops);

/* The register-only MFMA loop.  stamps: 4 x blocks uint64 (blocks from the
 * query); lane 0 of each workgroup writes its {s_memtime, s_memrealtime} at
 * the start and at the end of its loop. */
int fa_probe_mfma(int iters, uint64_t* stamps, fa_stream_t stream);

/* Rate of the constant-rate counter in kHz (hipDeviceAttributeWallClockRate). */
int fa_probe_wallclock_khz(int* khz);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_FA_PROBE_H */
