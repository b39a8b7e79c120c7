/*
 * moe_probes.h — measurement probes of the MI355X (gfx950) ceilings the roofline figures of the
 * MoE expert path are compared with.  They are not steps of the path: they measure what this
 * chip delivers under the same conditions the path's kernels run in, next to the datasheet peaks
 * (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16 MFMA).
 *
 * Conventions as in moe_mi355x.h: device pointers owned by the caller, work enqueued on `stream`
 * only, nothing allocated, MOE_OK or a negative moe_status (MOE_EINVAL before any launch for a
 * bad argument, MOE_ELAUNCH if the runtime refuses the launch), moe_last_error() for the text.
 */
#ifndef MOE_PROBES_H
#define MOE_PROBES_H

#include <stdint.h>

#include "moe_mi355x.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` bytes at `src` (16-byte aligned, bytes a multiple of 16) by
 * `blocks` workgroups of 256 threads, each thread loading 16-byte vectors in a grid-stride loop
 * and folding them into one 32-bit value.  `sink` (uint32 [blocks * 256]) receives those values
 * so the loads cannot be dropped.  Time it with events: bytes / time is the read ceiling the
 * weight-streaming kernels are compared with. */
moe_status moe_probe_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks, moe_stream stream);

/* Register-only bf16 MFMA loop: `blocks` workgroups of 256 threads (4 waves) each issue
 * iters * 8 v_mfma_f32_32x32x16_bf16 per wave on pseudo-random bf16 operands held in registers
 * (operands change from one instruction to the next, as in a GEMM), then write one fp32 value per
 * thread to `sink` (fp32 [blocks * 256]).  flops = blocks * 4 * iters * 8 * 32768; flops / time
 * is the MFMA ceiling under the clock this chip holds with that load. */
moe_status moe_probe_mfma_bf16(int64_t iters, float* sink, int32_t blocks, moe_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_PROBES_H */
