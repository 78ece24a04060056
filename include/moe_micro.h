/*
 * moe_micro.h - microbenchmarks of the two ceilings the MoE layer's kernels
 * are measured against on an MI355X (gfx950): HBM stream bandwidth and the
 * issue rate of the block-scaled MFMA the expert GEMMs use (the FP8 x MXFP4
 * arithmetic of vLLM recipe "XiaomiMiMo/MiMo-V2.6-Pro-RL", sections
 * "Overview" and "AMD (MI355X, TP4)").  Built as libmoe_micro.so beside the
 * layer's library; bench.py --micro runs them.  They compute nothing of the
 * layer.
 *
 * All pointers are DEVICE pointers owned by the caller; work is enqueued on
 * `stream` and not waited for (time it with events on that stream).  Return
 * 0 on success, 1 for an invalid argument, 2 for an unsupported operand
 * format, 4 for a failed launch.
 */
#ifndef MOE_MICRO_H
#define MOE_MICRO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

/* Read `bytes` (a multiple of 16) of buf with 16-byte loads, four in flight
 * per lane, `grid` workgroups of 256 threads.  pattern 0: grid-stride (each
 * load instruction of a wave covers 1 KiB of consecutive bytes); pattern 1:
 * one contiguous chunk per workgroup; patterns 2 and 3: the same two with
 * non-temporal loads.  out [grid * 256] uint32 receives the XOR of what each
 * thread read.                                                             */
int moe_micro_hbm_read(const void* buf, size_t bytes, uint32_t* out, int grid, int pattern, hipStream_t stream);

/* Read floor(bytes / (16 group_stride)) regions in the pattern of the
 * streaming expert GEMMs over packed weights: one workgroup of 4 waves per
 * region of 16 groups of group_bytes (a multiple of 4 KiB holding an even
 * number of 2 KiB stages), group_stride bytes apart; wave w reads groups
 * 4w .. 4w+3 in 1 KiB blocks, two blocks per group per stage, two stages in
 * flight.  skew 0: every wave walks the stages from the first; 1: wave w
 * starts at stage w * nstage / 4; 2: workgroup b starts at (b mod 8) *
 * nstage / 8 (both wrap around).  nontemporal != 0: non-temporal loads.
 * out [grid * 256] uint32 receives the XOR of what each thread read.       */
int moe_micro_hbm_read_groups(const void* buf, size_t bytes, size_t group_bytes, size_t group_stride, int skew,
                              uint32_t* out, int nontemporal, hipStream_t stream);

/* Write `bytes` (a multiple of 16) of buf with 16-byte grid-stride stores.  */
int moe_micro_hbm_write(void* buf, size_t bytes, int grid, hipStream_t stream);

/* `grid` workgroups of 4 waves (256 threads); each wave issues `iters` rounds
 * of 8 (shape 32: v_mfma_scale_f32_32x32x64_f8f6f4, 131072 FLOP each) or 16
 * (shape 16: v_mfma_scale_f32_16x16x128_f8f6f4, 65536 FLOP each)
 * independent block-scaled MFMAs on register operands with unit scales.
 * fmt_a / fmt_b: operand formats 4/0 (e2m1 x e4m3, as the expert GEMMs),
 * 0/0 (e4m3 x e4m3) or 4/4 (e2m1 x e2m1).  out [grid * 256] floats keep the
 * accumulators live; clocks[0] = shader-clock cycles and clocks[1] =
 * constant-clock (100 MHz) ticks spent by workgroup 0 in its MFMA loop.    */
int moe_micro_mfma(int fmt_a, int fmt_b, int shape, int iters, int grid, float* out, unsigned long long* clocks,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MICRO_H */
