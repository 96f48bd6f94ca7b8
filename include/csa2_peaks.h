/*
 * csa2_peaks.h -- measurement helpers of libcsa2.  They are not steps of
 * the path: the benchmark times them to report the device's practical
 * ceilings beside the datasheet peaks it prices the roofline against.
 */
#ifndef CSA2_PEAKS_H
#define CSA2_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue one streaming read of `bytes` (a multiple of 16, 16-byte aligned
 * device buffer `buf`) on `stream` by a grid-stride kernel of 16-byte loads
 * that writes nothing (sink: a device word array of 4096 entries that it
 * never writes in practice).  Returns 0, or 1 for bad arguments, 4 for a
 * launch error.  Bytes / kernel time is the kernel-level HBM read rate. */
int csa2_peak_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Enqueue `iters` iterations of four independent 32x32x16 bf16 MFMA chains
 * in each of 4096 waves (four per SIMD on 256 CUs) on `stream`; sink as
 * above (1024 floats).  Returns the dense bf16 FLOPs the launch performs
 * (flops / kernel time = the practical bf16 matrix rate), or -1 on error. */
double csa2_peak_mfma(int iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_PEAKS_H */
