/*
 * s5_peak.h - peak-rate probes of the roofline report (libs5_peak.so). They
 * measure the chip, not the S5 layer: the benchmark divides each forward
 * kernel's algorithmic bytes or flops per second by these measured rates
 * beside the vendor figures (HBM 8 TB/s, dense bf16 matrix cores 2.5 PF/s).
 *
 * Both run asynchronously on `stream`; time them with events on that stream.
 */
#ifndef S5_PEAK_H
#define S5_PEAK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

/*
 * s5_peak_copy - plain streaming copy dst[i] = src[i] of `bytes` bytes
 * (a multiple of 16; both device pointers 16-byte aligned, not overlapping):
 * 16-byte vector loads and stores (nontemporal != 0: streaming loads and
 * stores that bypass cache retention), grid-stride over all compute units.
 * One launch moves 2 * bytes of HBM traffic. Returns 0, or -1 for a bad
 * argument (nothing enqueued), or the HIP error code of the launch.
 */
int s5_peak_copy(const void* src, void* dst, int64_t bytes, int nontemporal, hipStream_t stream);

/*
 * s5_peak_mfma_bf16 - matrix-core throughput loop: `blocks` workgroups of
 * four waves, each wave running eight independent accumulation chains of
 * `iters` v_mfma_f32_16x16x32_bf16 instructions (16 x 16 x 32 multiply-adds,
 * 16384 flops each; iters a positive multiple of 4) on register operands,
 * with no memory traffic in the loop.
 * Flops per launch = blocks * 4 * 8 * iters * 16384. Each thread writes one
 * float of its sums to out[blocks * 256] (so the loop is not removed).
 * Returns 0, -1 for a bad argument (nothing enqueued), or the HIP error code.
 */
int s5_peak_mfma_bf16(int blocks, int iters, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* S5_PEAK_H */
