/*
 * fc_gguf_ceilings.h -- measured ceilings of the chip, for the benchmark
 * (libfcgceil.so; not part of the FC library).
 *
 * The FC kernels are reported against the published MI355X peaks (HBM3E
 * 8 TB/s; dense f16 matrix cores 2.5 PFLOP/s) and, beside them, against what
 * these two kernels reach on the same chip in the same run.
 *
 * Conventions: 0 on success, -1 on an invalid argument, -4 on a HIP launch
 * error.  Device pointers are HIP device memory of the current device;
 * `stream` is a hipStream_t (NULL = the null stream); launches are
 * asynchronous and stream-ordered.
 */
#ifndef FC_GGUF_CEILINGS_H
#define FC_GGUF_CEILINGS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * A plain coalesced read of `bytes` (a multiple of 16) of device memory
 * `src` (16-byte aligned): `grid` workgroups of 256 threads, each thread
 * reading `unroll` (1, 2, 4 or 8) 16-byte words per round with the rounds
 * strided over the grid.  Nothing is written in practice: `sink` (device,
 * 4 bytes) receives a word only if the read data fold to one fixed value.
 */
int fc_ceiling_stream_read(const void* src, int64_t bytes, int grid, int unroll, void* sink,
                           void* stream);

/*
 * Matrix-core rate: `grid` workgroups of 4 waves, each wave issuing `iters`
 * rounds of 4 independent 32x32 MFMAs: dtype 0 = v_mfma_f32_32x32x16_f16
 * (32768 flops each), dtype 1 = v_mfma_i32_32x32x32_i8 (65536 ops each).
 * `sink` (device, 4 bytes) is written only for one fixed result.
 */
int fc_ceiling_mfma(int dtype, int iters, int grid, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FC_GGUF_CEILINGS_H */
