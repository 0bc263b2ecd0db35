/*
 * dcu_measure.h -- measured peaks of the device, for roofline fractions against what a kernel on
 * this GPU actually reaches next to the nominal figures (MI355X: HBM 8 TB/s, dense bf16 MFMA
 * 2.5 PFLOP/s). Measurement utilities of this library, not steps of the method. Conventions as in
 * dcu.h (device pointers, asynchronous on `stream`, host-side argument checks).
 */
#ifndef DCU_MEASURE_H
#define DCU_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * dcu_measure_stream_read -- read `bytes` of device memory once, in 16-byte non-temporal loads
 * (each wave reads 1 KB contiguous runs, 4 loads in flight per lane), `grid` workgroups of 256
 * threads walking the buffer with a grid stride. The achieved bandwidth is bytes / kernel time.
 * buf   device buffer, 16-byte aligned; contents arbitrary.
 * sink  one uint32 the kernel may write (so the loads are kept); its value is meaningless.
 * Errors: EINVAL on NULL pointers, bytes <= 0 or grid <= 0; EUNSUPPORTED if bytes % 16 != 0 or
 *         buf is not 16-byte aligned.
 */
int dcu_measure_stream_read(const void* buf, int64_t bytes, int32_t grid, uint32_t* sink,
                            void* stream);

/*
 * dcu_measure_mfma_loop -- `grid` workgroups of 4 waves, each wave issuing iters x 8 independent
 * v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 multiply-adds, 32768 flops each) on register operands:
 * the matrix-core rate is grid * 4 * iters * 8 * 32768 / kernel time.
 * sink  256 floats the kernel may write (so the work is kept); values meaningless.
 * Errors: EINVAL on a NULL sink, grid <= 0 or iters <= 0.
 */
int dcu_measure_mfma_loop(int32_t grid, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DCU_MEASURE_H */
