/*
 * moe_bench.h -- measurement entry point of libmoe.so (not a step of the
 * layer): the MFMA ceiling that the grouped GEMMs' MFMA utilisation is read
 * against on MI355X (gfx950).
 *
 * moe_bench_mfma_ceiling runs the bf16 grouped GEMM's inner-loop pattern with
 * no global memory traffic: `blocks` workgroups of 512 threads (8
 * wavefronts, one workgroup per CU at a time since each takes all of LDS),
 * each wavefront doing `iters` rounds of 12 LDS fragment reads and 32
 * v_mfma_f32_16x16x32_bf16 in a ping-pong schedule (two barriers per round,
 * the second wavefront of each SIMD one phase behind the first).
 *   random_operands != 0: LDS holds random bf16 values (random mantissa and
 *     sign, exponents 2^-4..2^3), like the GEMMs' operands;
 *   random_operands == 0: LDS holds constant ones (the nominal MFMA rate).
 *   sink: device float array of blocks * 512 elements, caller-owned; the
 *     kernel writes one value per thread so its work is not removed.
 * Asynchronous on `stream` (a hipStream_t); time it with events.  The FLOPs
 * of one call are moe_bench_mfma_flops(blocks, iters).  Returns
 * MOE_ERR_INVALID_ARG for a NULL sink, blocks outside [1, 2^20] or iters < 1,
 * MOE_ERR_ALIGNMENT for a misaligned sink, MOE_ERR_HIP if the launch fails.
 */
#ifndef DROPLESS_MOE_BENCH_H
#define DROPLESS_MOE_BENCH_H

#include <stdint.h>

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

int64_t moe_bench_mfma_flops(int64_t blocks, int32_t iters);
moe_status_t moe_bench_mfma_ceiling(int32_t random_operands, int32_t iters, float* sink, int64_t blocks,
                                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DROPLESS_MOE_BENCH_H */
