/*
 * mfma_rate.h - gfx950 matrix-core rate microbenchmark (libmfma_rate.so, built
 * beside libattn.so; a measurement tool, not part of the attention ABI).
 *
 * It measures the whole chip's rate of v_mfma_f32_32x32x16_bf16, the instruction
 * of every attention product, with operands already in registers and nothing
 * else in the way, and the shader clock it runs at: the ceiling the attention
 * kernels' matrix work (Rao et al., "Scheduling Data to Compute: Hierarchical
 * Data Pipelining for LLM Training on AMD GPUs", section 2.1, whose data
 * pipeline exists to keep the compute units busy) is held against, on the
 * operand values they see.
 */
#ifndef MI355_MFMA_RATE_H
#define MI355_MFMA_RATE_H

#ifdef __cplusplus
extern "C" {
#endif

/*
 * One timed launch (after a one-iteration warm-up launch) of `blocks` workgroups
 * of 4 waves; every wave issues iters x 8 MFMAs (four accumulator chains, a
 * different operand pair for each of the 8 MFMAs of an iteration).
 *   operands     device pointer, 16-byte aligned, 16 x 64 x 16 bytes: the bf16x8
 *                operand of lane l for A operand k (k = 0..7) at byte
 *                16 (64 k + l), for B operand k at 16 (64 (8 + k) + l). Every
 *                wave uses the same values.
 *   blocks       workgroups; 256 per wave per SIMD of the 256 CUs
 *   ms_out       host pointer: the timed launch's duration (HIP events)
 *   sink         device pointer, blocks * 256 floats: each thread's sum of its
 *                64 accumulator values (keeps the products live)
 *   stamps       device pointer, 8-byte aligned, 4 * blocks words: per
 *                workgroup, the shader-clock counter (s_memtime) at the start
 *                and the end of its loop, then the 100 MHz real-time counter
 *                (s_memrealtime) at the same two points
 *   stream       hipStream_t as void*; the call synchronises on it
 * Returns 0 on success, 2 for bad sizes or pointers, 3 for a HIP error.
 */
int mfma_rate_bench(const void* operands, int blocks, int iters, float* ms_out, float* sink,
                    unsigned long long* stamps, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MI355_MFMA_RATE_H */
