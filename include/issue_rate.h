/*
 * issue_rate.h - gfx950 instruction-issue microbenchmark (libissue_rate.so, built
 * beside libattn.so; a measurement tool, not part of the attention ABI).
 *
 * The tile pipeline of Rao et al., "Scheduling Data to Compute: Hierarchical Data
 * Pipelining for LLM Training on AMD GPUs", section 2.1, keeps the compute units
 * busy while tiles stream. On gfx950 the streaming is global_load_lds copies that
 * each wave issues, and the softmax between the products is vector-unit work.
 * These two calls measure what a wave pays for each.
 */
#ifndef MI355_ISSUE_RATE_H
#define MI355_ISSUE_RATE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Modes of valu_issue_bench: 8 instructions per loop iteration, either on 8
 * independent chains or on one dependent chain. */
enum {
    VALU_FMA_INDEPENDENT = 0,  /* x_k = fma(x_k, a, 1), k = 0..7 */
    VALU_EXP_INDEPENDENT = 1,  /* x_k = exp2(-x_k) (v_exp_f32, negated source) */
    VALU_FMA_DEPENDENT = 2,    /* x_0 = fma(x_0, a, 1), 8 times */
    VALU_EXP_DEPENDENT = 3     /* x_0 = exp2(-x_0), 8 times */
};

/*
 * One launch of `blocks` workgroups of 4 waves (blocks = 256 x W gives W waves per
 * SIMD on the 256 CUs); each wave runs `iters` iterations of its mode.
 *   a       the fma multiplier
 *   sink    device pointer, blocks * 256 floats: each thread's sum of its 8 chain
 *           values after the loop (keeps the results live; lane l starts chain k at
 *           l/1024 + k/8)
 *   cycles  device pointer, 8-byte aligned, blocks * 4 words: per wave, the
 *           shader-clock counter (s_memtime) difference over its loop
 *   stream  hipStream_t as void*; the call synchronises on it
 * Returns 0 on success, 2 for a bad mode, size or pointer, 3 for a HIP error.
 */
int valu_issue_bench(int mode, int blocks, int iters, float a, float* sink, unsigned long long* cycles, void* stream);

/*
 * One launch of `blocks` workgroups of 8 waves (one per CU: 64 KB of LDS each).
 * In every iteration, after a workgroup barrier, each of waves 0 .. active-1
 * issues `copies` (1..8) global_load_lds_dwordx4 copies of 1 KB (64 lanes x 16
 * bytes) into its own LDS area, wave w's copy n from byte
 * 65536 b + 1024 (copies w + n) of src for workgroup b, and waits for them.
 *   src     device pointer, 16-byte aligned, blocks * 65536 bytes
 *   iters   iterations (the same source each time: after the first it is in L2)
 *   cycles  device pointer, 8-byte aligned, blocks * 8 * 2 words: per wave, the
 *           summed shader-clock cycles from the barrier to the last copy's issue,
 *           then to all its copies having landed
 *   dst     device pointer, 16-byte aligned, blocks * 65536 bytes: each active
 *           wave writes its LDS area back to the same offsets as its source
 *   stream  hipStream_t as void*; the call synchronises on it
 * Returns 0 on success, 2 for a bad size or pointer, 3 for a HIP error.
 */
int copy_issue_bench(const void* src, int blocks, int copies, int active, int iters, unsigned long long* cycles,
                     void* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MI355_ISSUE_RATE_H */
