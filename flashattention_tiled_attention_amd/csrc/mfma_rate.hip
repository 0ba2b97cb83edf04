// Matrix-core rate microbenchmark for gfx950 (MI355X).
//
// How fast do the matrix cores of the whole chip run v_mfma_f32_32x32x16_bf16,
// the instruction every attention product here is made of, when nothing else
// limits them: no LDS, no memory traffic, no vector-unit work, only four
// independent accumulator chains per wave with operands already in registers?
// And at what shader clock? The attention kernels' time is set by their matrix
// work (Rao et al., "Scheduling Data to Compute: Hierarchical Data Pipelining for
// LLM Training on AMD GPUs", section 2.1: the data pipeline exists to keep the
// compute units busy), so this rate, measured on the operands the kernels see,
// is the ceiling their throughput is held against next to the 2.4 GHz spec
// figure.
//
// Each wave holds eight A and eight B operands (bf16x8 per lane, from a device
// buffer the caller fills: random values, zeros, ...) and issues eight MFMAs per
// loop iteration, two on each of four accumulators, with a different operand pair
// for every MFMA of the iteration, so the matrix unit's inputs change from one
// instruction to the next as they do in the attention kernels. Wave 0 of each
// workgroup reads the shader-clock counter (s_memtime) and the 100 MHz real-time
// counter (s_memrealtime) after a workgroup barrier at the start and at the end
// of the loop; their ratio is the mean shader clock of that workgroup's run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "mfma_rate.h"

namespace {

using attn::bf16x8;
using attn::f32x16;
using attn::u32x4;

constexpr int kThreads = 256;  // one wave per SIMD
constexpr int kOperands = 8;

__global__ void __launch_bounds__(kThreads) mfma_rate_kernel(const u32x4* __restrict__ ops, int iters,
                                                             float* __restrict__ sink,
                                                             unsigned long long* __restrict__ stamps) {
    const int lane = threadIdx.x & 63;
    bf16x8 a[kOperands], b[kOperands];
#pragma unroll
    for (int k = 0; k < kOperands; ++k) {
        a[k] = __builtin_bit_cast(bf16x8, ops[k * 64 + lane]);
        b[k] = __builtin_bit_cast(bf16x8, ops[(kOperands + k) * 64 + lane]);
    }
    f32x16 acc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] = attn::zero16();

    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < kOperands; ++k) acc[k & 3] = attn::mfma32(a[k], b[(k + 3) % kOperands], acc[k & 3]);
    }
    __syncthreads();
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();

    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[c][r];
    sink[blockIdx.x * kThreads + threadIdx.x] = s;
    if (threadIdx.x == 0) {
        stamps[4 * blockIdx.x + 0] = t0;
        stamps[4 * blockIdx.x + 1] = t1;
        stamps[4 * blockIdx.x + 2] = r0;
        stamps[4 * blockIdx.x + 3] = r1;
    }
}

}  // namespace

extern "C" {

int mfma_rate_bench(const void* operands, int blocks, int iters, float* ms_out, float* sink,
                    unsigned long long* stamps, void* stream) {
    if (!operands || !ms_out || !sink || !stamps || blocks < 1 || iters < 1) return 2;
    if (((uintptr_t)operands & 15u) || ((uintptr_t)sink & 3u) || ((uintptr_t)stamps & 7u)) return 2;
    if ((double)blocks * kThreads >= 4294967296.0) return 2;
    hipStream_t s = (hipStream_t)stream;
    const u32x4* ops = (const u32x4*)operands;
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(kThreads), 0, s, ops, 1, sink, stamps);  // warm-up
    if (hipGetLastError() != hipSuccess) return 3;
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return 3;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return 3;
    }
    int rc = 0;
    float ms = 0.0f;
    if (hipEventRecord(e0, s) != hipSuccess) rc = 3;
    if (!rc) {
        hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(kThreads), 0, s, ops, iters, sink, stamps);
        if (hipGetLastError() != hipSuccess) rc = 3;
    }
    if (!rc && (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
        rc = 3;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    *ms_out = ms;
    return rc;
}

}  // extern "C"
