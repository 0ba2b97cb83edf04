// Instruction-issue microbenchmark for gfx950 (MI355X): the two issue costs that
// shape the attention kernels' schedules.
//
// The data pipeline of Rao et al., "Scheduling Data to Compute: Hierarchical Data
// Pipelining for LLM Training on AMD GPUs", section 2.1, keeps the compute units
// busy while tiles stream; on gfx950 a tile streams through
// global_load_lds_dwordx4 copies that each wave issues itself, and the softmax
// between two products is vector-unit work. How much of a wave's time do these
// take?
//
// valu_issue_kernel: each wave runs a loop of 8 vector instructions per iteration,
//   v_fma_f32 (x = x a + 1) or v_exp_f32 (x = 2^-x, the negation a source
//   modifier), on 8 independent chains or on one dependent chain, and records the
//   shader-clock counter (s_memtime) around its loop. Both chains stay finite.
// copy_issue_kernel: a workgroup of 8 waves; after a barrier, each of the first
//   `active` waves issues `n` 1 KB copies (64 lanes x 16 bytes) from global memory
//   into its own part of LDS and records the counter before the first and after
//   the last issue, and again once its copies have landed (vmcnt 0). After the last
//   iteration the waves copy their LDS back out, so the caller can check that the
//   copies moved what they claim.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "issue_rate.h"

namespace {

constexpr int kValuThreads = 256;  // 4 waves
constexpr int kCopyWaves = 8;
constexpr int kCopyThreads = 64 * kCopyWaves;
constexpr int kCopyBytesPerBlock = 65536;  // 8 waves x up to 8 copies x 1 KB

template <int MODE>
__global__ void __launch_bounds__(kValuThreads) valu_issue_kernel(int iters, float a, float* __restrict__ sink,
                                                                  unsigned long long* __restrict__ cycles) {
    float x[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) x[k] = (threadIdx.x & 63) * (1.0f / 1024.0f) + 0.125f * k;
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
        if (MODE == VALU_FMA_INDEPENDENT) {
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = fmaf(x[k], a, 1.0f);
        } else if (MODE == VALU_EXP_INDEPENDENT) {
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = __builtin_amdgcn_exp2f(-x[k]);
        } else if (MODE == VALU_FMA_DEPENDENT) {
#pragma unroll
            for (int k = 0; k < 8; ++k) x[0] = fmaf(x[0], a, 1.0f);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) x[0] = __builtin_amdgcn_exp2f(-x[0]);
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += x[k];
    sink[blockIdx.x * kValuThreads + threadIdx.x] = s;
    if ((threadIdx.x & 63) == 0) cycles[blockIdx.x * (kValuThreads / 64) + (threadIdx.x >> 6)] = t1 - t0;
}

template <int N>
__global__ void __launch_bounds__(kCopyThreads, 1) copy_issue_kernel(const unsigned char* __restrict__ src,
                                                                     int active, int iters,
                                                                     unsigned long long* __restrict__ cycles,
                                                                     unsigned char* __restrict__ dst) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const size_t part = (size_t)blockIdx.x * kCopyBytesPerBlock + (size_t)wave * N * 1024;
    const unsigned char* from = src + part;
    const uint32_t to = attn::lds_addr_of(lds) + wave * N * 1024;
    unsigned long long issue = 0, land = 0;
    for (int it = 0; it < iters; ++it) {
        __syncthreads();
        const unsigned long long t0 = __builtin_amdgcn_s_memtime();
        if (wave < active) {
#pragma unroll
            for (int n = 0; n < N; ++n) attn::copy16_to_lds_sa(from + n * 1024, lane * 16u, to + n * 1024);
        }
        const unsigned long long t1 = __builtin_amdgcn_s_memtime();
        attn::wait_copies();
        const unsigned long long t2 = __builtin_amdgcn_s_memtime();
        issue += t1 - t0;
        land += t2 - t0;
    }
    __syncthreads();
    if (wave < active) {
#pragma unroll
        for (int n = 0; n < N; ++n)
            *(attn::u32x4*)(dst + part + n * 1024 + lane * 16) = *(const attn::u32x4*)(lds + wave * N * 1024 + n * 1024 + lane * 16);
    }
    if (lane == 0) {
        cycles[((size_t)blockIdx.x * kCopyWaves + wave) * 2 + 0] = issue;
        cycles[((size_t)blockIdx.x * kCopyWaves + wave) * 2 + 1] = land;
    }
}

template <int N>
void launch_copy(const unsigned char* src, int blocks, int active, int iters, unsigned long long* cycles,
                 unsigned char* dst, hipStream_t s) {
    hipLaunchKernelGGL(copy_issue_kernel<N>, dim3(blocks), dim3(kCopyThreads), kCopyBytesPerBlock, s, src, active, iters,
                       cycles, dst);
}

}  // namespace

extern "C" {

int valu_issue_bench(int mode, int blocks, int iters, float a, float* sink, unsigned long long* cycles, void* stream) {
    if (mode < 0 || mode > 3 || blocks < 1 || iters < 1 || !sink || !cycles) return 2;
    if (((uintptr_t)sink & 3u) || ((uintptr_t)cycles & 7u)) return 2;
    if ((double)blocks * kValuThreads >= 4294967296.0) return 2;
    hipStream_t s = (hipStream_t)stream;
    switch (mode) {
        case VALU_FMA_INDEPENDENT:
            hipLaunchKernelGGL(valu_issue_kernel<VALU_FMA_INDEPENDENT>, dim3(blocks), dim3(kValuThreads), 0, s, iters, a, sink, cycles);
            break;
        case VALU_EXP_INDEPENDENT:
            hipLaunchKernelGGL(valu_issue_kernel<VALU_EXP_INDEPENDENT>, dim3(blocks), dim3(kValuThreads), 0, s, iters, a, sink, cycles);
            break;
        case VALU_FMA_DEPENDENT:
            hipLaunchKernelGGL(valu_issue_kernel<VALU_FMA_DEPENDENT>, dim3(blocks), dim3(kValuThreads), 0, s, iters, a, sink, cycles);
            break;
        default:
            hipLaunchKernelGGL(valu_issue_kernel<VALU_EXP_DEPENDENT>, dim3(blocks), dim3(kValuThreads), 0, s, iters, a, sink, cycles);
            break;
    }
    if (hipGetLastError() != hipSuccess) return 3;
    return hipStreamSynchronize(s) == hipSuccess ? 0 : 3;
}

int copy_issue_bench(const void* src, int blocks, int copies, int active, int iters, unsigned long long* cycles,
                     void* dst, void* stream) {
    if (!src || !cycles || !dst || blocks < 1 || iters < 1 || copies < 1 || copies > 8 || active < 1 || active > 8)
        return 2;
    if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u) || ((uintptr_t)cycles & 7u)) return 2;
    if ((double)blocks * kCopyBytesPerBlock >= 9.0e15) return 2;
    hipStream_t s = (hipStream_t)stream;
    static bool lds_raised = false;  // 64 KB of dynamic LDS for every instance
    if (!lds_raised) {
        hipError_t e = hipSuccess;
        const void* k[8] = {(const void*)copy_issue_kernel<1>, (const void*)copy_issue_kernel<2>,
                            (const void*)copy_issue_kernel<3>, (const void*)copy_issue_kernel<4>,
                            (const void*)copy_issue_kernel<5>, (const void*)copy_issue_kernel<6>,
                            (const void*)copy_issue_kernel<7>, (const void*)copy_issue_kernel<8>};
        for (int i = 0; i < 8 && e == hipSuccess; ++i)
            e = hipFuncSetAttribute(k[i], hipFuncAttributeMaxDynamicSharedMemorySize, kCopyBytesPerBlock);
        if (e != hipSuccess) return 3;
        lds_raised = true;
    }
    const unsigned char* from = (const unsigned char*)src;
    unsigned char* to = (unsigned char*)dst;
    switch (copies) {
        case 1: launch_copy<1>(from, blocks, active, iters, cycles, to, s); break;
        case 2: launch_copy<2>(from, blocks, active, iters, cycles, to, s); break;
        case 3: launch_copy<3>(from, blocks, active, iters, cycles, to, s); break;
        case 4: launch_copy<4>(from, blocks, active, iters, cycles, to, s); break;
        case 5: launch_copy<5>(from, blocks, active, iters, cycles, to, s); break;
        case 6: launch_copy<6>(from, blocks, active, iters, cycles, to, s); break;
        case 7: launch_copy<7>(from, blocks, active, iters, cycles, to, s); break;
        default: launch_copy<8>(from, blocks, active, iters, cycles, to, s); break;
    }
    if (hipGetLastError() != hipSuccess) return 3;
    return hipStreamSynchronize(s) == hipSuccess ? 0 : 3;
}

}  // extern "C"
