// LDS-to-register transpose microbenchmark for gfx950 (MI355X).
//
// Rao et al., "Scheduling Data to Compute: Hierarchical Data Pipelining for LLM
// Training on AMD GPUs", section 3.1.2 (Tables 4 and 5) and section 4.3.2
// (Table 10), compare ways of feeding a transposed operand from LDS to the
// matrix cores: the transpose load, strided 16-bit loads, and a plain row load
// followed by an XOR register shuffle, each against a plain row load of an
// operand that needs no transpose. This file measures the same four ways on
// gfx950, where the transpose load is ds_read_b64_tr_b16 (64 bits per lane).
//
// The operand is the one the attention kernels' P V product reads from the
// row-major V tile: for v_mfma_f32_32x32x16_bf16's A operand, lane l (column
// c = l % 32, half h = l / 32) needs 8 elements of one column, which in a
// row-major tile lie in 8 different rows. Methods:
//   0  ds_read_b128, no transpose: lane l reads 16 contiguous bytes. It delivers
//      an operand whose elements are adjacent in memory (the baseline), not the
//      transposed one.
//   1  ds_read_b64_tr_b16 x 2: the transpose load.
//   2  8 x 16-bit loads, one element from each row.
//   3  ds_read_b128 of 8 row elements, then an 8 x 8 transpose across groups
//      of 8 lanes in three XOR butterfly stages of DPP lane moves.
// Methods 1-3 deliver the same transposed operand, element e of lane (c, h)
// being V[8 (e / 4) + 4h + e % 4][c], the row order the transpose load produces
// and the attention kernels use (the check output holds every lane's operand at
// each of the eight positions a loop iteration loads). Every method reads 16 bytes of operand per lane per load. Each
// method reads the 64 x 64 bf16 tile in a layout free of bank conflicts for its
// access shape (checked with the LDS bank-conflict counter): the kernels'
// XOR-swizzled chunk order for the 16-byte row reads and the transpose load, a
// row pitch of 72 elements for the 16-bit column reads (the two half-waves read
// rows 4 apart). Method 3's row reads (8 rows x 2 chunks per 16 lanes, fixed by
// its shuffle partners) keep 2-way conflicts in every layout tried; its time is
// dominated by the shuffle's VALU work.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"
#include "lds_transpose.h"

namespace {

using attn::bf16x4;
using attn::bf16x8;
using attn::u32x4;

constexpr int kRows = 64, kCols = 64, kPitch2 = 72;
constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // operand loads per loop iteration

template <int METHOD>
__device__ __forceinline__ int tile_off(int row, int col) {
    return METHOD == 2 ? row * kPitch2 + col : attn::swz<kCols>(row, col);
}
// Row of element e of a lane in half h of the wave (the transpose load's order).
__device__ __forceinline__ int op_row(int e, int h) { return 8 * (e >> 2) + 4 * h + (e & 3); }

// Operand position p (0..kUnroll-1): a 16-row x 32-column block of the tile.
__device__ __forceinline__ int block_row(int p) { return 16 * (p & 3); }
__device__ __forceinline__ int block_col(int p) { return 32 * ((p >> 2) & 1); }

__device__ __forceinline__ uint32_t lo16(uint32_t x) { return x & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t x) { return x >> 16; }

// Lane exchanges inside rows of 16 lanes with DPP moves (VALU, no LDS traffic):
// xor 1 and xor 2 are quad permutations; xor 4 takes row_shl:4 (lane i reads
// lane i + 4) on lanes whose bit 2 is clear and row_shr:4 (lane i reads lane
// i - 4) on the others.
__device__ __forceinline__ uint32_t xchg1(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
}
__device__ __forceinline__ uint32_t xchg2(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
}
__device__ __forceinline__ uint32_t xchg4(uint32_t x, bool up) {
    const uint32_t from_above = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x104, 0xF, 0xF, false);
    const uint32_t from_below = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);
    return up ? from_below : from_above;
}

// Method 3's transpose: lanes 8q + i (i = 0..7) each hold row i of an 8 x 8 block
// of 16-bit elements (d[0..3], two elements per dword, element 2k in the low
// half of d[k]); afterwards lane i holds column i. Three butterfly stages
// exchange, with the lane at distance 4, 2, then 1, the elements whose index
// bit matches that distance.
__device__ __forceinline__ void transpose8x8(uint32_t (&d)[4], int i) {
    {   // distance 4: elements 4..7 (d2, d3) against the partner's 0..3 (d0, d1)
        const bool up = i & 4;
        const uint32_t s0 = up ? d[0] : d[2], s1 = up ? d[1] : d[3];
        const uint32_t r0 = xchg4(s0, up), r1 = xchg4(s1, up);
        if (up) { d[0] = r0; d[1] = r1; } else { d[2] = r0; d[3] = r1; }
    }
    {   // distance 2: elements 2, 3, 6, 7 (d1, d3) against the partner's 0, 1, 4, 5
        const bool up = i & 2;
        const uint32_t s0 = up ? d[0] : d[1], s1 = up ? d[2] : d[3];
        const uint32_t r0 = xchg2(s0), r1 = xchg2(s1);
        if (up) { d[0] = r0; d[2] = r1; } else { d[1] = r0; d[3] = r1; }
    }
    {   // distance 1: odd elements (high halves) against the partner's even ones
        const bool up = i & 1;
        // the halves to send, packed two per dword
        const uint32_t s0 = up ? (lo16(d[0]) | (lo16(d[1]) << 16)) : (hi16(d[0]) | (hi16(d[1]) << 16));
        const uint32_t s1 = up ? (lo16(d[2]) | (lo16(d[3]) << 16)) : (hi16(d[2]) | (hi16(d[3]) << 16));
        const uint32_t r0 = xchg1(s0), r1 = xchg1(s1);
        if (up) {   // received the partner's odd elements into our even slots
            d[0] = lo16(r0) | (d[0] & 0xffff0000u);
            d[1] = hi16(r0) | (d[1] & 0xffff0000u);
            d[2] = lo16(r1) | (d[2] & 0xffff0000u);
            d[3] = hi16(r1) | (d[3] & 0xffff0000u);
        } else {    // received the partner's even elements into our odd slots
            d[0] = lo16(d[0]) | (lo16(r0) << 16);
            d[1] = lo16(d[1]) | (hi16(r0) << 16);
            d[2] = lo16(d[2]) | (lo16(r1) << 16);
            d[3] = lo16(d[3]) | (hi16(r1) << 16);
        }
    }
}

template <int METHOD>
__device__ __forceinline__ u32x4 load_operand(const __bf16* tile, int p, int lane) {
    const int h = lane >> 5, c = lane & 31;
    const int r0 = block_row(p), c0 = block_col(p);
    if (METHOD == 0) {  // 16 contiguous bytes: the attention kernels' K-row reads,
                        // 32 rows at one 16-byte chunk per half-wave
        const int row = 32 * (p & 1) + c, col = 16 * ((p >> 1) & 3) + 8 * h;
        return __builtin_bit_cast(u32x4, attn::lds_read8(tile + tile_off<0>(row, col)));
    } else if (METHOD == 1) {  // transpose load: two 4-row halves
        const int row = r0 + 4 * h + ((lane & 15) >> 2);
        const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const bf16x4 a = attn::lds_read_tr(tile + tile_off<1>(row, col));
        const bf16x4 b = attn::lds_read_tr(tile + tile_off<1>(row + 8, col));
        return __builtin_bit_cast(u32x4, attn::concat(a, b));
    } else if (METHOD == 2) {  // one 16-bit element from each of 8 rows
        const uint16_t* t = (const uint16_t*)tile;
        uint32_t d[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t e0 = t[tile_off<2>(r0 + op_row(2 * k, h), c0 + c)];
            const uint32_t e1 = t[tile_off<2>(r0 + op_row(2 * k + 1, h), c0 + c)];
            d[k] = e0 | (e1 << 16);
        }
        return u32x4{d[0], d[1], d[2], d[3]};
    } else {  // row load + 8 x 8 shuffle transpose inside each group of 8 lanes
        const int i = c & 7, blk = c >> 3;  // lane i of column block blk
        const u32x4 row = __builtin_bit_cast(
            u32x4, attn::lds_read8(tile + tile_off<3>(r0 + op_row(i, h), c0 + 8 * blk)));
        uint32_t d[4] = {row[0], row[1], row[2], row[3]};
        transpose8x8(d, i);
        return u32x4{d[0], d[1], d[2], d[3]};
    }
}

template <int METHOD>
__global__ void __launch_bounds__(kThreads) lds_bench_kernel(int iters, uint32_t* operand_out,
                                                             uint32_t* checksum_out) {
    __shared__ __attribute__((aligned(16))) __bf16 tile[kRows * kPitch2];
    // element (r, c) holds the 16-bit pattern r * 64 + c, stored at its place in
    // this method's layout
    for (int k = threadIdx.x; k < kRows * kCols; k += kThreads) {
        const int r = k / kCols, c = k % kCols;
        ((uint16_t*)tile)[tile_off<METHOD>(r, c)] = (uint16_t)(r * kCols + c);
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    uint32_t acc[4] = {0u, 0u, 0u, 0u};  // four independent XOR chains
    if (blockIdx.x == 0 && threadIdx.x < 64) {
#pragma unroll
        for (int p = 0; p < kUnroll; ++p) {
            const u32x4 v = load_operand<METHOD>(tile, p, lane);
#pragma unroll
            for (int k = 0; k < 4; ++k) operand_out[(p * 64 + lane) * 4 + k] = v[k];
        }
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int p = 0; p < kUnroll; ++p) {
            const u32x4 v = load_operand<METHOD>(tile, p, lane);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] ^= v[k];
        }
        // the tile may have changed as far as the compiler knows: every iteration
        // loads again instead of reusing the first iteration's registers
        asm volatile("" ::: "memory");
    }
    checksum_out[blockIdx.x * kThreads + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <int METHOD>
hipError_t launch(int blocks, int iters, uint32_t* operand_out, uint32_t* checksum_out, hipStream_t s) {
    hipLaunchKernelGGL(lds_bench_kernel<METHOD>, dim3(blocks), dim3(kThreads), 0, s, iters, operand_out,
                       checksum_out);
    return hipGetLastError();
}

}  // namespace

extern "C" {

int lds_transpose_bench(int method, int blocks, int iters, int reps, float* ms_out,
                        unsigned int* operand_out, unsigned int* checksum_out, void* stream) {
    if (method < 0 || method > 3) return 1;
    if (blocks < 1 || iters < 1 || reps < 1 || !ms_out || !operand_out || !checksum_out) return 2;
    if (((uintptr_t)operand_out & 15u) || ((uintptr_t)checksum_out & 3u)) return 2;
    hipStream_t s = (hipStream_t)stream;
    auto run = [&](int n) -> hipError_t {
        switch (method) {
            case 0: return launch<0>(blocks, n, operand_out, checksum_out, s);
            case 1: return launch<1>(blocks, n, operand_out, checksum_out, s);
            case 2: return launch<2>(blocks, n, operand_out, checksum_out, s);
            default: return launch<3>(blocks, n, operand_out, checksum_out, s);
        }
    };
    if (run(1) != hipSuccess) return 3;  // warm-up
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return 3;
    if (hipEventCreate(&e1) != hipSuccess) { (void)hipEventDestroy(e0); return 3; }
    float best = 0.0f;
    int rc = 0;
    for (int r = 0; r < reps && !rc; ++r) {
        float ms = 0.0f;
        if (hipEventRecord(e0, s) != hipSuccess || run(iters) != hipSuccess ||
            hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
            hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
            rc = 3;
            break;
        }
        if (r == 0 || ms < best) best = ms;
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    *ms_out = best;
    return rc;
}

}  // extern "C"
