// Device helpers for the gfx950 attention kernels: MFMA operand types, bf16
// packing, LDS transpose loads and cross-half-wave reductions.
//
// MFMA lane layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64, lane l,
// half h = l / 32):
//   A (32 x 16): lane l holds A[l % 32][8h + e], e = 0..7
//   B (16 x 32): lane l holds B[8h + e][l % 32], e = 0..7
//   C (32 x 32): lane l, register r holds C[8 (r / 4) + 4h + (r % 4)][l % 32]
// A 32x32 accumulator therefore gives every lane one output column and 16 of
// its rows; used as the B operand of a following product, its rows become the
// contraction index in the order "k-slot 8h + e  <->  row 8 (e / 4) + 4h + e % 4"
// (for the first 16 rows; rows 16..31 likewise with r = 8..15). The matching A
// operand is read with that same row order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.0f;
    return z;
}

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                        float a6, float a7) {
    bf16x8 r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
    return r;
}

// Two fp32 values as one word of two bf16 (round to nearest even; x in the low half).
__device__ __forceinline__ uint32_t pack2_bf16(float x, float y) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r[0] = (__bf16)x;
    r[1] = (__bf16)y;
    return __builtin_bit_cast(uint32_t, r);
}

// Remainder of x after rounding it to bf16: x = bf16(x) + bf_lo(x) up to the
// rounding of the remainder, so a product with hi and lo bf16 operands carries
// about 16 significant bits of x.
__device__ __forceinline__ float bf_lo(float x) { return x - (float)(__bf16)x; }

__device__ __forceinline__ bf16x4 pack4(float a0, float a1, float a2, float a3) {
    bf16x4 r;
    r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
    return r;
}

__device__ __forceinline__ bf16x8 concat(bf16x4 lo, bf16x4 hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ds_read_b64_tr_b16. Each group of 16 lanes reads a 4-row x 16-column block of
// 16-bit elements: local lane 4r + c passes the address of row r, columns
// 4c..4c+3; local lane j receives column j, rows 0..3 as elements 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* lds_elem) {
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
    auto p = (ATTN_LDS v4bf*)((ATTN_LDS __bf16*)(lds_elem));
    v4bf r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p);
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 lds_read8(const __bf16* lds_elem) {
    return *(const bf16x8*)lds_elem;
}

// Element offset of (row, col) in an unpadded row-major bf16 tile of D columns
// whose 16-byte chunks are XOR-permuted per row. gfx950 LDS has 64 4-byte banks;
// ds_read_b128 serves 16 lanes per cycle and ds_read_b64_tr_b16 32 lanes per
// cycle. The permutation makes both access shapes the kernels use hit 16
// distinct 16-byte bank groups: 16 consecutive rows at one chunk (A-operand row
// reads) and 4 consecutive rows x 4 consecutive chunks (one transpose-read quad).
// The permutation depends on row & 15 only, so adding a multiple of 16 rows to
// an offset is a plain addition.
template <int D>
__device__ __forceinline__ int swz_f(int row) {
    static_assert(D == 64 || D == 128, "tile width");
    return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                    : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
    return row * D + ((((col >> 3) ^ swz_f<D>(row))) << 3) + (col & 7);
}

// Split of the direct copies of a [ROWS][W] bf16 tile (swz<W> order) over WAVES
// waves: one copy instruction moves 64 lanes x 16 bytes, a 1 KB run of whole rows.
template <int W, int ROWS, int WAVES>
struct CopyPlan {
    static constexpr int CH = W / 8;                        // 16-byte chunks per row
    static constexpr int ROWS_PER_COPY = 64 / CH;
    static constexpr int N = ROWS / ROWS_PER_COPY / WAVES;  // copies per wave
    static_assert(N >= 1 && N * ROWS_PER_COPY * WAVES == ROWS, "copy split");
};

// 32-bit LDS address of an LDS object named by a generic pointer: the generic
// address of LDS is the aperture base (zero in its low 32 bits) plus the LDS
// offset, so the low half is the LDS address. (An address-space cast would give
// the same value but tests the pointer for null first, which costs a 64-bit
// compare and a select in scalar registers for every copy.)
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    return (uint32_t)(uintptr_t)p;
}

// Asynchronous 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4):
// lane i's 16 bytes land at lds_wave_base + 16 i. lds_wave_base must be the same
// for every lane of the wave. Completion is tracked by vmcnt only: the caller
// waits with wait_copies() and then a workgroup barrier before any wave reads
// the destination. The instruction is issued from inline assembly on purpose:
// the compiler then does not know that LDS is being written behind its back, and
// does not make every later LDS read (of any slot) and every workgroup fence
// wait for the copy to land, which would expose the full copy latency in every
// step of the tile pipeline. The "memory" clobber keeps LDS accesses from moving
// across the copy. M0 (the LDS address of the copy) cannot be named as a clobber
// (the compiler reserves it); these kernels keep no value of their own in M0.
__device__ __forceinline__ void copy16_to_lds(const void* gsrc, void* lds_wave_base) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr_of(lds_wave_base));
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gsrc), "s"(lds)
        : "memory");
}
// The same copy from a wave-uniform base address held in scalar registers plus a
// per-lane 32-bit byte offset (the instruction's saddr form): a tile copy whose
// per-lane offsets are fixed then needs no vector address arithmetic per step.
// sbase must be the same for every lane of the wave.
__device__ __forceinline__ void copy16_to_lds_s(const void* sbase, uint32_t lane_byte_off, void* lds_wave_base) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr_of(lds_wave_base));
    // (readfirstlane returns a signed int: each half is taken back to 32 unsigned
    // bits before widening, or a low half with bit 31 set would fill the high half)
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t base = ((uint64_t)hi << 32) | lo;
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(lane_byte_off), "s"(base), "s"(lds)
        : "memory");
}
// The copies above with the LDS destination given as a 32-bit LDS address (no
// generic-to-LDS pointer conversion per copy); copy4_to_lds_a copies 4 bytes per
// lane (global_load_lds_dword): lane i's word lands at lds_addr + 4 i.
__device__ __forceinline__ void copy16_to_lds_sa(const void* sbase, uint32_t lane_byte_off, uint32_t lds_addr) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr);
    const uint64_t b = (uint64_t)(uintptr_t)sbase;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t base = ((uint64_t)hi << 32) | lo;
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(lane_byte_off), "s"(base), "s"(lds)
        : "memory");
}
__device__ __forceinline__ void copy16_to_lds_a(const void* gsrc, uint32_t lds_addr) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gsrc), "s"(lds)
        : "memory");
}
__device__ __forceinline__ void copy4_to_lds_a(const void* gsrc, uint32_t lds_addr) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, off"
        :
        : "v"(gsrc), "s"(lds)
        : "memory");
}
// s_waitcnt immediate that waits on the vector-memory counter alone: at most n of
// this wave's vector-memory operations (the copies above among them) in flight.
constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
// Workgroup barrier ordering LDS accesses only: it waits for this wave's LDS
// operations, not for its copies in flight (those are waited for by count).
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Wait until every copy this wave issued has landed in LDS (s_waitcnt 0). The
// compiler sees this wait, so it also knows that every vector-memory load it
// issued before is complete; otherwise it would keep counter waits for those
// loads inside the tile loop, and those would now also wait for the copies.
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0); }

// Combine a value with the same register of the lane 32 away (v_permlane32_swap).
__device__ __forceinline__ float halves_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// -inf where `mask` is all ones, else s, as one bitwise select (v_bfi_b32); mask is a
// sign-extended comparison (0 or all ones). The empty asm hides that origin from the
// compiler, which would otherwise turn the select back into a compare and a lane-mask
// select and fill the scalar registers with one 64-bit mask per score. Unlike adding
// -inf, the select also replaces a NaN score.
__device__ __forceinline__ float hide_if(int mask, float s) {
    asm("" : "+v"(mask));
    return __int_as_float((mask & (int)0xff800000u) | (~mask & __float_as_int(s)));
}

}  // namespace attn
