// Forward attention kernel for gfx950 (MI355X).
//
// Computes Eq. (1) of Rao et al., "Scheduling Data to Compute: Hierarchical
// Data Pipelining for LLM Training on AMD GPUs", section 2.1,
// O = softmax(Q K^T * scale) V, in the streaming form of that section's
// Algorithm 0: K/V tiles pass through LDS while each query row's running
// maximum m, running sum l and output accumulator stay in registers. The loop
// order is query tile outside, key/value tile inside, so the softmax state
// never leaves the chip (the same result as the algorithm's printed order).
//
// One workgroup = 4 waves = one tile of 128 query rows of one (batch, head);
// each wave owns 32 rows. Per 64-key tile:
//   S^T = K Q^T        v_mfma_f32_32x32x16_bf16, K from LDS (A), Q in registers (B)
//                      -> every lane holds one query column and 32 of its keys,
//                         so the row max/sum are lane-local plus one permlane32 swap
//   online softmax     exp2 with the scale folded into one fma per score
//   O^T += V^T P^T     P^T straight from the score registers (B), V^T read from
//                      the row-major V tile with ds_read_b64_tr_b16 (A)
// K/V tiles are double-buffered in LDS: the global loads of tile j+1 are in
// flight while tile j is multiplied. Causal tiles entirely above the diagonal
// are never loaded; the diagonal and ragged-tail tiles are masked.
#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kFwdBQ = 128;  // query rows per workgroup
constexpr int kFwdBK = 64;   // keys per LDS tile
constexpr int kFwdThreads = 256;

template <int D>
struct FwdTile {
    static constexpr int KP = D + 8;    // K row pitch in elements (conflict-free b128 reads)
    static constexpr int VP = D + 16;   // V row pitch (transpose reads)
    static constexpr int KTILE = kFwdBK * KP;
    static constexpr int VTILE = kFwdBK * VP;
    static constexpr int STAGE = KTILE + VTILE;
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static constexpr int CH = D / 8;                      // 16-byte chunks per row
    static constexpr int NLD = kFwdBK * CH / kFwdThreads;  // chunks per thread per tensor
};

// Work item of workgroup `bid`: (b, hq, query tile). Causal tiles are issued
// longest first. When the (b, kv-head) groups divide evenly over the 8 XCDs,
// all query heads of one group land on the same XCD (workgroups are dealt to
// XCDs round-robin by id), so its K/V stay in that XCD's L2.
__device__ __forceinline__ void decode_item(int bid, int nQ, int B, int Hkv, int G, bool causal,
                                            int& b, int& hq, int& qt) {
    const int C = B * Hkv;
    int rank, c, g;
    if ((C & 7) == 0) {
        const int x = bid & 7, s = bid >> 3, per = (C >> 3) * G;
        rank = s / per;
        const int rem = s - rank * per;
        c = (rem / G) * 8 + x;
        g = rem % G;
    } else {
        const int per = C * G;
        rank = bid / per;
        const int rem = bid - rank * per;
        c = rem / G;
        g = rem % G;
    }
    qt = causal ? nQ - 1 - rank : rank;
    b = c / Hkv;
    hq = (c % Hkv) * G + g;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kFwdThreads, 2) fwd_kernel(FwdArgs a) {
    using T = FwdTile<D>;
    constexpr int DK = D / 16;  // k-steps of the score product
    constexpr int DB = D / 32;  // 32-row blocks of O^T
    extern __shared__ __attribute__((aligned(16))) __bf16 smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    const int S = a.S;
    const int nQ = (S + kFwdBQ - 1) / kFwdBQ;
    int b, hq, qt;
    decode_item(blockIdx.x, nQ, a.B, a.Hkv, a.G, CAUSAL, b, hq, qt);
    const int hkv = hq / a.G;
    const size_t qbase = ((size_t)b * a.Hq + hq) * (size_t)S * D;
    const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)S * D;
    const uint16_t* Kp = a.k + kvbase;
    const uint16_t* Vp = a.v + kvbase;
    const int q0 = qt * kFwdBQ;
    const int qrow = q0 + 32 * wave + l32;
    const float c = a.scale_log2;

    // This lane's query row as B operands: Q[qrow][16 dk + 8h .. +7].
    bf16x8 qf[DK];
    if (qrow < S) {
        const u32x4* src = (const u32x4*)(a.q + qbase + (size_t)qrow * D + 8 * h);
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            u32x4 t = src[2 * dk];
            t ^= a.q_sign;
            qf[dk] = __builtin_bit_cast(bf16x8, t);
        }
    } else {
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) qf[dk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }

    const int nK = (S + kFwdBK - 1) / kFwdBK;
    const int jend = CAUSAL ? min(nK, (q0 + kFwdBQ - 1) / kFwdBK + 1) : nK;
    int wjend = CAUSAL ? min(jend, (q0 + 32 * wave + 31) / kFwdBK + 1) : jend;
    if (q0 + 32 * wave >= S) wjend = 0;  // a wave with no live rows only helps load

    u32x4 kst[T::NLD], vst[T::NLD];
    auto gload = [&](int j) {
        const int k0 = j * kFwdBK;
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const int ch = tid + kFwdThreads * i, row = ch / T::CH, col = (ch % T::CH) * 8;
            const int key = k0 + row;
            if (key < S) {
                kst[i] = *(const u32x4*)(Kp + (size_t)key * D + col);
                vst[i] = *(const u32x4*)(Vp + (size_t)key * D + col);
            } else {
                kst[i] = u32x4{0, 0, 0, 0};
                vst[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto lstore = [&](int stage) {
        __bf16* Ks = smem + stage * T::STAGE;
        __bf16* Vs = Ks + T::KTILE;
#pragma unroll
        for (int i = 0; i < T::NLD; ++i) {
            const int ch = tid + kFwdThreads * i, row = ch / T::CH, col = (ch % T::CH) * 8;
            *(u32x4*)(Ks + row * T::KP + col) = kst[i];
            *(u32x4*)(Vs + row * T::VP + col) = vst[i];
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = zero16();
    float m = -INFINITY, l = 0.0f;

    gload(0);
    lstore(0);
    __syncthreads();

    for (int j = 0; j < jend; ++j) {
        if (j + 1 < jend) gload(j + 1);
        if (j < wjend) {
            const __bf16* Ks = smem + (j & 1) * T::STAGE;
            const __bf16* Vs = Ks + T::KTILE;
            const int k0 = j * kFwdBK;

            f32x16 sacc[2] = {zero16(), zero16()};
#pragma unroll
            for (int dk = 0; dk < DK; ++dk) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const bf16x8 kf = lds_read8(Ks + (kb * 32 + l32) * T::KP + dk * 16 + 8 * h);
                    sacc[kb] = mfma32(kf, qf[dk], sacc[kb]);
                }
            }

            const bool need_mask = (k0 + kFwdBK > S) || (CAUSAL && k0 + kFwdBK - 1 > q0 + 32 * wave);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                        const bool ok = key < S && (!CAUSAL || key <= qrow);
                        if (!ok) sacc[kb][r] = -INFINITY;
                    }
            }

            float mx0 = sacc[0][0], mx1 = sacc[1][0];
#pragma unroll
            for (int r = 1; r < 16; ++r) {
                mx0 = fmaxf(mx0, sacc[0][r]);
                mx1 = fmaxf(mx1, sacc[1][r]);
            }
            const float mx = halves_max(fmaxf(mx0, mx1));
            const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
            const float mnew = fmaxf(m, mt);
            const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
            const float alpha = fast_exp2(m - muse);
            m = mnew;

            float rs0 = 0.f, rs1 = 0.f, rs2 = 0.f, rs3 = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; r += 2) {
                    const float s0 = sacc[kb][r], s1 = sacc[kb][r + 1];
                    float p0 = fast_exp2(fmaf(s0, c, -muse));
                    float p1 = fast_exp2(fmaf(s1, c, -muse));
                    if (need_mask) {
                        p0 = (s0 == -INFINITY) ? 0.0f : p0;
                        p1 = (s1 == -INFINITY) ? 0.0f : p1;
                    }
                    sacc[kb][r] = p0;
                    sacc[kb][r + 1] = p1;
                    if (kb == 0) { rs0 += p0; rs1 += p1; } else { rs2 += p0; rs3 += p1; }
                }
            l = l * alpha + ((rs0 + rs1) + (rs2 + rs3));
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

            // O^T += V^T P^T over four 16-key steps.
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const f32x16& sp = sacc[t >> 1];
                const int r0 = 8 * (t & 1);
                const bf16x8 pf = pack8(sp[r0], sp[r0 + 1], sp[r0 + 2], sp[r0 + 3], sp[r0 + 4],
                                        sp[r0 + 5], sp[r0 + 6], sp[r0 + 7]);
                const __bf16* vrow =
                    Vs + (16 * t + 4 * h + ((lane & 15) >> 2)) * T::VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x4 v1 = lds_read_tr(vrow + db * 32);
                    const bf16x4 v2 = lds_read_tr(vrow + db * 32 + 8 * T::VP);
                    oacc[db] = mfma32(concat(v1, v2), pf, oacc[db]);
                }
            }
        }
        if (j + 1 < jend) lstore((j + 1) & 1);
        __syncthreads();
    }

    const float lt = halves_sum(l);
    if (qrow < S) {
        const float inv = 1.0f / lt;
        uint16_t* op = a.o + qbase + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = db * 32 + 8 * g4 + 4 * h;
                const bf16x4 pk = pack4(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                                        oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
                *(bf16x4*)(op + d) = pk;
            }
        if (h == 0) a.lse[((size_t)b * a.Hq + hq) * S + qrow] = (m + log2f(lt)) * 0.69314718055994531f;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    const int nQ = (a.S + kFwdBQ - 1) / kFwdBQ;
    const long long blocks = (long long)a.B * a.Hq * nQ;
    hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(kFwdThreads),
                       FwdTile<D>::LDS_BYTES, stream, a);
    return hipGetLastError();
}

}  // namespace

// Raise the dynamic-LDS limit of every forward instance on the current device.
hipError_t fwd_setup_device() {
    hipError_t e;
    if ((e = hipFuncSetAttribute((const void*)fwd_kernel<64, false>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, FwdTile<64>::LDS_BYTES)))
        return e;
    if ((e = hipFuncSetAttribute((const void*)fwd_kernel<64, true>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, FwdTile<64>::LDS_BYTES)))
        return e;
    if ((e = hipFuncSetAttribute((const void*)fwd_kernel<128, false>,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, FwdTile<128>::LDS_BYTES)))
        return e;
    return hipFuncSetAttribute((const void*)fwd_kernel<128, true>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, FwdTile<128>::LDS_BYTES);
}

hipError_t launch_fwd(const FwdArgs& a, int D, hipStream_t stream) {
    if (D == 64) return a.causal ? launch_fwd_t<64, true>(a, stream) : launch_fwd_t<64, false>(a, stream);
    return a.causal ? launch_fwd_t<128, true>(a, stream) : launch_fwd_t<128, false>(a, stream);
}

}  // namespace attn
