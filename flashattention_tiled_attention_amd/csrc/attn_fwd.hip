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
// K and V tiles are double-buffered in LDS with K one tile ahead of V, so that
// each wave can overlap the score product of tile j+1 with the softmax of tile
// j, and the P V product of tile j with the row maxima of tile j+1; the global
// loads of the following tiles are in flight meanwhile. Causal tiles entirely
// above the diagonal are never loaded; the diagonal and ragged-tail tiles are
// masked.
#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr int kFwdBQ = 128;  // query rows per workgroup
constexpr int kFwdBK = 64;   // keys per LDS tile
constexpr int kFwdThreads = 256;

template <int D>
struct FwdTile {
    // K and V tiles are unpadded [64][D] bf16 with the swizzled chunk order of
    // swz<D>: conflict-free for the b128 row reads of K and the transpose reads of
    // V, and each 1 KB run of rows is contiguous, as the direct copies need.
    static constexpr int TILE = kFwdBK * D;               // elements
    static constexpr int LDS_BYTES = 4 * TILE * 2;        // 2 K slots + 2 V slots
    static constexpr int CH = D / 8;                      // 16-byte chunks per row
    static constexpr int ROWS_PER_COPY = 64 / CH;         // rows per wave copy (1 KB)
    static constexpr int COPIES = kFwdBK / ROWS_PER_COPY / 4;  // per wave per tensor
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

    // LDS: two K slots then two V slots.
    __bf16* const Kring = smem;
    __bf16* const Vring = smem + 2 * T::TILE;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);

    // Direct copies: copy n of this wave fills tile rows (wave*COPIES + n) *
    // ROWS_PER_COPY + lane / CH, physical chunk lane % CH, which holds logical
    // chunk (lane % CH) ^ swz_f(row). Rows past the end repeat row S-1: their
    // scores are masked and their probabilities are exactly 0.
    int crow[T::COPIES], ccol[T::COPIES];
#pragma unroll
    for (int n = 0; n < T::COPIES; ++n) {
        crow[n] = (wave_u * T::COPIES + n) * T::ROWS_PER_COPY + lane / T::CH;
        ccol[n] = (((lane % T::CH) ^ swz_f<D>(crow[n]))) * 8;
    }
    auto copy_tile = [&](const uint16_t* src, __bf16* dst, int j) {
        const int k0 = j * kFwdBK;
#pragma unroll
        for (int n = 0; n < T::COPIES; ++n) {
            const int key = min(k0 + crow[n], S - 1);
            copy16_to_lds(src + (size_t)key * D + ccol[n], dst + (wave_u * T::COPIES + n) * 512);
        }
    };
    // Per-lane read offsets (elements) into a slot: K rows (b128, A operand) for
    // each 16-wide k-step, and V transpose quads for each 32-column block and
    // row half; row offsets by multiples of 16 are added as constants.
    int koff[DK], voff[2][DB];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) koff[dk] = swz<D>(l32, dk * 16 + 8 * h);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < DB; ++db)
            voff[hf][db] = swz<D>(4 * h + ((lane & 15) >> 2) + 8 * hf,
                                  db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = zero16();
    float m = -INFINITY, l = 0.0f;
    bf16x8 pk[4];

    // S^T of key tile in K slot `slot` (two 32-key blocks).
    auto qk = [&](int slot, f32x16 (&sc)[2]) {
        const __bf16* Ks = Kring + slot * T::TILE;
        sc[0] = zero16();
        sc[1] = zero16();
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const bf16x8 kf = lds_read8(Ks + koff[dk] + kb * 32 * D);
                sc[kb] = mfma32(kf, qf[dk], sc[kb]);
            }
        }
    };
    // Causal diagonal / ragged tail: only a wave's last tile can hold invisible keys.
    auto mask = [&](int j, f32x16 (&sc)[2]) {
        const int lim = (CAUSAL ? min(qrow, S - 1) : S - 1) - j * kFwdBK - 4 * h;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) sc[kb][r] = -INFINITY;
    };
    // Row maximum of a tile (log2 units) and the lazy move of the running maximum:
    // m only moves when some row's maximum grows by more than max_slack (8 for
    // ordinary score spreads), so every exp2(t - m) stays <= 2^slack, carried by
    // fp32 and bf16 without loss, and the O rescale is skipped. The first tile
    // always moves it (m starts at -inf; key 0 is visible to every row).
    auto move_max = [&](const f32x16 (&sc)[2]) {
        float mx0 = fmaxf(sc[0][0], sc[0][1]), mx1 = fmaxf(sc[1][0], sc[1][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) {
            mx0 = fmaxf(mx0, sc[0][r]);
            mx1 = fmaxf(mx1, sc[1][r]);
        }
        const float mt = halves_max(fmaxf(mx0, mx1)) * c;  // c > 0
        if (__any(mt > m + a.max_slack)) {
            const float mnew = fmaxf(m, mt);
            const float alpha = fast_exp2(m - mnew);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
    };
    // P = exp2(t - m) as bf16 B operands (4 x 16 keys), row sums into l.
    auto softmax = [&](const f32x16 (&sc)[2]) {
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = fast_exp2(fmaf(sc[t >> 1][8 * (t & 1) + e], c, -m));
                rs[e & 3] += p[e];
            }
            pk[t] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        }
        l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    };
    // O^T += V^T P^T over four 16-key steps, V^T by transpose reads of slot `slot`.
    auto pv = [&](int slot) {
        const __bf16* Vs = Vring + slot * T::TILE;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x4 v1 = lds_read_tr(Vs + voff[0][db] + 16 * t * D);
                const bf16x4 v2 = lds_read_tr(Vs + voff[1][db] + 16 * t * D);
                oacc[db] = mfma32(concat(v1, v2), pk[t], oacc[db]);
            }
    };

    // Prologue: K0, V0 in slot 0, K1 in slot 1; scores of tile 0.
    copy_tile(Kp, Kring, 0);
    copy_tile(Vp, Vring, 0);
    if (jend > 1) copy_tile(Kp, Kring + T::TILE, 1);
    wait_copies();
    __syncthreads();

    f32x16 sa[2], sb[2];
    if (wjend > 0) {
        qk(0, sa);
        if (wjend == 1) mask(0, sa);
        move_max(sa);
    }
    // Iteration 0 refills K slot 0, which the scores above still read.
    __syncthreads();

    // Iteration j: K_{j+1} sits in K slot (j+1)&1 and V_j in V slot j&1, while
    // K_{j+2} and V_{j+1} stream from HBM straight into the slots the previous
    // iteration released. Steady iterations (tile j+1 exists and is unmasked for
    // this wave) are one branch-free block: the score product of tile j+1 is
    // interleaved with the exponentials of tile j, and the P V product of tile j
    // with the row maxima of tile j+1. Different waves of a workgroup may leave
    // the steady loop at different iterations; every iteration of either loop
    // ends in exactly one barrier, so the barrier counts stay equal.
    auto steady = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        copy_tile(Kp, Kring + (j & 1) * T::TILE, j + 2);
        copy_tile(Vp, Vring + ((j + 1) & 1) * T::TILE, j + 1);
        // Scheduling region 1: 16 x {score MFMA, K row read, 6 softmax VALU}.
        qk((j + 1) & 1, nxt);
        softmax(cur);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // Region 2: 16 x {P V MFMA, 2 V transpose reads, 2 row-max VALU}.
        pv(j & 1);
        float mx0 = fmaxf(nxt[0][0], nxt[0][1]), mx1 = fmaxf(nxt[1][0], nxt[1][1]);
#pragma unroll
        for (int r = 2; r < 16; ++r) {
            mx0 = fmaxf(mx0, nxt[0][r]);
            mx1 = fmaxf(mx1, nxt[1][r]);
        }
        const float mt = halves_max(fmaxf(mx0, mx1)) * c;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x402, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (__any(mt > m + a.max_slack)) {
            const float mnew = fmaxf(m, mt);
            const float alpha = fast_exp2(m - mnew);
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        }
        wait_copies();
        __syncthreads();
    };
    auto tail = [&](int j, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
        if (j + 2 < jend) copy_tile(Kp, Kring + (j & 1) * T::TILE, j + 2);
        if (j + 1 < jend) copy_tile(Vp, Vring + ((j + 1) & 1) * T::TILE, j + 1);
        if (j + 1 < wjend) {  // tile j+1 is this wave's last: masked
            qk((j + 1) & 1, nxt);
            softmax(cur);
            mask(j + 1, nxt);
            pv(j & 1);
            move_max(nxt);
        } else if (j + 1 == wjend) {
            softmax(cur);
            pv(j & 1);
        }
        wait_copies();
        __syncthreads();
    };

    const int jsteady = max(0, wjend - 2);
    int j = 0;
    for (; j + 1 < jsteady; j += 2) {
        steady(j, sa, sb);
        steady(j + 1, sb, sa);
    }
    if (j < jsteady) {
        steady(j, sa, sb);
        ++j;
    }
    // scores of tile j are in sa when j is even, in sb when j is odd
    for (; j < jend; ++j) {
        if (j & 1) tail(j, sb, sa);
        else tail(j, sa, sb);
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
