// Backward attention kernels for gfx950 (MI355X).
//
// Exact gradient of Eq. (1) of Rao et al., "Scheduling Data to Compute:
// Hierarchical Data Pipelining for LLM Training on AMD GPUs", section 2.1,
// with P recomputed from the forward's log-sum-exp. With
//   P = exp(scale Q K^T - lse),  dP = dO V^T,  delta = rowsum(dO * O),
//   dS = P * (dP - delta),
// the products are dQ = scale dS K and dK = scale dS^T Q (the two backward rows
// of that section's Table 3) and dV = P^T dO. Both Table 3 rows with a
// transposed operand read it with the gfx950 transpose load
// (ds_read_b64_tr_b16) from the row-major tile in LDS.
//
// Two stages, ordered on the caller's stream, no atomics (deterministic):
//   dq_kernel   one workgroup per (b, hq, 128-row query tile); K/V tiles stream
//               from HBM straight into double-buffered, swizzled LDS tiles
//               (global_load_lds). It also computes the exact delta of its rows
//               and a flag per 32-row block (below) and stores them in the
//               workspace, with lse * log2(e), as the row statistics of each
//               32-row block. With a sliding window, dq_win_kernel runs the
//               same body with the query heads of one kv head side by side in a
//               workgroup (fewer rows per head, so every wave uses nearly all of
//               the workgroup's key tiles).
//   dK/dV       one workgroup per (b, kv head, 64-key tile); 32-row Q/dO tiles of
//               every query head of the group stream from HBM into LDS, and wave
//               pairs split the (head, query tile) iterations; their dK/dV partial
//               sums are added in LDS at the end in a fixed order, so the
//               grouped-query sum never leaves the chip and is deterministic.
//               dkv_kernel (D or DV = 128): 8 waves, two per SIMD, in lock-step
//               through one barrier per step, K in registers, V in LDS, a
//               double-buffered stage per pair. dkv1_kernel (D = DV = 64): 4
//               waves, one per SIMD, K and V in registers, a ring of four stages
//               per pair fed three steps ahead, each wave software-pipelined
//               (the S/dP products of the next step under the vector work of this
//               one).

// delta is always the exact sum_j P_ij dP_ij in fp32, accumulated by the dQ
// kernel's pass (delta = rowsum(dO * O) from the bf16-stored O is off by up to
// 2^-9 of |dO| |O|, which the GQA sum carries into dK on rows with a large
// probability). Rows whose largest probability exceeds kPeakP, wherever the data
// puts them (the first rows of a causal problem, a key every later query points
// at, inputs of large norm), take the exact path: their P and dS operands are
// split into a bf16 high part plus a bf16 remainder (two MFMAs each), and their
// dQ pass is made with the exact delta. The dQ kernel finds such rows in its
// pass, makes the pass again for that workgroup, and flags each 32-row block for
// the dK/dV kernel, which chooses its body per workgroup from the flags of the
// query tiles it meets. The host asks for the exact path on every tile when
// |scale| * sqrt(D) > 2 (unit-variance inputs then spread their scores wide
// enough that most rows need it) or for a sliding window of fewer than 128 keys.
//
// Queries and keys have D columns and values DV (the d and d_v of Eq. (1)); each
// is 64 or 128, in any combination: Q, K, dQ and dK are D wide, V, O, dO and dV
// are DV wide.
//
// Sliding window (query i sees keys i-W+1 .. i, the window of the page's
// compressed sparse attention, Table 7): both kernels skip the tiles outside
// the band and mask the tiles that cross either of its edges.
#include "device.h"
#include "kernels.h"
#include <type_traits>

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// dQ (+ delta) kernel
// ---------------------------------------------------------------------------
constexpr int kDqBQ = 128;
constexpr int kDqBK = 64;
constexpr int kDqThreads = 256;

template <int D, int DV>
struct DqTile {
    // K tiles: unpadded [64][D], V tiles [64][DV] bf16 in the chunk order of swz
    // (the direct copies need 1 KB contiguous runs; swz keeps the K row reads,
    // the K transpose reads and the V row reads free of bank conflicts).
    static constexpr int KTILE = kDqBK * D;
    static constexpr int VTILE = kDqBK * DV;
    static constexpr int LDS_BYTES = 2 * (KTILE + VTILE) * 2;     // 2 K slots + 2 V slots
    using KCopy = CopyPlan<D, kDqBK, kDqThreads / 64>;
    using VCopy = CopyPlan<DV, kDqBK, kDqThreads / 64>;
};

// Work item of workgroup `bid` among nQ query-tile ranks: rank r is query tile
// qt_first - r when causal (longest first), qt_first + r otherwise; rank-major
// over the groups in both cases. (Group-major order, which the forward and the
// dK/dV kernels take without a causal edge, cuts this kernel's HBM reads at B=8,
// H=16, S=2048, D=64 from 3.6 to 1.0 times the algorithmic bytes, yet measured
// 6 % slower.)
__device__ __forceinline__ void decode_q_item(int bid, int nQ, int qt_first, int B, int Hkv, int G,
                                              bool causal, int& b, int& hq, int& qt) {
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
    qt = causal ? qt_first - rank : qt_first + rank;
    b = c / Hkv;
    hq = (c % Hkv) * G + g;
}


// One workgroup's share: query rows q0 .. q_last of the kv head that hq reads;
// this wave takes head hq, rows row0 .. row0+31.
//
// The plain body (PRECISE false) makes one pass: dS = P (dP - delta) with delta
// from the stored O and bf16 dS operands. In the same pass it accumulates the
// exact delta_i = sum_j P_ij dP_ij and each row's largest probability; it stores
// the exact delta and a flag per 32-row block (a row above kPeakP) for the dK/dV
// stage, and returns whether any row of the workgroup was above kPeakP. Then dQ is
// not stored: the caller runs the PRECISE body with delta_given, which makes the
// dQ pass again with the exact delta and split dS operands. Called without
// have_delta the PRECISE body first makes pass 0, which only accumulates the
// exact delta.
template <int D, int DV, bool CAUSAL, bool PRECISE>
__device__ __forceinline__ bool dq_body(const BwdArgs& a, __bf16* smem, int b, int hq, int q0, int q_last,
                                        int row0, bool have_delta, float& delta_io) {
    using T = DqTile<D, DV>;
    using KC = typename T::KCopy;
    using VC = typename T::VCopy;
    constexpr int DK = D / 16;    // k-steps of the score product
    constexpr int DKV = DV / 16;  // k-steps of the dP product
    constexpr int DKM = DK > DKV ? DK : DKV;
    constexpr int DB = D / 32;    // 32-row blocks of dQ^T

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int S = a.S;
    const int hkv = hq / a.G;
    const size_t rowbase = ((size_t)b * a.Hq + hq) * (size_t)S;
    const size_t kvrows = ((size_t)b * a.Hkv + hkv) * (size_t)S;
    const uint16_t* Kp = a.k + kvrows * D;
    const uint16_t* Vp = a.v + kvrows * DV;
    const int qrow = row0 + l32;
    const bool live = qrow < S;
    const float c = a.scale_log2;
    constexpr bool precise = PRECISE;

    // Q and dO rows as B operands; delta = rowsum(dO * O) from the stored O.
    bf16x8 qf[DK], df[DKV];
    float dpart = 0.0f;
    if (live) {
        const u32x4* qs = (const u32x4*)(a.q + (rowbase + qrow) * D + 8 * h);
        const u32x4* ds = (const u32x4*)(a.dout + (rowbase + qrow) * DV + 8 * h);
        const u32x4* os = (const u32x4*)(a.o + (rowbase + qrow) * DV + 8 * h);
#pragma unroll
        for (int dk = 0; dk < DKM; ++dk) {
            if (dk < DK) qf[dk] = __builtin_bit_cast(bf16x8, qs[2 * dk]);
            if (dk < DKV) {
                df[dk] = __builtin_bit_cast(bf16x8, ds[2 * dk]);
                const bf16x8 ov = __builtin_bit_cast(bf16x8, os[2 * dk]);
#pragma unroll
                for (int e = 0; e < 8; ++e) dpart += (float)df[dk][e] * (float)ov[e];
            }
        }
    } else {
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) qf[dk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
#pragma unroll
        for (int dk = 0; dk < DKV; ++dk) df[dk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }
    float delta = PRECISE && have_delta ? delta_io : halves_sum(dpart);
    const float lse2 = live ? a.lse[rowbase + qrow] * kLog2e : INFINITY;

    const int nK = (S + kDqBK - 1) / kDqBK;
    const int jend = CAUSAL ? min(nK, q_last / kDqBK + 1) : nK;
    int wjend = CAUSAL ? min(jend, (row0 + 31) / kDqBK + 1) : jend;
    if (row0 >= S) wjend = 0;
    const int W = CAUSAL ? a.window : 0;
    const int jstart = W > 0 ? max(0, q0 - W + 1) / kDqBK : 0;
    const int wjstart = W > 0 ? max(0, row0 - W + 1) / kDqBK : 0;

    __bf16* const Kring = smem;
    __bf16* const Vring = smem + 2 * T::KTILE;
    // Direct copies (as in the forward): rows past the end repeat row S-1; those
    // keys are masked (probability 0) on the last tile.
    int kcrow[KC::N], kccol[KC::N], vcrow[VC::N], vccol[VC::N];
#pragma unroll
    for (int n = 0; n < KC::N; ++n) {
        kcrow[n] = (wave * KC::N + n) * KC::ROWS_PER_COPY + lane / KC::CH;
        kccol[n] = (((lane % KC::CH) ^ swz_f<D>(kcrow[n]))) * 8;
    }
#pragma unroll
    for (int n = 0; n < VC::N; ++n) {
        vcrow[n] = (wave * VC::N + n) * VC::ROWS_PER_COPY + lane / VC::CH;
        vccol[n] = (((lane % VC::CH) ^ swz_f<DV>(vcrow[n]))) * 8;
    }
    auto copy_kv = [&](int slot, int j) {
        const int k0 = j * kDqBK;
        if (k0 + kDqBK <= S) {  // whole tile: scalar row address plus lane offsets made here
            const uint16_t* kb = Kp + (size_t)k0 * D;
            const uint16_t* vb = Vp + (size_t)k0 * DV;
#pragma unroll
            for (int n = 0; n < KC::N; ++n) {
                const int row = (wave * KC::N + n) * KC::ROWS_PER_COPY + lane / KC::CH;
                copy16_to_lds_s(kb, (uint32_t)(row * D + ((lane % KC::CH) ^ swz_f<D>(row)) * 8) * 2u,
                                Kring + slot * T::KTILE + (wave * KC::N + n) * 512);
            }
#pragma unroll
            for (int n = 0; n < VC::N; ++n) {
                const int row = (wave * VC::N + n) * VC::ROWS_PER_COPY + lane / VC::CH;
                copy16_to_lds_s(vb, (uint32_t)(row * DV + ((lane % VC::CH) ^ swz_f<DV>(row)) * 8) * 2u,
                                Vring + slot * T::VTILE + (wave * VC::N + n) * 512);
            }
            return;
        }
#pragma unroll
        for (int n = 0; n < KC::N; ++n) {
            const int key = min(k0 + kcrow[n], S - 1);
            copy16_to_lds(Kp + (uint32_t)(key * D + kccol[n]), Kring + slot * T::KTILE + (wave * KC::N + n) * 512);
        }
#pragma unroll
        for (int n = 0; n < VC::N; ++n) {
            const int key = min(k0 + vcrow[n], S - 1);
            copy16_to_lds(Vp + (uint32_t)(key * DV + vccol[n]), Vring + slot * T::VTILE + (wave * VC::N + n) * 512);
        }
    };
    // Per-lane LDS offsets: K and V rows (A operands of S^T and dP^T) per k-step,
    // and K transpose quads per 32-column block and row half (row offsets that
    // are multiples of 16 are added as constants).
    int roff[DK], rvoff[DKV], toff[2][DB];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) roff[dk] = swz<D>(l32, dk * 16 + 8 * h);
#pragma unroll
    for (int dk = 0; dk < DKV; ++dk) rvoff[dk] = swz<DV>(l32, dk * 16 + 8 * h);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < DB; ++db)
            toff[hf][db] = swz<D>(4 * h + ((lane & 15) >> 2) + 8 * hf,
                                  db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero16();

    // Pass 0 (exact body without a given delta) accumulates the exact delta; the
    // last pass forms dS and accumulates dQ^T += K^T dS^T. Tile j+1 is copied into
    // the other slot while tile j is multiplied.
    float dacc = 0.0f;     // sum_j P_ij dP_ij over this lane's keys
    bool peaked = false;   // plain body: some probability of the wave's rows above kPeakP
                           // (a wave-wide ballot, held in scalar registers)
    for (int pass = PRECISE && !have_delta ? 0 : 1; pass < 2; ++pass) {
        dacc = 0.0f;
        copy_kv(jstart & 1, jstart);
        wait_copies();
        __syncthreads();
        // Tiles in pairs, so that each tile's ring slot (par = j & 1) is a constant
        // and the slot offset folds into the LDS reads' immediate offsets.
        auto step = [&](int j, auto par) {
            if (j + 1 < jend) copy_kv((j + 1) & 1, j + 1);
            if (j >= wjstart && j < wjend) {
                constexpr int P = decltype(par)::value;
                const __bf16* Ks = Kring + P * T::KTILE;
                const __bf16* Vs = Vring + P * T::VTILE;
                const int k0 = j * kDqBK;
                const bool need_mask = j == wjend - 1 || (W > 0 && k0 < row0 + 32 - W);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    f32x16 s = zero16(), dp = zero16();
#pragma unroll
                    for (int dk = 0; dk < DKM; ++dk) {
                        bf16x8 kf, vf;
                        if (dk < DK) kf = lds_read8(Ks + roff[dk] + kb * 32 * D);
                        if (dk < DKV) vf = lds_read8(Vs + rvoff[dk] + kb * 32 * DV);
                        if (dk < DK) s = mfma32(kf, qf[dk], s);
                        if (dk < DKV) dp = mfma32(vf, df[dk], dp);
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], c, -lse2));
                    if (need_mask) {  // one uniform branch, taken on edge tiles only
                        // key k0 + kb*32 + 4h + off is visible iff lo <= off <= lim
                        const int lim = (CAUSAL ? min(qrow, S - 1) : S - 1) - k0 - kb * 32 - 4 * h;
                        const int lo = W > 0 ? qrow - W + 1 - k0 - kb * 32 - 4 * h : -(1 << 30);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int off = 8 * (r >> 2) + (r & 3);
                            s[r] = (off > lim || off < lo) ? 0.0f : s[r];
                        }
                    }
                    if (precise) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            dacc += s[r] * dp[r];  // used after pass 0 only
                            s[r] = s[r] * (dp[r] - delta);
                        }
                    } else {
                        float tmax = s[0];
#pragma unroll
                        for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
                        peaked |= __builtin_amdgcn_ballot_w64(tmax > kPeakP) != 0;
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float t = s[r] * dp[r];
                            dacc += t;
                            s[r] = fmaf(-s[r], delta, t);  // P (dP - delta)
                        }
                    }
                    if (pass == 0) continue;
                    // dQ^T += K^T dS^T over two 16-key steps; K^T via transpose loads.
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2) {
                        const int r0 = 8 * t2;
                        const bf16x8 hi = pack8(s[r0], s[r0 + 1], s[r0 + 2], s[r0 + 3], s[r0 + 4],
                                                s[r0 + 5], s[r0 + 6], s[r0 + 7]);
                        bf16x8 lo;
                        if (precise)
                            lo = pack8(bf_lo(s[r0]), bf_lo(s[r0 + 1]), bf_lo(s[r0 + 2]), bf_lo(s[r0 + 3]),
                                       bf_lo(s[r0 + 4]), bf_lo(s[r0 + 5]), bf_lo(s[r0 + 6]), bf_lo(s[r0 + 7]));
                        const int rb = (kb * 32 + 16 * t2) * D;
#pragma unroll
                        for (int db = 0; db < DB; ++db) {
                            const bf16x8 kt = concat(lds_read_tr(Ks + toff[0][db] + rb),
                                                     lds_read_tr(Ks + toff[1][db] + rb));
                            dq[db] = mfma32(kt, hi, dq[db]);
                            if (precise) dq[db] = mfma32(kt, lo, dq[db]);
                        }
                    }
                }
            }
            wait_copies();
            __syncthreads();
        };
        int j = jstart;
        if (j & 1) step(j++, std::integral_constant<int, 1>{});
        for (; j + 1 < jend; j += 2) {
            step(j, std::integral_constant<int, 0>{});
            step(j + 1, std::integral_constant<int, 1>{});
        }
        if (j < jend) step(j, std::integral_constant<int, 0>{});
        if (pass == 0) delta = halves_sum(dacc);
    }

    const int nQB = (S + 31) / 32;
    int* const peak = a.peak + ((size_t)b * a.Hq + hq) * nQB + row0 / 32;
    bool redo = false;
    if (!PRECISE) {
        // The ring is idle after the last step's barrier: a workgroup vote on
        // whether any row needs the exact path.
        delta = halves_sum(dacc);
        int* vote = (int*)smem;
        if (lane == 0) vote[wave] = peaked ? 1 : 0;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < kDqThreads / 64; ++w) redo |= vote[w] != 0;
        redo = __builtin_amdgcn_readfirstlane(redo ? 1 : 0) != 0;  // the same in every lane
        __syncthreads();  // the exact pass refills the ring
        if (lane == 0 && row0 < S) *peak = peaked ? 1 : 0;
        delta_io = delta;
    } else if (!have_delta && lane == 0 && row0 < S) {
        *peak = 1;
    }

    if (h == 0 && row0 < S) {  // every row of the 32-row block, those past S as (+inf, -0)
        const size_t S32 = (size_t)nQB * 32;
        float* blk = a.rowstat + (((size_t)b * a.Hq + hq) * S32 + row0) * 2;  // this block's 64 words
        blk[l32] = live ? a.lse[rowbase + qrow] * kLog2e : INFINITY;  // loaded again: not held across the loop
        blk[32 + l32] = live ? -delta : -0.0f;
    }
    if (live) {
        if (redo) return true;  // dQ is stored by the exact pass
        float* dst = a.dq + (rowbase + qrow) * D;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 v;
                v[0] = dq[db][4 * g4] * sc;
                v[1] = dq[db][4 * g4 + 1] * sc;
                v[2] = dq[db][4 * g4 + 2] * sc;
                v[3] = dq[db][4 * g4 + 3] * sc;
                *(f32x4*)(dst + db * 32 + 8 * g4 + 4 * h) = v;
            }
    }
    return redo;
}

// A workgroup's rows: the plain pass, then the exact one where the plain pass found
// a row above kPeakP (or on every workgroup, when the host asks for it). The
// exact workgroups run inside the same launch, in the tail of the longest-first
// schedule.
template <int D, int DV, bool CAUSAL>
__device__ __forceinline__ void dq_rows(const BwdArgs& a, __bf16* smem, int b, int hq, int q0, int q_last,
                                        int row0) {
    float delta = 0.0f;
    bool exact = a.precise_all != 0, have_delta = false;
    if (!exact) {
        exact = dq_body<D, DV, CAUSAL, false>(a, smem, b, hq, q0, q_last, row0, false, delta);
        have_delta = true;
    }
    if (exact)  // one inlined copy of the exact body serves both cases
        dq_body<D, DV, CAUSAL, true>(a, smem, b, hq, q0, q_last, row0, have_delta, delta);
}

// One launch over every query tile.
template <int D, int DV, bool CAUSAL>
__global__ void __launch_bounds__(kDqThreads, 2) dq_kernel(BwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
    const int nQ = (a.S + kDqBQ - 1) / kDqBQ;
    int b, hq, qt;
    decode_q_item(blockIdx.x, nQ, CAUSAL ? nQ - 1 : 0, a.B, a.Hkv, a.G, CAUSAL, b, hq, qt);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q0 = qt * kDqBQ;
    dq_rows<D, DV, CAUSAL>(a, smem, b, hq, q0, q0 + kDqBQ - 1, q0 + 32 * wave);
}

// Heads of one kv head that a sliding-window dQ workgroup takes together.
__host__ __device__ inline int dq_win_heads(int G) { return (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1; }

// Sliding window (as fwd_win_kernel does for the forward): the 4 waves take HW
// query heads of one kv head and 4/HW blocks of 32 rows, so every wave uses nearly
// all of the workgroup's key tiles. Every workgroup takes the exact path when the
// window is under 128 keys (precise_all), else as the rows' probabilities say.
template <int D, int DV>
__global__ void __launch_bounds__(kDqThreads, 2) dq_win_kernel(BwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
    const int HW = dq_win_heads(a.G), BQ = 32 * (4 / HW);
    const int nblk = a.G / HW;
    const int groups = a.B * a.Hkv * nblk;   // (b, kv head, head block)
    int qt, gid;
    const int bid = blockIdx.x;
    if ((groups & 7) == 0) {  // a head block stays on one XCD
        const int x = bid & 7, st = bid >> 3, per = groups >> 3;
        qt = st / per;
        gid = (st - qt * per) * 8 + x;
    } else {
        qt = bid / groups;
        gid = bid - qt * groups;
    }
    const int b = gid / (a.Hkv * nblk);
    const int rem = gid - b * (a.Hkv * nblk);
    const int hkv = rem / nblk, blk = rem - hkv * nblk;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hq = hkv * a.G + blk * HW + wave % HW;
    const int q0 = qt * BQ;
    const int row0 = q0 + 32 * (wave / HW);
    dq_rows<D, DV, true>(a, smem, b, hq, q0, q0 + BQ - 1, row0);
}

// ---------------------------------------------------------------------------
// dK/dV kernels: the work split both use, then dkv1_kernel (one wave per SIMD)
// ---------------------------------------------------------------------------
constexpr int kKvBK = 64;      // keys per workgroup (2 waves x 32)
constexpr int kKvBQ = 32;      // query rows per streamed tile
constexpr int kKv1Splits = 2;   // wave pairs that split the (head, query tile) iterations
constexpr int kKv1Ring = 4;     // stages per pair: the copies run three steps ahead
constexpr int kKv1Threads = 64 * 2 * kKv1Splits;   // one wave per SIMD

template <int D, int DV>
struct Kv1Tile {
    // Per pair a ring of kKv1Ring stages {Q [32][D], dO [32][DV], the 32 rows'
    // lse*log2e then their -delta}, the tiles bf16 in the swizzled chunk order of
    // swz (K and V rows of the workgroup's keys are held in registers).
    static constexpr int QTILE = kKvBQ * D;                          // elements
    static constexpr int DTILE = kKvBQ * DV;
    static constexpr int STAGE_BYTES = (QTILE + DTILE) * 2 + kKvBQ * 8;
    static constexpr int SPLIT_BYTES = kKv1Ring * STAGE_BYTES;
    static constexpr int TILE_BYTES = kKv1Splits * SPLIT_BYTES;
    // final sum: one pair hands over dK, the other dV, of both key halves
    static constexpr int XCHG_BYTES = 2 * (D / 32 + DV / 32) * 16 * 64 * 4;
    static constexpr int LDS_BYTES = TILE_BYTES > XCHG_BYTES ? TILE_BYTES : XCHG_BYTES;
    using QCopy = CopyPlan<D, kKvBQ, 2>;                             // per wave of a pair
    using DCopy = CopyPlan<DV, kKvBQ, 2>;
    // vector-memory operations of one stage fetch, per wave
    static constexpr int NF = QCopy::N + DCopy::N + 1;
};

// Which dK/dV kernel runs: the one-wave-per-SIMD pipelined kernel below for
// D = DV = 64, the two-waves-per-SIMD kernel further down otherwise. Measured on an
// MI355X in one process, the one-wave kernel takes 0.34 ms against 0.43 ms on a
// non-causal B=8, H=16, S=2048, D=64 problem, but 0.32 ms against 0.30 ms on the
// causal Llama-3.1-8B shape (D = 128): a single wave issues its instructions in
// order, and at D = 128 its vector work, copies and bookkeeping per step no longer
// fit under its matrix instructions, where two waves per SIMD issue theirs side by
// side.
template <int D, int DV>
constexpr bool kDkvOneWave = D == 64 && DV == 64;

// Work item of a dK/dV workgroup: (b, hkv, key tile); groups dealt to XCDs as in
// the forward: causal tiles rank-major, longest (lowest) first; otherwise
// group-major, so the workgroups an XCD holds at once stream one group's Q and dO
// (at B=8, H=16, S=2048, D=64 rank-major order fetched 10 times the algorithmic
// bytes from HBM, and the kernel took 6 % longer).
template <bool CAUSAL>
__device__ __forceinline__ void dkv_item(const BwdArgs& a, int& b, int& hkv, int& kt) {
    const int C = a.B * a.Hkv, bid = blockIdx.x;
    const bool spread = (C & 7) == 0;
    int rank, cgrp;
    if (CAUSAL) {
        if (spread) {
            const int x = bid & 7, st = bid >> 3, per = C >> 3;
            rank = st / per;
            cgrp = (st - rank * per) * 8 + x;
        } else {
            rank = bid / C;
            cgrp = bid - rank * C;
        }
    } else {
        const int nK = (a.S + kKvBK - 1) / kKvBK;
        const int st = spread ? bid >> 3 : bid;
        const int cl = st / nK;
        rank = st - cl * nK;
        cgrp = spread ? cl * 8 + (bid & 7) : cl;
    }
    kt = rank;  // ascending key tile = most query tiles first when causal
    b = cgrp / a.Hkv;
    hkv = cgrp % a.Hkv;
}

// The 32-row query tiles that see some key of key tile kt: all of them, from the
// tile holding key kt*64 on when causal, up to the last row that sees the tile's
// last key through a window.
template <bool CAUSAL>
__device__ __forceinline__ void dkv_range(const BwdArgs& a, int kt, int& qi_first, int& qi_last) {
    const int nQB = (a.S + kKvBQ - 1) / kKvBQ;
    const int kv0 = kt * kKvBK;
    const int W = CAUSAL ? a.window : 0;
    qi_first = CAUSAL ? kv0 / kKvBQ : 0;
    qi_last = W > 0 ? min(nQB - 1, (kv0 + kKvBK - 1 + W - 1) / kKvBQ) : nQB - 1;
}

// One past the last query tile, among those key tile kt meets, that the dQ stage
// flagged in any head of the group (qi_first when none is). Every wave scans the
// flags on its own with scalar loads (wave-uniform addresses, read through the
// constant address space: the dQ stage wrote them before this launch), so the scan
// needs no vector registers, no LDS and no barrier. Four 8-flag loads are in flight
// per round trip to the cache.
template <bool CAUSAL>
__device__ __forceinline__ int dkv_exact_end(const BwdArgs& a, int b, int hkv, int kt) {
    typedef const __attribute__((address_space(4))) int cint;
    typedef int i32x8 __attribute__((ext_vector_type(8)));
    typedef const __attribute__((address_space(4))) i32x8 cint8;
    int qi_first, qi_last;
    dkv_range<CAUSAL>(a, kt, qi_first, qi_last);
    const int per_g = qi_last - qi_first + 1, nQB = (a.S + kKvBQ - 1) / kKvBQ;
    int end = 0;  // one past the last flagged tile, relative to qi_first
    for (int g = 0; g < a.G; ++g) {
        const int* row = a.peak + ((size_t)b * a.Hq + (size_t)hkv * a.G + g) * nQB + qi_first;
        int i = 0;
        for (; i + 32 <= per_g; i += 32) {
            i32x8 f[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) f[u] = *(cint8*)(uintptr_t)(row + i + 8 * u);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) end = f[u][e] ? i + 8 * u + e + 1 : end;
        }
        for (; i + 8 <= per_g; i += 8) {
            const i32x8 f = *(cint8*)(uintptr_t)(row + i);
#pragma unroll
            for (int e = 0; e < 8; ++e) end = f[e] ? i + e + 1 : end;
        }
        for (; i < per_g; ++i) end = *(cint*)(uintptr_t)(row + i) ? i + 1 : end;
    }
    return qi_first + end;
}

// Query tiles qi_first .. qi_x - 1 (of every head of the group) run in a first loop
// whose iterations take the exact path where the dQ stage flagged their tile (or
// everywhere, when the host asks for it); tiles qi_x .. qi_last run in a second,
// plain loop. The accumulators carry from one loop into the other. qi_x comes from
// the flags (dkv_exact_end), read once the K rows and the V tile are on their way.
//
// One wave per SIMD: the wave keeps its own matrix core busy by software
// pipelining. The plain loop's step j issues the S/dP products of step j+1 with,
// between its matrix instructions (explicitly ordered scheduling regions), the
// vector work that turns step j's S/dP into bf16 P and dS operands and the copies
// of a stage three steps ahead; then step j's dV/dK products, in whose regions the
// next step's bookkeeping runs. Stage copies (Q, dO and the row statistics) go
// through a ring of four stages per pair, and every wait on them is a count of
// this wave's vector-memory operations. dP - delta is formed by the dP products
// themselves, their accumulator starting at -delta.
template <int D, int DV, bool CAUSAL>
__device__ __forceinline__ void dkv1_body(const BwdArgs& a, unsigned char* lds_raw, int b, int hkv, int kt) {
    using T = Kv1Tile<D, DV>;
    using QC = typename T::QCopy;
    using DC = typename T::DCopy;
    constexpr int NF = T::NF;
    constexpr int DK = D / 16;     // k-steps of the score product
    constexpr int DKV = DV / 16;   // k-steps of the dP product
    constexpr int DKM = DK > DKV ? DK : DKV;
    constexpr int DBK = D / 32;    // 32-row blocks of dK^T
    constexpr int DBV = DV / 32;   // 32-row blocks of dV^T
    constexpr int DBM = DBK > DBV ? DBK : DBV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int split = wave >> 1, w2 = wave & 1;
    const int S = a.S, G = a.G;
    const int nQB = (S + kKvBQ - 1) / kKvBQ;
    const size_t S32 = (size_t)nQB * kKvBQ;

    const int kv0 = kt * kKvBK;
    const int kw0 = kv0 + 32 * w2;  // this wave's first key
    const int key = kw0 + l32;      // this lane's key (column of S, dP)
    const size_t kvrow = ((size_t)b * a.Hkv + hkv) * (size_t)S;
    const float c = a.scale_log2;

    // K and V rows of this lane's key as B operands (zero past the end).
    bf16x8 kf[DK], vf[DKV];
    if (key < S) {
        const u32x4* ks = (const u32x4*)(a.k + (kvrow + key) * D + 8 * h);  // K is D wide
        const u32x4* vs = (const u32x4*)(a.v + (kvrow + key) * DV + 8 * h);  // V is DV wide
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) kf[dk] = __builtin_bit_cast(bf16x8, ks[2 * dk]);
#pragma unroll
        for (int dk = 0; dk < DKV; ++dk) vf[dk] = __builtin_bit_cast(bf16x8, vs[2 * dk]);
    } else {
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) kf[dk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
#pragma unroll
        for (int dk = 0; dk < DKV; ++dk) vf[dk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }

    // LDS: per pair the ring of stages.
    unsigned char* const split_base = lds_raw + split * T::SPLIT_BYTES;
    auto stage_q = [&](int sl) { return (__bf16*)(split_base + sl * T::STAGE_BYTES); };
    auto stage_do = [&](int sl) { return stage_q(sl) + T::QTILE; };
    auto stage_st = [&](int sl) {  // lse*log2e of the 32 rows, then their -delta
        return (float*)(split_base + sl * T::STAGE_BYTES + (T::QTILE + T::DTILE) * 2);
    };

    // Iterations of a loop over query tiles q_lo .. q_lo + nq - 1: (g, query tile qi)
    // for every head g of the group; pair p takes iterations p, p + kKv1Splits, ...
    const int W = CAUSAL ? a.window : 0;
    int qi_first, qi_last;
    dkv_range<CAUSAL>(a, kt, qi_first, qi_last);
    const int qi_x = a.precise_all ? qi_last + 1 : dkv_exact_end<CAUSAL>(a, b, hkv, kt);

    f32x16 dk[DBK], dv[DBV];
#pragma unroll
    for (int db = 0; db < DBK; ++db) dk[db] = zero16();
#pragma unroll
    for (int db = 0; db < DBV; ++db) dv[db] = zero16();

    // Per-lane LDS offsets: A-operand rows (Q; dO and V) per k-step; transpose
    // quads (Q^T; dO^T) per 32-column block and row half.
    int roff[DK], rvoff[DKV], toff[2][DBK], tvoff[2][DBV];
#pragma unroll
    for (int dk2 = 0; dk2 < DK; ++dk2) roff[dk2] = swz<D>(l32, dk2 * 16 + 8 * h);
#pragma unroll
    for (int dk2 = 0; dk2 < DKV; ++dk2) rvoff[dk2] = swz<DV>(l32, dk2 * 16 + 8 * h);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int db = 0; db < DBK; ++db)
            toff[hf][db] = swz<D>(4 * h + ((lane & 15) >> 2) + 8 * hf,
                                  db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
#pragma unroll
        for (int db = 0; db < DBV; ++db)
            tvoff[hf][db] = swz<DV>(4 * h + ((lane & 15) >> 2) + 8 * hf,
                                    db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    }

    // -delta of this lane's 16 rows (8(r/4) + 4h + r%4, r = 0..15) of the stage in
    // slot sl, as the initial value of the dP accumulator
    auto neg_delta = [&](int sl) {
        const float* Nd = stage_st(sl) + kKvBQ;
        f32x16 v;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 x = *(const f32x4*)(Nd + 8 * q + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e];
        }
        return v;
    };
    // S = Q K^T and dP - delta = dO V^T - delta of the stage in ring slot sl (32
    // queries x this wave's keys)
    auto sdp = [&](int sl, f32x16& sv, f32x16& dpv) {
        const __bf16* Qs = stage_q(sl);
        const __bf16* Ds = stage_do(sl);
        sv = zero16();
        dpv = neg_delta(sl);  // dP - delta: the products add onto -delta
#pragma unroll
        for (int dd = 0; dd < DKM; ++dd) {
            bf16x8 qa, da;
            if (dd < DK) qa = lds_read8(Qs + roff[dd]);
            if (dd < DKV) da = lds_read8(Ds + rvoff[dd]);
            if (dd < DK) sv = mfma32(qa, kf[dd], sv);
            if (dd < DKV) dpv = mfma32(da, vf[dd], dpv);
        }
    };
    // P = exp2(S c - lse log2 e) and dS = P (dP - delta) of the 16-query half t2
    // (dpv holds dP - delta); rows of sv/dpv are queries 8(r/4) + 4h + r%4, the
    // column is this lane's key. With the mask, keys outside a row's causal (or
    // window) range get P = 0.
    auto pds = [&](int sl, int qs0, auto mask_tag, const f32x16& sv, const f32x16& dpv, int t2,
                   float (&pv)[8], float (&dsv)[8]) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const float* St = stage_st(sl);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int r0 = 8 * (2 * t2 + half) + 4 * h;  // first of this lane's 4 rows
            const f32x4 l4 = *(const f32x4*)(St + r0);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * half + e;
                float p = fast_exp2(fmaf(sv[8 * t2 + i], c, -l4[e]));
                if (MASK) {
                    const int qrow = qs0 + r0 + e;
                    p = (key > qrow || (W > 0 && qrow >= key + W)) ? 0.0f : p;
                }
                pv[i] = p;
                dsv[i] = p * dpv[8 * t2 + i];
            }
        }
    };
    // dV^T += dO^T P and dK^T += Q^T dS for the 16-query half t2 (plus the remainder
    // operands on the exact path)
    auto dvdk = [&](int sl, int t2, const bf16x8& ph, const bf16x8& sh, bool precise, const bf16x8& pl,
                    const bf16x8& sl_) {
        const __bf16* Qs = stage_q(sl);
        const __bf16* Ds = stage_do(sl);
        const int rbk = 16 * t2 * D, rbv = 16 * t2 * DV;
#pragma unroll
        for (int db = 0; db < DBM; ++db) {
            bf16x8 dot, qt;
            if (db < DBV)
                dot = concat(lds_read_tr(Ds + tvoff[0][db] + rbv), lds_read_tr(Ds + tvoff[1][db] + rbv));
            if (db < DBK)
                qt = concat(lds_read_tr(Qs + toff[0][db] + rbk), lds_read_tr(Qs + toff[1][db] + rbk));
            if (db < DBV) dv[db] = mfma32(dot, ph, dv[db]);
            if (db < DBK) dk[db] = mfma32(qt, sh, dk[db]);
            if (precise) {
                if (db < DBV) dv[db] = mfma32(dot, pl, dv[db]);
                if (db < DBK) dk[db] = mfma32(qt, sl_, dk[db]);
            }
        }
    };
    auto pack_pv = [&](const float (&x)[8]) { return pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]); };
    auto pack_lo = [&](const float (&x)[8]) {
        return pack8(bf_lo(x[0]), bf_lo(x[1]), bf_lo(x[2]), bf_lo(x[3]), bf_lo(x[4]), bf_lo(x[5]), bf_lo(x[6]),
                     bf_lo(x[7]));
    };

    // A plain step without a mask, in explicitly ordered scheduling regions (the
    // compiler may not move instructions across a sched_barrier): one region per
    // k-step of the S/dP products of the next step (slot sln), each with two matrix
    // instructions, the LDS reads of the k-step two ahead, copy_k(dd) and the vector
    // work of 16/DKM of this step's 16 P/dS elements per lane (row statistics from
    // slot sl): P (fma, exp) of an element in its region, its dS and the bf16
    // packing of P and dS in the next, so that the exp's latency passes under the
    // next matrix instructions. Element e of a lane is query row 8(e/4) + 4h + e%4
    // of the tile, in the 16-query half e/8. The dV/dK products follow (dvdk_step).
    auto fast_sdp_pds = [&](int sl, int sln, const f32x16& sc, const f32x16& dc, f32x16& sn, f32x16& dn,
                            bf16x8 (&ph)[2], bf16x8 (&sh)[2], auto&& copy_k) {
        constexpr int EPK = 16 / DKM;  // elements per k-step
        const __bf16* Qn = stage_q(sln);
        const __bf16* Dn = stage_do(sln);
        const float* St = stage_st(sl);
        f32x4 xs[4];  // lse*log2e of this lane's 16 rows: row group q (rows 8q + 4h + 0..3)
        auto rds = [&](int q) { xs[q] = *(const f32x4*)(St + 8 * q + 4 * h); };  // one group ahead
        rds(0);
        bf16x8 qa[DKM], da[DKM];
        auto rd = [&](int dd) {
            if (dd < DK) qa[dd] = lds_read8(Qn + roff[dd]);
            if (dd < DKV) da[dd] = lds_read8(Dn + rvoff[dd]);
        };
        rd(0);
        if (DKM > 1) rd(1);
        sn = zero16();
        dn = neg_delta(sln);  // dP - delta: the products add onto -delta
        // Element e: P in region e / EPK (fma, exp), then dS and the bf16 packing of
        // P and dS in the next region, so that the exp's latency passes under the
        // next matrix instructions.
        float pe[16];
        uint32_t phw[8], shw[8];  // words of ph[0] (0..3) and ph[1] (4..7), likewise sh
        auto stage2 = [&](int dd) {  // dS and packing of region dd's elements
#pragma unroll
            for (int u = 0; u < EPK; u += 2) {
                const int e = dd * EPK + u;
                const float ds0 = pe[e] * dc[e], ds1 = pe[e + 1] * dc[e + 1];  // dc holds dP - delta
                phw[e >> 1] = pack2_bf16(pe[e], pe[e + 1]);
                shw[e >> 1] = pack2_bf16(ds0, ds1);
                asm volatile("" ::"v"(phw[e >> 1]), "v"(shw[e >> 1]));
            }
        };
#pragma unroll
        for (int dd = 0; dd < DKM; ++dd) {
            if (dd + 2 < DKM) rd(dd + 2);
            if ((dd * EPK) % 4 == 0 && dd * EPK / 4 + 1 < 4) rds(dd * EPK / 4 + 1);
            copy_k(dd);  // a share of the copies of the stage three steps ahead
            if (dd < DK) sn = mfma32(qa[dd], kf[dd], sn);
            if (dd < DKV) dn = mfma32(da[dd], vf[dd], dn);
#pragma unroll
            for (int u = 0; u < EPK; ++u) {
                const int e = dd * EPK + u;
                pe[e] = fast_exp2(fmaf(sc[e], c, -xs[e >> 2][e & 3]));
                // keeps the element's arithmetic in this region (pure arithmetic
                // could otherwise be placed anywhere before its first use)
                asm volatile("" ::"v"(pe[e]));
            }
            if (dd > 0) stage2(dd - 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        stage2(DKM - 1);
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            ph[t2] = __builtin_bit_cast(bf16x8, u32x4{phw[4 * t2], phw[4 * t2 + 1], phw[4 * t2 + 2], phw[4 * t2 + 3]});
            sh[t2] = __builtin_bit_cast(bf16x8, u32x4{shw[4 * t2], shw[4 * t2 + 1], shw[4 * t2 + 2], shw[4 * t2 + 3]});
        }
    };
    // dV^T += dO^T P and dK^T += Q^T dS of the stage in slot sl, one region per
    // (16-query half, 32-column block) pair, the transpose reads of the pair two
    // ahead; hook(pp) is the caller's work placed in region pp
    auto dvdk_step = [&](int sl, const bf16x8 (&ph)[2], const bf16x8 (&sh)[2], auto&& hook) {
        const __bf16* Qs = stage_q(sl);
        const __bf16* Ds = stage_do(sl);
        constexpr int NP = 2 * DBM;  // (t2, block) pairs
        bf16x8 dot[NP], qt[NP];
        auto rdt = [&](int pp) {
            const int t2 = pp / DBM, db = pp % DBM;
            const int rbk = 16 * t2 * D, rbv = 16 * t2 * DV;
            if (db < DBV)
                dot[pp] = concat(lds_read_tr(Ds + tvoff[0][db] + rbv), lds_read_tr(Ds + tvoff[1][db] + rbv));
            if (db < DBK)
                qt[pp] = concat(lds_read_tr(Qs + toff[0][db] + rbk), lds_read_tr(Qs + toff[1][db] + rbk));
        };
        rdt(0);
        rdt(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
            if (pp + 2 < NP) rdt(pp + 2);
            const int t2 = pp / DBM, db = pp % DBM;
            if (db < DBV) dv[db] = mfma32(dot[pp], ph[t2], dv[db]);
            if (db < DBK) dk[db] = mfma32(qt[pp], sh[t2], dk[db]);
            hook(pp);  // the caller's work for region pp
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    auto run = [&](int q_lo, int nq, auto exact_tag) {
        constexpr bool MAYBE_PRECISE = decltype(exact_tag)::value;
        const int total = G * nq;
        const int steps = (total + kKv1Splits - 1) / kKv1Splits;
        if (steps == 0) return;  // the same in every wave of the workgroup
        // Q / dO copies of a pair: copy n of wave w2 fills tile rows (w2*N + n) *
        // ROWS_PER_COPY + lane / CH, kept as this lane's byte offset within a tile of
        // whole rows. Rows past S repeat row S-1; their lse is +inf, so their
        // probabilities, and every term they touch, are exactly 0.
        uint32_t qcoff[QC::N], dcoff[DC::N];
#pragma unroll
        for (int n = 0; n < QC::N; ++n) {
            const int row = (w2 * QC::N + n) * QC::ROWS_PER_COPY + lane / QC::CH;
            qcoff[n] = (uint32_t)(row * D + ((lane % QC::CH) ^ swz_f<D>(row)) * 8) * 2u;
        }
#pragma unroll
        for (int n = 0; n < DC::N; ++n) {  // the same as qcoff when D == DV
            const int row = (w2 * DC::N + n) * DC::ROWS_PER_COPY + lane / DC::CH;
            dcoff[n] = D == DV ? 0u : (uint32_t)(row * DV + ((lane % DC::CH) ^ swz_f<DV>(row)) * 8) * 2u;
        }
        // The (head g, query tile q_lo + r) of a step's iteration it = g nq + r,
        // walked with counters (no division per step): one walk for the fetches,
        // which run kKv1Ring - 1 steps ahead, one for the steps computed. Every loop
        // iteration fetches, past the last step too (the last iteration again, into a
        // slot no later step reads), so that every fetch is NF vector-memory
        // operations of every wave and every wait is the same count.
        // A walk also carries the tile's first row among all query rows (row) and
        // among the padded rows of the row statistics (srow).
        struct Walk {
            int g, r;
            long long row, srow;
        };
        const long long head0 = (long long)b * a.Hq + (long long)hkv * G;  // the group's first query head
        auto walk_start = [&](Walk& w) {
            w.g = split / nq;
            w.r = split - w.g * nq;
            w.row = (head0 + w.g) * S + (long long)(q_lo + w.r) * kKvBQ;
            w.srow = (head0 + w.g) * (long long)S32 + (long long)(q_lo + w.r) * kKvBQ;
        };
        auto walk_next = [&](Walk& w) {
            w.r += kKv1Splits;
            w.row += kKv1Splits * kKvBQ;
            w.srow += kKv1Splits * kKvBQ;
            while (w.r >= nq) {
                w.r -= nq;
                ++w.g;
                w.row += S - (long long)nq * kKvBQ;
                w.srow += (long long)S32 - (long long)nq * kKvBQ;
            }
        };
        const uint32_t lds0 = lds_addr_of(split_base);  // this pair's ring, as an LDS address
        Walk wf;  // next step to fetch
        walk_start(wf);
        int fstep = 0;
        // the last iteration, which a fetch past the end copies again
        const long long last_row = (head0 + G - 1) * S + (long long)(q_lo + nq - 1) * kKvBQ;
        const long long last_srow = (head0 + G - 1) * (long long)S32 + (long long)(q_lo + nq - 1) * kKvBQ;
        // A fetch is planned once (addresses) and its NF copies issued one at a time,
        // so that the plain loop can spread them over its matrix instructions.
        struct Fetch {
            const uint16_t* qb;   // first row of the Q tile
            const uint16_t* db;   // first row of the dO tile
            const float* stat;    // this lane's word of the row statistics
            long long rb;         // the query head's first row
            int qr0;              // first query row of the tile within its head
            uint32_t st0;         // LDS address of the stage
            bool whole;           // the tile lies inside S
        };
        auto fetch_plan = [&]() {
            Fetch f;
            f.st0 = lds0 + (uint32_t)((fstep % kKv1Ring) * T::STAGE_BYTES);
            const bool past = wf.g >= G;  // past the last iteration: fetch the last one again
            const long long row = past ? last_row : wf.row, srow = past ? last_srow : wf.srow;
            f.qr0 = (q_lo + (past ? nq - 1 : wf.r)) * kKvBQ;
            f.rb = row - f.qr0;
            f.whole = f.qr0 + kKvBQ <= S;
            f.qb = a.q + row * D;
            f.db = a.dout + row * DV;
            // the 32 rows' (lse*log2e, delta): 256 bytes, one word per lane; both waves
            // of the pair copy the same words to the same place
            f.stat = a.rowstat + srow * 2 + lane;
            walk_next(wf);
            ++fstep;
            return f;
        };
        // copy k of NF; WHOLE: the tile lies inside S (known to the caller)
        auto fetch_copy_t = [&](const Fetch& f, int k, auto whole_tag) {
            constexpr bool WHOLE = decltype(whole_tag)::value;
            if (k < QC::N) {
                const int n = k;
                if (WHOLE) {  // scalar row address plus lane offsets
                    copy16_to_lds_sa(f.qb, qcoff[n], f.st0 + (w2 * QC::N + n) * 1024);
                } else {
                    const int row = (w2 * QC::N + n) * QC::ROWS_PER_COPY + lane / QC::CH;
                    const size_t off = (f.rb + min(f.qr0 + row, S - 1)) * D + ((lane % QC::CH) ^ swz_f<D>(row)) * 8;
                    copy16_to_lds_a(a.q + off, f.st0 + (w2 * QC::N + n) * 1024);
                }
            } else if (k < QC::N + DC::N) {
                const int n = k - QC::N;
                const uint32_t dst = f.st0 + T::QTILE * 2 + (w2 * DC::N + n) * 1024;
                if (WHOLE) {
                    copy16_to_lds_sa(f.db, D == DV ? qcoff[n] : dcoff[n], dst);
                } else {
                    const int row = (w2 * DC::N + n) * DC::ROWS_PER_COPY + lane / DC::CH;
                    const size_t off = (f.rb + min(f.qr0 + row, S - 1)) * DV + ((lane % DC::CH) ^ swz_f<DV>(row)) * 8;
                    copy16_to_lds_a(a.dout + off, dst);
                }
            } else {
                copy4_to_lds_a(f.stat, f.st0 + (T::QTILE + T::DTILE) * 2);
            }
        };
        auto fetch_all = [&](const Fetch& f) {
            if (f.whole) {
#pragma unroll
                for (int k = 0; k < NF; ++k) fetch_copy_t(f, k, std::true_type{});
            } else {
#pragma unroll
                for (int k = 0; k < NF; ++k) fetch_copy_t(f, k, std::false_type{});
            }
        };
        auto fetch = [&]() { fetch_all(fetch_plan()); };  // plan and issue all copies
        // Does the wave work at the step of walk w, and with which rows? It skips a
        // step whose queries all precede its keys, or (window) all lie past the band
        // of its last key; the mask is needed where the rows cross either edge.
        Walk wi;  // the step computed
        walk_start(wi);
        auto item = [&](int& qs0, bool& need_mask) {
            qs0 = (q_lo + wi.r) * kKvBQ;
            need_mask = (CAUSAL && qs0 < kw0 + 31) || (W > 0 && qs0 + 31 > kw0 + W - 1);
            const bool skip = (CAUSAL && qs0 + 31 < kw0) || qs0 >= S || (W > 0 && qs0 > kw0 + 31 + W - 1);
            return wi.g < G && !skip;
        };

        // prologue: the first kKv1Ring - 1 fetches; wait for the first
#pragma unroll
        for (int p = 0; p < kKv1Ring - 1; ++p) fetch();
        __builtin_amdgcn_s_waitcnt(vm_wait_imm((kKv1Ring - 2) * NF));
        barrier_lds();

        if constexpr (MAYBE_PRECISE) {
            for (int j = 0; j < steps; ++j) {
                if (j > 0) {  // step j's stage has landed; every wave is done with step j-1's
                    __builtin_amdgcn_s_waitcnt(vm_wait_imm((kKv1Ring - 2) * NF));
                    barrier_lds();
                }
                fetch();
                int qs0;
                bool msk;
                if (item(qs0, msk)) {
                    const int sl = j % kKv1Ring;
                    const size_t hrow = (size_t)b * a.Hq + hkv * G + wi.g;
                    const bool precise = a.precise_all ||
                        *(const __attribute__((address_space(4))) int*)(uintptr_t)(a.peak + hrow * nQB + q_lo + wi.r) != 0;
                    f32x16 sv, dpv;
                    sdp(sl, sv, dpv);
#pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2) {
                        float pv[8], dsv[8];
                        if (msk)
                            pds(sl, qs0, std::true_type{}, sv, dpv, t2, pv, dsv);
                        else
                            pds(sl, qs0, std::false_type{}, sv, dpv, t2, pv, dsv);
                        const bf16x8 ph = pack_pv(pv), sh = pack_pv(dsv);
                        bf16x8 pl = ph, sl2 = sh;
                        if (precise) {
                            pl = pack_lo(pv);
                            sl2 = pack_lo(dsv);
                        }
                        dvdk(sl, t2, ph, sh, precise, pl, sl2);
                    }
                }
                walk_next(wi);
            }
        } else {
            f32x16 sc, dc;  // S/dP of the current step
            sdp(0, sc, dc);
            // the bookkeeping of a step (its fetch's addresses, whether and how it
            // works) is done in the previous step's dV/dK region, whose matrix
            // instructions leave the wave's issue slots free
            Fetch f = fetch_plan();
            int qs0;
            bool msk;
            bool act = item(qs0, msk);
            for (int j = 0; j < steps; ++j) {
                // step j+1's stage has landed (own copies, then everyone's); every
                // wave is done with step j-1's stage, which the next fetch refills
                __builtin_amdgcn_s_waitcnt(vm_wait_imm((kKv1Ring - 3) * NF));
                barrier_lds();
                const int sl = j % kKv1Ring, sn_ = (j + 1) % kKv1Ring;
                f32x16 sn, dn;
                bf16x8 ph[2], sh[2];
                if (act && !msk && f.whole) {
                    // S/dP of step j+1 (on a stale stage past the last step, never
                    // used) with P and dS of step j between its matrix instructions,
                    // and the copies of the stage three steps ahead spread over them
                    constexpr int DKM_ = DKM;
                    fast_sdp_pds(sl, sn_, sc, dc, sn, dn, ph, sh, [&](int dd) {
#pragma unroll
                        for (int k = dd * NF / DKM_; k < (dd + 1) * NF / DKM_; ++k)
                            fetch_copy_t(f, k, std::true_type{});
                    });
                } else {
                    fetch_all(f);
                    sdp(sn_, sn, dn);
                    if (act) {  // an edge step (the mask), or the stage ahead is a ragged tile
#pragma unroll
                        for (int t2 = 0; t2 < 2; ++t2) {
                            float pv[8], dsv[8];
                            if (msk)
                                pds(sl, qs0, std::true_type{}, sc, dc, t2, pv, dsv);
                            else
                                pds(sl, qs0, std::false_type{}, sc, dc, t2, pv, dsv);
                            ph[t2] = pack_pv(pv);
                            sh[t2] = pack_pv(dsv);
                        }
                    } else {  // nothing to add
                        const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
                        ph[0] = ph[1] = sh[0] = sh[1] = z;
                    }
                }
                // one copy of the dV/dK products for every path, with the next step's
                // bookkeeping in its regions
                dvdk_step(sl, ph, sh, [&](int pp) {
                    if (pp == 0) {
                        walk_next(wi);
                        f = fetch_plan();
                    } else if (pp == 1) {
                        act = item(qs0, msk);
                    }
                });
                sc = sn;
                dc = dn;
            }
        }
        // the ring is reused by the next loop (or the final sum): every copy has
        // landed and every wave is done reading
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        barrier_lds();
    };
    run(qi_first, qi_x - qi_first, std::true_type{});
    run(qi_x, qi_last + 1 - qi_x, std::false_type{});

    // Sum the two pairs' partials (same keys, disjoint iterations) in a fixed order:
    // pair 1 hands its dK to pair 0 and pair 0 its dV to pair 1, then each adds the
    // other's partial to its own. Layout [w2][blocks][r][lane].
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
    barrier_lds();
    float* const xk = (float*)lds_raw;                 // pair 1's dK
    float* const xv = xk + 2 * DBK * 16 * 64;          // pair 0's dV
    if (split == 1) {
#pragma unroll
        for (int db = 0; db < DBK; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) xk[((w2 * DBK + db) * 16 + r) * 64 + lane] = dk[db][r];
    } else {
#pragma unroll
        for (int db = 0; db < DBV; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) xv[((w2 * DBV + db) * 16 + r) * 64 + lane] = dv[db][r];
    }
    barrier_lds();
    if (split == 0 && key < S) {  // dK = scale * (own + pair 1's), D wide
        float* out = a.dk + (kvrow + key) * D;
#pragma unroll
        for (int db = 0; db < DBK; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = (dk[db][4 * g4 + e] + xk[((w2 * DBK + db) * 16 + 4 * g4 + e) * 64 + lane]) * a.scale;
                *(f32x4*)(out + db * 32 + 8 * g4 + 4 * h) = v;
            }
    } else if (split == 1 && key < S) {  // dV = own + pair 0's, DV wide
        float* out = a.dv + (kvrow + key) * DV;
#pragma unroll
        for (int db = 0; db < DBV; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = dv[db][4 * g4 + e] + xv[((w2 * DBV + db) * 16 + 4 * g4 + e) * 64 + lane];
                *(f32x4*)(out + db * 32 + 8 * g4 + 4 * h) = v;
            }
    }
}

template <int D, int DV, bool CAUSAL>
__global__ void __launch_bounds__(kKv1Threads, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
dkv1_kernel(BwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    int b, hkv, kt;
    dkv_item<CAUSAL>(a, b, hkv, kt);
    dkv1_body<D, DV, CAUSAL>(a, lds_raw, b, hkv, kt);
}

// ---------------------------------------------------------------------------
// dK/dV kernel with two waves per SIMD (for D or DV = 128): 8 waves = 4 pairs,
// each pair a double-buffered Q/dO stage, the waves in lock-step through one
// barrier per step; the two waves on a SIMD cover each other's latencies.
// ---------------------------------------------------------------------------
constexpr int kKvSplits = 4;   // wave pairs that split the (head, query tile) iterations
constexpr int kKvThreads = 64 * 2 * kKvSplits;   // two waves per SIMD

template <int D, int DV>
struct KvTile {
    // V tile [64][DV] and per-split double-buffered Q [32][D] and dO [32][DV]
    // tiles, all bf16 in the swizzled chunk order of swz; lse*log2e and delta per
    // query row.
    static constexpr int QTILE = kKvBQ * D;                          // elements
    static constexpr int DTILE = kKvBQ * DV;
    static constexpr int STAGE_BYTES = (QTILE + DTILE) * 2 + 2 * kKvBQ * 4;
    static constexpr int SPLIT_BYTES = 2 * STAGE_BYTES;
    static constexpr int VTILE_BYTES = kKvBK * DV * 2;
    static constexpr int TILE_BYTES = VTILE_BYTES + kKvSplits * SPLIT_BYTES;
    // final sum: two splits hand over dK and dV of both key halves
    static constexpr int XCHG_BYTES = 2 * 2 * (D / 32 + DV / 32) * 16 * 64 * 4;
    static constexpr int LDS_BYTES = TILE_BYTES > XCHG_BYTES ? TILE_BYTES : XCHG_BYTES;
    using QCopy = CopyPlan<D, kKvBQ, 2>;                             // per wave of a pair
    using DCopy = CopyPlan<DV, kKvBQ, 2>;
    using VCopy = CopyPlan<DV, kKvBK, 2 * kKvSplits>;                // per wave
};

// Query tiles qi_first .. qi_x - 1 (of every head of the group) run in a first loop
// whose iterations take the exact path where the dQ stage flagged their tile (or
// everywhere, when the host asks for it); tiles qi_x .. qi_last run in a second,
// plain loop, where the per-iteration test is compiled out and the dV/dK product
// loop is straight-line code. The accumulators carry from one loop into the other.
// qi_x comes from the flags (dkv_exact_end), read once the K rows and the V tile
// are on their way, so that their latencies overlap.
template <int D, int DV, bool CAUSAL>
__device__ __forceinline__ void dkv_body(const BwdArgs& a, unsigned char* lds_raw, int b, int hkv, int kt) {
    using T = KvTile<D, DV>;
    using QC = typename T::QCopy;
    using DC = typename T::DCopy;
    using VC = typename T::VCopy;
    constexpr int DK = D / 16;     // k-steps of the score product
    constexpr int DKV = DV / 16;   // k-steps of the dP product
    constexpr int DKM = DK > DKV ? DK : DKV;
    constexpr int DBK = D / 32;    // 32-row blocks of dK^T
    constexpr int DBV = DV / 32;   // 32-row blocks of dV^T
    constexpr int DBM = DBK > DBV ? DBK : DBV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int split = wave >> 1, w2 = wave & 1, ptid = tid & 127;
    const int S = a.S, G = a.G;
    const int nQB = (S + kKvBQ - 1) / kKvBQ;

    const int kv0 = kt * kKvBK;
    const int kw0 = kv0 + 32 * w2;  // this wave's first key
    const int key = kw0 + l32;      // this lane's key (column of S, dP)
    const size_t kvrow = ((size_t)b * a.Hkv + hkv) * (size_t)S;
    const float c = a.scale_log2;

    // K rows of this lane's key as B operands (zero past the end).
    bf16x8 kf[DK];
    if (key < S) {
        const u32x4* ks = (const u32x4*)(a.k + (kvrow + key) * D + 8 * h);  // K is D wide
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) kf[dk] = __builtin_bit_cast(bf16x8, ks[2 * dk]);
    } else {
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) kf[dk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
    }

    // LDS: V tile, then per split two stages of {Q, dO, lse*log2e, delta}.
    __bf16* const Vs = (__bf16*)lds_raw;
    unsigned char* const split_base = lds_raw + T::VTILE_BYTES + split * T::SPLIT_BYTES;
    auto stage_q = [&](int st) { return (__bf16*)(split_base + st * T::STAGE_BYTES); };
    auto stage_do = [&](int st) { return stage_q(st) + T::QTILE; };
    auto stage_lse = [&](int st) {
        return (float*)(split_base + st * T::STAGE_BYTES + (T::QTILE + T::DTILE) * 2);
    };
    auto stage_dl = [&](int st) { return stage_lse(st) + kKvBQ; };

    // V tile: every wave copies VCOPIES rows-runs (rows past the end repeat S-1;
    // those keys' columns are never stored).
#pragma unroll
    for (int n = 0; n < VC::N; ++n) {
        const int row = (wave * VC::N + n) * VC::ROWS_PER_COPY + lane / VC::CH;
        const int col = (((lane % VC::CH) ^ swz_f<DV>(row))) * 8;
        const int kr = min(kv0 + row, S - 1);
        copy16_to_lds(a.v + (kvrow + kr) * DV + col, Vs + (wave * VC::N + n) * 512);
    }

    // Iterations of a loop over query tiles q_lo .. q_lo + nq - 1: (g, query tile qi)
    // for every head g of the group; split p takes iterations p, p + kKvSplits, ...
    const int W = CAUSAL ? a.window : 0;
    int qi_first, qi_last;
    dkv_range<CAUSAL>(a, kt, qi_first, qi_last);
    const int qi_x = a.precise_all ? qi_last + 1 : dkv_exact_end<CAUSAL>(a, b, hkv, kt);

    f32x16 dk[DBK], dv[DBV];
#pragma unroll
    for (int db = 0; db < DBK; ++db) dk[db] = zero16();
#pragma unroll
    for (int db = 0; db < DBV; ++db) dv[db] = zero16();

    auto run = [&](int q_lo, int nq, auto exact_tag) {
        constexpr bool MAYBE_PRECISE = decltype(exact_tag)::value;
        const int total = G * nq;
        const int steps = (total + kKvSplits - 1) / kKvSplits;
        if (steps == 0) return;  // the same in every wave of the workgroup
        // per-lane offsets are made in each loop: live across both, they would be
        // spilled in both
        // Q / dO copies of a pair: copy n of wave w2 fills tile rows (w2*N + n) *
        // ROWS_PER_COPY + lane / CH, kept as this lane's byte offset within a tile of
        // whole rows. Rows past S repeat row S-1; their lse is +inf, so their
        // probabilities, and every term they touch, are exactly 0.
        uint32_t qcoff[QC::N], dcoff[DC::N];
    #pragma unroll
        for (int n = 0; n < QC::N; ++n) {
            const int row = (w2 * QC::N + n) * QC::ROWS_PER_COPY + lane / QC::CH;
            qcoff[n] = (uint32_t)(row * D + ((lane % QC::CH) ^ swz_f<D>(row)) * 8) * 2u;
        }
    #pragma unroll
        for (int n = 0; n < DC::N; ++n) {  // the same as qcoff when D == DV
            const int row = (w2 * DC::N + n) * DC::ROWS_PER_COPY + lane / DC::CH;
            dcoff[n] = D == DV ? 0u : (uint32_t)(row * DV + ((lane % DC::CH) ^ swz_f<DV>(row)) * 8) * 2u;
        }
        // Per-lane LDS offsets: A-operand rows (Q; dO and V) per k-step; transpose
        // quads (Q^T; dO^T) per 32-column block and row half.
        int roff[DK], rvoff[DKV], toff[2][DBK], tvoff[2][DBV];
    #pragma unroll
        for (int dk = 0; dk < DK; ++dk) roff[dk] = swz<D>(l32, dk * 16 + 8 * h);
    #pragma unroll
        for (int dk = 0; dk < DKV; ++dk) rvoff[dk] = swz<DV>(l32, dk * 16 + 8 * h);
    #pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
    #pragma unroll
            for (int db = 0; db < DBK; ++db)
                toff[hf][db] = swz<D>(4 * h + ((lane & 15) >> 2) + 8 * hf,
                                      db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    #pragma unroll
            for (int db = 0; db < DBV; ++db)
                tvoff[hf][db] = swz<DV>(4 * h + ((lane & 15) >> 2) + 8 * hf,
                                        db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
        }
        float lst = 0.f, dlst = 0.f;
        int peak_next = 0;  // exact body: the dQ stage's flag of the iteration being fetched
        auto fetch = [&](int step) {  // async copies of Q/dO + lse/delta into registers
            const int it = kKvSplits * step + split;
            if (it >= total) return;
            const int st = step & 1;
            const int g = it / nq, qi = q_lo + it % nq;
            const size_t hrow = (size_t)b * a.Hq + hkv * G + g;  // the query head's index
            const size_t rb = hrow * (size_t)S;
            const int qr0 = qi * kKvBQ;
            // A whole tile inside S: its first row's address (scalar) plus lane offsets.
            // The body with the exact path keeps per-lane addresses: it has no
            // registers to spare for the scalar form's.
            if (!MAYBE_PRECISE && qr0 + kKvBQ <= S) {
                const uint16_t* qb = a.q + (rb + qr0) * D;
                const uint16_t* db = a.dout + (rb + qr0) * DV;
    #pragma unroll
                for (int n = 0; n < QC::N; ++n)
                    copy16_to_lds_s(qb, qcoff[n], stage_q(st) + (w2 * QC::N + n) * 512);
    #pragma unroll
                for (int n = 0; n < DC::N; ++n)
                    copy16_to_lds_s(db, D == DV ? qcoff[n] : dcoff[n], stage_do(st) + (w2 * DC::N + n) * 512);
            } else if (D == DV) {  // one address for both tensors
    #pragma unroll
                for (int n = 0; n < QC::N; ++n) {
                    const int row = (w2 * QC::N + n) * QC::ROWS_PER_COPY + lane / QC::CH;
                    const size_t off = (rb + min(qr0 + row, S - 1)) * D + ((lane % QC::CH) ^ swz_f<D>(row)) * 8;
                    copy16_to_lds(a.q + off, stage_q(st) + (w2 * QC::N + n) * 512);
                    copy16_to_lds(a.dout + off, stage_do(st) + (w2 * QC::N + n) * 512);
                }
            } else {
    #pragma unroll
                for (int n = 0; n < QC::N; ++n) {
                    const int row = (w2 * QC::N + n) * QC::ROWS_PER_COPY + lane / QC::CH;
                    const size_t off = (rb + min(qr0 + row, S - 1)) * D + ((lane % QC::CH) ^ swz_f<D>(row)) * 8;
                    copy16_to_lds(a.q + off, stage_q(st) + (w2 * QC::N + n) * 512);
                }
    #pragma unroll
                for (int n = 0; n < DC::N; ++n) {
                    const int row = (w2 * DC::N + n) * DC::ROWS_PER_COPY + lane / DC::CH;
                    const size_t off = (rb + min(qr0 + row, S - 1)) * DV + ((lane % DC::CH) ^ swz_f<DV>(row)) * 8;
                    copy16_to_lds(a.dout + off, stage_do(st) + (w2 * DC::N + n) * 512);
                }
            }
            if (ptid < kKvBQ) {
                // raw values only: any use of a loaded value here would make the wave
                // wait for its vector-memory counter, which also counts the tile
                // copies just issued, and so for the whole prefetch
                const int qr = qr0 + ptid;
                lst = qr < S ? a.lse[rb + qr] : INFINITY;
                // -delta of the row (0 past S), negated at publish; the index is below
                // B*Hq*(2S + 64) < 2^32
                dlst = a.rowstat[(uint32_t)hrow * (uint32_t)(nQB * kKvBQ * 2) + (uint32_t)(qr0 * 2 + kKvBQ + ptid)];
            }
            // The flag's address is the same in every lane: a scalar load through the
            // constant address space (the dQ stage wrote it before this launch) keeps it
            // in a scalar register; it is read one step later.
            if (MAYBE_PRECISE)
                peak_next = *(const __attribute__((address_space(4))) int*)(uintptr_t)(a.peak + hrow * nQB + qi);
        };
        auto publish = [&](int step) {  // row statistics into the stage the copies fill
            const int it = kKvSplits * step + split;
            if (it >= total) return;
            if (ptid < kKvBQ) {
                stage_lse(step & 1)[ptid] = lst * kLog2e;
                stage_dl(step & 1)[ptid] = -dlst;
            }
        };

        fetch(0);
        publish(0);
        wait_copies();
        __syncthreads();
        for (int step = 0; step < steps; ++step) {
            // this iteration's flag, loaded one step ago (complete since the last wait)
            const bool peak_cur = MAYBE_PRECISE && peak_next != 0;
            if (step + 1 < steps) fetch(step + 1);
            const int it = kKvSplits * step + split;
            if (it < total) {
                const int st = step & 1;
                const __bf16* Qs = stage_q(st);
                const __bf16* Ds = stage_do(st);
                const float* Ls = stage_lse(st);
                const float* Dl = stage_dl(st);
                const int qs0 = (q_lo + it % nq) * kKvBQ;
                const bool precise = MAYBE_PRECISE && (a.precise_all || peak_cur);
                // skip when every query precedes every key of the wave, or (window)
                // every query lies past the band of the wave's last key
                const bool skip = (CAUSAL && qs0 + 31 < kw0) || qs0 >= S || (W > 0 && qs0 > kw0 + 31 + W - 1);
                if (!skip) {
                    const bool need_mask = (CAUSAL && qs0 < kw0 + 31) || (W > 0 && qs0 + 31 > kw0 + W - 1);
                    f32x16 s = zero16(), dp = zero16();
    #pragma unroll
                    for (int dd = 0; dd < DKM; ++dd) {
                        bf16x8 qa, da, vb;
                        if (dd < DK) qa = lds_read8(Qs + roff[dd]);
                        if (dd < DKV) {
                            da = lds_read8(Ds + rvoff[dd]);
                            vb = lds_read8(Vs + rvoff[dd] + w2 * 32 * DV);
                        }
                        if (dd < DK) s = mfma32(qa, kf[dd], s);
                        if (dd < DKV) dp = mfma32(da, vb, dp);
                    }
                    // rows of s/dp are queries 8(r/4) + 4h + r%4; the column is this lane's key.
                    // dV^T += dO^T P and dK^T += Q^T dS over two 16-query steps.
    #pragma unroll
                    for (int t2 = 0; t2 < 2; ++t2) {
                        float pv[8], dsv[8], dl[8];
    #pragma unroll
                        for (int half = 0; half < 2; ++half) {
                            const int rg = 2 * t2 + half;
                            const f32x4 l4 = *(const f32x4*)(Ls + 8 * rg + 4 * h);
                            const f32x4 d4 = *(const f32x4*)(Dl + 8 * rg + 4 * h);
    #pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                pv[4 * half + e] = fast_exp2(fmaf(s[4 * rg + e], c, -l4[e]));
                                dl[4 * half + e] = d4[e];
                            }
                        }
                        if (need_mask) {  // one uniform branch, taken on edge tiles only
    #pragma unroll
                            for (int i = 0; i < 8; ++i) {
                                const int qrow = qs0 + 8 * (2 * t2 + (i >> 2)) + 4 * h + (i & 3);
                                pv[i] = (key > qrow || (W > 0 && qrow >= key + W)) ? 0.0f : pv[i];
                            }
                        }
    #pragma unroll
                        for (int i = 0; i < 8; ++i) dsv[i] = pv[i] * (dp[8 * t2 + i] - dl[i]);
                        const bf16x8 ph = pack8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
                        const bf16x8 sh = pack8(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
                        bf16x8 pl, sl;
                        if (precise) {
                            pl = pack8(bf_lo(pv[0]), bf_lo(pv[1]), bf_lo(pv[2]), bf_lo(pv[3]), bf_lo(pv[4]),
                                       bf_lo(pv[5]), bf_lo(pv[6]), bf_lo(pv[7]));
                            sl = pack8(bf_lo(dsv[0]), bf_lo(dsv[1]), bf_lo(dsv[2]), bf_lo(dsv[3]), bf_lo(dsv[4]),
                                       bf_lo(dsv[5]), bf_lo(dsv[6]), bf_lo(dsv[7]));
                        }
                        const int rbk = 16 * t2 * D, rbv = 16 * t2 * DV;
    #pragma unroll
                        for (int db = 0; db < DBM; ++db) {
                            bf16x8 dot, qt;
                            if (db < DBV)
                                dot = concat(lds_read_tr(Ds + tvoff[0][db] + rbv), lds_read_tr(Ds + tvoff[1][db] + rbv));
                            if (db < DBK)
                                qt = concat(lds_read_tr(Qs + toff[0][db] + rbk), lds_read_tr(Qs + toff[1][db] + rbk));
                            if (db < DBV) dv[db] = mfma32(dot, ph, dv[db]);
                            if (db < DBK) dk[db] = mfma32(qt, sh, dk[db]);
                            if (precise) {
                                if (db < DBV) dv[db] = mfma32(dot, pl, dv[db]);
                                if (db < DBK) dk[db] = mfma32(qt, sl, dk[db]);
                            }
                        }
                    }
                }
            }
            if (step + 1 < steps) publish(step + 1);
            wait_copies();
            __syncthreads();
        }
    };
    run(qi_first, qi_x - qi_first, std::true_type{});
    run(qi_x, qi_last + 1 - qi_x, std::false_type{});

    // Sum the four splits' partials (same keys, disjoint iterations) in a fixed
    // order: splits 2,3 hand over to splits 0,1; then split 1 hands dK to split 0
    // and split 0 hands dV to split 1. Layout [slot][w2][dK blocks, dV blocks][r][lane].
    float* xchg = (float*)lds_raw;
    auto slot = [&](int sl, int tensor, int db, int r) {
        return xchg + ((((sl * 2 + w2) * (DBK + DBV) + tensor * DBK + db) * 16 + r) * 64) + lane;
    };
    if (split >= 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int db = 0; db < DBK; ++db) *slot(split - 2, 0, db, r) = dk[db][r];
#pragma unroll
            for (int db = 0; db < DBV; ++db) *slot(split - 2, 1, db, r) = dv[db][r];
        }
    }
    __syncthreads();
    if (split < 2) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
#pragma unroll
            for (int db = 0; db < DBK; ++db) dk[db][r] += *slot(split, 0, db, r);
#pragma unroll
            for (int db = 0; db < DBV; ++db) dv[db][r] += *slot(split, 1, db, r);
        }
    }
    __syncthreads();
    if (split == 1) {
#pragma unroll
        for (int db = 0; db < DBK; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) *slot(0, 0, db, r) = dk[db][r];
    } else if (split == 0) {
#pragma unroll
        for (int db = 0; db < DBV; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) *slot(1, 1, db, r) = dv[db][r];
    }
    __syncthreads();
    if (split == 0 && key < S) {  // dK = scale * (own + split 1's), D wide
        float* out = a.dk + (kvrow + key) * D;
#pragma unroll
        for (int db = 0; db < DBK; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (dk[db][4 * g4 + e] + *slot(0, 0, db, 4 * g4 + e)) * a.scale;
                *(f32x4*)(out + db * 32 + 8 * g4 + 4 * h) = v;
            }
    } else if (split == 1 && key < S) {  // dV = own + split 0's, DV wide
        float* out = a.dv + (kvrow + key) * DV;
#pragma unroll
        for (int db = 0; db < DBV; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = dv[db][4 * g4 + e] + *slot(1, 1, db, 4 * g4 + e);
                *(f32x4*)(out + db * 32 + 8 * g4 + 4 * h) = v;
            }
    }
}

template <int D, int DV, bool CAUSAL>
__global__ void __launch_bounds__(kKvThreads, 1) dkv_kernel(BwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    int b, hkv, kt;
    dkv_item<CAUSAL>(a, b, hkv, kt);
    dkv_body<D, DV, CAUSAL>(a, lds_raw, b, hkv, kt);
}

template <int D, int DV, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& args, int stages, hipStream_t stream) {
    BwdArgs a = args;
    if (stages & 1) {
        // Query tiles whose rows need the exact path: all of them when asked for,
        // else tile 0 of a causal problem or the single tile of S <= 128.
        const int nQ = (a.S + kDqBQ - 1) / kDqBQ;
        constexpr int lds = DqTile<D, DV>::LDS_BYTES;
        if (CAUSAL && a.window > 0) {
            const int HW = dq_win_heads(a.G), BQ = 32 * (4 / HW);
            const long long wblocks = (long long)((a.S + BQ - 1) / BQ) * a.B * a.Hkv * (a.G / HW);
            hipLaunchKernelGGL((dq_win_kernel<D, DV>), dim3((unsigned)wblocks), dim3(kDqThreads), lds, stream, a);
        } else {
            const long long blocks = (long long)a.B * a.Hq * nQ;
            hipLaunchKernelGGL((dq_kernel<D, DV, CAUSAL>), dim3((unsigned)blocks), dim3(kDqThreads), lds, stream, a);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (stages & 2) {
        const int nKB = (a.S + kKvBK - 1) / kKvBK;
        const long long kvblocks = (long long)a.B * a.Hkv * nKB;
        if constexpr (kDkvOneWave<D, DV>) {
            constexpr int lds = Kv1Tile<D, DV>::LDS_BYTES;
            hipLaunchKernelGGL((dkv1_kernel<D, DV, CAUSAL>), dim3((unsigned)kvblocks), dim3(kKv1Threads), lds, stream, a);
        } else {
            constexpr int lds = KvTile<D, DV>::LDS_BYTES;
            hipLaunchKernelGGL((dkv_kernel<D, DV, CAUSAL>), dim3((unsigned)kvblocks), dim3(kKvThreads), lds, stream,
                               a);
        }
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename K>
hipError_t set_lds(K kernel, int bytes) {
    return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int D, int DV>
hipError_t setup_pair() {
    hipError_t e;
    if ((e = set_lds(dq_kernel<D, DV, false>, DqTile<D, DV>::LDS_BYTES))) return e;
    if ((e = set_lds(dq_kernel<D, DV, true>, DqTile<D, DV>::LDS_BYTES))) return e;
    if ((e = set_lds(dq_win_kernel<D, DV>, DqTile<D, DV>::LDS_BYTES))) return e;
    if constexpr (kDkvOneWave<D, DV>) {
        if ((e = set_lds(dkv1_kernel<D, DV, false>, Kv1Tile<D, DV>::LDS_BYTES))) return e;
        return set_lds(dkv1_kernel<D, DV, true>, Kv1Tile<D, DV>::LDS_BYTES);
    } else {
        if ((e = set_lds(dkv_kernel<D, DV, false>, KvTile<D, DV>::LDS_BYTES))) return e;
        return set_lds(dkv_kernel<D, DV, true>, KvTile<D, DV>::LDS_BYTES);
    }
}

template <int D, int DV>
hipError_t launch_pair(const BwdArgs& a, int stages, hipStream_t stream) {
    return a.causal ? launch_bwd_t<D, DV, true>(a, stages, stream) : launch_bwd_t<D, DV, false>(a, stages, stream);
}

}  // namespace

hipError_t bwd_setup_device() {
    hipError_t e;
    if ((e = setup_pair<64, 64>())) return e;
    if ((e = setup_pair<128, 128>())) return e;
    if ((e = setup_pair<64, 128>())) return e;
    return setup_pair<128, 64>();
}

hipError_t launch_bwd(const BwdArgs& a, int D, int DV, int stages, hipStream_t stream) {
    if (D == 64) return DV == 64 ? launch_pair<64, 64>(a, stages, stream) : launch_pair<64, 128>(a, stages, stream);
    return DV == 128 ? launch_pair<128, 128>(a, stages, stream) : launch_pair<128, 64>(a, stages, stream);
}

}  // namespace attn
