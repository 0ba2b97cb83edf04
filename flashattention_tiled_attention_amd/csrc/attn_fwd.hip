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
// One workgroup = 8 waves = one tile of 256 query rows of one (batch, head);
// each wave owns 32 rows (with a sliding window, fwd_win_kernel gives the 8
// waves several query heads of one kv head instead, see there). When queries,
// keys and values are all 128 wide, the running-maximum slack is on and S is a
// multiple of 256, fwd1_kernel (further down) takes the same tiles with 4 waves
// of 64 rows each instead. Per key tile j
// (64 keys; 128 when queries, keys and values are all 64 wide), a wave does
//   S^T = K Q^T        v_mfma_f32_32x32x16_bf16, K from LDS (A), Q in registers (B)
//                      -> every lane holds one query column and 32 of its keys,
//                         so the row max/sum are lane-local plus one permlane32 swap
//   online softmax     exp2 with the scale folded into one fma per score
//   O^T += V^T P^T     P^T from the score registers (B), V^T read from the
//                      row-major V tile with ds_read_b64_tr_b16 (A)
//
// Ping-pong: the waves form two groups of four, and each SIMD holds one wave of
// each group. Time is cut into phases separated by workgroup barriers; in every
// phase one group runs its matrix work (the P V product of tile j-1 and the
// score product of tile j: 32 MFMAs) while the other group runs the
// softmax of its previous tile on the vector unit, so each SIMD's matrix unit
// always has one wave feeding it. The matrix-phase wave raises its issue
// priority so its MFMAs are not starved by the softmax wave.
//
// K and V tiles stream from HBM straight into LDS (global_load_lds), two tiles
// ahead of use, into unpadded tiles with a per-row XOR order of 16-byte chunks
// that keeps both the K row reads and the V transpose reads free of bank
// conflicts. Causal tiles entirely above the diagonal are never loaded; each
// wave masks only its last tile (the diagonal, or the ragged end of S).
//
// Rows that see few keys carry large probabilities, where rounding P to bf16 for
// the P V product would cost up to about 2^-9 of |V| in O. For those rows (a
// window of fewer than 128 keys, the first query tile of a causal or windowed
// problem, a single tile of S <= 128) the workgroup takes a PRECISE body that splits P into
// a bf16 high part and a bf16 remainder and runs the P V product on both. Both
// bodies live in one launch, so the few exact-path workgroups run in the tail
// of the longest-first schedule instead of in a launch of their own.
//
// Queries and keys have D columns and values DV (the d and d_v of Eq. (1)); each
// is 64 or 128, in any combination.
//
// With a sliding window of W keys (query i sees keys i-W+1 .. i, the window of
// the page's compressed sparse attention, Table 7) the tiles entirely below the
// band are skipped as well, and a wave also masks the tiles that cross the
// band's lower edge.
#include "device.h"
#include "kernels.h"
#include <type_traits>

namespace attn {
namespace {

constexpr int kFwdBQ = 256;     // query rows per workgroup
constexpr int kFwdWaves = 8;
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr int kLook = 4;        // LDS operand reads in flight ahead of the MFMAs

// Keys per LDS tile of a body: 128 for the plain body when queries, keys and
// values are all 64 wide, so a matrix phase has 32 MFMAs as it does at 128 (with
// 64-key tiles a D = 64 phase had 16, too few to cover the softmax phase and the
// barriers); 64 otherwise. The exact body keeps 64: its split probabilities need
// the registers that 128-key scores would take.
template <int D, int DV, bool PRECISE>
constexpr int fwd_keys_per_tile() { return (D == 64 && DV == 64 && !PRECISE) ? 128 : 64; }

template <int D, int DV, int BK_ = 64>
struct FwdTile {
    static constexpr int BK = BK_;
    // K tiles are unpadded [BK][D] and V tiles [BK][DV] bf16, in the chunk order
    // of swz<D> and swz<DV>, so each 1 KB run of rows is contiguous, as the
    // direct copies need.
    static constexpr int KTILE = BK * D;                          // elements
    static constexpr int VTILE = BK * DV;
    static constexpr int LDS_BYTES = 2 * (KTILE + VTILE) * 2;     // 2 K slots + 2 V slots
    using KCopy = CopyPlan<D, BK, kFwdWaves>;
    using VCopy = CopyPlan<DV, BK, kFwdWaves>;
};

// Dynamic LDS of a forward launch: the larger of its two bodies' rings.
template <int D, int DV>
constexpr int fwd_lds_bytes() { return FwdTile<D, DV, fwd_keys_per_tile<D, DV, false>()>::LDS_BYTES; }

// Work item of workgroup `bid` among nQ query-tile ranks: rank r is query tile
// qt_first - r when causal (longest first), qt_first + r otherwise. When the
// (b, kv-head) groups divide evenly over the 8 XCDs, all query heads of one
// group land on the same XCD (workgroups are dealt to XCDs round-robin by id),
// so its K/V stay in that XCD's L2. Causal items go rank-major over the groups,
// so the longest tiles start first; the others go group-major, so the 32
// workgroups an XCD holds at once read the K/V of one to four groups: at B=8,
// H=16, S=2048, D=64 rank-major order has 16 groups' K/V (8 MiB) in flight per
// XCD, against a 4 MiB L2, and fetches 3 times the algorithmic bytes from HBM.
__device__ __forceinline__ void decode_item(int bid, int nQ, int qt_first, int B, int Hkv, int G,
                                            bool causal, int& b, int& hq, int& qt) {
    const int C = B * Hkv;
    int rank, c, g;
    if (causal) {  // rank-major: the longest tiles of every group go first
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
    } else {  // group-major: the workgroups an XCD holds at once share few groups' K/V
        const int per = nQ * G;
        const bool spread = (C & 7) == 0;
        const int s = spread ? bid >> 3 : bid;
        const int cl = s / per, rem = s - cl * per;
        rank = rem / G;
        g = rem - rank * G;
        c = spread ? cl * 8 + (bid & 7) : cl;
    }
    qt = causal ? qt_first - rank : qt_first + rank;
    b = c / Hkv;
    hq = (c % Hkv) * G + g;
}

// One workgroup's share: query rows q0 .. q_last of the kv head that hq reads;
// this wave takes head hq, rows row0 .. row0+31.
template <int D, int DV, bool CAUSAL, bool PRECISE>
__device__ __forceinline__ void fwd_body(const FwdArgs& a, __bf16* smem, int b, int hq, int q0, int q_last,
                                         int row0) {
    using T = FwdTile<D, DV, fwd_keys_per_tile<D, DV, PRECISE>()>;
    using KC = typename T::KCopy;
    using VC = typename T::VCopy;
    constexpr int BK = T::BK;    // keys per tile
    constexpr int NKB = BK / 32; // 32-key blocks of a tile's scores
    constexpr int NT = BK / 16;  // 16-key steps of its P V product
    constexpr int DK = D / 16;   // k-steps of the score product
    constexpr int DB = DV / 32;  // 32-row blocks of O^T

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;  // ping-pong group; waves w and w+4 share a SIMD
    const int h = lane >> 5, l32 = lane & 31;
    const int S = a.S;
    const int hkv = hq / a.G;
    const size_t qrows = ((size_t)b * a.Hq + hq) * (size_t)S;
    const size_t kvrows = ((size_t)b * a.Hkv + hkv) * (size_t)S;
    const size_t qbase = qrows * D;
    const uint16_t* Kp = a.k + kvrows * D;
    const uint16_t* Vp = a.v + kvrows * DV;
    const int qrow = row0 + l32;
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

    const int nK = (S + BK - 1) / BK;
    const int jend = CAUSAL ? min(nK, q_last / BK + 1) : nK;
    int wjend = CAUSAL ? min(jend, (row0 + 31) / BK + 1) : jend;
    if (row0 >= S) wjend = 0;  // a wave with no live rows only helps load
    // Window: the workgroup's first tile holds the first row's first key, a wave's
    // first tile its first row's; tiles with keys below row0 + 32 - W are masked.
    const int W = CAUSAL ? a.window : 0;
    const int jstart = W > 0 ? max(0, q0 - W + 1) / BK : 0;
    const int wjstart = W > 0 ? max(0, row0 - W + 1) / BK : 0;

    __bf16* const Kring = smem;
    __bf16* const Vring = smem + 2 * T::KTILE;

    // Direct copies: copy n of this wave fills tile rows (wave*N + n) *
    // ROWS_PER_COPY + lane / CH, physical chunk lane % CH, which holds logical
    // chunk (lane % CH) ^ swz_f(row). Rows past the end repeat row S-1: their
    // scores are masked and their probabilities are exactly 0.
    // This lane's copy n as a byte offset within a tile of whole rows: a tile that
    // lies inside S is copied from its first row's address (scalar) plus these.
    uint32_t kcoff[KC::N], vcoff[VC::N];
#pragma unroll
    for (int n = 0; n < KC::N; ++n) {
        const int row = (wave * KC::N + n) * KC::ROWS_PER_COPY + lane / KC::CH;
        kcoff[n] = (uint32_t)(row * D + ((lane % KC::CH) ^ swz_f<D>(row)) * 8) * 2u;
    }
#pragma unroll
    for (int n = 0; n < VC::N; ++n) {
        const int row = (wave * VC::N + n) * VC::ROWS_PER_COPY + lane / VC::CH;
        vcoff[n] = (uint32_t)(row * DV + ((lane % VC::CH) ^ swz_f<DV>(row)) * 8) * 2u;
    }
    auto copy_k = [&](__bf16* dst, int j) {
        const int k0 = j * BK;
        if (k0 + BK <= S) {
            const uint16_t* base = Kp + (size_t)k0 * D;
#pragma unroll
            for (int n = 0; n < KC::N; ++n) copy16_to_lds_s(base, kcoff[n], dst + (wave * KC::N + n) * 512);
            return;
        }
#pragma unroll
        for (int n = 0; n < KC::N; ++n) {  // the last tile: rows past S repeat row S-1
            const int e = kcoff[n] >> 1, key = min(k0 + e / D, S - 1);
            copy16_to_lds(Kp + (uint32_t)(key * D + e % D), dst + (wave * KC::N + n) * 512);
        }
    };
    auto copy_v = [&](__bf16* dst, int j) {
        const int k0 = j * BK;
        if (k0 + BK <= S) {
            const uint16_t* base = Vp + (size_t)k0 * DV;
#pragma unroll
            for (int n = 0; n < VC::N; ++n) copy16_to_lds_s(base, vcoff[n], dst + (wave * VC::N + n) * 512);
            return;
        }
#pragma unroll
        for (int n = 0; n < VC::N; ++n) {
            const int e = vcoff[n] >> 1, key = min(k0 + e / DV, S - 1);
            copy16_to_lds(Vp + (uint32_t)(key * DV + e % DV), dst + (wave * VC::N + n) * 512);
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
            voff[hf][db] = swz<DV>(4 * h + ((lane & 15) >> 2) + 8 * hf,
                                   db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = zero16();
    // m starts finite: a row whose keys in its first tiles all fall below the
    // window keeps m, and exp2(-inf - m) is then 0 rather than NaN; the first
    // visible key moves it, and exp2(m - mnew) is 0 as it would be from -inf.
    float m = -1e30f, l = 0.0f;
    f32x16 sc[NKB];  // scores of the tile between its matrix and softmax phases
    bf16x8 pk[NT];   // probabilities of the tile between its softmax and P V phases
    bf16x8 pl[NT];   // their bf16 remainders (PRECISE only)

    // Matrix phase of tile j: O^T += V_{j-1}^T P_{j-1}^T, then S^T_j = K_j Q^T.
    // par: std::integral_constant holding j & 1, or -1 to take it from j at run time.
    auto matrix_phase = [&](int j, auto par) {
        constexpr int PC = decltype(par)::value;
        const int P = PC < 0 ? (j & 1) : PC;  // a constant parity folds the slot into the reads' offsets
        __builtin_amdgcn_s_setprio(1);
        if (j - 1 >= wjstart && j - 1 < wjend) {
            const __bf16* Vs = Vring + (PC < 0 ? ((j - 1) & 1) : (P ^ 1)) * T::VTILE;
            constexpr int MPER = PRECISE ? 2 : 1;  // MFMAs per V^T operand
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x4 v1 = lds_read_tr(Vs + voff[0][db] + 16 * t * DV);
                    const bf16x4 v2 = lds_read_tr(Vs + voff[1][db] + 16 * t * DV);
                    const bf16x8 vt = concat(v1, v2);
                    oacc[db] = mfma32(vt, pk[t], oacc[db]);
                    if (PRECISE) oacc[db] = mfma32(vt, pl[t], oacc[db]);
                }
            // transpose reads run LOOK operands ahead of the MFMAs: enough to
            // cover LDS latency with bounded register use
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * kLook, 0);
#pragma unroll
            for (int i = 0; i < NT * DB - kLook; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, MPER, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kLook * MPER, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (j >= wjstart && j < wjend) {
            const __bf16* Ks = Kring + P * T::KTILE;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sc[kb] = zero16();
#pragma unroll
            for (int dk = 0; dk < DK; ++dk)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const bf16x8 kf = lds_read8(Ks + koff[dk] + kb * 32 * D);
                    sc[kb] = mfma32(kf, qf[dk], sc[kb]);
                }
            __builtin_amdgcn_sched_group_barrier(0x100, kLook, 0);
#pragma unroll
            for (int i = 0; i < NKB * DK - kLook; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, kLook, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
    };

    // Probabilities exp2(s c - m) of the tile as bf16 B operands (and their bf16
    // remainders on the exact path); returns this lane's sum of its BK/2.
    auto probs = [&]() {
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = fast_exp2(fmaf(sc[t >> 1][8 * (t & 1) + e], c, -m));
                rs[e & 3] += p[e];
            }
            pk[t] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
            if (PRECISE)
                pl[t] = pack8(bf_lo(p[0]), bf_lo(p[1]), bf_lo(p[2]), bf_lo(p[3]), bf_lo(p[4]), bf_lo(p[5]),
                              bf_lo(p[6]), bf_lo(p[7]));
        }
        return (rs[0] + rs[1]) + (rs[2] + rs[3]);
    };
    // The maximum can be skipped only where the running maximum may lag
    // (slack > 0); with slack 0 it is tracked exactly.
    const bool fast_max = a.max_slack >= 1.0f;
    const float max_bound = exp2f(a.max_slack - 1.0f);

    // Softmax phase of tile j: mask (last tile only), row maxima, lazy move of
    // the running maximum, probabilities as bf16 B operands, row sums.
    auto softmax_phase = [&](int j) {
        if (j < wjstart || j >= wjend) return;
        if (j == wjend - 1 || (W > 0 && j * BK < row0 + 32 - W)) {
            // key j*BK + 4h + off is visible iff lo <= off <= lim
            const int base = j * BK + 4 * h;
            const int lim = (CAUSAL ? min(qrow, S - 1) : S - 1) - base;
            const int lo = W > 0 ? qrow - W + 1 - base : -(1 << 30);
            // -inf goes in under a sign-extended mask, not through a compare and
            // select: that keeps the 2 * BK/2 comparisons out of the scalar
            // registers, which lane masks would fill. With a causal or window edge
            // it goes in by a bitwise select (hide_if), which also hides a NaN score
            // of a key the row must not see; without one the only hidden keys are
            // the ragged end's, copies of key S-1 that every row sees, and adding
            // -inf (or +0.0) is enough.
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                    const int hidden = ((lim - off) | (off - lo)) >> 31;  // all ones iff off > lim or off < lo
                    if constexpr (CAUSAL)
                        sc[kb][r] = hide_if(hidden, sc[kb][r]);
                    else
                        sc[kb][r] += __int_as_float(hidden & (int)0xff800000u);
                }
        }
        // Past a wave's first tile the maximum is usually not needed: if every
        // lane's BK/2 probabilities against the current m sum to at most
        // 2^(slack-1), each of them is at most that, so the tile maximum is
        // within slack-1 of m (one unit of margin covers the rounding of the two
        // forms) and the rule below would leave m alone. The probabilities and
        // sums are then exactly those of the full step; otherwise (a new
        // maximum, an overflow, a NaN) the full step runs on the unchanged
        // scores.
        bool need_max = PRECISE || !fast_max || j <= wjstart;
        float tot = 0.0f;
        if (!need_max) {
            tot = probs();
            need_max = __any(!(tot <= max_bound));
        }
        if (need_max) {
            float mx[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                mx[kb] = fmaxf(sc[kb][0], sc[kb][1]);
#pragma unroll
                for (int r = 2; r < 16; ++r) mx[kb] = fmaxf(mx[kb], sc[kb][r]);
            }
#pragma unroll
            for (int kb = 1; kb < NKB; ++kb) mx[0] = fmaxf(mx[0], mx[kb]);
            const float mt = halves_max(mx[0]) * c;  // c > 0
            // The running maximum only moves when some row's grows by more than
            // max_slack (log2 units; 8 for ordinary score spreads): until then
            // every exp2(t - m) <= 2^slack, carried by fp32 and bf16 without
            // loss, and the O rescale is skipped. A row's first visible key
            // always moves it.
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
            tot = probs();
        }
        l += tot;
    };

    // Prologue: tile j sits in slot j & 1 of its ring; the first two K tiles and
    // the first V tile.
    copy_k(Kring + (jstart & 1) * T::KTILE, jstart);
    if (jstart + 1 < jend) copy_k(Kring + ((jstart + 1) & 1) * T::KTILE, jstart + 1);
    copy_v(Vring + (jstart & 1) * T::VTILE, jstart);
    wait_copies();
    __syncthreads();

    // Two phases per step s, each closed by a workgroup barrier. Group 0 runs the
    // matrix phase of tile s then its softmax; group 1 runs the softmax of tile
    // s-1 then the matrix phase of tile s, so on every SIMD one wave multiplies
    // while the other exponentiates. Steps run from the first tile the workgroup
    // needs to one past its last. Tiles K_s and V_{s-1} are read in step s;
    // at the start of step s+1 the copies of K_{s+2} and V_{s+1} go into the
    // slots those two released, and they are complete before the barrier that
    // ends step s+1. Every wave passes every barrier; waves with fewer tiles idle
    // in their late phases.
    auto refill = [&](int s) {
        if (s > jstart) {
            if (s + 1 < jend) copy_k(Kring + ((s - 1) & 1) * T::KTILE, s + 1);
            if (s < jend) copy_v(Vring + (s & 1) * T::VTILE, s);
        }
    };
    //
    // Causal (and windowed) at D = DV = 128, the steps run in pairs, so that each
    // step's slot parity is a constant and the slot offsets fold into the LDS
    // reads' immediate offsets (16 address additions fewer per matrix phase). At
    // D = 64 the doubled loop body measured slower, and the non-causal D = 128
    // kernel, whose exact body is larger, runs out of registers with it; there the
    // parity stays a run-time value.
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    using AnyParity = std::integral_constant<int, -1>;
    constexpr bool kPaired = CAUSAL && D == 128 && DV == 128;
    if constexpr (kPaired) {
        auto run_steps = [&](auto step) {
            int s = jstart;
            if (s & 1) step(s++, Odd{});
            for (; s + 1 <= jend; s += 2) {
                step(s, Even{});
                step(s + 1, Odd{});
            }
            if (s <= jend) step(s, Even{});
        };
        if (grp == 0) {
            run_steps([&](int s, auto par) {
                refill(s);
                matrix_phase(s, par);
                __syncthreads();
                softmax_phase(s);
                wait_copies();
                __syncthreads();
            });
        } else {
            run_steps([&](int s, auto par) {
                refill(s);
                softmax_phase(s - 1);
                __syncthreads();
                matrix_phase(s, par);
                wait_copies();
                __syncthreads();
            });
        }
    } else if (grp == 0) {
        for (int s = jstart; s <= jend; ++s) {
            refill(s);
            matrix_phase(s, AnyParity{});
            __syncthreads();
            softmax_phase(s);
            wait_copies();
            __syncthreads();
        }
    } else {
        for (int s = jstart; s <= jend; ++s) {
            refill(s);
            softmax_phase(s - 1);
            __syncthreads();
            matrix_phase(s, AnyParity{});
            wait_copies();
            __syncthreads();
        }
    }

    const float lt = halves_sum(l);
    if (qrow < S) {
        const float inv = 1.0f / lt;
        uint16_t* op = a.o + (qrows + qrow) * DV;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = db * 32 + 8 * g4 + 4 * h;
                const bf16x4 pkd = pack4(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                                         oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
                *(bf16x4*)(op + d) = pkd;
            }
        if (h == 0) a.lse[((size_t)b * a.Hq + hq) * S + qrow] = (m + log2f(lt)) * 0.69314718055994531f;
    }
}

// One head, 256 query rows per workgroup. Query tiles 0 .. a.precise_tiles-1
// take the exact P V product.
template <int D, int DV, bool CAUSAL>
__global__ void __launch_bounds__(kFwdThreads, 1) fwd_kernel(FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
    const int nQ = (a.S + kFwdBQ - 1) / kFwdBQ;
    int b, hq, qt;
    decode_item(blockIdx.x, nQ, CAUSAL ? nQ - 1 : 0, a.B, a.Hkv, a.G, CAUSAL, b, hq, qt);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q0 = qt * kFwdBQ;
    // Rows interleave between the ping-pong groups (group 0: 0-31, 64-95, ...;
    // group 1: 32-63, 96-127, ...) so both see the same number of causal tiles.
    const int row0 = q0 + 64 * (wave & 3) + 32 * (wave >> 2);
    if (qt < a.precise_tiles)
        fwd_body<D, DV, CAUSAL, true>(a, smem, b, hq, q0, q0 + kFwdBQ - 1, row0);
    else
        fwd_body<D, DV, CAUSAL, false>(a, smem, b, hq, q0, q0 + kFwdBQ - 1, row0);
}

// Heads of one kv head that a sliding-window workgroup takes together.
__host__ __device__ inline int win_heads(int G) {
    return (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
}

// Sliding window: a band of W keys gives 256 rows of one head about twice the key
// tiles any one wave needs. Here the 8 waves take HW query heads of one kv head
// (HW = 8, 4, 2 or 1, a divisor of G) and 8/HW blocks of 32 rows, so a workgroup
// covers only 32*8/HW rows and every wave uses nearly all of its key tiles.
// Workgroups whose rows may see fewer than 128 keys (W < 128, or the first 256
// rows) take the exact P V product.
template <int D, int DV>
__global__ void __launch_bounds__(kFwdThreads, 1) fwd_win_kernel(FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
    const int HW = win_heads(a.G), BQ = 32 * (8 / HW);
    const int nQ = (a.S + BQ - 1) / BQ;
    const int groups = a.B * a.Hkv * (a.G / HW);   // (b, kv head, head block)
    int qt, gid;
    const int bid = blockIdx.x;
    if ((groups & 7) == 0) {  // a head block stays on one XCD (workgroups are dealt round-robin)
        const int x = bid & 7, st = bid >> 3, per = groups >> 3;
        qt = st / per;
        gid = (st - qt * per) * 8 + x;
    } else {
        qt = bid / groups;
        gid = bid - qt * groups;
    }
    const int nblk = a.G / HW;
    const int b = gid / (a.Hkv * nblk);
    const int rem = gid - b * (a.Hkv * nblk);
    const int hkv = rem / nblk, blk = rem - hkv * nblk;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hq = hkv * a.G + blk * HW + wave % HW;
    const int q0 = qt * BQ;
    const int row0 = q0 + 32 * (wave / HW);
    if (a.window < 128 || q0 < 256)
        fwd_body<D, DV, true, true>(a, smem, b, hq, q0, q0 + BQ - 1, row0);
    else
        fwd_body<D, DV, true, false>(a, smem, b, hq, q0, q0 + BQ - 1, row0);
}

// ---------------------------------------------------------------------------
// fwd1_kernel: queries, keys and values 128 wide, with the running-maximum slack
// on (max_slack >= 1) and S a multiple of 256. Four waves, one per SIMD, take
// the same 256 query rows per workgroup as fwd_kernel, each wave 64 of them in two
// 32-row blocks (rows q0 + 32 w + 128 r, r = 0, 1). Every K and V^T operand a
// wave reads from LDS then feeds two MFMAs, one per row block, which halves the
// LDS operand traffic per MFMA against 32 rows per wave; the 512 registers of a
// SIMD hold both blocks' scores, probabilities and O accumulators.
//
// With one wave per SIMD there is no partner wave whose MFMAs could cover the
// softmax, so the wave interleaves the two itself, a 32-key block at a time. Each
// step handles key tile j + 1's scores and tile j's P V product in two regions:
//   region 0: S^T of block 0 of tile j+1 and P V of block 0 of tile j, under the
//             softmax of block 1 of tile j;
//   region 1: S^T of block 1 of tile j+1 and P V of block 1 of tile j, under the
//             softmax of block 0 of tile j+1;
// a region's 16 score and 16 P V MFMAs (both row blocks) go out over 8 slots,
// each with its share of the exponentials and bf16 packing, and the step's tile
// copies go out one per slot of region 0.
//
// The loop never rescales O. Each row's reference maximum m is taken exactly
// from the first key tile, and the probabilities exp2(s c - m) of the later
// tiles are only summed. After the loop each lane's sum is checked against
// 2^(slack-1) times the number of 32-key blocks: it passes whenever every block
// would have passed fwd_body's per-tile test (each lane's sum of a block at most
// 2^(slack-1)), and passing bounds every probability by the lane's sum, so P
// stays exact in bf16 and l and O stay far from overflow. Where a sum fails (a
// score far above m, an overflow, a NaN) the wave raises a flag in LDS and the
// whole workgroup recomputes its rows in fwd1_careful, which moves the maximum as
// fwd_body does and splits P into a bf16 high part and remainder. Keeping the
// conditional rescale of all 128 O registers out of the loop is what keeps the
// loop free of register copies and spills. The first query tile of a causal
// problem (rows that see at most 256 keys) always takes fwd1_careful, as it takes
// fwd_body's exact instance in fwd_kernel.
//
// The build compiles this file with MFMA results in VGPRs (build.py): a kernel
// that may use 512 registers otherwise gets every accumulator in AGPRs, and the
// softmax would need an extra instruction to read each score out.
// ---------------------------------------------------------------------------
constexpr int kF1Waves = 4;
constexpr int kF1Threads = 64 * kF1Waves;
constexpr int kF1BK = 64;  // keys per LDS tile
constexpr int kF1Rows = 2; // 32-row blocks per wave

struct F1Tile {
    static constexpr int D = 128, DV = 128;
    static constexpr int KTILE = kF1BK * D;  // elements
    static constexpr int VTILE = kF1BK * DV;
    static constexpr int RING_BYTES = 2 * (KTILE + VTILE) * 2;  // 2 K slots + 2 V slots
    static constexpr int LDS_BYTES = RING_BYTES + 16;           // + the workgroup's flag word
    using KCopy = CopyPlan<D, kF1BK, kF1Waves>;
    using VCopy = CopyPlan<DV, kF1BK, kF1Waves>;
};

// Per-lane offsets shared by both bodies: copy source offsets (bytes within a
// tile) and LDS read offsets (elements within a slot), as in fwd_body.
struct F1Lane {
    static constexpr int D = F1Tile::D, DV = F1Tile::DV, DK = D / 16, DB = DV / 32;
    using KC = F1Tile::KCopy;
    using VC = F1Tile::VCopy;
    uint32_t kcoff[KC::N], vcoff[VC::N];
    int koff[DK], voff[2][DB];
    __device__ __forceinline__ F1Lane(int wave, int lane) {
        const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
        for (int n = 0; n < KC::N; ++n) {
            const int row = (wave * KC::N + n) * KC::ROWS_PER_COPY + lane / KC::CH;
            kcoff[n] = (uint32_t)(row * D + ((lane % KC::CH) ^ swz_f<D>(row)) * 8) * 2u;
        }
#pragma unroll
        for (int n = 0; n < VC::N; ++n) {
            const int row = (wave * VC::N + n) * VC::ROWS_PER_COPY + lane / VC::CH;
            vcoff[n] = (uint32_t)(row * DV + ((lane % VC::CH) ^ swz_f<DV>(row)) * 8) * 2u;
        }
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) koff[dk] = swz<D>(l32, dk * 16 + 8 * h);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                voff[hf][db] = swz<DV>(4 * h + ((lane & 15) >> 2) + 8 * hf,
                                       db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
    }
};

// Sets the scores of keys past this lane's query row to -inf (a bitwise select, so
// that a NaN score of a hidden key does not reach the row): element e of a 32-key
// block starting at key k0 holds key k0 + 8 (e / 4) + 4 h + e % 4.
__device__ __forceinline__ void f1_mask(f32x16& s, int k0, int qrow, int h) {
    const int lim = qrow - k0 - 4 * h;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int off = 8 * (e >> 2) + (e & 3);
        s[e] = hide_if((lim - off) >> 31, s[e]);  // all ones iff off > lim
    }
}

// Exact body: each wave takes its two row blocks one after the other, 32 rows at
// a time. Per key tile all waves copy K and V into slot 0 of the ring; then the
// scores, the row maximum moved as fwd_body moves it, the probabilities split
// into bf16 high parts and remainders, and the P V product on both.
template <bool CAUSAL, int NR>
__device__ __forceinline__ void fwd1_careful(const FwdArgs& a, __bf16* smem, int b, int hq, int q0) {
    using T = F1Tile;
    constexpr int D = T::D, DV = T::DV, BK = kF1BK, DK = D / 16, DB = DV / 32, NT = BK / 16;
    using KC = T::KCopy;
    using VC = T::VCopy;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int S = a.S;
    const size_t qrows = ((size_t)b * a.Hq + hq) * (size_t)S;
    const size_t kvrows = ((size_t)b * a.Hkv + hq / a.G) * (size_t)S;
    const uint16_t* Kp = a.k + kvrows * D;
    const uint16_t* Vp = a.v + kvrows * DV;
    const float c = a.scale_log2;
    const F1Lane ln(wave, lane);
    const __bf16* Ks = smem;
    const __bf16* Vs = smem + T::KTILE;
    const uint32_t kdst = lds_addr_of(smem) + wave * KC::N * 1024;
    const uint32_t vdst = lds_addr_of(smem + T::KTILE) + wave * VC::N * 1024;
    for (int r = 0; r < NR; ++r) {
        const int row0 = q0 + 128 * r + 32 * wave;
        const int qrow = row0 + l32;
        bf16x8 qf[DK];
        const u32x4* src = (const u32x4*)(a.q + (qrows + qrow) * D + 8 * h);
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            u32x4 t = src[2 * dk];
            t ^= a.q_sign;
            qf[dk] = __builtin_bit_cast(bf16x8, t);
        }
        // tiles the workgroup's rows of this pass see, and this wave's rows
        const int jend = CAUSAL ? (q0 + 128 * r + 127) / BK + 1 : S / BK;
        const int wjend = CAUSAL ? (row0 + 31) / BK + 1 : jend;
        f32x16 oacc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = zero16();
        float m = -1e30f, l = 0.0f;
        for (int j = 0; j < jend; ++j) {
            barrier_lds();  // every wave is done with the previous tile
            const uint16_t* kb = Kp + (size_t)j * BK * D;
            const uint16_t* vb = Vp + (size_t)j * BK * DV;
#pragma unroll
            for (int n = 0; n < KC::N; ++n) copy16_to_lds_sa(kb, ln.kcoff[n], kdst + n * 1024);
#pragma unroll
            for (int n = 0; n < VC::N; ++n) copy16_to_lds_sa(vb, ln.vcoff[n], vdst + n * 1024);
            wait_copies();
            barrier_lds();
            if (j >= wjend) continue;  // past this wave's diagonal (wave-uniform)
            f32x16 sc[2] = {zero16(), zero16()};
#pragma unroll
            for (int dk = 0; dk < DK; ++dk)
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
                    sc[kb2] = mfma32(lds_read8(Ks + ln.koff[dk] + kb2 * 32 * D), qf[dk], sc[kb2]);
            if (CAUSAL && j == wjend - 1) {
                f1_mask(sc[0], j * BK, qrow, h);
                f1_mask(sc[1], j * BK + 32, qrow, h);
            }
            float mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
            for (int e = 1; e < 16; ++e) mx = fmaxf(mx, fmaxf(sc[0][e], sc[1][e]));
            const float mt = halves_max(mx) * c;
            if (__any(mt > m + a.max_slack)) {
                const float mnew = fmaxf(m, mt);
                const float alpha = fast_exp2(m - mnew);
                m = mnew;
                l *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
            }
            bf16x8 pk[NT], pl[NT];
            float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = fast_exp2(fmaf(sc[t >> 1][8 * (t & 1) + e], c, -m));
                    rs[e & 3] += p[e];
                }
                pk[t] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
                pl[t] = pack8(bf_lo(p[0]), bf_lo(p[1]), bf_lo(p[2]), bf_lo(p[3]), bf_lo(p[4]), bf_lo(p[5]),
                              bf_lo(p[6]), bf_lo(p[7]));
            }
            l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const bf16x8 vt = concat(lds_read_tr(Vs + ln.voff[0][db] + 16 * t * DV),
                                             lds_read_tr(Vs + ln.voff[1][db] + 16 * t * DV));
                    oacc[db] = mfma32(vt, pk[t], oacc[db]);
                    oacc[db] = mfma32(vt, pl[t], oacc[db]);
                }
        }
        const float lt = halves_sum(l);
        const float inv = 1.0f / lt;
        uint16_t* op = a.o + (qrows + qrow) * DV;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = db * 32 + 8 * g4 + 4 * h;
                *(bf16x4*)(op + d) = pack4(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                                           oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
            }
        if (h == 0) a.lse[qrows + qrow] = (m + log2f(lt)) * 0.69314718055994531f;
    }
}

// Pipelined body; returns false (workgroup-uniform, nothing written) when some
// wave's probabilities left the bound, true once O and lse are written.
template <bool CAUSAL, int NR>
__device__ __forceinline__ bool fwd1_fast(const FwdArgs& a, __bf16* smem, int b, int hq, int q0) {
    using T = F1Tile;
    constexpr int D = T::D, DV = T::DV, BK = kF1BK;
    constexpr int DK = D / 16;    // k-steps of a block's S^T
    constexpr int DB = DV / 32;   // 32-column blocks of O^T
    constexpr int NT = BK / 16;   // 16-key P V steps of a tile
    constexpr int NPV = 2 * DB;   // P V MFMAs of a key block per row block
    constexpr int NSL = DK > NPV ? DK : NPV;  // slots of a region
    constexpr int EPS = 16 / NSL; // softmax elements per row block per slot
    using KC = T::KCopy;
    using VC = T::VCopy;
    constexpr int NCP = KC::N + VC::N;  // copies per wave per step
    static_assert(16 % NSL == 0 && EPS % 2 == 0 && NCP <= NSL, "region slots");
    static_assert(DK == NSL && NPV == NSL, "every slot has one k-step and one P V step");
    const int S = a.S;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const size_t qrows = ((size_t)b * a.Hq + hq) * (size_t)S;
    const size_t kvrows = ((size_t)b * a.Hkv + hq / a.G) * (size_t)S;
    const uint16_t* Kp = a.k + kvrows * D;
    const uint16_t* Vp = a.v + kvrows * DV;
    const int qrow0 = q0 + 32 * wave + l32;  // row of block r: qrow0 + 128 r
    const float c = a.scale_log2;
    int* const flag = (int*)((char*)smem + T::RING_BYTES);

    bf16x8 qf[NR][DK];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const u32x4* src = (const u32x4*)(a.q + (qrows + qrow0 + 128 * r) * D + 8 * h);
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            u32x4 t = src[2 * dk];
            t ^= a.q_sign;
            qf[r][dk] = __builtin_bit_cast(bf16x8, t);
        }
    }
    // Tiles of the workgroup; a causal one masks tiles from q0 / BK on (its
    // first row's tile; earlier tiles are visible to all of its rows).
    const int nK = CAUSAL ? q0 / BK + 128 * NR / BK : S / BK;
    __bf16* const Kring = smem;
    __bf16* const Vring = smem + 2 * T::KTILE;
    const uint32_t kbase = lds_addr_of(Kring) + wave * KC::N * 1024;
    const uint32_t vbase = lds_addr_of(Vring) + wave * VC::N * 1024;
    const F1Lane ln(wave, lane);
    // copy k of the step's NCP: K_jk into K slot ks, V_jv into V slot vs
    auto copy_one = [&](int k, int ks, int jk, int vs, int jv) {
        if (k < KC::N)
            copy16_to_lds_sa(Kp + (size_t)jk * BK * D, ln.kcoff[k], kbase + (uint32_t)(ks * T::KTILE * 2 + k * 1024));
        else
            copy16_to_lds_sa(Vp + (size_t)jv * BK * DV, ln.vcoff[k - KC::N],
                             vbase + (uint32_t)(vs * T::VTILE * 2 + (k - KC::N) * 1024));
    };

    f32x16 oacc[NR][DB];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[r][db] = zero16();
    // m: each row's reference maximum; l4: four partial sums of this lane's share
    // of its probabilities, carried through the loop
    float m[NR], l4[NR][4];

    // Sb[r][kb]: scores of key block kb of the current tile for row block r;
    // Pb[r][t]: the bf16 probabilities of its 16-key step t.
    f32x16 Sb[NR][2];
    bf16x8 Pb[NR][NT];
    auto qk_op = [&](const __bf16* Ks, int kb, int dk) { return lds_read8(Ks + ln.koff[dk] + kb * 32 * D); };
    auto pv_op = [&](const __bf16* Vs, int t, int db) {
        return concat(lds_read_tr(Vs + ln.voff[0][db] + 16 * t * DV), lds_read_tr(Vs + ln.voff[1][db] + 16 * t * DV));
    };
    // One region: the DK k-steps of S^T of key block kb of the tile in Ks (when
    // WITH_QK) and the NPV P V MFMAs of key block pb (V tile in Vs), both row
    // blocks, one k-step or P V step per slot, with the softmax of key block sb
    // (of tile jt, masked when MASK) spread over the slots and copies k0 .. of the
    // step issued one per slot.
    auto region = [&](auto with_qk, auto mask, const __bf16* Ks, int kb, const __bf16* Vs, int pb, int sb, int jt,
                      auto&& copy, int k0) __attribute__((always_inline)) {
        constexpr bool WITH_QK = decltype(with_qk)::value;
        constexpr bool MASK = decltype(mask)::value;
        if (MASK) {
#pragma unroll
            for (int r = 0; r < NR; ++r) f1_mask(Sb[r][sb], jt * BK + 32 * sb, qrow0 + 128 * r, h);
        }
        float pe[NR][16];
        uint32_t pw[NR][8];
        bf16x8 kr[DK], vr[NPV];
        if (WITH_QK) {
#pragma unroll
            for (int r = 0; r < NR; ++r) Sb[r][kb] = zero16();
            kr[0] = qk_op(Ks, kb, 0);
        }
        vr[0] = pv_op(Vs, 2 * pb, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NSL; ++i) {
            if (WITH_QK && i + 1 < DK) kr[i + 1] = qk_op(Ks, kb, i + 1);
            if (i + 1 < NPV) vr[i + 1] = pv_op(Vs, 2 * pb + (i + 1) / DB, (i + 1) % DB);
            copy(k0 + i);
            // the P V product first: its operand was read after the K operand, so
            // the one wait for it covers both
            if (i < NPV) {
#pragma unroll
                for (int r = 0; r < NR; ++r)
                    oacc[r][i % DB] = mfma32(vr[i], Pb[r][2 * pb + i / DB], oacc[r][i % DB]);
            }
            if (WITH_QK && i < DK) {
#pragma unroll
                for (int r = 0; r < NR; ++r) Sb[r][kb] = mfma32(kr[i], qf[r][i], Sb[r][kb]);
            }
#pragma unroll
            for (int r = 0; r < NR; ++r) {
#pragma unroll
                for (int u = 0; u < EPS; ++u) {
                    const int e = EPS * i + u;
                    pe[r][e] = fast_exp2(fmaf(Sb[r][sb][e], c, -m[r]));
                    l4[r][e & 3] += pe[r][e];
                    asm volatile("" ::"v"(pe[r][e]), "v"(l4[r][e & 3]));
                }
#pragma unroll
                for (int u = 0; u < EPS; u += 2) {
                    const int e = EPS * i + u;
                    pw[r][e >> 1] = pack2_bf16(pe[r][e], pe[r][e + 1]);
                    asm volatile("" ::"v"(pw[r][e >> 1]));
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int t2 = 0; t2 < 2; ++t2)
                Pb[r][2 * sb + t2] = __builtin_bit_cast(
                    bf16x8, u32x4{pw[r][4 * t2], pw[r][4 * t2 + 1], pw[r][4 * t2 + 2], pw[r][4 * t2 + 3]});
    };
    auto no_copy = [&](int) {};
    using False = std::integral_constant<bool, false>;
    using True = std::integral_constant<bool, true>;

    // prologue: K_0, K_1 and V_0; tile 0's scores; m from its 64 keys; block 0's
    // probabilities
    if (tid == 0) *flag = 0;
#pragma unroll
    for (int k = 0; k < NCP; ++k) copy_one(k, 0, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < KC::N; ++k) copy_one(k, 1, 1, 0, 0);
    wait_copies();
    barrier_lds();
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        Sb[r][0] = zero16();
        Sb[r][1] = zero16();
    }
#pragma unroll
    for (int dk = 0; dk < DK; ++dk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 kf = qk_op(Kring, kb, dk);
#pragma unroll
            for (int r = 0; r < NR; ++r) Sb[r][kb] = mfma32(kf, qf[r][dk], Sb[r][kb]);
        }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        float mx = fmaxf(Sb[r][0][0], Sb[r][1][0]);
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, fmaxf(Sb[r][0][e], Sb[r][1][e]));
        m[r] = halves_max(mx) * c;
#pragma unroll
        for (int e = 0; e < 4; ++e) l4[r][e] = 0.0f;
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p[e] = fast_exp2(fmaf(Sb[r][0][8 * t2 + e], c, -m[r]));
                l4[r][e & 3] += p[e];
            }
            Pb[r][t2] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        }
    }
    barrier_lds();  // every wave is done with K slot 0 before K_2 goes there

    // Step j (0 <= j <= nK-2): copies of K_{j+2} (past the end the last tile
    // again, into a slot no later step reads) and V_{j+1} into the slots of K_j and
    // V_{j-1}; tile j's P V and block-1 softmax, tile j+1's scores and block-0
    // softmax. The slot parity is a template constant.
    auto step = [&](int j, auto par, auto mask) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value;  // j & 1
        const int jk = min(j + 2, nK - 1), jv = j + 1;
        auto copy = [&](int k) {
            if (k < NCP) copy_one(k, P, jk, P ^ 1, jv);
        };
        const __bf16* Ks = Kring + (P ^ 1) * T::KTILE;
        const __bf16* Vs = Vring + P * T::VTILE;
        region(True{}, mask, Ks, 0, Vs, 0, 1, j, copy, 0);
        region(True{}, mask, Ks, 1, Vs, 1, 0, j + 1, copy, NSL);
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        barrier_lds();
    };
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    // Unmasked steps 0 .. jm-1; a causal workgroup's last four steps (from
    // q0 / BK - 1, an odd step, on) handle its diagonal tiles and mask.
    const int jm = CAUSAL ? q0 / BK - 1 : nK - 1;
    int j = 0;
    for (; j + 2 <= jm; j += 2) {
        step(j, Even{}, False{});
        step(j + 1, Odd{}, False{});
    }
    if (j < jm) step(j++, Even{}, False{});
    if constexpr (CAUSAL) {
#pragma unroll
        for (int t = 0; t < NR; ++t, j += 2) {
            step(j, Odd{}, True{});
            step(j + 1, Even{}, True{});
        }
    }
    // tail: tile nK-1's P V and its block-1 softmax
    {
        const __bf16* Vs = Vring + ((nK - 1) & 1) * T::VTILE;
        region(False{}, std::integral_constant<bool, CAUSAL>{}, Kring, 0, Vs, 0, 1, nK - 1, no_copy, 0);
#pragma unroll
        for (int i = 0; i < NPV; ++i) {
            const bf16x8 vt = pv_op(Vs, 2 + i / DB, i % DB);
#pragma unroll
            for (int r = 0; r < NR; ++r) oacc[r][i % DB] = mfma32(vt, Pb[r][2 + i / DB], oacc[r][i % DB]);
        }
    }
    // Every probability is at most its lane's sum. The sum of 2 nK blocks passes
    // whenever each block's sum is at most 2^(slack-1), the bound fwd_body tests
    // per tile, and passing caps every probability at 2^(slack-1) * 2 nK: P stays
    // exact in bf16 and O and l far from overflow.
    float l[NR];
    bool bad = false;
    const float bound = exp2f(a.max_slack - 1.0f) * (float)(2 * nK);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        l[r] = (l4[r][0] + l4[r][1]) + (l4[r][2] + l4[r][3]);
        bad |= !(l[r] <= bound);  // also a NaN or an infinity
    }
    if (__any(bad) && lane == 0) *(volatile int*)flag = 1;
    barrier_lds();
    if (*(volatile int*)flag) return false;

#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int qrow = qrow0 + 128 * r;
        const float lt = halves_sum(l[r]);
        const float inv = 1.0f / lt;
        uint16_t* op = a.o + (qrows + qrow) * DV;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = db * 32 + 8 * g4 + 4 * h;
                *(bf16x4*)(op + d) = pack4(oacc[r][db][4 * g4] * inv, oacc[r][db][4 * g4 + 1] * inv,
                                           oacc[r][db][4 * g4 + 2] * inv, oacc[r][db][4 * g4 + 3] * inv);
            }
        if (h == 0) a.lse[qrows + qrow] = (m[r] + log2f(lt)) * 0.69314718055994531f;
    }
    return true;
}

// NR row blocks per wave: 2 (one wave per SIMD, 256 rows per workgroup) or 1 (two
// workgroups of 128 rows per CU, two waves per SIMD).
template <bool CAUSAL, int NR>
__global__ void __launch_bounds__(kF1Threads, 3 - NR) __attribute__((amdgpu_waves_per_eu(3 - NR, 3 - NR)))
fwd1_kernel(FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) __bf16 smem[];
    constexpr int BQ = 128 * NR;
    const int nQ = a.S / BQ;
    int b, hq, qt;
    decode_item(blockIdx.x, nQ, CAUSAL ? nQ - 1 : 0, a.B, a.Hkv, a.G, CAUSAL, b, hq, qt);
    const int q0 = qt * BQ;
    // rows below precise_tiles * 256 (the first 256 rows of a causal problem) take the exact body
    if (q0 >= a.precise_tiles * kFwdBQ && fwd1_fast<CAUSAL, NR>(a, smem, b, hq, q0)) return;
    fwd1_careful<CAUSAL, NR>(a, smem, b, hq, q0);
}

template <int D, int DV, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& args, hipStream_t stream) {
    // Rows that see at most 128 keys take the exact P V product: tile 0 of a
    // causal problem (rows 0..255 see at most 256 keys; the first 128 of them, the
    // ones that need it, are there) or the single tile of S <= 128. Windowed
    // problems go to fwd_win_kernel, which makes that choice per workgroup.
    const int nQ = (args.S + kFwdBQ - 1) / kFwdBQ;
    FwdArgs a = args;
    constexpr int lds = fwd_lds_bytes<D, DV>();
    if (CAUSAL && a.window > 0) {
        const int HW = win_heads(a.G), BQ = 32 * (8 / HW);
        const long long wblocks = (long long)((a.S + BQ - 1) / BQ) * a.B * a.Hkv * (a.G / HW);
        hipLaunchKernelGGL((fwd_win_kernel<D, DV>), dim3((unsigned)wblocks), dim3(kFwdThreads), lds, stream, a);
        return hipGetLastError();
    }
    a.precise_tiles = (CAUSAL || a.S <= 128) ? 1 : 0;
    // 128-wide heads with the slack on and whole 256-row tiles: fwd1_kernel (its
    // own exact body covers the first causal tile). Otherwise fwd_kernel.
    if constexpr (D == 128 && DV == 128) {
        if (a.max_slack >= 1.0f && a.S % kFwdBQ == 0 && a.S > 128) {
            constexpr int NR = kF1Rows;
            hipLaunchKernelGGL((fwd1_kernel<CAUSAL, NR>), dim3((unsigned)((long long)a.B * a.Hq * (a.S / (128 * NR)))),
                               dim3(kF1Threads), F1Tile::LDS_BYTES, stream, a);
            return hipGetLastError();
        }
    }
    const long long blocks = (long long)a.B * a.Hq * nQ;
    hipLaunchKernelGGL((fwd_kernel<D, DV, CAUSAL>), dim3((unsigned)blocks), dim3(kFwdThreads), lds, stream, a);
    return hipGetLastError();
}

template <typename K>
hipError_t set_lds(K kernel, int bytes) {
    return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int D, int DV>
hipError_t setup_pair() {
    hipError_t e = set_lds(fwd_kernel<D, DV, false>, fwd_lds_bytes<D, DV>());
    if (!e) e = set_lds(fwd_kernel<D, DV, true>, fwd_lds_bytes<D, DV>());
    if (!e && D == 128 && DV == 128) e = set_lds(fwd1_kernel<false, kF1Rows>, F1Tile::LDS_BYTES);
    if (!e && D == 128 && DV == 128) e = set_lds(fwd1_kernel<true, kF1Rows>, F1Tile::LDS_BYTES);
    return e ? e : set_lds(fwd_win_kernel<D, DV>, fwd_lds_bytes<D, DV>());
}

template <int D, int DV>
hipError_t launch_pair(const FwdArgs& a, hipStream_t stream) {
    return a.causal ? launch_fwd_t<D, DV, true>(a, stream) : launch_fwd_t<D, DV, false>(a, stream);
}

}  // namespace

// Raise the dynamic-LDS limit of every forward instance on the current device.
hipError_t fwd_setup_device() {
    hipError_t e;
    if ((e = setup_pair<64, 64>())) return e;
    if ((e = setup_pair<128, 128>())) return e;
    if ((e = setup_pair<64, 128>())) return e;
    return setup_pair<128, 64>();
}

hipError_t launch_fwd(const FwdArgs& a, int D, int DV, hipStream_t stream) {
    if (D == 64) return DV == 64 ? launch_pair<64, 64>(a, stream) : launch_pair<64, 128>(a, stream);
    return DV == 128 ? launch_pair<128, 128>(a, stream) : launch_pair<128, 64>(a, stream);
}

}  // namespace attn
