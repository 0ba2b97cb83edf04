// Sparse attention over per-token index lists, for gfx950 (MI355X).
//
// The compressed sparse attention of Rao et al., "Scheduling Data to Compute:
// Hierarchical Data Pipelining for LLM Training on AMD GPUs" (section 2.1;
// Table 7 for its shapes), gives every query token a top-k list of key/value
// rows: a sliding window of recent tokens plus rows of a compressed pool. The
// forward gathers the listed rows, scores them and streams their values into the
// output accumulator (Eq. (1) over the listed rows). The backward gathers the
// same rows to form dQ, produces one dK/dV contribution per (token, list slot),
// and reduces those contributions by the inverse of the index map. The kernels
// here follow that data flow:
//
//   sparse_fwd_kernel     one workgroup per (b, token, kv head, block of 64 query
//                         heads). The token's list is compacted into LDS (empty
//                         slots dropped, order kept); 32-row K/V tiles are
//                         gathered from HBM straight into double-buffered,
//                         swizzled LDS tiles by per-lane global_load_lds
//                         addresses (MI355X has no gather engine, so each lane
//                         names its own row); S^T = K Q^T, online softmax and
//                         O^T += V^T P^T as in the dense forward.
//   sparse_dq_kernel      the same gather; dP^T = V dO^T, dS = P (dP - delta),
//                         dQ^T += K^T dS^T; writes delta for the next stage.
//   sparse_kv_partial     one workgroup per (b, token, kv head, 128 list slots):
//                         the token's query heads are the rows of one Q and one
//                         dO tile in LDS, each lane owns one slot; it writes
//                         scale dS^T Q and P^T dO for every non-empty slot.
//   sp_count, sp_scan_chunks, sp_scan_rows, sp_offset_chunks, sp_scatter
//                         the inverse of the index map: for every key/value row,
//                         the (token, slot) entries that name it, in token order
//                         (deterministic: counts are order-free, and positions
//                         are handed out chunk by chunk, token by token).
//   sp_reduce             dK, dV of every row: the sum of its entries'
//                         contributions in that order, in a fixed association.
//
// The sum over a token's query heads happens inside the partial kernel's MFMAs
// (the heads are their contraction index), so the per-slot contribution is one
// D-vector per kv head. In the forward and dQ kernels, rows that see few keys (at
// most 256 non-empty slots) take the exact path of the dense kernels: P and dS
// split into a bf16 high part and a bf16 remainder, and delta recomputed as
// sum_s P dP. The per-slot contributions always take the split P and dS.
#include "device.h"
#include "kernels.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSpBK = 32;            // list slots per gathered K/V tile (dQ)
constexpr int kSpFwdBK = 32;         // list slots per gathered K/V tile (forward)
constexpr int kSpRows = 64;          // query heads per forward / dQ workgroup
constexpr int kSpThreads = 128;      // 2 waves x 32 heads
constexpr int kSpPreciseSlots = 256; // tokens with at most this many keys take the exact path
constexpr int kSpSlotsPerWG = 128;   // partial kernel: list slots per workgroup (4 waves x 32)
constexpr int kSpPartThreads = 256;
constexpr int kSpMaxG = 128;         // query heads per kv head
constexpr int kSpChunk = 16;         // tokens per inverse-map chunk
constexpr int kSpXcdTokens = 64;     // tokens per XCD chunk (forward, dQ, partial)
constexpr int kSpLdsRows = 16384;    // inverse map: per-chunk row counters in LDS up to this N

__device__ __forceinline__ bool slot_valid(int j, int N) { return j >= 0 && j < N; }

// Work item of workgroup `bid` among `total` items ordered (b, token, kv head,
// block), `per` items per token. Workgroup bid runs on XCD bid % 8. Tokens go to
// the XCDs in chunks of kSpXcdTokens, so neighbouring tokens (whose windows
// overlap) share one L2, dealt round robin from the last chunk down: every XCD
// gets the same mix of short and long lists (later tokens list more pool rows),
// and the longest start first. When the items do not split into whole rounds of
// chunks, each XCD takes a contiguous range (total divisible by 8), else launch
// order.
__device__ __forceinline__ int xcd_item(int bid, int total, int per) {
    const long long chunk = (long long)kSpXcdTokens * per;  // 64-bit: per can be large
    const int x = bid & 7, r = bid >> 3;
    if (total % (8 * chunk) == 0) {  // then 8 * chunk <= total < 2^31
        const long long rounds = total / (8 * chunk);
        return (int)(((rounds - 1 - r / chunk) * 8 + x) * chunk + r % chunk);
    }
    if ((total & 7) == 0) return x * (total >> 3) + r;
    return bid;
}

// Compact the token's list into LDS: the non-empty entries in slot order.
// Returns their number (the same in every lane). 128 threads; red: 16 LDS ints.
// Entries are read eight 128-entry rounds at a time, all loads in flight together;
// each round's two wave counts go to LDS, and one barrier per batch publishes them.
__device__ __forceinline__ int compact_list(const int32_t* src, int topk, int N, int* out, int* red) {
    constexpr int R = 8;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int total = 0;
    for (int base = 0; base < topk; base += R * kSpThreads) {
        int j[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int s = base + r * kSpThreads + tid;
            j[r] = s < topk ? src[s] : -1;
        }
        unsigned long long m[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            m[r] = __ballot(slot_valid(j[r], N));
            if (lane == 0) red[2 * r + wave] = __popcll(m[r]);
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int c0 = red[2 * r], c1 = red[2 * r + 1];
            if (slot_valid(j[r], N)) out[total + (wave ? c0 : 0) + __popcll(m[r] & ((1ull << lane) - 1ull))] = j[r];
            total += c0 + c1;
        }
        __syncthreads();
    }
    return total;
}

template <int D, int BK = kSpBK>
struct SpTile {
    static constexpr int TILE = BK * D;                        // elements
    static constexpr int KV_BYTES = 4 * TILE * 2;             // 2 K slots + 2 V slots
    using Copy = CopyPlan<D, BK, 2>;
    static int lds_bytes(int topk) { return KV_BYTES + ((topk * 4 + 15) & ~15) + 64; }
};

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
// Work item of a forward / dQ workgroup: (b, token i, kv head, block hb of 64
// query heads).
struct SpItem {
    int b, i, hkv, hb;
};
__device__ __forceinline__ SpItem sp_item(const SparseArgs& a) {
    const int nHB = (a.G + kSpRows - 1) / kSpRows;
    int w = xcd_item(blockIdx.x, a.B * a.S * a.Hkv * nHB, a.Hkv * nHB);
    SpItem it;
    it.hb = w % nHB; w /= nHB;
    it.hkv = w % a.Hkv; w /= a.Hkv;
    it.i = w % a.S;
    it.b = w / a.S;
    return it;
}

// The body after the list is compacted into LDS (n entries). PRECISE is the exact
// path, chosen once per workgroup, so the loop is straight-line code either way.
template <int D, bool PRECISE>
__device__ __forceinline__ void sparse_fwd_body(const SparseArgs& a, unsigned char* lds_raw, const SpItem& it,
                                                const int* list, int n) {
    constexpr int BK = kSpFwdBK;   // list slots per tile
    constexpr int NB = BK / 32;    // 32-slot blocks per tile
    using T = SpTile<D, BK>;
    using C = typename T::Copy;
    constexpr int DK = D / 16;
    constexpr int DB = D / 32;
    __bf16* const Kring = (__bf16*)lds_raw;
    __bf16* const Vring = Kring + 2 * T::TILE;
    const int b = it.b, i = it.i, hkv = it.hkv;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int head = it.hb * kSpRows + 32 * wave + l32;
    const bool live = head < a.G;
    const int hq = hkv * a.G + head;
    const size_t row = ((size_t)b * a.Hq + hq) * a.S + i;   // flat query row (when live)
    const float c = a.scale_log2;

    bf16x8 qf[DK];
    if (live) {
        const u32x4* src = (const u32x4*)(a.q + row * D + 8 * h);
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

    const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)a.N * D;
    const uint16_t* Kp = a.k + kvbase;
    const uint16_t* Vp = a.v + kvbase;
    // Gathered copies: copy m of this wave fills tile rows (wave*N + m) * ROWS_PER_COPY
    // + lane / CH with the row its compacted slot names; slots past the end repeat
    // the last one (their scores are masked, their probabilities exactly 0).
    int crow[C::N], ccol[C::N];
#pragma unroll
    for (int m = 0; m < C::N; ++m) {
        crow[m] = (wave * C::N + m) * C::ROWS_PER_COPY + lane / C::CH;
        ccol[m] = (((lane % C::CH) ^ swz_f<D>(crow[m]))) * 8;
    }
    auto copy_tile = [&](int slot, int t) {
#pragma unroll
        for (int m = 0; m < C::N; ++m) {
            const int j = list[min(t * BK + crow[m], n - 1)];
            const uint32_t off = (uint32_t)j * D + ccol[m];
            copy16_to_lds(Kp + off, Kring + slot * T::TILE + (wave * C::N + m) * 512);
            copy16_to_lds(Vp + off, Vring + slot * T::TILE + (wave * C::N + m) * 512);
        }
    };
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
    float m = -1e30f, l = 0.0f;
    const bool fast_max = a.max_slack >= 1.0f;
    const float max_bound = exp2f(a.max_slack - 1.0f);

    const int nT = (n + BK - 1) / BK;
    if (nT > 0) {
        copy_tile(0, 0);
        wait_copies();
        __syncthreads();
    }
    for (int t = 0; t < nT; ++t) {
        if (t + 1 < nT) copy_tile((t + 1) & 1, t + 1);
        const __bf16* Ks = Kring + (t & 1) * T::TILE;
        const __bf16* Vs = Vring + (t & 1) * T::TILE;
        f32x16 sc[NB];
#pragma unroll
        for (int kb = 0; kb < NB; ++kb) sc[kb] = zero16();
#pragma unroll
        for (int dk = 0; dk < DK; ++dk)
#pragma unroll
            for (int kb = 0; kb < NB; ++kb) sc[kb] = mfma32(lds_read8(Ks + koff[dk] + kb * 32 * D), qf[dk], sc[kb]);
        if (t == nT - 1) {  // slot t*BK + 4h + off exists iff off < lim
            const int lim = n - t * BK - 4 * h;
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) sc[kb][r] = -INFINITY;
        }
        bf16x8 pk[2 * NB], pl[2 * NB];
        auto probs = [&]() {  // exp2(s c - m) as bf16 operands; this lane's sum
            float rs = 0.0f;
#pragma unroll
            for (int t2 = 0; t2 < 2 * NB; ++t2) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = fast_exp2(fmaf(sc[t2 >> 1][8 * (t2 & 1) + e], c, -m));
                    rs += p[e];
                }
                pk[t2] = pack8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
                if (PRECISE)
                    pl[t2] = pack8(bf_lo(p[0]), bf_lo(p[1]), bf_lo(p[2]), bf_lo(p[3]), bf_lo(p[4]),
                                   bf_lo(p[5]), bf_lo(p[6]), bf_lo(p[7]));
            }
            return rs;
        };
        // As in the dense forward, past the first tile the maximum is taken only
        // when some lane's probabilities against the current m sum past
        // 2^(slack-1); below that the rule that follows would leave m alone, so
        // the result is the same.
        bool need_max = PRECISE || !fast_max || t == 0;
        float tot = 0.0f;
        if (!need_max) {
            tot = probs();
            need_max = __any(!(tot <= max_bound));
        }
        if (need_max) {
            float mx = fmaxf(sc[0][0], sc[0][1]);
#pragma unroll
            for (int kb = 0; kb < NB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
            const float mt = halves_max(mx) * c;  // c > 0
            // As in the dense forward, the running maximum only moves when some
            // row's grows by more than max_slack (log2 units): until then every
            // probability is at most 2^slack, exact enough in fp32 and bf16, and O
            // is not rescaled.
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
        // O^T += V^T P^T over 16-slot steps; V^T through transpose loads.
#pragma unroll
        for (int t2 = 0; t2 < 2 * NB; ++t2)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 vt = concat(lds_read_tr(Vs + voff[0][db] + 16 * t2 * D),
                                         lds_read_tr(Vs + voff[1][db] + 16 * t2 * D));
                oacc[db] = mfma32(vt, pk[t2], oacc[db]);
                if (PRECISE) oacc[db] = mfma32(vt, pl[t2], oacc[db]);
            }
        wait_copies();
        __syncthreads();
    }

    const float lt = halves_sum(l);
    if (live) {
        uint16_t* op = a.out + row * D;
        const float inv = n > 0 ? 1.0f / lt : 0.0f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d = db * 32 + 8 * g4 + 4 * h;
                *(bf16x4*)(op + d) = pack4(oacc[db][4 * g4] * inv, oacc[db][4 * g4 + 1] * inv,
                                           oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv);
            }
        if (h == 0) a.lse[row] = n > 0 ? (m + log2f(lt)) * 0.69314718055994531f : -INFINITY;
    }
}

template <int D>
__global__ void __launch_bounds__(kSpThreads, 2) sparse_fwd_kernel(SparseArgs a) {
    using T = SpTile<D, kSpFwdBK>;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    int* const list = (int*)(lds_raw + T::KV_BYTES);
    int* const red = list + ((a.topk + 3) & ~3);
    const SpItem it = sp_item(a);
    const int n = compact_list(a.idx + ((size_t)it.b * a.S + it.i) * a.topk, a.topk, a.N, list, red);
    if (a.precise_all || n <= kSpPreciseSlots)
        sparse_fwd_body<D, true>(a, lds_raw, it, list, n);
    else
        sparse_fwd_body<D, false>(a, lds_raw, it, list, n);
}

// ---------------------------------------------------------------------------
// dQ (+ delta)
// ---------------------------------------------------------------------------
// The plain body (PRECISE false) makes one pass with delta from the stored O and
// bf16 dS operands; in the same pass it accumulates the exact delta = sum_s P dP,
// which it stores for the contribution kernel, and looks for a probability above
// kPeakP in any of the workgroup's rows. It returns whether it found one: then dQ is
// not stored and the caller runs the PRECISE body with that delta (have_delta),
// which makes the pass again with split dS operands. Called without have_delta the
// PRECISE body first makes a pass that only accumulates the exact delta.
template <int D, bool PRECISE>
__device__ __forceinline__ bool sparse_dq_body(const SparseArgs& a, unsigned char* lds_raw, const SpItem& it,
                                               const int* list, int n, bool have_delta, float& delta_io) {
    using T = SpTile<D>;
    using C = typename T::Copy;
    constexpr int DK = D / 16;
    constexpr int DB = D / 32;
    __bf16* const Kring = (__bf16*)lds_raw;
    __bf16* const Vring = Kring + 2 * T::TILE;
    const int b = it.b, i = it.i, hkv = it.hkv;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int head = it.hb * kSpRows + 32 * wave + l32;
    const bool live = head < a.G;
    const int hq = hkv * a.G + head;
    const size_t row = ((size_t)b * a.Hq + hq) * a.S + i;
    const float c = a.scale_log2;  // signed

    // Q and dO rows as B operands; delta = rowsum(dO * O) from the stored O.
    bf16x8 qf[DK], df[DK];
    float dpart = 0.0f;
    if (live) {
        const u32x4* qs = (const u32x4*)(a.q + row * D + 8 * h);
        const u32x4* ds = (const u32x4*)(a.dout + row * D + 8 * h);
        const u32x4* os = (const u32x4*)(a.o + row * D + 8 * h);
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            qf[dk] = __builtin_bit_cast(bf16x8, qs[2 * dk]);
            df[dk] = __builtin_bit_cast(bf16x8, ds[2 * dk]);
            const bf16x8 ov = __builtin_bit_cast(bf16x8, os[2 * dk]);
#pragma unroll
            for (int e = 0; e < 8; ++e) dpart += (float)df[dk][e] * (float)ov[e];
        }
    } else {
#pragma unroll
        for (int dk = 0; dk < DK; ++dk) {
            qf[dk] = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0});
            df[dk] = qf[dk];
        }
    }
    float delta = PRECISE && have_delta ? delta_io : halves_sum(dpart);
    const float lse2 = (live && n > 0) ? a.lse[row] * kLog2e : INFINITY;

    const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)a.N * D;
    const uint16_t* Kp = a.k + kvbase;
    const uint16_t* Vp = a.v + kvbase;
    int crow[C::N], ccol[C::N];
#pragma unroll
    for (int m = 0; m < C::N; ++m) {
        crow[m] = (wave * C::N + m) * C::ROWS_PER_COPY + lane / C::CH;
        ccol[m] = (((lane % C::CH) ^ swz_f<D>(crow[m]))) * 8;
    }
    auto copy_tile = [&](int slot, int t) {
#pragma unroll
        for (int m = 0; m < C::N; ++m) {
            const int j = list[min(t * kSpBK + crow[m], n - 1)];
            const uint32_t off = (uint32_t)j * D + ccol[m];
            copy16_to_lds(Kp + off, Kring + slot * T::TILE + (wave * C::N + m) * 512);
            copy16_to_lds(Vp + off, Vring + slot * T::TILE + (wave * C::N + m) * 512);
        }
    };
    int roff[DK], toff[2][DB];
#pragma unroll
    for (int dk = 0; dk < DK; ++dk) roff[dk] = swz<D>(l32, dk * 16 + 8 * h);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < DB; ++db)
            toff[hf][db] = swz<D>(4 * h + ((lane & 15) >> 2) + 8 * hf,
                                  db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    f32x16 dq[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dq[db] = zero16();

    // Pass 0 (exact body without a given delta) accumulates delta = sum_s P dP; the
    // last pass forms dS and accumulates dQ^T += K^T dS^T.
    const int nT = (n + kSpBK - 1) / kSpBK;
    float dacc = 0.0f;
    bool peaked = false;  // plain body: a probability above kPeakP (a wave-wide ballot)
    for (int pass = PRECISE && !have_delta ? 0 : 1; pass < 2; ++pass) {
        dacc = 0.0f;
        if (nT > 0) {
            copy_tile(0, 0);
            wait_copies();
            __syncthreads();
        }
        for (int t = 0; t < nT; ++t) {
            if (t + 1 < nT) copy_tile((t + 1) & 1, t + 1);
            const __bf16* Ks = Kring + (t & 1) * T::TILE;
            const __bf16* Vs = Vring + (t & 1) * T::TILE;
            f32x16 s = zero16(), dp = zero16();
#pragma unroll
            for (int dk = 0; dk < DK; ++dk) {
                s = mfma32(lds_read8(Ks + roff[dk]), qf[dk], s);
                dp = mfma32(lds_read8(Vs + roff[dk]), df[dk], dp);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], c, -lse2));
            if (t == nT - 1) {
                const int lim = n - t * kSpBK - 4 * h;
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = (8 * (r >> 2) + (r & 3) >= lim) ? 0.0f : s[r];
            }
            if (PRECISE) {
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
            if (pass == 1) {
#pragma unroll
                for (int t2 = 0; t2 < 2; ++t2) {
                    const int r0 = 8 * t2;
                    const bf16x8 hi = pack8(s[r0], s[r0 + 1], s[r0 + 2], s[r0 + 3], s[r0 + 4], s[r0 + 5],
                                            s[r0 + 6], s[r0 + 7]);
                    bf16x8 lo;
                    if (PRECISE)
                        lo = pack8(bf_lo(s[r0]), bf_lo(s[r0 + 1]), bf_lo(s[r0 + 2]), bf_lo(s[r0 + 3]),
                                   bf_lo(s[r0 + 4]), bf_lo(s[r0 + 5]), bf_lo(s[r0 + 6]), bf_lo(s[r0 + 7]));
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const bf16x8 kt = concat(lds_read_tr(Ks + toff[0][db] + 16 * t2 * D),
                                                 lds_read_tr(Ks + toff[1][db] + 16 * t2 * D));
                        dq[db] = mfma32(kt, hi, dq[db]);
                        if (PRECISE) dq[db] = mfma32(kt, lo, dq[db]);
                    }
                }
            }
            wait_copies();
            __syncthreads();
        }
        if (pass == 0) delta = halves_sum(dacc);
    }

    bool redo = false;
    if (!PRECISE) {
        // a workgroup vote in the K/V ring, idle once every wave is past its last
        // tile (the barrier; with no tiles the ring was never used)
        delta = halves_sum(dacc);
        int* vote = (int*)lds_raw;
        __syncthreads();
        if (lane == 0) vote[wave] = peaked ? 1 : 0;
        __syncthreads();
        redo = __builtin_amdgcn_readfirstlane((vote[0] | vote[1]) ? 1 : 0) != 0;
        __syncthreads();  // the exact pass refills the ring
        delta_io = delta;
    }

    if (live) {
        if (h == 0) a.delta[row] = delta;
        if (redo) return true;  // dQ is stored by the exact pass
        float* dst = a.dq + row * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = dq[db][4 * g4 + e] * a.scale;
                *(f32x4*)(dst + db * 32 + 8 * g4 + 4 * h) = v;
            }
    }
    return redo;
}

template <int D>
__global__ void __launch_bounds__(kSpThreads, 2) sparse_dq_kernel(SparseArgs a) {
    using T = SpTile<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    int* const list = (int*)(lds_raw + T::KV_BYTES);
    int* const red = list + ((a.topk + 3) & ~3);
    const SpItem it = sp_item(a);
    const int n = compact_list(a.idx + ((size_t)it.b * a.S + it.i) * a.topk, a.topk, a.N, list, red);
    // Tokens with at most kSpPreciseSlots keys (or all, on request) take the exact
    // body from the start; the others when their pass finds a probability above
    // kPeakP.
    float delta = 0.0f;
    bool exact = a.precise_all || n <= kSpPreciseSlots, have_delta = false;
    if (!exact) {
        exact = sparse_dq_body<D, false>(a, lds_raw, it, list, n, false, delta);
        have_delta = true;
    }
    if (exact) sparse_dq_body<D, true>(a, lds_raw, it, list, n, have_delta, delta);
}

// ---------------------------------------------------------------------------
// per-(token, slot) dK / dV contributions
// ---------------------------------------------------------------------------
template <int D>
struct PartTile {
    // Q and dO tiles [Gp][D] of the token's query heads and the V rows of the
    // workgroup's 128 slots [128][D], all in swz<D> order; lse*log2e and delta
    // per head.
    __host__ __device__ static int tile_bytes(int Gp) { return (2 * Gp * D + kSpSlotsPerWG * D) * 2; }
    __host__ __device__ static int lds_bytes(int Gp) { return tile_bytes(Gp) + 2 * Gp * 4; }
};

// One of the two products of this wave's 32 slots, summed over every head of the
// token, as a [slot][d] accumulator (lane = column d, registers = slots
// 8(r/4) + 4h + r%4):
//   DK = false:  dV = P^T dO
//   DK = true:   dK = dS^T Q   (without the scale)
// Each pass recomputes S (and dP for dK) for the token's heads in groups of 32:
// two accumulators do not fit in the registers of two waves per SIMD, one does.
// P^T / dS^T are the A operands straight from the score registers (lane = slot,
// heads as contraction index in the order the score layout gives); dO / Q are
// the B operands, read with transpose loads in that same head order.
template <int D, bool PRECISE, bool DK>
__device__ __forceinline__ void part_product(const __bf16* Qt, const __bf16* Dt, const __bf16* Vt,
                                             const float* Ls, const float* Dl, const bf16x8 (&kf)[D / 16],
                                             bool valid, int wave, int lane, int Gp, float c,
                                             f32x16 (&acc)[D / 32]) {
    constexpr int NK = D / 16;
    constexpr int DB = D / 32;
    const int h = lane >> 5, l32 = lane & 31;
    int roff[NK], toff[2][DB];
#pragma unroll
    for (int d = 0; d < NK; ++d) roff[d] = swz<D>(l32, d * 16 + 8 * h);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < DB; ++db)
            toff[hf][db] = swz<D>(4 * h + ((lane & 15) >> 2) + 8 * hf,
                                  db * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = zero16();
    const __bf16* Bt = DK ? Qt : Dt;   // B operand tile of the product
    for (int hs = 0; hs < Gp / 32; ++hs) {
        // rows of s / dp are heads 32 hs + 8(r/4) + 4h + r%4; the column is this lane's slot
        f32x16 s = zero16(), dp = zero16();
#pragma unroll
        for (int dd = 0; dd < NK; ++dd) {
            s = mfma32(lds_read8(Qt + hs * 32 * D + roff[dd]), kf[dd], s);
            if (DK) dp = mfma32(lds_read8(Dt + hs * 32 * D + roff[dd]), lds_read8(Vt + wave * 32 * D + roff[dd]), dp);
        }
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
            float x[8];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int rg = 2 * t2 + half;
                const f32x4 l4 = *(const f32x4*)(Ls + hs * 32 + 8 * rg + 4 * h);
                f32x4 d4;
                if (DK) d4 = *(const f32x4*)(Dl + hs * 32 + 8 * rg + 4 * h);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = valid ? fast_exp2(fmaf(s[4 * rg + e], c, -l4[e])) : 0.0f;
                    x[4 * half + e] = DK ? p * (dp[4 * rg + e] - d4[e]) : p;
                }
            }
            const bf16x8 xh = pack8(x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]);
            bf16x8 xl;
            if (PRECISE)
                xl = pack8(bf_lo(x[0]), bf_lo(x[1]), bf_lo(x[2]), bf_lo(x[3]), bf_lo(x[4]), bf_lo(x[5]),
                           bf_lo(x[6]), bf_lo(x[7]));
            const int rb = (hs * 32 + 16 * t2) * D;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const bf16x8 bt = concat(lds_read_tr(Bt + toff[0][db] + rb), lds_read_tr(Bt + toff[1][db] + rb));
                acc[db] = mfma32(xh, bt, acc[db]);
                if (PRECISE) acc[db] = mfma32(xl, bt, acc[db]);
            }
        }
    }
}

// Store a [slot][d] accumulator (lane = column) times `mul` into rows
// dst[slot][0..D) for slots < nslots: each store writes two 128-byte row pieces.
// The contributions are read once, by the reduction, long after: the stores are
// non-temporal, so they stream to memory instead of filling the L2.
template <int D>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[D / 32], float mul, float* dst, int nslots,
                                           int lane) {
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int slot = 8 * (r >> 2) + 4 * h + (r & 3);
        if (slot < nslots) {
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                __builtin_nontemporal_store(acc[db][r] * mul, dst + (size_t)slot * D + db * 32 + l32);
        }
    }
}

// Every contribution takes the split (bf16 high part + remainder) P and dS: one
// contribution sums up to 128 query heads, and rounding P to bf16 there alone moves
// dV by up to 1e-2 at the 128-head cr4 shape. The products are cheap next to the
// stores of this kernel.
template <int D>
__device__ __forceinline__ void part_both(const __bf16* Qt, const __bf16* Dt, const __bf16* Vt, const float* Ls,
                                          const float* Dl, const bf16x8 (&kf)[D / 16], bool valid, int wave,
                                          int lane, int Gp, const SparseArgs& a, size_t e0, int nslots) {
    f32x16 acc[D / 32];
    part_product<D, true, false>(Qt, Dt, Vt, Ls, Dl, kf, valid, wave, lane, Gp, a.scale_log2, acc);
    store_rows<D>(acc, 1.0f, a.inter_v + e0 * D, nslots, lane);
    part_product<D, true, true>(Qt, Dt, Vt, Ls, Dl, kf, valid, wave, lane, Gp, a.scale_log2, acc);
    store_rows<D>(acc, a.scale, a.inter_k + e0 * D, nslots, lane);
}

template <int D>
__global__ void __launch_bounds__(kSpPartThreads, 2) sparse_kv_partial_kernel(SparseArgs a) {
    constexpr int NK = D / 16;
    constexpr int CH = D / 8, RPC = 64 / CH;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const int G = a.G, Gp = (G + 31) & ~31;
    __bf16* const Qt = (__bf16*)lds_raw;
    __bf16* const Dt = Qt + Gp * D;
    __bf16* const Vt = Dt + Gp * D;
    float* const Ls = (float*)(lds_raw + PartTile<D>::tile_bytes(Gp));
    float* const Dl = Ls + Gp;

    const int nSB = (a.topk + kSpSlotsPerWG - 1) / kSpSlotsPerWG;
    int w = xcd_item(blockIdx.x, a.B * a.S * a.Hkv * nSB, a.Hkv * nSB);
    const int sb = w % nSB; w /= nSB;
    const int hkv = w % a.Hkv; w /= a.Hkv;
    const int i = w % a.S;
    const int b = w / a.S;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int32_t* lst = a.idx + ((size_t)b * a.S + i) * a.topk;
    const int slot0 = sb * kSpSlotsPerWG + 32 * wave;        // this wave's first list slot
    const int slot = slot0 + l32;                            // this lane's list slot
    const int jraw = slot < a.topk ? lst[slot] : -1;
    const bool valid = slot_valid(jraw, a.N);
    const int j = valid ? jraw : 0;
    // A block of empty slots (the unused tail of a short list) has nothing to write:
    // the whole workgroup leaves before loading anything.
    if (!__syncthreads_or(valid)) return;

    // Q / dO rows of the token's heads (rows past G repeat head G-1; their lse is
    // +inf, so they add exactly 0), and the V rows of this workgroup's slots.
    const size_t qrow0 = ((size_t)b * a.Hq + hkv * G) * a.S + i;   // head g at qrow0 + g*S
    for (int cpy = wave; cpy < Gp / RPC; cpy += 4) {
        const int r = cpy * RPC + lane / CH;
        const int col = (((lane % CH) ^ swz_f<D>(r))) * 8;
        const size_t src = (qrow0 + (size_t)min(r, G - 1) * a.S) * D + col;
        copy16_to_lds(a.q + src, Qt + cpy * 512);
        copy16_to_lds(a.dout + src, Dt + cpy * 512);
    }
    const size_t kvbase = ((size_t)b * a.Hkv + hkv) * (size_t)a.N * D;
    for (int cpy = wave; cpy < kSpSlotsPerWG / RPC; cpy += 4) {
        const int r = cpy * RPC + lane / CH;
        const int col = (((lane % CH) ^ swz_f<D>(r))) * 8;
        const int s2 = sb * kSpSlotsPerWG + r;
        const int jr = s2 < a.topk ? lst[s2] : -1;
        copy16_to_lds(a.v + kvbase + (size_t)(slot_valid(jr, a.N) ? jr : 0) * D + col, Vt + cpy * 512);
    }
    for (int g = tid; g < Gp; g += kSpPartThreads) {
        const size_t r = qrow0 + (size_t)g * a.S;
        Ls[g] = g < G ? a.lse[r] * kLog2e : INFINITY;
        Dl[g] = g < G ? a.delta[r] : 0.0f;
    }
    // this lane's K row as B operands
    bf16x8 kf[NK];
    {
        const u32x4* ks = (const u32x4*)(a.k + kvbase + (size_t)j * D + 8 * h);
#pragma unroll
        for (int d = 0; d < NK; ++d) kf[d] = __builtin_bit_cast(bf16x8, ks[2 * d]);
    }
    wait_copies();
    __syncthreads();
    if (__ballot(valid) == 0) return;  // no non-empty slot in this wave (no barrier follows)

    const int nslots = min(32, a.topk - slot0);  // rows of this wave inside the token's list
    const size_t e0 = (((size_t)b * a.Hkv + hkv) * a.S + i) * a.topk + slot0;
    part_both<D>(Qt, Dt, Vt, Ls, Dl, kf, valid, wave, lane, Gp, a, e0, nslots);
}

// ---------------------------------------------------------------------------
// inverse of the index map
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) sp_fill_zero(int* p, size_t n) {
    for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (size_t)gridDim.x * 256) p[x] = 0;
}

// cnt[b][c][j] = number of entries of chunk c (tokens 16c .. 16c+15) naming row j.
// Counts do not depend on order, so the workgroup walks the chunk's lists as one
// contiguous range, eight loads in flight per thread. With LDS_ROWS the chunk's N
// counters live in LDS (N <= kSpLdsRows): a window row is named by up to 16 tokens
// of a chunk, and LDS atomics take that contention far faster than the L2's; the
// counters, zeros included, then go out in one coalesced pass. Otherwise the
// atomics go to the zero-filled global counters.
template <bool LDS_ROWS>
__global__ void __launch_bounds__(256) sp_count(SparseArgs a) {
    constexpr int U = 8;
    extern __shared__ int lds_cnt[];
    const int b = blockIdx.x / a.nchunks, ch = blockIdx.x % a.nchunks;
    int* cnt = a.cnt + ((size_t)b * a.nchunks + ch) * a.N;
    int* ctr = LDS_ROWS ? lds_cnt : cnt;
    if (LDS_ROWS) {
        for (int j = threadIdx.x; j < a.N; j += 256) lds_cnt[j] = 0;
        __syncthreads();
    }
    const int i0 = ch * kSpChunk, i1 = min(a.S, i0 + kSpChunk);
    const int32_t* lst = a.idx + ((size_t)b * a.S + i0) * a.topk;
    const int n = (i1 - i0) * a.topk;
    for (int base = 0; base < n; base += 256 * U) {
        int j[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = base + u * 256 + (int)threadIdx.x;
            j[u] = e < n ? lst[e] : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (slot_valid(j[u], a.N)) atomicAdd(ctr + j[u], 1);
    }
    if (LDS_ROWS) {
        __syncthreads();
        for (int j = threadIdx.x; j < a.N; j += 256) cnt[j] = lds_cnt[j];
    }
}

// Per row j: chunk counts -> exclusive chunk bases (in place); row totals.
__global__ void __launch_bounds__(256) sp_scan_chunks(SparseArgs a) {
    const size_t x = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= (size_t)a.B * a.N) return;
    const int b = (int)(x / a.N), j = (int)(x % a.N);
    int* col = a.cnt + (size_t)b * a.nchunks * a.N + j;   // chunk ch at col[ch * N]
    int run = 0;
    int ch = 0;
    for (; ch + 16 <= a.nchunks; ch += 16) {  // sixteen loads in flight, then the running sum
        int v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = col[(size_t)(ch + u) * a.N];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            col[(size_t)(ch + u) * a.N] = run;
            run += v[u];
        }
    }
    for (; ch < a.nchunks; ++ch) {
        const int v = col[(size_t)ch * a.N];
        col[(size_t)ch * a.N] = run;
        run += v;
    }
    a.rowstart[(size_t)b * (a.N + 1) + j] = run;
}

// rowstart[b][0..N] = exclusive prefix sum of the row totals (one workgroup per b).
__global__ void __launch_bounds__(1024) sp_scan_rows(SparseArgs a) {
    __shared__ int buf[1024];
    int* rs = a.rowstart + (size_t)blockIdx.x * (a.N + 1);
    int base = 0;
    for (int j0 = 0; j0 < a.N; j0 += 1024) {
        const int j = j0 + threadIdx.x;
        const int v = j < a.N ? rs[j] : 0;
        buf[threadIdx.x] = v;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
            const int add = threadIdx.x >= off ? buf[threadIdx.x - off] : 0;
            __syncthreads();
            buf[threadIdx.x] += add;
            __syncthreads();
        }
        if (j < a.N) rs[j] = base + buf[threadIdx.x] - v;
        base += buf[1023];
        __syncthreads();
    }
    if (threadIdx.x == 0) rs[a.N] = base;
}

// cnt[b][c][j] += rowstart[b][j]: each chunk's base for row j becomes the place,
// in the entry list, of that chunk's first entry naming j.
__global__ void __launch_bounds__(256) sp_offset_chunks(SparseArgs a) {
    const size_t per_b = (size_t)a.nchunks * a.N, n = (size_t)a.B * per_b;
    for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (size_t)gridDim.x * 256) {
        const int b = (int)(x / per_b), j = (int)(x % a.N);
        a.cnt[x] += a.rowstart[(size_t)b * (a.N + 1) + j];
    }
}

// list[b][rowstart[j] + k] = the k-th entry (i*topk + s, in token order) naming
// row j. A workgroup walks its chunk's tokens in order; a returning atomic on the
// chunk's place for row j gives each entry its place (in LDS with LDS_ROWS, as in
// sp_count). Slot s of a token is thread s % 256's entry s / 256 (PER = entries
// per thread, a power of two covering topk); the next token's entries load while
// this token's atomics run.
template <int PER, bool LDS_ROWS>
__global__ void __launch_bounds__(256) sp_scatter(SparseArgs a) {
    extern __shared__ int lds_cur[];
    const int b = blockIdx.x / a.nchunks, ch = blockIdx.x % a.nchunks;
    int* cur = a.cnt + ((size_t)b * a.nchunks + ch) * a.N;
    if (LDS_ROWS) {
        for (int j = threadIdx.x; j < a.N; j += 256) lds_cur[j] = cur[j];
        __syncthreads();
        cur = lds_cur;
    }
    int* out = a.list + (size_t)b * a.S * a.topk;
    const int i0 = ch * kSpChunk, i1 = min(a.S, i0 + kSpChunk);
    auto load = [&](int i, int (&j)[PER]) {
        const int32_t* lst = a.idx + ((size_t)b * a.S + i) * a.topk;
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int s = u * 256 + (int)threadIdx.x;
            j[u] = s < a.topk ? lst[s] : -1;
        }
    };
    int jc[PER], jn[PER];
    load(i0, jc);
    for (int i = i0; i < i1; ++i) {
        if (i + 1 < i1) load(i + 1, jn);
#pragma unroll
        for (int u = 0; u < PER; ++u)
            if (slot_valid(jc[u], a.N)) out[atomicAdd(cur + jc[u], 1)] = i * a.topk + u * 256 + (int)threadIdx.x;
        __syncthreads();  // token i's places are taken before token i+1's
#pragma unroll
        for (int u = 0; u < PER; ++u) jc[u] = jn[u];
    }
}

// dK, dV of row (b, hkv, j): the sum of its entries' contributions in list order.
// The row's entries are split into four contiguous quarters, one per wave; a wave
// reads 64 entry numbers at once (one per lane) and then walks them eight at a
// time, the entry number broadcast from a scalar register, so sixteen row loads
// are in flight; each contribution is read once, so the loads are non-temporal.
// The four partial sums are added in wave order. Lane l holds columns 2l, 2l+1.
template <int D>
__global__ void __launch_bounds__(256) sp_reduce(SparseArgs a) {
    typedef float fv __attribute__((ext_vector_type(2)));
    constexpr int PER = 2;
    __shared__ fv part[2][4][64];
    const int j = blockIdx.x % a.N;
    const int bh = blockIdx.x / a.N;   // b * Hkv + hkv
    const int b = bh / a.Hkv;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool on = lane < D / PER;  // D = 64 uses 32 lanes of each wave
    const int* rs = a.rowstart + (size_t)b * (a.N + 1);
    const int* ent = a.list + (size_t)b * a.S * a.topk;
    const int e0 = rs[j], e1 = rs[j + 1];
    const int quarter = (e1 - e0 + 3) / 4;
    const int w0 = min(e1, e0 + wave * quarter), w1 = min(e1, w0 + quarter);
    const float* ik = a.inter_k + (size_t)bh * a.S * a.topk * D + (on ? lane * PER : 0);
    const float* iv = a.inter_v + (size_t)bh * a.S * a.topk * D + (on ? lane * PER : 0);
    fv sk = {}, sv = {};
    for (int base = w0; base < w1; base += 64) {
        const int cntb = min(64, w1 - base);
        const int mine = lane < cntb ? ent[base + lane] : 0;
        int u = 0;
        for (; u + 8 <= cntb; u += 8) {
            fv k8[8], v8[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const size_t x = (size_t)__builtin_amdgcn_readlane(mine, u + t) * D;
                k8[t] = __builtin_nontemporal_load((const fv*)(ik + x));
                v8[t] = __builtin_nontemporal_load((const fv*)(iv + x));
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                sk += k8[t];
                sv += v8[t];
            }
        }
        for (; u < cntb; ++u) {
            const size_t x = (size_t)__builtin_amdgcn_readlane(mine, u) * D;
            sk += __builtin_nontemporal_load((const fv*)(ik + x));
            sv += __builtin_nontemporal_load((const fv*)(iv + x));
        }
    }
    part[0][wave][lane] = sk;
    part[1][wave][lane] = sv;
    __syncthreads();
    if (wave < 2 && on) {
        fv r = part[wave][0][lane];
        r += part[wave][1][lane];
        r += part[wave][2][lane];
        r += part[wave][3][lane];
        float* dst = (wave == 0 ? a.dk : a.dv) + ((size_t)bh * a.N + j) * D + lane * PER;
        *(fv*)dst = r;
    }
}

template <typename K>
hipError_t set_lds(K kernel, int bytes) {
    return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

template <int D>
hipError_t launch_fwd_t(const SparseArgs& a, hipStream_t stream) {
    const int nHB = (a.G + kSpRows - 1) / kSpRows;
    const long long blocks = (long long)a.B * a.S * a.Hkv * nHB;
    const int lds = SpTile<D, kSpFwdBK>::lds_bytes(a.topk);
    hipLaunchKernelGGL((sparse_fwd_kernel<D>), dim3((unsigned)blocks), dim3(kSpThreads), lds, stream, a);
    return hipGetLastError();
}

template <bool LDS_ROWS>
void launch_scatter(const SparseArgs& a, dim3 grid, int lds, hipStream_t stream) {
    if (a.topk <= 256)
        hipLaunchKernelGGL((sp_scatter<1, LDS_ROWS>), grid, dim3(256), lds, stream, a);
    else if (a.topk <= 512)
        hipLaunchKernelGGL((sp_scatter<2, LDS_ROWS>), grid, dim3(256), lds, stream, a);
    else if (a.topk <= 1024)
        hipLaunchKernelGGL((sp_scatter<4, LDS_ROWS>), grid, dim3(256), lds, stream, a);
    else if (a.topk <= 2048)
        hipLaunchKernelGGL((sp_scatter<8, LDS_ROWS>), grid, dim3(256), lds, stream, a);
    else
        hipLaunchKernelGGL((sp_scatter<16, LDS_ROWS>), grid, dim3(256), lds, stream, a);
}

template <int D>
hipError_t launch_bwd_t(const SparseArgs& a, hipStream_t stream) {
    hipError_t e;
    const size_t ncnt = (size_t)a.B * a.nchunks * a.N;
    const bool lds_rows = a.N <= kSpLdsRows;
    if (!lds_rows)
        hipLaunchKernelGGL(sp_fill_zero, dim3((unsigned)min((size_t)4096, (ncnt + 255) / 256)), dim3(256), 0, stream,
                           a.cnt, ncnt);
    const int nHB = (a.G + kSpRows - 1) / kSpRows;
    const long long qblocks = (long long)a.B * a.S * a.Hkv * nHB;
    const int qlds = SpTile<D>::lds_bytes(a.topk);
    hipLaunchKernelGGL((sparse_dq_kernel<D>), dim3((unsigned)qblocks), dim3(kSpThreads), qlds, stream, a);
    const int nSB = (a.topk + kSpSlotsPerWG - 1) / kSpSlotsPerWG;
    const long long pblocks = (long long)a.B * a.S * a.Hkv * nSB;
    const int plds = PartTile<D>::lds_bytes((a.G + 31) & ~31);
    hipLaunchKernelGGL((sparse_kv_partial_kernel<D>), dim3((unsigned)pblocks), dim3(kSpPartThreads), plds, stream,
                       a);
    const dim3 cgrid((unsigned)(a.B * a.nchunks));
    const int rows_lds = lds_rows ? a.N * 4 : 0;
    if (lds_rows)
        hipLaunchKernelGGL(sp_count<true>, cgrid, dim3(256), rows_lds, stream, a);
    else
        hipLaunchKernelGGL(sp_count<false>, cgrid, dim3(256), 0, stream, a);
    hipLaunchKernelGGL(sp_scan_chunks, dim3((unsigned)(((size_t)a.B * a.N + 255) / 256)), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(sp_scan_rows, dim3((unsigned)a.B), dim3(1024), 0, stream, a);
    hipLaunchKernelGGL(sp_offset_chunks, dim3((unsigned)min((size_t)65536, (ncnt + 255) / 256)), dim3(256), 0,
                       stream, a);
    if (lds_rows)
        launch_scatter<true>(a, cgrid, rows_lds, stream);
    else
        launch_scatter<false>(a, cgrid, 0, stream);
    hipLaunchKernelGGL((sp_reduce<D>), dim3((unsigned)((size_t)a.B * a.Hkv * a.N)), dim3(256), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return hipSuccess;
}

}  // namespace

int sparse_tokens_per_chunk() { return kSpChunk; }
int sparse_max_heads_per_kv() { return kSpMaxG; }

// Raise the dynamic-LDS limit of every sparse instance on the current device.
hipError_t sparse_setup_device() {
    hipError_t e;
    if ((e = set_lds(sparse_fwd_kernel<64>, 65536))) return e;
    if ((e = set_lds(sparse_fwd_kernel<128>, 65536))) return e;
    if ((e = set_lds(sparse_dq_kernel<64>, 65536))) return e;
    if ((e = set_lds(sparse_dq_kernel<128>, 65536))) return e;
    if ((e = set_lds(sparse_kv_partial_kernel<64>, PartTile<64>::lds_bytes(kSpMaxG)))) return e;
    return set_lds(sparse_kv_partial_kernel<128>, PartTile<128>::lds_bytes(kSpMaxG));
}

hipError_t launch_sparse_fwd(const SparseArgs& a, int D, hipStream_t stream) {
    return D == 64 ? launch_fwd_t<64>(a, stream) : launch_fwd_t<128>(a, stream);
}

hipError_t launch_sparse_bwd(const SparseArgs& a, int D, hipStream_t stream) {
    return D == 64 ? launch_bwd_t<64>(a, stream) : launch_bwd_t<128>(a, stream);
}

}  // namespace attn
