// Internal interface between the C ABI (attn_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int B, Hq, Hkv, S, G;
    int causal;
    int window;          // causal only: > 0 limits query i to keys i-window+1 .. i; 0 = no limit
    float scale_log2;    // max(|scale| * log2(e), 2^-100)
    uint32_t q_sign;     // 0x80008000 when scale < 0 (Q is negated on load), else 0
    float max_slack;     // log2 growth of a row maximum tolerated before rescaling O
    int precise_tiles;   // query tiles 0 .. precise_tiles-1 take the exact (split-P) path
};

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const float* lse;
    const uint16_t* dout;
    float* dq;
    float* dk;
    float* dv;
    float* rowstat;      // workspace: [B][Hq][ceil(S/32)][64]: per block of 32 query rows, the
                         // rows' lse_i * log2(e), then their -delta_i (delta_i = sum_j P_ij
                         // dP_ij); rows past S hold +inf and -0, so that whole blocks can be
                         // copied
    int* peak;           // workspace: [B][Hq][ceil(S/32)], 1 where a row of the 32-row block has
                         // a probability above kPeakP (written by the dQ stage)
    int B, Hq, Hkv, S, G;
    int causal;
    int window;          // as in FwdArgs
    float scale;         // signed scale
    float scale_log2;    // scale * log2(e) (signed)
    int precise_all;     // split P/dS operands on every tile, whatever the data
};

// A row whose largest probability exceeds this takes the backward's exact path: its
// P and dS operands are split into a bf16 high part and a bf16 remainder. Below it,
// the bf16 rounding of P and dS (at most 2^-9 of each) kept dQ, dK and dV within
// 0.56 of the 1e-2 bar in a CPU emulation of that arithmetic: all heads of two kv
// groups of the causal Llama-3.1-8B shape (S = 4096, D = 128), the same with a
// 128-key window, and every peaked input of the backward tests. A threshold of 1/2
// missed the bar there (4.6e-2); 1/8 put 81 % of the 128-key window's 32-row
// blocks on the exact path, against 8 % at 1/4.
constexpr float kPeakP = 0.25f;

// Sparse attention over per-token index lists (attn_sparse_* entry points).
struct SparseArgs {
    const uint16_t* q;       // [B][Hq][S][D]
    const uint16_t* k;       // [B][Hkv][N][D]
    const uint16_t* v;       // [B][Hkv][N][D]
    const int32_t* idx;      // [B][S][topk]; entries outside [0, N) are empty slots
    const uint16_t* o;       // backward: the forward's output
    const uint16_t* dout;    // backward: [B][Hq][S][D]
    uint16_t* out;           // forward output [B][Hq][S][D]
    float* lse;              // [B][Hq][S] (written by the forward, read by the backward)
    float* dq;               // [B][Hq][S][D]
    float* dk;               // [B][Hkv][N][D]
    float* dv;
    // backward workspace
    float* delta;            // [B][Hq][S]
    float* inter_k;          // [B][Hkv][S][topk][D]: scale * dS^T Q per (token, slot)
    float* inter_v;          // [B][Hkv][S][topk][D]: P^T dO per (token, slot)
    int* cnt;                // [B][nchunks][N]: per-chunk row counts, then chunk bases
    int* rowstart;           // [B][N+1]: start of each row's entries in `list`
    int* list;               // [B][S*topk]: entries i*topk + s grouped by row, token order
    int B, Hq, Hkv, S, N, G, topk, nchunks;
    float scale;             // signed scale (backward)
    float scale_log2;        // forward: max(|scale| * log2(e), 2^-100); backward: scale * log2(e)
    uint32_t q_sign;         // forward: 0x80008000 when scale < 0, else 0
    int precise_all;         // every workgroup takes the exact (split P / dS) path
    float max_slack;         // forward: log2 growth of a row maximum tolerated before rescaling O
};

// Each launcher enqueues its kernels on `stream` and returns hipGetLastError().
// D: query/key head dimension, DV: value head dimension (each 64 or 128).
hipError_t launch_fwd(const FwdArgs& a, int D, int DV, hipStream_t stream);
// stages: bit 0 = dQ and delta, bit 1 = dK/dV (in that order when both are set)
hipError_t launch_bwd(const BwdArgs& a, int D, int DV, int stages, hipStream_t stream);
// D: head dimension (64 or 128); G = Hq / Hkv <= 128.
hipError_t launch_sparse_fwd(const SparseArgs& a, int D, hipStream_t stream);
hipError_t launch_sparse_bwd(const SparseArgs& a, int D, hipStream_t stream);

}  // namespace attn
