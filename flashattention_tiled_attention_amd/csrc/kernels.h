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
    float* delta;        // workspace: [B][Hq][S]
    int B, Hq, Hkv, S, G;
    int causal;
    int window;          // as in FwdArgs
    float scale;         // signed scale
    float scale_log2;    // scale * log2(e) (signed)
    int precise_all;     // exact delta and split P/dS operands on every tile
    int precise_tiles;   // dQ query tiles 0 .. precise_tiles-1 take that exact path (set by launch_bwd)
};

// Each launcher enqueues its kernels on `stream` and returns hipGetLastError().
// D: query/key head dimension, DV: value head dimension (each 64 or 128).
hipError_t launch_fwd(const FwdArgs& a, int D, int DV, hipStream_t stream);
// stages: bit 0 = dQ and delta, bit 1 = dK/dV (in that order when both are set)
hipError_t launch_bwd(const BwdArgs& a, int D, int DV, int stages, hipStream_t stream);

}  // namespace attn
