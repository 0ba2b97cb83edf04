/*
 * attn.h - C ABI of the MI355X (gfx950) fused attention library.
 *
 * The operation is scaled dot-product attention as stated in Rao et al.,
 * "Scheduling Data to Compute: Hierarchical Data Pipelining for LLM Training on
 * AMD GPUs", section 2.1, Eq. (1): O = softmax(Q K^T * scale) V, computed the
 * way that section's Algorithm 0 describes: K/V blocks stream through on-chip
 * memory while the online-softmax state (running max m, running sum l) and the
 * output accumulator stay on chip. The backward pass is the exact gradient of
 * Eq. (1), recomputing P from the saved log-sum-exp; its products are the ones
 * the same section's Table 3 lists (dQ = dS K, dK = dS^T Q) plus dV = P^T dO.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer on the current HIP device, in
 *    contiguous [B][H][S][D] layout (row-major; D fastest), 16-byte aligned.
 *    q, o, dout, dq: H = Hq.  k, v, dk, dv: H = Hkv.  lse: [B][Hq][S].
 *  - bf16 tensors are passed as raw 16-bit storage (const void*).
 *  - Grouped-query attention: query head hq reads key/value head hq / (Hq/Hkv)
 *    (consecutive query heads share a key/value head). Hq % Hkv must be 0.
 *  - causal != 0: query row i sees key rows j <= i (query and key lengths are
 *    both S). causal == 0: every row sees all S keys.
 *  - scale: any finite float; the usual value is 1/sqrt(D).
 *  - D must be 64 or 128. S, B, Hq, Hkv >= 1, B*Hq*S*D < 2^40 and S*D < 2^31
 *    (the kernels address rows within one head with 32-bit offsets), and every
 *    launch must fit a grid of fewer than 2^32 work-items (ATTN_ERR_SHAPE).
 *  - stream: a hipStream_t passed as void*; NULL means the null stream. The
 *    header uses void* so that C callers and foreign-function bindings need no
 *    HIP header; the value is cast back to hipStream_t inside the library.
 *    Calls are asynchronous: ATTN_OK means the kernels were enqueued. A device
 *    fault surfaces at the caller's next synchronisation.
 *  - The caller owns every buffer (inputs, outputs, workspace) and keeps it
 *    alive until the stream has finished the call. The library allocates no
 *    device memory and keeps no per-call state.
 *  - Outputs must not alias inputs or each other. Every output element is
 *    overwritten; none needs to be cleared beforehand.
 *  - Arguments are validated before any HIP call; on an error nothing is
 *    launched and nothing is written.
 */
#ifndef MI355_ATTN_H
#define MI355_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,          /* a required pointer is NULL */
    ATTN_ERR_SHAPE = 2,         /* B, Hq, Hkv, S, D or Dv < 1, B*Hq*S*max(D, Dv) >= 2^40,
                                   S*max(D, Dv) >= 2^31, or a launch grid of 2^32
                                   work-items or more: B*Hq*(2S+512) or B*Hkv*(8S+512) */
    ATTN_ERR_GQA = 3,           /* Hq is not a multiple of Hkv */
    ATTN_ERR_UNSUPPORTED_D = 4, /* D (or Dv) is neither 64 nor 128 */
    ATTN_ERR_ALIGN = 5,         /* a tensor or workspace pointer is not 16-byte aligned */
    ATTN_ERR_WORKSPACE = 6,     /* workspace is NULL or smaller than attn_bwd_workspace_bytes() */
    ATTN_ERR_SCALE = 7,         /* scale is NaN or infinite */
    ATTN_ERR_HIP = 8,           /* the HIP runtime failed (no device, launch error) */
    ATTN_ERR_DEVICE = 9,        /* the current device is not a gfx950 GPU */
    ATTN_ERR_WINDOW = 10,       /* a sliding window of fewer than 1 key (vdim: < 0, or set without causal) */
    ATTN_ERR_SPARSE = 11,       /* sparse: topk > 4096, Hq/Hkv > 128, N*D or S*topk >= 2^31,
                                   or a launch grid of 2^32 work-items or more:
                                   B*S*Hkv*ceil(Hq/Hkv/64)*128, B*S*Hkv*ceil(topk/128)*256
                                   or B*Hkv*N*256 */
    ATTN_ERR_SCRATCH = 12       /* attn_bwd_noalloc: the sizes need more workspace than its
                                   static scratch holds */
};

/*
 * Forward pass, Eq. (1) with Algorithm 0's streaming (section 2.1).
 *   q    [B][Hq][S][D]  bf16, read
 *   k, v [B][Hkv][S][D] bf16, read
 *   o    [B][Hq][S][D]  bf16, written: softmax(q k^T * scale) v, accumulated in
 *                       fp32 and rounded to nearest even once at the end
 *   lse  [B][Hq][S]     fp32, written: natural-log log-sum-exp of each row's
 *                       scaled scores, ln(sum_j exp(scale * q_i . k_j))
 * Returns an attn_status.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int S, int D, int causal, float scale, void* stream);

/*
 * Bytes of device workspace attn_bwd needs for these sizes: the row statistics,
 * per block of 32 query rows their lse_i * log2(e) then their -delta_i (delta_i =
 * sum_j P_ij dP_ij), fp32 ([B][Hq][ceil(S/32)][64]; rows past S hold +inf and
 * -0), and one int32 flag per block of 32 query rows ([B][Hq][ceil(S/32)]: 1
 * where a row of the block has a probability above 1/4, whose gradient terms
 * then take the exact path), each part 256-byte aligned. Returns 0 when the sizes
 * are invalid (attn_bwd would reject them).
 */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D);

/*
 * Backward pass: exact gradient of Eq. (1) (section 2.1; Table 3 lists its
 * dQ and dK products), with P recomputed from lse.
 *   q, k, v        as in attn_fwd, read
 *   o              [B][Hq][S][D] bf16, read: attn_fwd's output for the same inputs
 *   lse            [B][Hq][S] fp32, read: attn_fwd's lse for the same inputs
 *   dout           [B][Hq][S][D] bf16, read: gradient of the loss w.r.t. o
 *   dq             [B][Hq][S][D] fp32, written
 *   dk, dv         [B][Hkv][S][D] fp32, written; each key/value head's gradient
 *                  is summed over the Hq/Hkv query heads that read it
 *   workspace      device scratch of at least attn_bwd_workspace_bytes() bytes,
 *                  16-byte aligned; its contents on entry do not matter and on
 *                  return are unspecified
 * Calls that share a workspace must be ordered on one stream.
 * Returns an attn_status.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, float* dq, float* dk, float* dv,
             int B, int Hq, int Hkv, int S, int D, int causal, float scale,
             void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation, arguments and results as attn_bwd, without the workspace
 * arguments. Its workspace is a static device array of the library, 16 MiB per
 * GPU (attn_bwd_noalloc_max_workspace_bytes()), held from the first call on a
 * device until the process ends; the call itself allocates nothing. Sizes with
 * attn_bwd_workspace_bytes() above that limit return ATTN_ERR_SCRATCH before
 * anything is launched (for example B*Hq*S up to 2,000,000 query rows fit). Every
 * call on one GPU shares that GPU's array: calls that may overlap on one GPU
 * (different streams, or other threads) race and must be ordered by the caller.
 * Nothing in the array needs clearing between calls: each call writes every
 * value it later reads.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, float* dq, float* dk, float* dv,
                     int B, int Hq, int Hkv, int S, int D, int causal, float scale, void* stream);
size_t attn_bwd_noalloc_max_workspace_bytes(void);

/*
 * The two stages attn_bwd runs, for callers that schedule them separately
 * (attn_bwd is exactly attn_bwd_dq followed by attn_bwd_dkdv on one stream).
 * Arguments and errors are those of attn_bwd.
 *   attn_bwd_dq    writes the row statistics (lse_i * log2(e), delta_i =
 *                  sum_j P_ij dP_ij) and the per-block flags into the workspace,
 *                  and dq = scale * dS K (section 2.1, Table 3, query gradient
 *                  row). dk and dv are not touched.
 *   attn_bwd_dkdv  reads the row statistics and the flags from the workspace (it must hold
 *                  attn_bwd_dq's result for the same inputs) and writes
 *                  dk = scale * dS^T Q
 *                  (Table 3, key gradient row) and dv = P^T dO, each summed over
 *                  the query heads of its group. dq is not touched.
 */
int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, float* dq, float* dk, float* dv,
                int B, int Hq, int Hkv, int S, int D, int causal, float scale,
                void* workspace, size_t workspace_bytes, void* stream);
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, float* dq, float* dk, float* dv,
                  int B, int Hq, int Hkv, int S, int D, int causal, float scale,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sliding-window causal attention: query row i sees only the `window` most
 * recent keys, i - window < j <= i. This is the window every query of the
 * compressed sparse attention on the same page attends to (Table 7, window =
 * 128; section 3.1.1 describes its sliding-window kernels); within the band,
 * Eq. (1) and its gradient are computed exactly as by attn_fwd / attn_bwd with
 * causal != 0. window >= S gives the plain causal result. Tiles outside the
 * band are neither loaded nor multiplied, so the work is O(S * window).
 *   window  >= 1, else ATTN_ERR_WINDOW (checked before anything else)
 * Every other argument, the layouts and the errors are those of attn_fwd and
 * attn_bwd; attn_bwd_window takes a workspace of
 * attn_bwd_workspace_bytes(B, Hq, Hkv, S, D) bytes, and needs o and lse
 * from attn_fwd_window with the same window.
 */
int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int S, int D, int window, float scale, void* stream);
int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, float* dq, float* dk, float* dv,
                    int B, int Hq, int Hkv, int S, int D, int window, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Separate value head dimension: Eq. (1) (section 2.1) gives queries and keys
 * d columns and values d_v columns, which need not be equal. Here d = D and
 * d_v = Dv, each 64 or 128 (else ATTN_ERR_UNSUPPORTED_D), in any combination:
 *   q, dq   [B][Hq][S][D]     k, dk   [B][Hkv][S][D]
 *   o, dout [B][Hq][S][Dv]    v, dv   [B][Hkv][S][Dv]      lse [B][Hq][S]
 * causal and window combine as in the entry points above: window = 0 means no
 * window; window >= 1 needs causal != 0 (else, or for window < 0,
 * ATTN_ERR_WINDOW). Scores are q . k over D columns, so the usual scale is
 * 1/sqrt(D). attn_bwd_vdim's workspace is attn_bwd_workspace_bytes(B, Hq, Hkv,
 * S, D) bytes (its row statistics do not depend on Dv), and it
 * needs o and lse from attn_fwd_vdim with the same arguments. With Dv == D these
 * are attn_fwd / attn_bwd (window = 0) and attn_fwd_window / attn_bwd_window.
 * Every other rule, layout and error is that of attn_fwd and attn_bwd, with
 * B*Hq*S*max(D, Dv) < 2^40 and S*max(D, Dv) < 2^31.
 */
int attn_fwd_vdim(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int S, int D, int Dv, int causal, int window,
                  float scale, void* stream);
int attn_bwd_vdim(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, float* dq, float* dk, float* dv,
                  int B, int Hq, int Hkv, int S, int D, int Dv, int causal, int window,
                  float scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse attention over per-token index lists: the compressed sparse attention
 * of the same page (section 2.1; Table 7 gives its list shapes) gives every
 * query token a top-k list of key/value rows, a sliding window of recent tokens
 * plus rows of a compressed pool. The forward gathers the listed rows, scores
 * them and streams their values into the output: Eq. (1) restricted to the
 * token's list, one term per list slot. The backward gathers the same rows for
 * dQ, forms one dK/dV contribution per (token, slot), and reduces those by the
 * inverse of the index map (section 2.1's description of the CSA backward).
 *   q, o, dout, dq [B][Hq][S][D]   (o, dout bf16; dq fp32)
 *   k, v           [B][Hkv][N][D] bf16: N key/value rows per kv head (for the
 *                  compressed attention, the S raw tokens followed by the pool)
 *   dk, dv         [B][Hkv][N][D] fp32: every row is written (0 where no list
 *                  names it), summed over the query heads of its group
 *   idx            [B][S][topk] int32, device memory, shared by all query heads
 *                  of a token; entry s of token i names row idx[b][i][s]; an
 *                  entry outside [0, N) is an empty slot. A row listed twice
 *                  counts twice. The lists carry every causal or window
 *                  restriction; nothing else masks.
 *   lse            [B][Hq][S] fp32 (natural log); -inf for a token whose list is
 *                  empty, whose O row is 0 (and whose dQ row is 0)
 * D is 64 or 128, topk in [1, 4096], Hq/Hkv <= 128, N*D and S*topk < 2^31,
 * and every launch within a grid of fewer than 2^32 work-items (the reduction
 * takes 256 per key/value row, so B*Hkv*N < 2^24) (ATTN_ERR_SPARSE otherwise). attn_sparse_bwd needs o and lse from
 * attn_sparse_fwd with the same arguments, and a workspace of
 * attn_sparse_bwd_workspace_bytes() bytes: delta, the per-(token, slot)
 * contributions (2 * B*Hkv*S*topk*D fp32) and the inverse map; its contents on
 * entry do not matter. Results are deterministic (no floating-point atomics).
 * Every other rule is that of attn_fwd / attn_bwd.
 */
int attn_sparse_fwd(const void* q, const void* k, const void* v, const int* idx, void* o, float* lse,
                    int B, int Hq, int Hkv, int S, int N, int D, int topk, float scale,
                    void* stream);
size_t attn_sparse_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int N, int D, int topk);
int attn_sparse_bwd(const void* q, const void* k, const void* v, const int* idx, const void* o,
                    const float* lse, const void* dout, float* dq, float* dk, float* dv,
                    int B, int Hq, int Hkv, int S, int N, int D, int topk, float scale,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MI355_ATTN_H */
