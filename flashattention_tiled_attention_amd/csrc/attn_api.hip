// C ABI of the attention library: argument validation, per-device set-up and
// kernel launch on the caller's stream. Declarations and the contract of each
// entry point are in include/attn.h.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "attn.h"
#include "kernels.h"

namespace attn {
hipError_t fwd_setup_device();
hipError_t bwd_setup_device();
hipError_t sparse_setup_device();
int sparse_tokens_per_chunk();
int sparse_max_heads_per_kv();
}  // namespace attn

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_status[kMaxDevices];

// Backward scratch of attn_bwd_noalloc: one copy per GPU, held until the process
// ends. In host code `scratch` names a host-side stand-in, not device memory; the
// device address of each GPU's copy is taken once per device at set-up
// (g_scratch) and only that address is ever passed to a kernel.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch[kMaxDevices];

// Once per device: check that it is a gfx950 GPU and raise the kernels'
// dynamic-LDS limit. Returns an attn_status.
int setup_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return ATTN_ERR_HIP;
    }
    if (dev >= kMaxDevices) return ATTN_ERR_DEVICE;
    std::call_once(g_dev_once[dev], [dev]() {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            g_dev_status[dev] = ATTN_ERR_HIP;
            return;
        }
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            g_dev_status[dev] = ATTN_ERR_DEVICE;
            return;
        }
        if (attn::fwd_setup_device() != hipSuccess || attn::bwd_setup_device() != hipSuccess ||
            attn::sparse_setup_device() != hipSuccess) {
            (void)hipGetLastError();
            g_dev_status[dev] = ATTN_ERR_HIP;
            return;
        }
        // this device's copy of the no-allocation scratch (the device is current)
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            g_dev_status[dev] = ATTN_ERR_HIP;
            return;
        }
        g_scratch[dev] = ptr;
        g_dev_status[dev] = ATTN_OK;
    });
    return g_dev_status[dev];
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

// D: query/key head dimension; Dv: value head dimension.
int check_sizes(int B, int Hq, int Hkv, int S, int D, int Dv) {
    if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || D < 1 || Dv < 1) return ATTN_ERR_SHAPE;
    const double elems = (double)B * Hq * S * (D > Dv ? D : Dv);
    if (elems >= 1099511627776.0) return ATTN_ERR_SHAPE;  // 2^40
    // row offsets within one head are 32-bit in the kernels' tile copies
    if ((double)S * (D > Dv ? D : Dv) >= 2147483648.0) return ATTN_ERR_SHAPE;  // 2^31
    // Every launch's work-items (workgroups x threads) must fit the 32-bit grid.
    // Per query head the forward launches at most 2*S + 512 of them (256 rows, or
    // 256/HW rows of HW heads, per 512-thread workgroup) and the dQ kernel at most
    // 2*S + 256 (128 rows per 256 threads); per kv head the dK/dV kernel launches
    // ceil(S/64) workgroups of 512 threads, at most 8*S + 512.
    if ((double)B * Hq * (2.0 * S + 512.0) >= 4294967296.0) return ATTN_ERR_SHAPE;
    if ((double)B * Hkv * (8.0 * S + 512.0) >= 4294967296.0) return ATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_GQA;
    if ((D != 64 && D != 128) || (Dv != 64 && Dv != 128)) return ATTN_ERR_UNSUPPORTED_D;
    return ATTN_OK;
}

// Dense backward workspace: the row statistics [B][Hq][ceil(S/32)][64] fp32 (per
// block of 32 query rows their lse * log2(e), then their -delta; rows past S hold
// +inf and -0), then the per-32-row-block exact-path flags [B][Hq][ceil(S/32)]
// int32, each part 256-byte aligned.
size_t rowstat_bytes(int B, int Hq, int S) {
    return (((size_t)B * Hq * ((S + 31) / 32) * 32 * 2 * sizeof(float)) + 255) & ~(size_t)255;
}
size_t peak_bytes(int B, int Hq, int S) {
    return (((size_t)B * Hq * ((S + 31) / 32) * sizeof(int)) + 255) & ~(size_t)255;
}

constexpr int kSparseMaxTopk = 4096;

// Sizes of the sparse entry points: D is the head dimension of q, k, v; N the
// number of key/value rows; topk the list length.
int check_sparse_sizes(int B, int Hq, int Hkv, int S, int N, int D, int topk) {
    if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || N < 1 || D < 1 || topk < 1) return ATTN_ERR_SHAPE;
    if ((double)B * Hq * S * D >= 1099511627776.0 || (double)B * Hkv * N * D >= 1099511627776.0)
        return ATTN_ERR_SHAPE;
    if (Hq % Hkv != 0) return ATTN_ERR_GQA;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED_D;
    if (topk > kSparseMaxTopk || Hq / Hkv > attn::sparse_max_heads_per_kv()) return ATTN_ERR_SPARSE;
    // 32-bit row offsets within a head, 32-bit list entries, 32-bit grids
    if ((double)N * D >= 2147483647.0 || (double)S * topk >= 2147483647.0) return ATTN_ERR_SPARSE;
    // Work-items (workgroups x threads) of every launch within the 32-bit grid: the
    // forward and dQ kernels (128 threads per 64 query heads of a token), the partial
    // kernel (256 threads per 128 list slots of a token and kv head) and the reduction
    // (256 threads per key/value row).
    const double heads = (double)B * S * Hkv * ((Hq / Hkv + 63) / 64);
    if (heads * 128.0 >= 4294967296.0) return ATTN_ERR_SPARSE;
    if ((double)B * S * Hkv * ((topk + 127) / 128) * 256.0 >= 4294967296.0) return ATTN_ERR_SPARSE;
    if ((double)B * Hkv * N * 256.0 >= 4294967296.0) return ATTN_ERR_SPARSE;
    return ATTN_OK;
}

// Backward workspace: delta, the two per-(token, slot) contribution arrays, and
// the inverse of the index map (chunk counts, row starts, entry list).
struct SparseWs {
    size_t delta, inter_k, inter_v, cnt, rowstart, list, total;
    int nchunks;
};

SparseWs sparse_ws(int B, int Hq, int Hkv, int S, int N, int D, int topk) {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    SparseWs w;
    w.nchunks = (S + attn::sparse_tokens_per_chunk() - 1) / attn::sparse_tokens_per_chunk();
    size_t off = 0;
    w.delta = off;    off += al((size_t)B * Hq * S * 4);
    w.inter_k = off;  off += al((size_t)B * Hkv * S * topk * D * 4);
    w.inter_v = off;  off += al((size_t)B * Hkv * S * topk * D * 4);
    w.cnt = off;      off += al((size_t)B * w.nchunks * N * 4);
    w.rowstart = off; off += al((size_t)B * (N + 1) * 4);
    w.list = off;     off += al((size_t)B * S * topk * 4);
    w.total = off;
    return w;
}

}  // namespace

extern "C" {

const char* attn_status_str(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "B, Hq, Hkv, S, D and Dv must be >= 1 and B*Hq*S*max(D, Dv) < 2^40";
        case ATTN_ERR_GQA: return "Hq must be a multiple of Hkv";
        case ATTN_ERR_UNSUPPORTED_D: return "head dimensions D and Dv must be 64 or 128";
        case ATTN_ERR_ALIGN: return "tensor and workspace pointers must be 16-byte aligned";
        case ATTN_ERR_WORKSPACE: return "workspace is NULL or smaller than attn_bwd_workspace_bytes()";
        case ATTN_ERR_SCALE: return "scale must be finite";
        case ATTN_ERR_HIP: return "HIP runtime error";
        case ATTN_ERR_DEVICE: return "the current device is not a gfx950 (MI355X) GPU";
        case ATTN_ERR_WINDOW: return "window must be >= 1 (>= 0 and causal for the vdim entry points)";
        case ATTN_ERR_SPARSE:
            return "sparse sizes out of range: topk <= 4096, Hq/Hkv <= 128, N*D and S*topk < 2^31";
        case ATTN_ERR_SCRATCH:
            return "attn_bwd_noalloc: attn_bwd_workspace_bytes() for these sizes exceeds its 16 MiB static scratch";
        default: return "unknown attn status";
    }
}

static int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int Hq, int Hkv, int S, int D, int Dv, int causal, int window, float scale,
                    void* stream) {
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    int rc = check_sizes(B, Hq, Hkv, S, D, Dv);
    if (rc) return rc;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse))
        return ATTN_ERR_ALIGN;
    if ((rc = setup_current_device())) return rc;

    attn::FwdArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (uint16_t*)o;
    a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S; a.G = Hq / Hkv;
    a.causal = causal ? 1 : 0;
    a.window = window;
    // The kernel needs a strictly positive factor (masked scores are -inf); a zero
    // scale becomes 2^-100, which leaves every exp2 of a finite score at exactly 1.
    a.scale_log2 = fmaxf(fabsf(scale) * 1.4426950408889634f, 7.888609052210118e-31f);
    a.q_sign = scale < 0.0f ? 0x80008000u : 0u;
    // A stale row maximum leaves the dominant weight of a peaked row (|scale| *
    // sqrt(D) > 2 for unit-variance inputs) off 1.0 and so exposed to bf16
    // rounding; there the maximum is tracked exactly.
    a.max_slack = fabsf(scale) * sqrtf((float)D) > 2.0f ? 0.0f : 8.0f;
    a.precise_tiles = 0;  // set by the launcher, which knows the tile size
    if (attn::launch_fwd(a, D, Dv, (hipStream_t)stream) != hipSuccess) return ATTN_ERR_HIP;
    return ATTN_OK;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int S, int D, int causal, float scale, void* stream) {
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, S, D, D, causal, 0, scale, stream);
}

int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int Hq, int Hkv, int S, int D, int window, float scale, void* stream) {
    if (window < 1) return ATTN_ERR_WINDOW;
    // a window of S or more keys is the whole causal triangle
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, S, D, D, 1, window >= S ? 0 : window, scale, stream);
}

int attn_fwd_vdim(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int Hq, int Hkv, int S, int D, int Dv, int causal, int window, float scale,
                  void* stream) {
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_WINDOW;
    return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, S, D, Dv, causal, window >= S ? 0 : window,
                    scale, stream);
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D) {
    if (check_sizes(B, Hq, Hkv, S, D, D) != ATTN_OK) return 0;
    return rowstat_bytes(B, Hq, S) + peak_bytes(B, Hq, S);
}

// use_scratch: the workspace is this device's static scratch (attn_bwd_noalloc);
// workspace and workspace_bytes are then ignored.
static int bwd_stages(int stages, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, float* dq, float* dk, float* dv, int B,
                      int Hq, int Hkv, int S, int D, int Dv, int causal, int window, float scale,
                      void* workspace, size_t workspace_bytes, void* stream, bool use_scratch = false) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
    int rc = check_sizes(B, Hq, Hkv, S, D, Dv);
    if (rc) return rc;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (use_scratch) {
        if (attn_bwd_workspace_bytes(B, Hq, Hkv, S, D) > kScratchBytes) return ATTN_ERR_SCRATCH;
    } else if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, Hq, Hkv, S, D)) {
        return ATTN_ERR_WORKSPACE;
    }
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse) ||
        misaligned(dout) || misaligned(dq) || misaligned(dk) || misaligned(dv) ||
        (!use_scratch && misaligned(workspace)))
        return ATTN_ERR_ALIGN;
    if ((rc = setup_current_device())) return rc;
    if (use_scratch) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices || !g_scratch[dev]) {
            (void)hipGetLastError();
            return ATTN_ERR_HIP;
        }
        workspace = g_scratch[dev];
    }

    attn::BwdArgs a;
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.o = (const uint16_t*)o;
    a.lse = lse;
    a.dout = (const uint16_t*)dout;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.rowstat = (float*)workspace;
    a.peak = (int*)((unsigned char*)workspace + rowstat_bytes(B, Hq, S));
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S; a.G = Hq / Hkv;
    a.causal = causal ? 1 : 0;
    a.window = window;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    // Rows with a probability above kPeakP take the exact path wherever the data
    // puts them (the dQ stage finds them). Every tile takes it from the start when
    // most rows will need it: a score spread |scale| * sqrt(D) > 2 for
    // unit-variance inputs, or a window of fewer than 128 keys, where every row sees
    // fewer keys than the first causal rows do. A window of 128 keys or more is left
    // to the data, as the causal problem is: with every row on 128 keys, bf16 P and
    // dS keep dQ, dK and dV within 5e-3 of fp64 at the Llama-3.1-8B shape
    // (unit-variance inputs).
    a.precise_all = (fabsf(scale) * sqrtf((float)D) > 2.0f || (window > 0 && window < 128)) ? 1 : 0;
    if (attn::launch_bwd(a, D, Dv, stages, (hipStream_t)stream) != hipSuccess) return ATTN_ERR_HIP;
    return ATTN_OK;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int S,
             int D, int causal, float scale, void* workspace, size_t workspace_bytes,
             void* stream) {
    return bwd_stages(3, q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, S, D, D, causal, 0, scale,
                      workspace, workspace_bytes, stream);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int S,
                     int D, int causal, float scale, void* stream) {
    return bwd_stages(3, q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, S, D, D, causal, 0, scale,
                      nullptr, 0, stream, true);
}

size_t attn_bwd_noalloc_max_workspace_bytes(void) { return kScratchBytes; }

int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse,
                const void* dout, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int S,
                int D, int causal, float scale, void* workspace, size_t workspace_bytes,
                void* stream) {
    return bwd_stages(1, q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, S, D, D, causal, 0, scale,
                      workspace, workspace_bytes, stream);
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, float* dq, float* dk, float* dv, int B, int Hq, int Hkv, int S,
                  int D, int causal, float scale, void* workspace, size_t workspace_bytes,
                  void* stream) {
    return bwd_stages(2, q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, S, D, D, causal, 0, scale,
                      workspace, workspace_bytes, stream);
}

int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, float* dq, float* dk, float* dv, int B, int Hq, int Hkv,
                    int S, int D, int window, float scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (window < 1) return ATTN_ERR_WINDOW;
    return bwd_stages(3, q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, S, D, D, 1,
                      window >= S ? 0 : window, scale, workspace, workspace_bytes, stream);
}

int attn_bwd_vdim(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, float* dq, float* dk, float* dv, int B, int Hq, int Hkv,
                  int S, int D, int Dv, int causal, int window, float scale, void* workspace,
                  size_t workspace_bytes, void* stream) {
    if (window < 0 || (window > 0 && !causal)) return ATTN_ERR_WINDOW;
    return bwd_stages(3, q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, S, D, Dv, causal,
                      window >= S ? 0 : window, scale, workspace, workspace_bytes, stream);
}

int attn_sparse_fwd(const void* q, const void* k, const void* v, const int* idx, void* o, float* lse,
                    int B, int Hq, int Hkv, int S, int N, int D, int topk, float scale,
                    void* stream) {
    if (!q || !k || !v || !idx || !o || !lse) return ATTN_ERR_NULL;
    int rc = check_sparse_sizes(B, Hq, Hkv, S, N, D, topk);
    if (rc) return rc;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(idx) || misaligned(o) ||
        misaligned(lse))
        return ATTN_ERR_ALIGN;
    if ((rc = setup_current_device())) return rc;
    attn::SparseArgs a = {};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.idx = (const int32_t*)idx;
    a.out = (uint16_t*)o;
    a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S; a.N = N; a.G = Hq / Hkv; a.topk = topk;
    a.scale = scale;
    a.scale_log2 = fmaxf(fabsf(scale) * 1.4426950408889634f, 7.888609052210118e-31f);
    a.q_sign = scale < 0.0f ? 0x80008000u : 0u;
    a.precise_all = fabsf(scale) * sqrtf((float)D) > 2.0f ? 1 : 0;
    a.max_slack = a.precise_all ? 0.0f : 8.0f;  // exact running maximum for peaked rows
    if (attn::launch_sparse_fwd(a, D, (hipStream_t)stream) != hipSuccess) return ATTN_ERR_HIP;
    return ATTN_OK;
}

size_t attn_sparse_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int N, int D, int topk) {
    if (check_sparse_sizes(B, Hq, Hkv, S, N, D, topk) != ATTN_OK) return 0;
    return sparse_ws(B, Hq, Hkv, S, N, D, topk).total;
}

int attn_sparse_bwd(const void* q, const void* k, const void* v, const int* idx, const void* o,
                    const float* lse, const void* dout, float* dq, float* dk, float* dv, int B,
                    int Hq, int Hkv, int S, int N, int D, int topk, float scale, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (!q || !k || !v || !idx || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
    int rc = check_sparse_sizes(B, Hq, Hkv, S, N, D, topk);
    if (rc) return rc;
    if (!isfinite(scale)) return ATTN_ERR_SCALE;
    const SparseWs w = sparse_ws(B, Hq, Hkv, S, N, D, topk);
    if (!workspace || workspace_bytes < w.total) return ATTN_ERR_WORKSPACE;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(idx) || misaligned(o) ||
        misaligned(lse) || misaligned(dout) || misaligned(dq) || misaligned(dk) || misaligned(dv) ||
        misaligned(workspace))
        return ATTN_ERR_ALIGN;
    if ((rc = setup_current_device())) return rc;
    attn::SparseArgs a = {};
    a.q = (const uint16_t*)q;
    a.k = (const uint16_t*)k;
    a.v = (const uint16_t*)v;
    a.idx = (const int32_t*)idx;
    a.o = (const uint16_t*)o;
    a.dout = (const uint16_t*)dout;
    a.lse = (float*)lse;  // read only by the backward kernels
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    unsigned char* ws = (unsigned char*)workspace;
    a.delta = (float*)(ws + w.delta);
    a.inter_k = (float*)(ws + w.inter_k);
    a.inter_v = (float*)(ws + w.inter_v);
    a.cnt = (int*)(ws + w.cnt);
    a.rowstart = (int*)(ws + w.rowstart);
    a.list = (int*)(ws + w.list);
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.S = S; a.N = N; a.G = Hq / Hkv; a.topk = topk;
    a.nchunks = w.nchunks;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.precise_all = fabsf(scale) * sqrtf((float)D) > 2.0f ? 1 : 0;
    if (attn::launch_sparse_bwd(a, D, (hipStream_t)stream) != hipSuccess) return ATTN_ERR_HIP;
    return ATTN_OK;
}

}  // extern "C"
