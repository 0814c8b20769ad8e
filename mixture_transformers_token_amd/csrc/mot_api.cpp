// C-ABI layer of libmot: argument validation (fail closed, before anything is
// enqueued), device selection from the caller's stream, and kernel dispatch.
// The layer allocates nothing and keeps no state between calls.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mot.h"
#include "mot_internal.h"

namespace {

constexpr int64_t kWsAlign = 256;

int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void *a, int64_t a_bytes, const void *b, int64_t b_bytes) {
    if (a_bytes <= 0 || b_bytes <= 0) return false;  // an empty range overlaps nothing
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

// Makes the stream's device current for the duration of a call (launches go to
// the device that owns the caller's stream, not to whatever device is current).
class DeviceGuard {
  public:
    explicit DeviceGuard(hipStream_t s) {
        if (hipGetDevice(&prev_) != hipSuccess) {
            ok_ = false;
            return;
        }
        int dev = prev_;
        if (s != nullptr && hipStreamGetDevice(s, &dev) != hipSuccess) {
            ok_ = false;
            return;
        }
        if (dev != prev_) {
            if (hipSetDevice(dev) != hipSuccess) {
                ok_ = false;
                return;
            }
            switched_ = true;
        }
    }
    ~DeviceGuard() {
        if (switched_) (void)hipSetDevice(prev_);
    }
    bool ok() const { return ok_; }

  private:
    int prev_ = 0;
    bool ok_ = true;
    bool switched_ = false;
};

constexpr int64_t kAttnHeadDim = 128;
constexpr int64_t kAttnMaxHeads = 256;

// the attention reads V in place: one sequence needs no workspace, packed
// sequences only the header with the lengths check's error word
size_t attn_ws_bytes(int64_t, int64_t) { return 0; }

size_t attn_varlen_ws_bytes(int64_t Tk, int64_t n_seqs, int64_t hkv) {
    if (Tk < 0 || n_seqs <= 0 || hkv <= 0) return 0;
    return (size_t)MOT_WS_HEADER_BYTES;
}

constexpr int64_t kLatentMaxC = 4096;

size_t latent_ws_bytes(int64_t n_req, int64_t max_rows) {
    if (n_req <= 0 || max_rows <= 0 || n_req > MOT_MAX_T || max_rows > MOT_MAX_T) return 0;
    return (size_t)(MOT_WS_HEADER_BYTES + n_req * (int64_t)mot::latent_chunks(max_rows) * 2 * 4);
}

// Checks shared by the latent-step calls; 0 if fine.
int validate_latent(int64_t n_req, int64_t rows, int64_t C, int64_t max_rows, const int32_t *cu,
                    void *workspace, size_t workspace_bytes) {
    if (n_req < 0 || rows < 0 || C <= 0 || max_rows < 1) return MOT_ERR_INVALID_ARG;
    if (C % 4 || C > kLatentMaxC || rows > MOT_MAX_T || n_req > MOT_MAX_T || max_rows > MOT_MAX_T)
        return MOT_ERR_UNSUPPORTED_SHAPE;
    if (n_req * (int64_t)mot::latent_chunks(max_rows) >= (int64_t(1) << 31)) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (!cu) return MOT_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(cu) & 3u) return MOT_ERR_MISALIGNED;
    if (!workspace || workspace_bytes < latent_ws_bytes(n_req, max_rows)) return MOT_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1)) != 0) return MOT_ERR_MISALIGNED;
    return MOT_OK;
}

size_t ws_bytes(int64_t T) {
    return (size_t)(MOT_WS_HEADER_BYTES + round_up(4 * (T > 0 ? T : 0), kWsAlign));
}

struct RoutedCall {
    const uint16_t *x;
    int64_t ldx;
    const uint16_t *w_und, *w_gen;
    const uint8_t *modality;
    void *y;
    int64_t ldy;
    int64_t T, K, N;       // N: output columns (F for SwiGLU)
    int64_t w_rows;        // rows of each weight matrix (N, or 2F)
    const float *rstd;
    const uint16_t *nw_und, *nw_gen;
    void *workspace;
    size_t workspace_bytes;
    unsigned flags;
    int out_f32 = 0;       // 1: y is fp32 [T][ldy]
    const mot::QkArgs *qk = nullptr;  // fused QK norm + rotary epilogue (qkv, ld, T unused)
    // 1: the weights are contraction-major, [K][N] with pitch N (the forward's
    // weights of dX = dY W): big tiles only, no prologue, bf16 output
    int wtok = 0;
};

int validate_routed(const RoutedCall &c) {
    if (c.T < 0 || c.K < 0 || c.N < 0) return MOT_ERR_INVALID_ARG;
    if (c.T == 0) return MOT_OK;
    if (!c.x || !c.w_und || !c.w_gen || !c.modality || !c.y) return MOT_ERR_INVALID_ARG;
    if (c.T > MOT_MAX_T) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (c.K == 0 || c.N == 0 || c.K % 64 || c.N % 64 || c.K > MOT_MAX_DIM || c.N > MOT_MAX_DIM)
        return MOT_ERR_UNSUPPORTED_SHAPE;
    if ((c.flags & ~(MOT_FLAG_PLAN_READY | MOT_FLAG_TILE_MASK)) != 0) return MOT_ERR_INVALID_ARG;
    if (c.ldx < c.K || c.ldy < c.N || c.ldx > (int64_t(1) << 32) || c.ldy > (int64_t(1) << 32))
        return MOT_ERR_INVALID_ARG;
    if (c.ldx % 8 || c.ldy % 8) return MOT_ERR_MISALIGNED;
    const int npro = (c.rstd != nullptr) + (c.nw_und != nullptr) + (c.nw_gen != nullptr);
    if (npro != 0 && npro != 3) return MOT_ERR_INVALID_ARG;
    if (npro == 3 && c.K > mot::kMaxPrologueK) return MOT_ERR_UNSUPPORTED_SHAPE;
    if ((c.flags & MOT_FLAG_TILE_MASK) == MOT_FLAG_TILE_MASK) return MOT_ERR_INVALID_ARG;
    if (c.out_f32 && (npro != 0 || (c.flags & MOT_FLAG_TILE_MASK) != 0)) return MOT_ERR_INVALID_ARG;
    if (!aligned16(c.x) || !aligned16(c.w_und) || !aligned16(c.w_gen) || !aligned16(c.y))
        return MOT_ERR_MISALIGNED;
    if (npro == 3 && (!aligned16(c.nw_und) || !aligned16(c.nw_gen) ||
                      (reinterpret_cast<uintptr_t>(c.rstd) & 3u)))
        return MOT_ERR_MISALIGNED;
    if (!c.workspace || c.workspace_bytes < ws_bytes(c.T)) return MOT_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(c.workspace) & (kWsAlign - 1)) != 0) return MOT_ERR_MISALIGNED;
    const int64_t x_bytes = ((c.T - 1) * c.ldx + c.K) * 2;
    const int64_t y_bytes = ((c.T - 1) * c.ldy + c.N) * (c.out_f32 ? 4 : 2);
    if (overlaps(c.x, x_bytes, c.y, y_bytes)) return MOT_ERR_INVALID_ARG;
    const int64_t w_bytes = c.w_rows * c.K * 2;
    if (overlaps(c.w_und, w_bytes, c.y, y_bytes) || overlaps(c.w_gen, w_bytes, c.y, y_bytes))
        return MOT_ERR_INVALID_ARG;
    if (overlaps(c.workspace, (int64_t)ws_bytes(c.T), c.y, y_bytes)) return MOT_ERR_INVALID_ARG;
    // the kernels address each operand with 32-bit byte offsets
    if (x_bytes >= (int64_t(1) << 32) || w_bytes >= (int64_t(1) << 32) ||
        y_bytes >= (int64_t(1) << 32))
        return MOT_ERR_UNSUPPORTED_SHAPE;
    return MOT_OK;
}

int run_routed(const RoutedCall &c, bool swiglu, void *stream) {
    const int v = validate_routed(c);
    if (v != MOT_OK || c.T == 0) return v;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    int32_t *hdr = static_cast<int32_t *>(c.workspace);
    int32_t *perm = reinterpret_cast<int32_t *>(static_cast<char *>(c.workspace) + MOT_WS_HEADER_BYTES);
    const bool plan_ready = (c.flags & MOT_FLAG_PLAN_READY) != 0;
    const bool inline_route = !plan_ready && c.T <= mot::kInlineRouteMaxT;
    if (!plan_ready && !inline_route) {
        if (mot::launch_plan(c.modality, c.T, hdr, perm, s) != hipSuccess) return MOT_ERR_DEVICE;
    }
    mot::GemmArgs a;
    a.modality = c.modality;
    a.hdr_out = hdr;
    a.perm_out = perm;
    a.x = c.x;
    a.ldx = c.ldx;
    a.w_und = c.w_und;
    a.w_gen = c.w_gen;
    a.y = c.y;
    a.ldy = c.ldy;
    a.hdr = hdr;
    a.perm = perm;
    a.rstd = c.rstd;
    a.nw_und = c.nw_und;
    a.nw_gen = c.nw_gen;
    a.T = c.T;
    a.K = (int)c.K;
    a.N = (int)c.N;
    a.wrows = (int)c.w_rows;
    switch (c.flags & MOT_FLAG_TILE_MASK) {
    case MOT_FLAG_TILE_256x256: a.tile_mode = 1; break;
    case MOT_FLAG_TILE_128x128: a.tile_mode = 2; break;
    default: a.tile_mode = 0;
    }
    a.x_bytes = (uint32_t)(((c.T - 1) * c.ldx + c.K) * 2);
    a.w_bytes = (uint32_t)(c.w_rows * c.K * 2);
    a.y_bytes = (uint32_t)(((c.T - 1) * c.ldy + c.N) * (c.out_f32 ? 4 : 2));
    a.out_f32 = c.out_f32;
    if (c.qk != nullptr && c.T <= mot::kSkinnyMaxT && a.tile_mode == 0) {
        // small pack: the weight-bound GEMM (its 32-column slabs split heads),
        // then the standalone QK kernel on its rows, which does nothing if
        // the GEMM's error word is set
        if (mot::launch_gemm(a, false, inline_route, s) != hipSuccess) return MOT_ERR_DEVICE;
        mot::QkArgs q = *c.qk;
        q.qkv = static_cast<uint16_t *>(c.y);
        q.ld = c.ldy;
        q.T = c.T;
        q.err = hdr;
        q.after_gemm = 1;
        return mot::launch_qk_norm_rope(q, s) == hipSuccess ? MOT_OK : MOT_ERR_DEVICE;
    }
    if (c.qk != nullptr) {
        a.qk_heads = c.qk->hq + c.qk->hk;
        a.qk_hq = c.qk->hq;
        a.qw_und = c.qk->qw_und;
        a.qw_gen = c.qk->qw_gen;
        a.kw_und = c.qk->kw_und;
        a.kw_gen = c.qk->kw_gen;
        a.positions = c.qk->positions;
        a.cos_t = c.qk->cos_t;
        a.sin_t = c.qk->sin_t;
        a.n_pos = c.qk->n_pos;
        a.qk_eps = c.qk->eps;
        // the in-kernel segment list raises errors by atomic maximum in a
        // cleared word (the plan kernel writes the word itself)
        if (inline_route && mot::launch_set_word(hdr, 0, s) != hipSuccess) return MOT_ERR_DEVICE;
    }
    if (c.wtok) {
        a.ldw = c.N;
        a.tile_mode = 1;
        return mot::launch_gemm_wtok(a, inline_route, s) == hipSuccess ? MOT_OK : MOT_ERR_DEVICE;
    }
    if (mot::launch_gemm(a, swiglu, inline_route, s) != hipSuccess) return MOT_ERR_DEVICE;
    return MOT_OK;
}

// ---- allocation-free routed GEMM --------------------------------------------
//
// The scratch of mot_routed_gemm_noalloc: one routed workspace (header and
// segment list) for packs of up to MOT_NOALLOC_MAX_T rows, in device memory
// that the library holds from load to process end, one copy per GPU.  In host
// code `scratch` names a host-side stand-in, not the device address: the
// address is taken once per device with hipGetSymbolAddress (that device
// current) and only that pointer is ever passed to kernels.
static __device__ __attribute__((aligned(256))) uint8_t scratch[MOT_WS_HEADER_BYTES + 4 * (size_t)MOT_NOALLOC_MAX_T];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (nullptr on failure).
void *device_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int mot_routed_gemm_noalloc(const uint16_t *x, int64_t ldx, const uint16_t *w_und, const uint16_t *w_gen,
                            const uint8_t *modality, uint16_t *y, int64_t ldy, int64_t T, int64_t K, int64_t N,
                            const float *rstd, const uint16_t *nw_und, const uint16_t *nw_gen,
                            int32_t *error_out, unsigned flags, void *stream) {
    if (T < 0) return MOT_ERR_INVALID_ARG;
    if (T > MOT_NOALLOC_MAX_T) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (flags & MOT_FLAG_PLAN_READY) return MOT_ERR_INVALID_ARG;  // the scratch holds no caller's plan
    if (reinterpret_cast<uintptr_t>(error_out) & 3u) return MOT_ERR_MISALIGNED;
    if (error_out && y && T > 0 && overlaps(error_out, 4, y, ((T - 1) * ldy + N) * 2)) return MOT_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    void *ws = device_scratch();
    if (ws == nullptr) return MOT_ERR_DEVICE;
    RoutedCall c{x, ldx, w_und, w_gen, modality, y, ldy, T, K, N, N,
                 rstd, nw_und, nw_gen, ws, sizeof(scratch), flags};
    const int v = validate_routed(c);
    if (v != MOT_OK || T == 0) return v;
    const int st = run_routed(c, false, stream);
    if (st != MOT_OK || error_out == nullptr) return st;
    return mot::launch_copy_word(static_cast<const int32_t *>(ws), error_out, s) == hipSuccess ? MOT_OK
                                                                                              : MOT_ERR_DEVICE;
}

int mot_abi_version(void) { return MOT_ABI_VERSION; }

const char *mot_status_string(int status) {
    switch (status) {
    case MOT_OK: return "MOT_OK";
    case MOT_ERR_INVALID_ARG: return "MOT_ERR_INVALID_ARG: invalid argument";
    case MOT_ERR_UNSUPPORTED_SHAPE: return "MOT_ERR_UNSUPPORTED_SHAPE: unsupported shape";
    case MOT_ERR_MISALIGNED: return "MOT_ERR_MISALIGNED: pointer or leading dimension misaligned";
    case MOT_ERR_WORKSPACE: return "MOT_ERR_WORKSPACE: workspace missing or too small";
    case MOT_ERR_DEVICE: return "MOT_ERR_DEVICE: HIP runtime or launch failure";
    case MOT_ERR_MODALITY: return "MOT_ERR_MODALITY: modality byte not 0 or 1";
    case MOT_ERR_POSITION: return "MOT_ERR_POSITION: position outside the rotary table";
    case MOT_ERR_SEQLENS: return "MOT_ERR_SEQLENS: packed sequence lengths invalid";
    case MOT_ERR_PLAN: return "MOT_ERR_PLAN: the ready plan does not describe this pack";
    case MOT_ERR_SCHEDULE: return "MOT_ERR_SCHEDULE: a step's timesteps are outside 0 <= t_next < t <= 1 (or t not finite)";
    case MOT_ERR_INDEX_SET: return "MOT_ERR_INDEX_SET: a row is not in exactly one index set, or an index is out of range";
    default: return "unknown mot_status";
    }
}

size_t mot_workspace_bytes(int64_t T) { return ws_bytes(T); }

int mot_routing_plan(const uint8_t *modality, int64_t T, void *workspace, size_t workspace_bytes,
                     void *stream) {
    if (T < 0) return MOT_ERR_INVALID_ARG;
    if (T == 0) return MOT_OK;
    if (!modality) return MOT_ERR_INVALID_ARG;
    if (T > MOT_MAX_T) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (!workspace || workspace_bytes < ws_bytes(T)) return MOT_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1)) != 0) return MOT_ERR_MISALIGNED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    int32_t *hdr = static_cast<int32_t *>(workspace);
    int32_t *perm = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + MOT_WS_HEADER_BYTES);
    return mot::launch_plan(modality, T, hdr, perm, s) == hipSuccess ? MOT_OK : MOT_ERR_DEVICE;
}

int mot_modality_from_index_sets(const int32_t *und_idx, int64_t n_und, const int32_t *gen_idx, int64_t n_gen,
                                 uint8_t *modality, int64_t T, void *workspace, size_t workspace_bytes,
                                 void *stream) {
    if (T < 0 || n_und < 0 || n_gen < 0) return MOT_ERR_INVALID_ARG;
    if (T > MOT_MAX_T) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (n_und + n_gen != T) return MOT_ERR_INVALID_ARG;  // some row is in neither list, or in more than one
    if (T == 0) return MOT_OK;
    if (!modality || (n_und > 0 && !und_idx) || (n_gen > 0 && !gen_idx)) return MOT_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(und_idx) & 3u) || (reinterpret_cast<uintptr_t>(gen_idx) & 3u))
        return MOT_ERR_MISALIGNED;
    if (!workspace || workspace_bytes < ws_bytes(T)) return MOT_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1)) != 0) return MOT_ERR_MISALIGNED;
    const int64_t wsb = (int64_t)ws_bytes(T);
    if (overlaps(modality, T, workspace, wsb) || (n_und > 0 && overlaps(modality, T, und_idx, 4 * n_und)) ||
        (n_gen > 0 && overlaps(modality, T, gen_idx, 4 * n_gen)) ||
        (n_und > 0 && overlaps(workspace, wsb, und_idx, 4 * n_und)) ||
        (n_gen > 0 && overlaps(workspace, wsb, gen_idx, 4 * n_gen)))
        return MOT_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    int32_t *err = static_cast<int32_t *>(workspace);
    uint32_t *cnt = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + MOT_WS_HEADER_BYTES);
    return mot::launch_index_sets(und_idx, n_und, gen_idx, n_gen, modality, T, err, cnt, s) == hipSuccess
               ? MOT_OK
               : MOT_ERR_DEVICE;
}

int mot_routed_gemm(const uint16_t *x, int64_t ldx, const uint16_t *w_und, const uint16_t *w_gen,
                    const uint8_t *modality, uint16_t *y, int64_t ldy, int64_t T, int64_t K,
                    int64_t N, const float *rstd, const uint16_t *nw_und, const uint16_t *nw_gen,
                    void *workspace, size_t workspace_bytes, unsigned flags, void *stream) {
    RoutedCall c{x, ldx, w_und, w_gen, modality, y, ldy, T, K, N, N,
                 rstd, nw_und, nw_gen, workspace, workspace_bytes, flags};
    return run_routed(c, false, stream);
}

int mot_routed_gemm_qk_norm_rope(const uint16_t *x, int64_t ldx, const uint16_t *w_und, const uint16_t *w_gen,
                                 const uint8_t *modality, uint16_t *y, int64_t ldy, int64_t T, int64_t K, int64_t N,
                                 int64_t n_q_heads, int64_t n_k_heads, const uint16_t *qw_und, const uint16_t *qw_gen,
                                 const uint16_t *kw_und, const uint16_t *kw_gen, const int32_t *positions,
                                 const uint16_t *cos_table, const uint16_t *sin_table, int64_t n_pos, float eps,
                                 void *workspace, size_t workspace_bytes, unsigned flags, void *stream) {
    if (n_q_heads < 0 || n_k_heads < 0 || n_q_heads + n_k_heads == 0) return MOT_ERR_INVALID_ARG;
    if (!(eps > 0.0f) || !isfinite(eps)) return MOT_ERR_INVALID_ARG;
    if (flags & MOT_FLAG_PLAN_READY) return MOT_ERR_INVALID_ARG;  // the call raises errors in its own plan's word
    RoutedCall c{x, ldx, w_und, w_gen, modality, y, ldy, T, K, N, N,
                 nullptr, nullptr, nullptr, workspace, workspace_bytes, flags};
    const int v = validate_routed(c);
    if (v != MOT_OK || T == 0) return v;
    if (128 * (n_q_heads + n_k_heads) > N) return MOT_ERR_INVALID_ARG;
    if (!qw_und || !qw_gen || !kw_und || !kw_gen || !positions || !cos_table || !sin_table || n_pos <= 0)
        return MOT_ERR_INVALID_ARG;
    if (n_pos > MOT_MAX_T) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(qw_und) || !aligned16(qw_gen) || !aligned16(kw_und) || !aligned16(kw_gen) || !aligned16(positions) ||
        !aligned16(cos_table) || !aligned16(sin_table))
        return MOT_ERR_MISALIGNED;
    const int64_t y_bytes = ((T - 1) * ldy + N) * 2;
    const void *ins[] = {qw_und, qw_gen, kw_und, kw_gen, positions, cos_table, sin_table};
    const int64_t in_bytes[] = {256, 256, 256, 256, 4 * T, 128 * n_pos, 128 * n_pos};
    for (int i = 0; i < 7; ++i)
        if (overlaps(y, y_bytes, ins[i], in_bytes[i])) return MOT_ERR_INVALID_ARG;
    mot::QkArgs q;
    q.hq = (int)n_q_heads;
    q.hk = (int)n_k_heads;
    q.modality = modality;
    q.qw_und = qw_und;
    q.qw_gen = qw_gen;
    q.kw_und = kw_und;
    q.kw_gen = kw_gen;
    q.positions = positions;
    q.cos_t = cos_table;
    q.sin_t = sin_table;
    q.n_pos = (int)n_pos;
    q.eps = eps;
    c.qk = &q;
    return run_routed(c, false, stream);
}

int mot_routed_gemm_f32(const uint16_t *x, int64_t ldx, const uint16_t *w_und, const uint16_t *w_gen,
                        const uint8_t *modality, float *y, int64_t ldy, int64_t T, int64_t K, int64_t N,
                        void *workspace, size_t workspace_bytes, unsigned flags, void *stream) {
    RoutedCall c{x, ldx, w_und, w_gen, modality, y, ldy, T, K, N, N,
                 nullptr, nullptr, nullptr, workspace, workspace_bytes, flags, 1};
    return run_routed(c, false, stream);
}

int mot_routed_gemm_swiglu(const uint16_t *x, int64_t ldx, const uint16_t *wgu_und,
                           const uint16_t *wgu_gen, const uint8_t *modality, uint16_t *act,
                           int64_t ldact, int64_t T, int64_t K, int64_t F, const float *rstd,
                           const uint16_t *nw_und, const uint16_t *nw_gen, void *workspace,
                           size_t workspace_bytes, unsigned flags, void *stream) {
    RoutedCall c{x, ldx, wgu_und, wgu_gen, modality, act, ldact, T, K, F, 2 * F,
                 rstd, nw_und, nw_gen, workspace, workspace_bytes, flags};
    return run_routed(c, true, stream);
}

int mot_fused_add_rmsnorm(const uint16_t *x, uint16_t *residual, const uint16_t *w_und,
                          const uint16_t *w_gen, const uint8_t *modality, float eps,
                          uint16_t *out, float *rstd_out, int64_t T, int64_t H, void *workspace,
                          void *stream) {
    if (T < 0 || H < 0) return MOT_ERR_INVALID_ARG;
    if (!(eps > 0.0f) || !isfinite(eps)) return MOT_ERR_INVALID_ARG;
    if (T == 0) return MOT_OK;
    if (!x || !w_und || !w_gen || !modality) return MOT_ERR_INVALID_ARG;
    if (!out && !rstd_out) return MOT_ERR_INVALID_ARG;
    if (T > MOT_MAX_T) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (H == 0 || H % 64 || H > 16384) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (!aligned16(x) || !aligned16(w_und) || !aligned16(w_gen) ||
        (residual && !aligned16(residual)) || (out && !aligned16(out)) ||
        (rstd_out && (reinterpret_cast<uintptr_t>(rstd_out) & 3u)) ||
        (workspace && (reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1))))
        return MOT_ERR_MISALIGNED;
    const int64_t bytes = T * H * 2;
    if (out && (overlaps(out, bytes, x, bytes) || (residual && overlaps(out, bytes, residual, bytes))))
        return MOT_ERR_INVALID_ARG;
    if (residual && overlaps(residual, bytes, x, bytes)) return MOT_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    int32_t *err = workspace ? static_cast<int32_t *>(workspace) : nullptr;
    return mot::launch_norm(x, residual, w_und, w_gen, modality, eps, out, rstd_out, T, (int)H, err,
                            s) == hipSuccess
               ? MOT_OK
               : MOT_ERR_DEVICE;
}

int mot_transpose_bf16(const uint16_t *in, int64_t ld_in, int64_t rows, int64_t cols,
                       const uint8_t *modality, int keep, uint16_t *out, int64_t ld_out,
                       int64_t rows_pad, void *stream) {
    if (rows < 0 || cols < 0 || rows_pad < rows) return MOT_ERR_INVALID_ARG;
    if (rows_pad == 0 || cols == 0) return MOT_OK;
    if (!in && rows > 0) return MOT_ERR_INVALID_ARG;
    if (!out || (modality && keep != 0 && keep != 1)) return MOT_ERR_INVALID_ARG;
    if (rows_pad > MOT_MAX_T || cols > MOT_MAX_DIM) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (ld_in < cols || ld_out < rows_pad) return MOT_ERR_INVALID_ARG;
    if (ld_in % 8 || ld_out % 8) return MOT_ERR_MISALIGNED;
    if ((in && !aligned16(in)) || !aligned16(out)) return MOT_ERR_MISALIGNED;
    const int64_t in_bytes = rows > 0 ? ((rows - 1) * ld_in + cols) * 2 : 0;
    const int64_t out_bytes = ((cols - 1) * ld_out + rows_pad) * 2;
    if (in && overlaps(in, in_bytes, out, out_bytes)) return MOT_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    return mot::launch_transpose(in, ld_in, rows, cols, modality, keep, out, ld_out, rows_pad, s) == hipSuccess
               ? MOT_OK
               : MOT_ERR_DEVICE;
}

int mot_routed_gemm_dx(const uint16_t *dy, int64_t lddy, const uint16_t *w_und, const uint16_t *w_gen,
                       const uint8_t *modality, uint16_t *dx, int64_t lddx, int64_t T, int64_t N, int64_t K,
                       void *workspace, size_t workspace_bytes, unsigned flags, void *stream) {
    if ((flags & ~MOT_FLAG_PLAN_READY) != 0) return MOT_ERR_INVALID_ARG;
    // the routed GEMM's contract with the contraction over N and K output
    // columns; the weights [N][K] are the same bytes as its [K][N] operand's
    // transpose
    RoutedCall c{dy, lddy, w_und, w_gen, modality, dx, lddx, T, N, K, K,
                 nullptr, nullptr, nullptr, workspace, workspace_bytes, flags};
    c.wtok = 1;
    const int v = validate_routed(c);
    if (v != MOT_OK || T == 0) return v;
    // the last 256-column tile reads up to 256 columns past K in W's rows
    if ((N * K + 256) * 2 >= (int64_t(1) << 32)) return MOT_ERR_UNSUPPORTED_SHAPE;
    return run_routed(c, false, stream);
}

int mot_grad_w(const uint16_t *dy, int64_t lddy, const uint16_t *x, int64_t ldx, const uint8_t *modality,
               int keep, int64_t T, int64_t N, int64_t K, void *out, int64_t ldo, int out_f32, void *stream) {
    if (T < 0 || N < 0 || K < 0 || (keep != 0 && keep != 1) || (out_f32 != 0 && out_f32 != 1))
        return MOT_ERR_INVALID_ARG;
    if (N == 0 || K == 0) return MOT_OK;
    if (!out || (T > 0 && (!dy || !x || !modality))) return MOT_ERR_INVALID_ARG;
    if (T > MOT_MAX_T || N > MOT_MAX_T || K % 64 || K > MOT_MAX_DIM) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (lddy < N || ldx < K || ldo < K) return MOT_ERR_INVALID_ARG;
    if (lddy % 8 || ldx % 8 || ldo % 8) return MOT_ERR_MISALIGNED;
    if (!aligned16(dy) || !aligned16(x) || !aligned16(out)) return MOT_ERR_MISALIGNED;
    const int64_t esz = out_f32 ? 4 : 2;
    if (T == 0) dy = x = nullptr, modality = nullptr;  // nothing is read
    const int64_t dy_bytes = T > 0 ? ((T - 1) * lddy + N) * 2 : 0;
    const int64_t x_bytes = T > 0 ? ((T - 1) * ldx + K) * 2 : 0;
    const int64_t o_bytes = ((N - 1) * ldo + K) * esz;
    // byte offsets the kernel forms: token rows up to T rounded up to 64,
    // columns up to the last 256-column tile's end (and an out-of-range
    // sentinel just below 2^32 for the rows it drops)
    const int64_t tp = round_up(T > 0 ? T : 1, 64);
    const int64_t lim = (int64_t(1) << 32) - 256;
    if ((tp * lddy + round_up(N, 256)) * 2 >= lim || (tp * ldx + round_up(K, 256)) * 2 >= lim ||
        o_bytes >= (int64_t(1) << 32))
        return MOT_ERR_UNSUPPORTED_SHAPE;
    if (overlaps(out, o_bytes, dy, dy_bytes) || overlaps(out, o_bytes, x, x_bytes) ||
        overlaps(out, o_bytes, modality, T))
        return MOT_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    mot::GemmArgs a;
    a.x = dy;
    a.ldx = lddy;
    a.w_und = x;
    a.w_gen = x;
    a.ldw = ldx;
    a.y = out;
    a.ldy = ldo;
    a.modality = modality;
    a.keep = keep;
    a.t_tok = (int)T;
    a.T = N;
    a.K = (int)tp;
    a.N = (int)K;
    a.wrows = (int)K;
    a.x_bytes = (uint32_t)dy_bytes;
    a.w_bytes = (uint32_t)x_bytes;
    a.y_bytes = (uint32_t)o_bytes;
    a.out_f32 = out_f32;
    return mot::launch_grad_w(a, s) == hipSuccess ? MOT_OK : MOT_ERR_DEVICE;
}

size_t mot_attention_workspace_bytes(int64_t Tk, int64_t n_kv_heads) {
    return attn_ws_bytes(Tk, n_kv_heads);
}

int mot_joint_attention(const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk, const uint16_t *v,
                        int64_t ldv, uint16_t *out, int64_t ldo, int64_t Tq, int64_t Tk, int64_t n_q_heads,
                        int64_t n_kv_heads, int64_t head_dim, int causal, void *workspace,
                        size_t workspace_bytes, void *stream) {
    if (Tq < 0 || Tk < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads)
        return MOT_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return MOT_ERR_INVALID_ARG;
    if (Tq == 0) return MOT_OK;
    if (head_dim != kAttnHeadDim || n_q_heads > kAttnMaxHeads) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (Tq > MOT_MAX_T || Tk > MOT_MAX_T) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (!q || !out || (Tk > 0 && (!k || !v))) return MOT_ERR_INVALID_ARG;
    const int64_t qw = n_q_heads * kAttnHeadDim, kw = n_kv_heads * kAttnHeadDim;
    if (ldq < qw || ldo < qw || (Tk > 0 && (ldk < kw || ldv < kw))) return MOT_ERR_INVALID_ARG;
    if (ldq % 8 || ldo % 8 || (Tk > 0 && (ldk % 8 || ldv % 8))) return MOT_ERR_MISALIGNED;
    if (!aligned16(q) || !aligned16(out) || (Tk > 0 && (!aligned16(k) || !aligned16(v))))
        return MOT_ERR_MISALIGNED;
    (void)workspace;
    (void)workspace_bytes;
    const int64_t q_bytes = ((Tq - 1) * ldq + qw) * 2, o_bytes = ((Tq - 1) * ldo + qw) * 2;
    if (overlaps(out, o_bytes, q, q_bytes)) return MOT_ERR_INVALID_ARG;
    if (Tk > 0) {
        const int64_t k_bytes = ((Tk - 1) * ldk + kw) * 2, v_bytes = ((Tk - 1) * ldv + kw) * 2;
        // the kernel addresses K and V (up to their last key block's end)
        // with 32-bit byte offsets
        if ((round_up(Tk, 64) * ldk + kw) * 2 >= (int64_t(1) << 32) ||
            (round_up(Tk, 64) * ldv + kw) * 2 >= (int64_t(1) << 32))
            return MOT_ERR_UNSUPPORTED_SHAPE;
        if (overlaps(out, o_bytes, k, k_bytes) || overlaps(out, o_bytes, v, v_bytes)) return MOT_ERR_INVALID_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    mot::AttnArgs a;
    a.q = q;
    a.ldq = ldq;
    a.k = k;
    a.ldk = ldk;
    a.v = v;
    a.ldv = ldv;
    a.out = out;
    a.ldo = ldo;
    a.Tq = Tq;
    a.Tk = Tk;
    a.hq = (int)n_q_heads;
    a.hkv = (int)n_kv_heads;
    a.causal = causal;
    a.scale_log2e = (float)(1.4426950408889634074 / sqrt((double)kAttnHeadDim));
    return mot::launch_attention(a, s) == hipSuccess ? MOT_OK : MOT_ERR_DEVICE;
}

size_t mot_attention_varlen_workspace_bytes(int64_t Tk, int64_t n_seqs, int64_t n_kv_heads) {
    return attn_varlen_ws_bytes(Tk, n_seqs, n_kv_heads);
}

int mot_joint_attention_varlen(const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk, const uint16_t *v,
                               int64_t ldv, uint16_t *out, int64_t ldo, const int32_t *cu_q, const int32_t *cu_k,
                               int64_t n_seqs, int64_t Tq, int64_t Tk, int64_t max_q, int64_t n_q_heads,
                               int64_t n_kv_heads, int64_t head_dim, int causal, void *workspace,
                               size_t workspace_bytes, void *stream) {
    if (Tq < 0 || Tk < 0 || n_seqs < 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads)
        return MOT_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return MOT_ERR_INVALID_ARG;
    if (Tq == 0) return MOT_OK;
    if (n_seqs == 0 || max_q < 1) return MOT_ERR_INVALID_ARG;
    if (head_dim != kAttnHeadDim || n_q_heads > kAttnMaxHeads) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (Tq > MOT_MAX_T || Tk > MOT_MAX_T || max_q > MOT_MAX_T || n_seqs > 65536) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (n_seqs * n_q_heads * ((max_q + 127) / 128) >= (int64_t(1) << 31)) return MOT_ERR_UNSUPPORTED_SHAPE;
    if (!q || !out || !cu_q || !cu_k || (Tk > 0 && (!k || !v))) return MOT_ERR_INVALID_ARG;
    const int64_t qw = n_q_heads * kAttnHeadDim, kw = n_kv_heads * kAttnHeadDim;
    if (ldq < qw || ldo < qw || (Tk > 0 && (ldk < kw || ldv < kw))) return MOT_ERR_INVALID_ARG;
    if (ldq % 8 || ldo % 8 || (Tk > 0 && (ldk % 8 || ldv % 8))) return MOT_ERR_MISALIGNED;
    if (!aligned16(q) || !aligned16(out) || (Tk > 0 && (!aligned16(k) || !aligned16(v))) ||
        (reinterpret_cast<uintptr_t>(cu_q) & 3u) || (reinterpret_cast<uintptr_t>(cu_k) & 3u))
        return MOT_ERR_MISALIGNED;
    const size_t wsb = attn_varlen_ws_bytes(Tk, n_seqs, n_kv_heads);
    if (!workspace || workspace_bytes < wsb) return MOT_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & (kWsAlign - 1)) != 0) return MOT_ERR_MISALIGNED;
    const int64_t q_bytes = ((Tq - 1) * ldq + qw) * 2, o_bytes = ((Tq - 1) * ldo + qw) * 2;
    if (overlaps(out, o_bytes, q, q_bytes) || overlaps(out, o_bytes, workspace, (int64_t)wsb) ||
        overlaps(workspace, (int64_t)wsb, q, q_bytes))
        return MOT_ERR_INVALID_ARG;
    if (Tk > 0) {
        const int64_t k_bytes = ((Tk - 1) * ldk + kw) * 2, v_bytes = ((Tk - 1) * ldv + kw) * 2;
        if ((round_up(Tk, 64) * ldk + kw) * 2 >= (int64_t(1) << 32) ||
            (round_up(Tk, 64) * ldv + kw) * 2 >= (int64_t(1) << 32))
            return MOT_ERR_UNSUPPORTED_SHAPE;
        if (overlaps(out, o_bytes, k, k_bytes) || overlaps(out, o_bytes, v, v_bytes) ||
            overlaps(workspace, (int64_t)wsb, k, k_bytes) || overlaps(workspace, (int64_t)wsb, v, v_bytes))
            return MOT_ERR_INVALID_ARG;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    int32_t *err = static_cast<int32_t *>(workspace);
    if (mot::launch_seqlens_check(cu_q, cu_k, (int)n_seqs, Tq, Tk, max_q, err, s) != hipSuccess)
        return MOT_ERR_DEVICE;
    mot::AttnArgs a;
    a.q = q;
    a.ldq = ldq;
    a.k = k;
    a.ldk = ldk;
    a.v = v;
    a.ldv = ldv;
    a.out = out;
    a.ldo = ldo;
    a.Tq = Tq;
    a.Tk = Tk;
    a.hq = (int)n_q_heads;
    a.hkv = (int)n_kv_heads;
    a.causal = causal;
    a.scale_log2e = (float)(1.4426950408889634074 / sqrt((double)kAttnHeadDim));
    a.cu_q = cu_q;
    a.cu_k = cu_k;
    a.nseq = (int)n_seqs;
    a.nqb = (int)((max_q + 127) / 128);
    a.err = err;
    return mot::launch_attention(a, s) == hipSuccess ? MOT_OK : MOT_ERR_DEVICE;
}

int mot_qk_norm_rope(uint16_t *qkv, int64_t ld, int64_t T, int64_t n_q_heads, int64_t n_k_heads,
                     const uint8_t *modality, const uint16_t *qw_und, const uint16_t *qw_gen,
                     const uint16_t *kw_und, const uint16_t *kw_gen, const int32_t *positions,
                     const uint16_t *cos_table, const uint16_t *sin_table, int64_t n_pos, float eps,
                     void *workspace, size_t workspace_bytes, void *stream) {
    if (T < 0 || n_q_heads < 0 || n_k_heads < 0) return MOT_ERR_INVALID_ARG;
    if (!(eps > 0.0f) || !isfinite(eps)) return MOT_ERR_INVALID_ARG;
    if (T == 0) return MOT_OK;
    if (!qkv || !modality || !qw_und || !qw_gen || !kw_und || !kw_gen || !positions || !cos_table ||
        !sin_table)
        return MOT_ERR_INVALID_ARG;
    if (n_q_heads + n_k_heads == 0 || n_pos <= 0) return MOT_ERR_INVALID_ARG;
    if (T > MOT_MAX_T || n_pos > MOT_MAX_T || 128 * (n_q_heads + n_k_heads) > MOT_MAX_DIM)
        return MOT_ERR_UNSUPPORTED_SHAPE;
    const int64_t cols = 128 * (n_q_heads + n_k_heads);
    if (ld < cols) return MOT_ERR_INVALID_ARG;
    if (ld % 8) return MOT_ERR_MISALIGNED;
    if (!aligned16(qkv) || !aligned16(qw_und) || !aligned16(qw_gen) || !aligned16(kw_und) ||
        !aligned16(kw_gen) || !aligned16(positions) || !aligned16(cos_table) || !aligned16(sin_table))
        return MOT_ERR_MISALIGNED;
    if (!workspace || workspace_bytes < MOT_WS_HEADER_BYTES) return MOT_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOT_ERR_MISALIGNED;
    // the rows are rewritten in place: no input may overlap them
    const int64_t qkv_bytes = ((T - 1) * ld + cols) * 2;
    const void *ins[] = {modality, qw_und, qw_gen, kw_und, kw_gen, positions, cos_table, sin_table, workspace};
    const int64_t in_bytes[] = {T, 256, 256, 256, 256, 4 * T, 128 * n_pos, 128 * n_pos, 16};
    for (int i = 0; i < 9; ++i)
        if (overlaps(qkv, qkv_bytes, ins[i], in_bytes[i])) return MOT_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    mot::QkArgs a;
    a.qkv = qkv;
    a.ld = ld;
    a.T = T;
    a.hq = (int)n_q_heads;
    a.hk = (int)n_k_heads;
    a.modality = modality;
    a.qw_und = qw_und;
    a.qw_gen = qw_gen;
    a.kw_und = kw_und;
    a.kw_gen = kw_gen;
    a.positions = positions;
    a.cos_t = cos_table;
    a.sin_t = sin_table;
    a.n_pos = (int)n_pos;
    a.eps = eps;
    a.err = static_cast<int32_t *>(workspace);
    return mot::launch_qk_norm_rope(a, s) == hipSuccess ? MOT_OK : MOT_ERR_DEVICE;
}

size_t mot_latent_workspace_bytes(int64_t n_req, int64_t max_rows) { return latent_ws_bytes(n_req, max_rows); }

int mot_cfg_combine_renorm(const float *v_cond, const float *v_text_uncond, const float *v_img_uncond, float *out,
                           const int32_t *cu_rows, int64_t n_req, int64_t rows, int64_t C, int64_t max_rows,
                           const float *t, float s_text, float s_img, float t_lo, float t_hi, float renorm_min,
                           int renorm_type, void *workspace, size_t workspace_bytes, void *stream) {
    if (n_req == 0 && rows == 0 && C > 0) return MOT_OK;
    const int v = validate_latent(n_req, rows, C, max_rows, cu_rows, workspace, workspace_bytes);
    if (v != MOT_OK) return v;
    if (n_req == 0) return MOT_ERR_INVALID_ARG;  // rows without requests
    // (with no rows the row arrays are not read and may be NULL)
    if ((rows > 0 && (!v_cond || !v_text_uncond || !out)) || !t) return MOT_ERR_INVALID_ARG;
    if (renorm_type < 0 || renorm_type > 2) return MOT_ERR_INVALID_ARG;
    if (!isfinite(s_text) || !isfinite(s_img) || !isfinite(t_lo) || !isfinite(t_hi) ||
        !(renorm_min >= 0.0f && renorm_min <= 1.0f))
        return MOT_ERR_INVALID_ARG;
    if (!aligned16(v_cond) || !aligned16(v_text_uncond) || (v_img_uncond && !aligned16(v_img_uncond)) ||
        !aligned16(out) || (reinterpret_cast<uintptr_t>(t) & 3u))
        return MOT_ERR_MISALIGNED;
    const int64_t bytes = rows * C * 4;
    const int64_t wsb = (int64_t)latent_ws_bytes(n_req, max_rows);
    const void *ins[] = {v_cond, v_text_uncond, v_img_uncond, cu_rows, t, workspace};
    const int64_t in_bytes[] = {bytes, bytes, bytes, 4 * (n_req + 1), 4 * n_req, wsb};
    for (int i = 0; i < 6; ++i)
        if (ins[i] && overlaps(out, bytes, ins[i], in_bytes[i])) return MOT_ERR_INVALID_ARG;
    for (int i = 0; i < 5; ++i)
        if (ins[i] && overlaps(workspace, wsb, ins[i], in_bytes[i])) return MOT_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    int32_t *err = static_cast<int32_t *>(workspace);
    float *part = reinterpret_cast<float *>(static_cast<char *>(workspace) + MOT_WS_HEADER_BYTES);
    return mot::launch_cfg_combine(v_cond, v_text_uncond, v_img_uncond, out, cu_rows, (int)n_req, rows, (int)C,
                                   max_rows, t, s_text, s_img, t_lo, t_hi, renorm_min, renorm_type, err, part,
                                   s) == hipSuccess
               ? MOT_OK
               : MOT_ERR_DEVICE;
}

int mot_flow_sde_step_logp(const float *x, const float *v, const float *noise, const float *x_next_in,
                           float *x_next_out, float *logp, const int32_t *cu_rows, int64_t n_req, int64_t rows,
                           int64_t C, int64_t max_rows, const float *t_cur, const float *t_next, float eta,
                           void *workspace, size_t workspace_bytes, void *stream) {
    if (n_req == 0 && rows == 0 && C > 0) return MOT_OK;
    const int vs = validate_latent(n_req, rows, C, max_rows, cu_rows, workspace, workspace_bytes);
    if (vs != MOT_OK) return vs;
    if (n_req == 0) return MOT_ERR_INVALID_ARG;
    // (with no rows the row arrays are not read and may be NULL: every
    // request is empty and its log-probability is 0)
    if ((rows > 0 && (!x || !v)) || !logp || !t_cur || !t_next) return MOT_ERR_INVALID_ARG;
    const bool sample = noise != nullptr;
    if (rows > 0 && (sample ? (!x_next_out || x_next_in) : (!x_next_in || x_next_out))) return MOT_ERR_INVALID_ARG;
    if (!(eta > 0.0f) || !isfinite(eta)) return MOT_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(v) || (noise && !aligned16(noise)) || (x_next_in && !aligned16(x_next_in)) ||
        (x_next_out && !aligned16(x_next_out)) || (reinterpret_cast<uintptr_t>(logp) & 3u) ||
        (reinterpret_cast<uintptr_t>(t_cur) & 3u) || (reinterpret_cast<uintptr_t>(t_next) & 3u))
        return MOT_ERR_MISALIGNED;
    const int64_t bytes = rows * C * 4;
    const int64_t wsb = (int64_t)latent_ws_bytes(n_req, max_rows);
    const void *ins[] = {x, v, noise, x_next_in, cu_rows, t_cur, t_next, workspace};
    const int64_t in_bytes[] = {bytes, bytes, bytes, bytes, 4 * (n_req + 1), 4 * n_req, 4 * n_req, wsb};
    for (int i = 0; i < 8; ++i) {
        if (!ins[i]) continue;
        if (x_next_out && overlaps(x_next_out, bytes, ins[i], in_bytes[i])) return MOT_ERR_INVALID_ARG;
        if (overlaps(logp, 4 * n_req, ins[i], in_bytes[i])) return MOT_ERR_INVALID_ARG;
        if (i < 7 && overlaps(workspace, wsb, ins[i], in_bytes[i])) return MOT_ERR_INVALID_ARG;
    }
    if (x_next_out && overlaps(x_next_out, bytes, logp, 4 * n_req)) return MOT_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    int32_t *err = static_cast<int32_t *>(workspace);
    float *part = reinterpret_cast<float *>(static_cast<char *>(workspace) + MOT_WS_HEADER_BYTES);
    return mot::launch_sde_step(x, v, noise, x_next_in, x_next_out, logp, cu_rows, (int)n_req, rows, (int)C, max_rows,
                                t_cur, t_next, eta, err, part, s) == hipSuccess
               ? MOT_OK
               : MOT_ERR_DEVICE;
}

int mot_read_device_error(const void *workspace, void *stream) {
    if (!workspace) return MOT_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    DeviceGuard guard(s);
    if (!guard.ok()) return MOT_ERR_DEVICE;
    int32_t host = 0;
    if (hipMemcpyAsync(&host, workspace, sizeof host, hipMemcpyDeviceToHost, s) != hipSuccess)
        return MOT_ERR_DEVICE;
    if (hipStreamSynchronize(s) != hipSuccess) return MOT_ERR_DEVICE;
    return host == 0 ? MOT_OK : host;
}

}  // extern "C"
