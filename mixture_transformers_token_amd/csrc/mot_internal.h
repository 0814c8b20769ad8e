// Internal interface between the C-ABI layer (mot_api.cpp) and the HIP
// kernels (mot_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mot {

// Largest K the routed-RMSNorm prologue supports (its norm weights are
// staged in LDS).
constexpr int kMaxPrologueK = 8192;

// Packs of at most this many rows build their segment list inside the GEMM
// kernel (every workgroup scans the modality bytes); larger packs run the
// plan kernel first.
constexpr int64_t kInlineRouteMaxT = 8192;

// Packs of at most this many rows (without the norm prologue, with the
// library's own tile choice) take the weight-bound small-pack kernel.
constexpr int64_t kSkinnyMaxT = 128;

// Arguments of one routed GEMM launch.  Sizes are validated by the caller.
struct GemmArgs {
    const uint16_t *x;
    int64_t ldx;
    const uint16_t *w_und;
    const uint16_t *w_gen;
    void *y;              // bf16 output, or fp32 when out_f32
    int64_t ldy;
    const uint8_t *modality;  // [T]; read by the in-kernel segment list
    const int32_t *hdr;   // workspace header: error, n_und, n_gen, T
    const int32_t *perm;  // workspace segment list
    int32_t *hdr_out;     // same header and list, written by the in-kernel segment list
    int32_t *perm_out;
    const float *rstd;    // prologue (nullptr: none)
    const uint16_t *nw_und;
    const uint16_t *nw_gen;
    int64_t T;
    int K;
    int N;                // output columns (F for SwiGLU)
    int wrows;            // weight rows per set (N, or 2F for SwiGLU)
    int tile_mode;        // 0: big tiles for whole rounds, small for the rest;
                          // 1: big (256x256) tiles only; 2: small (128x128) only
    uint32_t x_bytes;     // extent of x from its base (bytes, < 4 GiB)
    uint32_t w_bytes;     // extent of one weight matrix (bytes, < 4 GiB)
    uint32_t y_bytes;     // extent of y from its base (bytes, < 4 GiB)
    int out_f32;          // 1: y is fp32 (plain GEMM, 256 x 256 tiles only)
    // Fused per-head QK RMSNorm + rotary epilogue (the QKV projection's
    // mot_qk_norm_rope step inside the GEMM; qk_heads == 0: none).  Heads are
    // 128 output columns from column 0: qk_hq q heads, then k heads, up to
    // qk_heads; later columns (v) are stored plain.  Position errors raise
    // MOT_ERR_POSITION in hdr_out[0] by atomic maximum.
    int qk_heads = 0;
    int qk_hq = 0;
    const uint16_t *qw_und = nullptr, *qw_gen = nullptr, *kw_und = nullptr, *kw_gen = nullptr;
    const int32_t *positions = nullptr;
    const uint16_t *cos_t = nullptr, *sin_t = nullptr;  // [n_pos][64] bf16
    int n_pos = 0;
    float qk_eps = 0.0f;
    // Weight gradient (launch_grad_w): token-major operands, x = dY [t_tok][ldx]
    // and the weight side X [t_tok][ldw]; X rows whose modality byte is not
    // keep count as zeros; K = t_tok rounded up to 64.
    int64_t ldw = 0;
    int keep = 1;
    int t_tok = 0;
};

// Routed per-head QK RMSNorm + rotary embedding, in place on QKV rows.
struct QkArgs {
    uint16_t *qkv;        // [T][ld] bf16: q heads, then k heads, 128 columns each
    int64_t ld;
    int64_t T;
    int hq, hk;           // q and k heads
    const uint8_t *modality;
    const uint16_t *qw_und, *qw_gen, *kw_und, *kw_gen;  // [128] bf16 norm weights
    const int32_t *positions;                           // [T]
    const uint16_t *cos_t, *sin_t;                      // [n_pos][64] bf16
    int n_pos;
    float eps;
    int32_t *err;         // error word (cleared by the launch, unless after_gemm)
    int after_gemm = 0;   // 1: runs after the routed GEMM that wrote these rows: the word
                          // holds the GEMM's result; if set, nothing is done
};

// Shared joint attention, head dimension 128 (mot_attention.hip).
struct AttnArgs {
    const uint16_t *q;    // [Tq][ldq] bf16: q heads of 128 columns
    int64_t ldq;
    const uint16_t *k;    // [Tk][ldk] bf16: kv heads of 128 columns
    int64_t ldk;
    const uint16_t *v;    // [Tk][ldv] bf16: kv heads of 128 columns
    int64_t ldv;
    uint16_t *out;        // [Tq][ldo] bf16
    int64_t ldo;
    int64_t Tq, Tk;
    int hq, hkv;          // hq % hkv == 0
    int causal;           // 1: query i sees keys j <= i + (Tk - Tq)
    float scale_log2e;    // fp32 rounding of log2(e)/sqrt(128)
    // packed sequences (cu_q == nullptr: one sequence of Tq rows, Tk keys)
    const int32_t *cu_q = nullptr, *cu_k = nullptr;  // [nseq + 1] cumulative rows / keys
    int nseq = 0;
    int nqb = 0;                   // query blocks of 128 per sequence (longest)
    const int32_t *err = nullptr;  // lengths check result; the kernel exits if non-zero
};

// dW[n][k] = sum over token rows t with modality[t] == keep of dY[t][n] X[t][k]
// (GemmArgs: x = dY, w_und = X, y = dW, T = rows n, K = tokens rounded up to
// 64, N = wrows = columns k; out_f32 as for the GEMM).
hipError_t launch_grad_w(const GemmArgs &a, hipStream_t stream);

// Routed GEMM whose weights are contraction-major (W [K][ldw], the x side
// [T][ldx] as usual): dX = dY W with the forward's [N][K] weights read as they
// lie.  Big tiles only (a.tile_mode must be 1).
hipError_t launch_gemm_wtok(const GemmArgs &a, bool inline_route, hipStream_t stream);

hipError_t launch_attention(const AttnArgs &a, hipStream_t stream);
hipError_t launch_seqlens_check(const int32_t *cu_q, const int32_t *cu_k, int n, int64_t Tq, int64_t Tk,
                                int64_t max_q, int32_t *err, hipStream_t stream);

// Latent step (mot_latent.hip): chunk slots of one request, and the launches.
int latent_chunks(int64_t max_rows);
hipError_t launch_cfg_combine(const float *vc, const float *vt, const float *vi, float *out, const int32_t *cu,
                              int n, int64_t rows, int C, int64_t max_rows, const float *t, float s_text, float s_img,
                              float t_lo, float t_hi, float rmin, int type, int32_t *err, float *part,
                              hipStream_t stream);
hipError_t launch_sde_step(const float *x, const float *v, const float *noise, const float *xn_in, float *xn_out,
                           float *logp, const int32_t *cu, int n, int64_t rows, int C, int64_t max_rows,
                           const float *t_cur, const float *t_next, float eta, int32_t *err, float *part,
                           hipStream_t stream);

hipError_t launch_plan(const uint8_t *modality, int64_t T, int32_t *hdr, int32_t *perm,
                       hipStream_t stream);
// Modality bytes from the und / gen index lists; cnt: T words of scratch.
hipError_t launch_index_sets(const int32_t *und_idx, int64_t n_und, const int32_t *gen_idx, int64_t n_gen,
                             uint8_t *modality, int64_t T, int32_t *err, uint32_t *cnt, hipStream_t stream);
// Launches the persistent routed GEMM (one workgroup per CU at most).  With
// inline_route the kernel builds (and publishes) the segment list itself.
hipError_t launch_gemm(const GemmArgs &a, bool swiglu, bool inline_route, hipStream_t stream);
hipError_t launch_qk_norm_rope(const QkArgs &a, hipStream_t stream);
// *dst = v on the device (one thread), in stream order.
hipError_t launch_set_word(int32_t *dst, int32_t v, hipStream_t stream);
// *dst = *src on the device (one thread), in stream order.
hipError_t launch_copy_word(const int32_t *src, int32_t *dst, hipStream_t stream);
hipError_t launch_transpose(const uint16_t *in, int64_t ld_in, int64_t rows, int64_t cols,
                            const uint8_t *modality, int keep, uint16_t *out, int64_t ld_out,
                            int64_t rows_pad, hipStream_t stream);
hipError_t launch_norm(const uint16_t *x, uint16_t *residual, const uint16_t *w_und,
                       const uint16_t *w_gen, const uint8_t *modality, float eps,
                       uint16_t *out, float *rstd_out, int64_t T, int H, int32_t *err_word,
                       hipStream_t stream);

}  // namespace mot
