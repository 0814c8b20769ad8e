/*
 * mot.h -- C ABI of libmot, the MI355X (gfx950) Mixture-of-Transformers
 * token-routed projection.
 *
 * The method: BAGEL-7B-MoT's Qwen2.5-7B-shaped decoder holds two full weight
 * sets, "understanding" (und) and "generation" (gen), that share attention.
 * In every GEMM and norm each packed token row is routed to one set by a
 * per-row modality index (there is no learned router), and an output row's
 * bytes may not change with the other rows packed beside it (RL-Kernel RFC
 * page "[RFC][BAGEL-7B-MoT][CUDA/ROCm] WS1/WS2 kernel roadmap and integration
 * plan", section 1, item 1).  Every call keeps that page's numerical rules
 * (section 3): one fp32 accumulation order per output element, no reduction
 * split across workgroups and no atomics, no fast math, rounding only where
 * the interface declares it, and an error status instead of a guess for a
 * shape it does not support.  The operations are the
 * page's "mot_routed_gemm", "mot_swiglu_mlp" (its gate/up + SwiGLU half),
 * "mot_fused_add_rmsnorm" and "mot_qk_norm_rope" work items (section 5), the
 * routed GEMM's fp32 sums uncast (mot_routed_gemm_f32, for fp32 gradients), the
 * shared attention of both sets ("gen_joint_attention", section 5), and
 * the routed backward (section 1: Phase A trains the generation set, the
 * frozen understanding operators still pass dX back): the transpose that
 * prepares its operands and the weight gradient over token rows.
 *
 * Conventions shared by every call
 *  - bf16 tensors are passed as uint16_t bit patterns; all tensors are
 *    row-major.  Weights use the nn.Linear layout W[n][k]: y = x * W^T.
 *  - modality[t] is one byte per row: 0 = und, 1 = gen.  Any other value is a
 *    data error detected on the device (see mot_read_device_error).
 *  - Every pointer except `stream` is a DEVICE pointer owned by the caller.
 *    The library allocates nothing and keeps no state between calls.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Work is enqueued on
 *    it and runs on the stream's device; no call synchronises except
 *    mot_read_device_error.
 *  - Every host-checkable error is returned before anything is enqueued, and
 *    the outputs are then untouched.  T == 0 is a no-op returning MOT_OK.
 *  - Calls that share a workspace must be ordered (same stream, or events).
 *
 * Result bytes of the row-wise calls (GEMMs, norm, QK norm + rotary) are
 * batch-invariant: each output row depends only on its own input row, its
 * modality byte (and position) and the weights, bit for bit, whatever the
 * pack's size, order or mix.
 */
#ifndef MOT_H
#define MOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOT_ABI_VERSION 14

typedef enum mot_status {
    MOT_OK = 0,
    MOT_ERR_INVALID_ARG = 1,       /* null pointer, negative size, bad leading dimension, aliasing, eps */
    MOT_ERR_UNSUPPORTED_SHAPE = 2, /* K, N or F not a positive multiple of 64, or above the limits below */
    MOT_ERR_MISALIGNED = 3,        /* a tensor pointer not 16-byte aligned, or a leading dimension not a multiple of 8 */
    MOT_ERR_WORKSPACE = 4,         /* workspace missing or smaller than mot_workspace_bytes(T) */
    MOT_ERR_DEVICE = 5,            /* a HIP runtime call or a kernel launch failed */
    MOT_ERR_MODALITY = 6,          /* a modality byte was neither 0 nor 1 (reported by mot_read_device_error) */
    MOT_ERR_POSITION = 7,          /* a rotary position outside its table (reported by mot_read_device_error) */
    MOT_ERR_SEQLENS = 8,           /* packed sequence lengths invalid (reported by mot_read_device_error) */
    MOT_ERR_PLAN = 9,              /* a plan passed with MOT_FLAG_PLAN_READY does not describe the call's
                                      T rows (reported by mot_read_device_error; since ABI 8) */
    MOT_ERR_INDEX_SET = 10,        /* a row in neither index set, in both, or twice in one; or an index
                                      outside [0, T) (reported by mot_read_device_error; since ABI 8) */
    MOT_ERR_SCHEDULE = 11          /* a latent step's timesteps break 0 <= t_next < t <= 1, or a CFG t is
                                      not finite (reported by mot_read_device_error; since ABI 10) */
} mot_status;

/* Limits checked on the host. */
#define MOT_MAX_T (1 << 24)
#define MOT_MAX_DIM (1 << 20)

/* Workspace layout (device memory, 256-byte aligned, caller-owned):
 *   bytes [0, 16)      int32 header[4] = { error, n_und, n_gen, T }
 *                      error is MOT_OK or MOT_ERR_MODALITY (MOT_ERR_PLAN, MOT_ERR_INDEX_SET:
 *                      see below); on error n_und = n_gen = 0.
 *   bytes [256, 256+4T) int32 perm[T]: the rows with modality 0 in ascending
 *                      order, then the rows with modality 1 in ascending order.
 * This stable partition is the pack's segment list: routed kernels cut it into
 * per-set row tiles, so no tile mixes weight sets. */
#define MOT_WS_HEADER_BYTES 256

/* ABI version of the loaded library (compare with MOT_ABI_VERSION; a Python
 * binding refuses to run on a mismatch). */
int mot_abi_version(void);

/* Static, human-readable name of a mot_status value. */
const char *mot_status_string(int status);

/* Bytes of workspace the routed calls need for a pack of T rows (T >= 0). */
size_t mot_workspace_bytes(int64_t T);

/* Routing plan (the segment list): from modality[T] build the header and perm
 * described above in `workspace`.  The routed GEMM calls run this step
 * themselves unless MOT_FLAG_PLAN_READY is given (for packs of up to 8192
 * rows inside the GEMM kernel, which also writes the header and perm).
 * Errors: MOT_ERR_INVALID_ARG (T < 0, null pointers with T > 0),
 * MOT_ERR_UNSUPPORTED_SHAPE (T > MOT_MAX_T), MOT_ERR_WORKSPACE, MOT_ERR_DEVICE. */
int mot_routing_plan(const uint8_t *modality, int64_t T,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Modality bytes from the pack's two index sets.  The RFC page (section 1,
 * item 1) selects each row's weight set by a fixed index set: the rows of
 * the understanding branch and those of the generation branch.  This call
 * turns the two lists into the per-row byte the routed calls read:
 *   modality[und_idx[i]] = 0,  modality[gen_idx[i]] = 1.
 *   und_idx [n_und], gen_idx [n_gen]: int32 device arrays of row indices, in
 *        any order; modality [T] uint8 device array, written.
 *   Every row must appear exactly once over the two lists: n_und + n_gen
 *   must equal T (checked on the host: MOT_ERR_INVALID_ARG).  On the device,
 *   a row that is in neither list, in both or twice in one, and any index
 *   outside [0, T), raise MOT_ERR_INDEX_SET in the workspace's error word
 *   (read it with mot_read_device_error; it is cleared by the call); such
 *   rows get the invalid byte 0xFF, so a routed call on these bytes writes
 *   nothing and reports MOT_ERR_MODALITY.  The result does not depend on the
 *   lists' order.
 *   workspace: >= mot_workspace_bytes(T) bytes, 256-byte aligned; its plan
 *   (header and perm) is overwritten (per-row counts), so build the plan
 *   afterwards.  No argument may overlap another.
 * Errors: MOT_ERR_INVALID_ARG, MOT_ERR_UNSUPPORTED_SHAPE, MOT_ERR_MISALIGNED,
 * MOT_ERR_WORKSPACE, MOT_ERR_DEVICE.  T == 0 (with empty lists) is a no-op.
 * Since ABI 8. */
int mot_modality_from_index_sets(const int32_t *und_idx, int64_t n_und, const int32_t *gen_idx, int64_t n_gen,
                                 uint8_t *modality, int64_t T, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Flags of the routed GEMM calls. */
#define MOT_FLAG_PLAN_READY 1u /* workspace already holds the plan of this `modality`,
                                  built earlier in stream order; skip rebuilding it.
                                  A plan whose header does not describe T rows makes the
                                  call write nothing and raise MOT_ERR_PLAN (since ABI 8);
                                  a plan whose error word is set makes it write nothing.
                                  (Plain GEMM packs of at most 256 rows and SwiGLU packs
                                  of at most 128 rebuild their segment list from
                                  `modality` whatever this flag says; above 128 rows
                                  they still check the plan's header as above.) */
/* Tile shapes (token rows x weight rows per workgroup).  By default the
 * kernel runs 256x256 tiles for whole rounds of the GPU and 128x128 tiles for
 * the rest, chosen on the device from the pack's set sizes; these flags force
 * one shape, for tuning and tests.  Every shape runs the same per-element k
 * order, so the output bytes do not depend on the shape.  Setting both bits
 * is MOT_ERR_INVALID_ARG. */
#define MOT_FLAG_TILE_AUTO    0x00u
#define MOT_FLAG_TILE_256x256 0x10u
#define MOT_FLAG_TILE_128x128 0x20u
#define MOT_FLAG_TILE_MASK    0x30u

/* Routed GEMM (QKV, O and down projections):
 *   y[t][n] = bf16_rne( sum_k A[t][k] * W_{modality[t]}[n][k] ),  0 <= n < N,
 * fp32 accumulation over k in one fixed ascending order, one writer per
 * element.  A = x, or with the routed-RMSNorm prologue (rstd, nw_und and
 * nw_gen all non-NULL) A[t][k] = bf16_rne((x[t][k] * rstd[t]) * nw_{modality[t]}[k])
 * computed in fp32 -- bit-identical to feeding the output of
 * mot_fused_add_rmsnorm to the plain GEMM.
 *   x      [T][ldx] bf16, first K columns read; ldx >= K, ldx % 8 == 0.
 *   w_und, w_gen [N][K] bf16 each; both required.
 *   modality [T] uint8.
 *   y      [T][ldy] bf16, columns [0, N) written; ldy >= N, ldy % 8 == 0;
 *          must not overlap x.
 *   rstd [T] fp32, nw_und / nw_gen [K] bf16: all three NULL (no prologue)
 *          or all three non-NULL.
 *   K % 64 == 0, N % 64 == 0, 0 < K, N <= MOT_MAX_DIM, 0 <= T <= MOT_MAX_T.
 *   workspace: >= mot_workspace_bytes(T) bytes, 256-byte aligned.
 * Rows whose modality byte is invalid make the whole call write nothing; the
 * error is reported by mot_read_device_error. */
int mot_routed_gemm(const uint16_t *x, int64_t ldx,
                    const uint16_t *w_und, const uint16_t *w_gen,
                    const uint8_t *modality,
                    uint16_t *y, int64_t ldy,
                    int64_t T, int64_t K, int64_t N,
                    const float *rstd, const uint16_t *nw_und, const uint16_t *nw_gen,
                    void *workspace, size_t workspace_bytes,
                    unsigned flags, void *stream);

/* The QKV projection with the per-head routed QK RMSNorm and rotary
 * embedding in its epilogue: the "mot_qk_norm_rope" work item of the RFC page
 * (section 5) fused into "mot_routed_gemm", in the order of the page's
 * reference hazards (QK norm in fp32, then the rotation with Q/K in bf16).
 * The output bytes are those of mot_routed_gemm followed by mot_qk_norm_rope
 * on its rows (same arithmetic, bit for bit), without writing and re-reading
 * the q and k columns in between.
 *   Arguments of mot_routed_gemm (no prologue) and of mot_qk_norm_rope:
 *   y [T][ldy] with N >= 128 * (n_q_heads + n_k_heads): q heads at columns
 *   [0, 128 n_q_heads), k heads next, the rest (v) stored as the GEMM's
 *   bytes.  flags: tile-shape flags only (MOT_FLAG_PLAN_READY is
 *   MOT_ERR_INVALID_ARG: the call builds its plan, whose error word it
 *   uses).  Rows whose position is outside the table keep the GEMM's bytes and
 *   raise MOT_ERR_POSITION in the workspace's error word; an invalid modality
 *   byte makes the call write nothing and raises MOT_ERR_MODALITY (the larger
 *   code wins).
 * Errors: those of both calls.  Since ABI 11. */
int mot_routed_gemm_qk_norm_rope(const uint16_t *x, int64_t ldx, const uint16_t *w_und, const uint16_t *w_gen,
                                 const uint8_t *modality, uint16_t *y, int64_t ldy, int64_t T, int64_t K, int64_t N,
                                 int64_t n_q_heads, int64_t n_k_heads, const uint16_t *qw_und, const uint16_t *qw_gen,
                                 const uint16_t *kw_und, const uint16_t *kw_gen, const int32_t *positions,
                                 const uint16_t *cos_table, const uint16_t *sin_table, int64_t n_pos, float eps,
                                 void *workspace, size_t workspace_bytes, unsigned flags, void *stream);

/* Largest pack of mot_routed_gemm_noalloc. */
#define MOT_NOALLOC_MAX_T 65536

/* mot_routed_gemm without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The call's workspace (the
 * routing header and segment list, MOT_WS_HEADER_BYTES + 4 * T bytes) lives
 * in a static device array of the library, sized for MOT_NOALLOC_MAX_T rows
 * (256 KiB + 256 bytes), one copy per GPU, held until the process ends.  The
 * call allocates nothing.  Every call on one GPU shares that GPU's array and
 * leaves its contents there: calls that overlap on one GPU (other streams,
 * other threads) race and must be ordered by the caller.
 *   error_out: NULL, or a device int32 that receives the call's device error
 *        word in stream order (MOT_OK, or MOT_ERR_MODALITY if a modality byte
 *        was invalid, in which case nothing was written to y).
 *   flags: tile-shape flags only; MOT_FLAG_PLAN_READY is MOT_ERR_INVALID_ARG.
 * Other arguments, the result bytes (identical to mot_routed_gemm's) and the
 * errors as mot_routed_gemm, plus MOT_ERR_UNSUPPORTED_SHAPE for
 * T > MOT_NOALLOC_MAX_T.  Since ABI 9. */
int mot_routed_gemm_noalloc(const uint16_t *x, int64_t ldx,
                            const uint16_t *w_und, const uint16_t *w_gen,
                            const uint8_t *modality,
                            uint16_t *y, int64_t ldy,
                            int64_t T, int64_t K, int64_t N,
                            const float *rstd, const uint16_t *nw_und, const uint16_t *nw_gen,
                            int32_t *error_out, unsigned flags, void *stream);

/* Routed GEMM with fp32 output: the fp32 sums of mot_routed_gemm, before
 * their bf16 cast (the bf16 output of mot_routed_gemm is bf16_rne of this
 * one's, bit for bit).  It serves fp32 weight gradients for a master-weight
 * optimizer: the RFC page (section 1) trains the generation expert while the
 * understanding one stays frozen, and the MoE route/combine PR page folds
 * weight gradients over rows in ascending order in fp32; with the operands of
 * mot_transpose_bf16 below, this call returns that fp32 fold uncast.
 *   y      [T][ldy] fp32, columns [0, N) written; ldy >= N, ldy % 8 == 0,
 *          16-byte aligned; must not overlap x, the weights or the workspace.
 *   flags  MOT_FLAG_PLAN_READY only (no tile override, no prologue): every
 *          row block runs as a 256 x 256 tile.
 * Other arguments and the errors as mot_routed_gemm.  Since ABI 5. */
int mot_routed_gemm_f32(const uint16_t *x, int64_t ldx,
                        const uint16_t *w_und, const uint16_t *w_gen,
                        const uint8_t *modality,
                        float *y, int64_t ldy,
                        int64_t T, int64_t K, int64_t N,
                        void *workspace, size_t workspace_bytes,
                        unsigned flags, void *stream);

/* Routed gate/up GEMM with the SwiGLU epilogue (the gate/up half of the MLP):
 *   g = sum_k A[t][k] * W_m[j][k],  u = sum_k A[t][k] * W_m[F + j][k]  (fp32),
 *   act[t][j] = bf16_rne( (g / (1 + expf(-g))) * u ),  0 <= j < F,
 * with accurate expf (no fast intrinsic) and one bf16 cast (RL-Kernel MoE
 * route/combine PR page: gate_up GEMM, SwiGLU in fp32, then bf16).
 *   wgu_und, wgu_gen [2F][K] bf16: rows [0, F) gate, rows [F, 2F) up.
 *   act [T][ldact] bf16, ldact >= F, ldact % 8 == 0.  F % 64 == 0.
 * Other arguments, the prologue and the errors as mot_routed_gemm. */
int mot_routed_gemm_swiglu(const uint16_t *x, int64_t ldx,
                           const uint16_t *wgu_und, const uint16_t *wgu_gen,
                           const uint8_t *modality,
                           uint16_t *act, int64_t ldact,
                           int64_t T, int64_t K, int64_t F,
                           const float *rstd, const uint16_t *nw_und, const uint16_t *nw_gen,
                           void *workspace, size_t workspace_bytes,
                           unsigned flags, void *stream);

/* Routed fused add-RMSNorm, per row t with m = modality[t]:
 *   h = bf16_rne(x[t] + residual[t])   (fp32 add; h = x[t] when residual is NULL)
 *   residual[t] = h                    (in place, when residual is non-NULL)
 *   rstd = 1 / sqrtf(sum_k(h_k^2) / H + eps)   fp32, correctly rounded divide
 *          and sqrt, one fixed reduction tree per row that does not depend on T
 *   out[t][k] = bf16_rne((h_k * rstd) * w_m[k])   fp32, one cast
 *   rstd_out[t] = rstd
 * (RMSNorm convention of the RL-Kernel MoE route/combine PR page: the weight
 * is applied in fp32, the result is rounded once, and a row's reduction order
 * depends on H alone.)
 *   x, residual, out: [T][H] bf16, contiguous; out may be NULL (prologue mode:
 *   the routed GEMMs then read h and rstd); rstd_out [T] fp32 or NULL; at least
 *   one of out / rstd_out non-NULL.  w_und, w_gen [H] bf16.
 *   H % 64 == 0, 0 < H <= 16384; eps > 0 and finite.
 *   workspace: NULL, or a routed workspace whose header error word is SET to
 *   MOT_ERR_MODALITY if a byte is invalid (rows with an invalid byte are not
 *   written).  This call never clears the error word.
 * Errors: MOT_ERR_INVALID_ARG, MOT_ERR_UNSUPPORTED_SHAPE, MOT_ERR_MISALIGNED,
 * MOT_ERR_DEVICE. */
int mot_fused_add_rmsnorm(const uint16_t *x, uint16_t *residual,
                          const uint16_t *w_und, const uint16_t *w_gen,
                          const uint8_t *modality, float eps,
                          uint16_t *out, float *rstd_out,
                          int64_t T, int64_t H,
                          void *workspace, void *stream);

/* bf16 transpose, the operand preparation of the routed backward on
 * transposed copies (mot_routed_gemm_dx and mot_grad_w below compute the same
 * products, with the same bytes, from the operands as they lie).  The RFC
 * page (section 1) trains only the generation expert in Phase A while the
 * frozen understanding operators still need dX, and the MoE route/combine PR
 * page folds weight gradients over rows in ascending order in fp32.  With it:
 *   dX = dY * W_{m(t)}  (per row t): mot_routed_gemm(dY, W_und^T, W_gen^T),
 *        the same routed kernel and k order, W^T = this call on each [N][K] set;
 *   dW_gen = sum over gen rows t of dY[t]^T X[t]: mot_routed_gemm(dY^T, Xg^T,
 *        Xg^T, all rows set 0) over the tokens, where Xg^T is this call on X
 *        with modality and keep = 1 (und rows zeroed) and both transposes are
 *        padded to a multiple of 64 rows; the MFMA chain then folds the rows
 *        in ascending 16-row chunks, in fp32.
 *   out[c][r] = in[r][c]                  for r < rows, c < cols, except
 *   out[c][r] = 0  where modality != NULL and modality[r] != keep, and for
 *                  rows <= r < rows_pad.
 *   in  [rows][ld_in] bf16, ld_in >= cols;  out [cols][ld_out], ld_out >= rows_pad;
 *   ld_in % 8 == ld_out % 8 == 0, pointers 16-byte aligned, in and out disjoint,
 *   keep 0 or 1; rows_pad <= MOT_MAX_T, cols <= MOT_MAX_DIM.
 * Errors: MOT_ERR_INVALID_ARG, MOT_ERR_UNSUPPORTED_SHAPE, MOT_ERR_MISALIGNED,
 * MOT_ERR_DEVICE.  rows_pad == 0 or cols == 0 is a no-op. */
int mot_transpose_bf16(const uint16_t *in, int64_t ld_in, int64_t rows, int64_t cols,
                       const uint8_t *modality, int keep, uint16_t *out, int64_t ld_out,
                       int64_t rows_pad, void *stream);

/* Routed input gradient with the forward's weights as they lie: the dX of
 * the routed backward (the RFC page, section 1: the frozen understanding
 * operators still pass dX back), with no transposed copy of either set.
 *   dx[t][k] = bf16_rne( fp32 sum over n of dy[t][n] * W_{modality[t]}[n][k] )
 * the n in ascending 16-step MFMA chunks: the k order, and so the bytes, of
 * mot_routed_gemm(dy, W_und^T, W_gen^T) (W^T from mot_transpose_bf16).
 *   dy [T][lddy] bf16, columns [0, N); w_und, w_gen [N][K] bf16 (nn.Linear
 *   layout of the forward y = x W^T, pitch K); dx [T][lddx] bf16, columns
 *   [0, K) written; N % 64 == 0, K % 64 == 0.
 *   flags: MOT_FLAG_PLAN_READY only.  Every row block runs as a 256 x 256
 *   tile (partial blocks included).
 * Modality bytes, workspace, plan, error word and the other errors as
 * mot_routed_gemm (with its K the contraction length N here and its N the
 * output width K).  Since ABI 14. */
int mot_routed_gemm_dx(const uint16_t *dy, int64_t lddy, const uint16_t *w_und, const uint16_t *w_gen,
                       const uint8_t *modality, uint16_t *dx, int64_t lddx, int64_t T, int64_t N, int64_t K,
                       void *workspace, size_t workspace_bytes, unsigned flags, void *stream);

/* Weight gradient of one set, from the operands as they lie in memory (no
 * transposed copies): the generation-set dW of the routed backward (the RFC
 * page, section 1: Phase A trains the generation expert), or the other set's
 * with keep = 0.
 *   out[n][k] = sum over rows t < T with modality[t] == keep of
 *               dy[t][n] * x[t][k]
 * in fp32, the rows folded in ascending order in 16-row MFMA steps over all
 * T rows (rows of the other set, or with any other byte, count as zero rows,
 * so the fold is the one mot_routed_gemm gives on mot_transpose_bf16's
 * operands above, bit for bit), stored as bf16 (round to nearest even once)
 * or, with out_f32 = 1, as the fp32 sums.
 *   dy  [T][lddy] bf16, columns [0, N);  x [T][ldx] bf16, columns [0, K);
 *   modality [T] bytes;  out [N][ldo] bf16 (fp32 when out_f32), columns
 *   [0, K) written; must not overlap dy, x or modality.
 *   K % 64 == 0, K <= MOT_MAX_DIM, N <= MOT_MAX_T, T <= MOT_MAX_T; lddy >= N,
 *   ldx >= K, ldo >= K, all % 8 == 0; dy, x, out 16-byte aligned; keep and
 *   out_f32 0 or 1.  The kernel addresses dy and x (their rows up to T
 *   rounded up to 64, 256-column tiles) and out with 32-bit byte offsets:
 *   larger extents are MOT_ERR_UNSUPPORTED_SHAPE.
 * Errors: MOT_ERR_INVALID_ARG, MOT_ERR_UNSUPPORTED_SHAPE, MOT_ERR_MISALIGNED,
 * MOT_ERR_DEVICE.  N == 0 or K == 0 is a no-op; T == 0 writes zeros (dy, x
 * and modality may then be NULL).  Since ABI 13. */
int mot_grad_w(const uint16_t *dy, int64_t lddy, const uint16_t *x, int64_t ldx,
               const uint8_t *modality, int keep, int64_t T, int64_t N, int64_t K,
               void *out, int64_t ldo, int out_f32, void *stream);

/* Routed per-head QK RMSNorm, then the rotary embedding, in place on the
 * rows of the QKV projection's output: the "mot_qk_norm_rope" work item of
 * the RL-Kernel RFC page (section 5), in the order its reference hazards fix
 * (QK norm in fp32, then the rotation with Q/K in bf16).  Row t uses weight
 * set m = modality[t]; each of its heads of 128 columns (q heads at columns
 * [0, 128*n_q_heads), k heads right after; other columns untouched) becomes
 *   rstd = 1/sqrt(mean_j(x_j^2) + eps),  y_j = bf16((x_j * rstd) * w[j])
 *   with w the set's q or k norm weight, then, with c, s the row of
 *   cos_table and sin_table at positions[t] (entry j mod 64):
 *   out_j    = bf16(bf16(y_j * c_j)      + bf16(-y_{j+64} * s_j))   j < 64
 *   out_j+64 = bf16(bf16(y_{j+64} * c_j) + bf16( y_j * s_j))
 *   (rotate-half pairs; each bf16() one round-to-nearest-even).
 *   qkv [T][ld] bf16, ld >= 128*(n_q_heads+n_k_heads), ld % 8 == 0;
 *   qw_*, kw_* [128] bf16; positions [T] int32; cos_table, sin_table
 *   [n_pos][64] bf16; device pointers, 16-byte aligned, none overlapping the
 *   rows; eps > 0 and finite; workspace: at least MOT_WS_HEADER_BYTES, its
 *   error word is cleared and then raised (MOT_ERR_MODALITY, MOT_ERR_POSITION;
 *   the larger wins) for rows whose byte or position is invalid, which keep
 *   their bytes.  The tables are data (cos and sin of the model's angles).
 * Errors: MOT_ERR_INVALID_ARG, MOT_ERR_UNSUPPORTED_SHAPE, MOT_ERR_MISALIGNED,
 * MOT_ERR_WORKSPACE, MOT_ERR_DEVICE.  T == 0 is a no-op. */
int mot_qk_norm_rope(uint16_t *qkv, int64_t ld, int64_t T, int64_t n_q_heads, int64_t n_k_heads,
                     const uint8_t *modality, const uint16_t *qw_und, const uint16_t *qw_gen,
                     const uint16_t *kw_und, const uint16_t *kw_gen, const int32_t *positions,
                     const uint16_t *cos_table, const uint16_t *sin_table, int64_t n_pos, float eps,
                     void *workspace, size_t workspace_bytes, void *stream);

/* Synchronises `stream` and returns the workspace's device error word:
 * MOT_OK, MOT_ERR_MODALITY, MOT_ERR_POSITION, MOT_ERR_SEQLENS, MOT_ERR_PLAN,
 * MOT_ERR_INDEX_SET, MOT_ERR_SCHEDULE, or MOT_ERR_DEVICE if the copy fails. */
int mot_read_device_error(const void *workspace, void *stream);

/* Workspace bytes of mot_joint_attention: 0 (V is read in place; until
 * ABI 11 the call kept a transposed copy of V there).  Since ABI 6. */
size_t mot_attention_workspace_bytes(int64_t Tk, int64_t n_kv_heads);

/* Shared joint attention: the "gen_joint_attention" work item of the RFC
 * page (section 5).  Both weight sets share it, so it is not routed: every
 * query row of the pack attends over the same keys, of both modalities.
 * For query row i and q head h, with kv head g = h / (n_q_heads / n_kv_heads):
 *   s_j = fp32 sum_d q[i][128h+d] * k[j][128g+d] for each key j that row i
 *         sees (the softmax of s_j / sqrt(128));
 *   out[i][128h+d] = bf16_rne( sum_j p_j v[j][128g+d] / sum_j p_j ),
 *         p_j = 2^(c s_j - c m) (hardware exp2), c = log2(e)/sqrt(128)
 *         rounded once to fp32, m a per-row reference that follows the
 *         running maximum of the scores and moves only when a block's
 *         maximum exceeds it by more than 8/c (so p_j <= 2^8); keys in blocks
 *         of 64 from key 0 upwards, the sums and the rescale by 2^(c m_old -
 *         c m_new) in fp32; the p_j enter the products with v as bf16.
 * Visible keys: all Tk when causal == 0.  With causal == 1 the mask is
 * aligned at the bottom-right corner, as the same page's reference hazards
 * require for a cached prefill: row i sees keys j <= i + (Tk - Tq).  A row
 * that sees no key gets zeros.  One accumulation order per element, no
 * split over keys (the page's section 3); a row's bytes depend only on its
 * q row, the keys it sees and the v rows, not on the other rows of the pack.
 *   q   [Tq][ldq] bf16, heads at columns [0, 128*n_q_heads); ldq % 8 == 0.
 *   k, v [Tk][ldk], [Tk][ldv] bf16, kv heads at columns [0, 128*n_kv_heads)
 *        (q, k and v may be column ranges of one QKV buffer).
 *   out [Tq][ldo] bf16, columns [0, 128*n_q_heads) written; must not overlap
 *        q, k, v or the workspace.
 *   head_dim == 128; n_q_heads % n_kv_heads == 0; n_q_heads <= 256;
 *   Tq, Tk <= MOT_MAX_T; causal 0 or 1; pointers 16-byte aligned.
 *   workspace, workspace_bytes: unused (may be NULL, 0); kept for callers
 *        that size one with mot_attention_workspace_bytes.
 *   The kernel addresses K and V with 32-bit byte offsets: (round_up(Tk, 64)
 *        * ldk + 128 * n_kv_heads) * 2 and the same with ldv stay below 2^32.
 * Errors: MOT_ERR_INVALID_ARG, MOT_ERR_UNSUPPORTED_SHAPE, MOT_ERR_MISALIGNED,
 * MOT_ERR_DEVICE.  Tq == 0 is a no-op.  Since ABI 6. */
int mot_joint_attention(const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk,
                        const uint16_t *v, int64_t ldv, uint16_t *out, int64_t ldo,
                        int64_t Tq, int64_t Tk, int64_t n_q_heads, int64_t n_kv_heads,
                        int64_t head_dim, int causal, void *workspace, size_t workspace_bytes,
                        void *stream);

/* Workspace bytes of mot_joint_attention_varlen: MOT_WS_HEADER_BYTES, the
 * header whose first int32 is the lengths check's error word (until ABI 11
 * a transposed copy of V followed it).  0 for invalid sizes.  Since ABI 7. */
size_t mot_attention_varlen_workspace_bytes(int64_t Tk, int64_t n_seqs, int64_t n_kv_heads);

/* mot_joint_attention over packed sequences: sequence b has the query rows
 * [cu_q[b], cu_q[b+1]) and the keys [cu_k[b], cu_k[b+1]); each row attends
 * only over its own sequence's keys, with the causal mask aligned at the
 * bottom-right corner of that sequence (row i of a sequence of Lq rows and
 * Lk keys sees its keys j <= i + Lk - Lq).  Several requests (the branches of
 * a CFG step, prompts of a batch) then share one call, and a row's bytes are
 * those it gets when its sequence runs alone: the softmax order is fixed per
 * sequence, from its first key.
 *   cu_q, cu_k [n_seqs + 1] int32 device arrays: 0 = cu[0] <= ... <=
 *        cu[n_seqs] = Tq (resp. Tk); no sequence longer than max_q rows.
 *        They are checked on the device; if they break these rules nothing is
 *        written and the workspace's error word is MOT_ERR_SEQLENS (read it
 *        with mot_read_device_error; it is 0 after a valid call).
 *   max_q: an upper bound on the rows of one sequence (host value; the grid
 *        is n_seqs x ceil(max_q / 128) x n_q_heads workgroups).
 *   workspace: >= mot_attention_varlen_workspace_bytes(Tk, n_seqs,
 *        n_kv_heads) bytes, 256-byte aligned, overwritten.
 * Other arguments, the arithmetic and the errors as mot_joint_attention.
 * Tq == 0 is a no-op.  Since ABI 7. */
int mot_joint_attention_varlen(const uint16_t *q, int64_t ldq, const uint16_t *k, int64_t ldk,
                               const uint16_t *v, int64_t ldv, uint16_t *out, int64_t ldo,
                               const int32_t *cu_q, const int32_t *cu_k, int64_t n_seqs,
                               int64_t Tq, int64_t Tk, int64_t max_q,
                               int64_t n_q_heads, int64_t n_kv_heads, int64_t head_dim, int causal,
                               void *workspace, size_t workspace_bytes, void *stream);

/* ---- latent step: renormalised CFG and the flow SDE step (since ABI 10) ----
 *
 * The "cfg_combine_renorm" and "flow_sde_step_logp" work items of the RFC
 * page (section 5).  The page gives the rules they keep, not their formulas
 * (section 1, item 3; section 3, its rules for BAGEL): the combine takes up to
 * three branches and two guidance scales, guides only inside a window of t
 * tested in fp32, and rescales by a clamped ratio of norms taken for each
 * request on its own, never across the pack; the step and its
 * log-probability are fp32, sigma equals t (the path x_t = (1 - t) x_0 +
 * t noise), the step goes down from t_i to t_{i+1} (a positive dt), and the
 * log-probability adds up the request's latent elements in an order fixed in
 * advance.  The formulas below are this library's readings of those rules.
 *
 * Layout: fp32 [rows][C] arrays, C % 4 == 0, C <= 4096, packed by request:
 * request b owns rows [cu_rows[b], cu_rows[b+1]) (cu_rows: int32 device
 * array of n_req + 1 entries, 0 = cu[0] <= ... <= cu[n_req] = rows, no
 * request longer than max_rows >= 1, n_req >= 1; empty requests are allowed,
 * and their log-probability is 0; checked on the device, and a violation
 * writes nothing and raises MOT_ERR_SEQLENS).  Work goes in chunks of 64 rows
 * of one request; request-wide sums add the chunks' fp32 sums in ascending
 * order, so a request's results do not depend on the other requests of the
 * pack.  workspace: >= mot_latent_workspace_bytes(n_req, max_rows) bytes,
 * 256-byte aligned; its error word is set by every call. */
size_t mot_latent_workspace_bytes(int64_t n_req, int64_t max_rows);

#define MOT_RENORM_NONE 0
#define MOT_RENORM_GLOBAL 1   /* one ratio per request, over all its elements */
#define MOT_RENORM_CHANNEL 2  /* one ratio per latent row, over its C channels */

/* Guided velocity of each request b, in fp32:
 *   inside the window t_lo < t[b] <= t_hi:
 *     g = v_tu + s_text (v_c - v_tu);  three branches: g = v_iu + s_img (g - v_iu)
 *     r = min(1, max(renorm_min, ||v_c|| / ||g||)) over the request (GLOBAL)
 *         or over each row (CHANNEL), r = 1 when ||g|| = 0; r = 1 (NONE)
 *     out = r g
 *   outside the window: out = v_c.
 *   v_cond, v_text_uncond: [rows][C] fp32; v_img_uncond: [rows][C] or NULL
 *   (two branches); out [rows][C], overlapping no input; t [n_req] fp32
 *   device array (finite, else MOT_ERR_SCHEDULE and nothing written);
 *   scales and window finite, 0 <= renorm_min <= 1.
 * Errors: MOT_ERR_INVALID_ARG, MOT_ERR_UNSUPPORTED_SHAPE, MOT_ERR_MISALIGNED
 * (16-byte aligned arrays, 4-byte aligned cu_rows and t), MOT_ERR_WORKSPACE,
 * MOT_ERR_DEVICE.  n_req == 0 with rows == 0 is a no-op. */
int mot_cfg_combine_renorm(const float *v_cond, const float *v_text_uncond, const float *v_img_uncond, float *out,
                           const int32_t *cu_rows, int64_t n_req, int64_t rows, int64_t C, int64_t max_rows,
                           const float *t, float s_text, float s_img, float t_lo, float t_hi, float renorm_min,
                           int renorm_type, void *workspace, size_t workspace_bytes, void *stream);

/* One SDE step of each request b from t = t_cur[b] down to t_next[b], in
 * fp32 (the Euler-Maruyama step of rectified flow's reverse SDE published
 * with Flow-GRPO; v is the model's velocity dx/dt):
 *   dt = t - t_next > 0,  s = eta sqrt(t / (1 - t)) (1 - t_next in the
 *   denominator at the first step t = 1),  k = s^2 / (2 t)
 *   mu = x - dt (v + k (x + (1 - t) v)),  sd = s sqrt(dt)
 *   sampling (noise != NULL):  x_next_out = mu + sd noise
 *   either mode, with x_next the sample or x_next_in:
 *     logp[b] = -q / (2 sd^2) - n (log(sd) + log(2 pi) / 2),
 *     q = sum over the request's n = rows_b * C elements of (x_next - mu)^2
 *   (the same arithmetic in both modes, so evaluating a sample's x_next gives
 *   the sampling call's logp bit for bit).
 *   x, v, noise, x_next_in, x_next_out: [rows][C] fp32; exactly one mode:
 *   noise and x_next_out non-NULL with x_next_in NULL, or x_next_in alone.
 *   logp [n_req] fp32; t_cur, t_next [n_req] fp32 device arrays with
 *   0 <= t_next < t_cur <= 1 (else MOT_ERR_SCHEDULE, nothing written);
 *   eta > 0 and finite.  Outputs overlap no input.
 * Errors as mot_cfg_combine_renorm. */
int mot_flow_sde_step_logp(const float *x, const float *v, const float *noise, const float *x_next_in,
                           float *x_next_out, float *logp, const int32_t *cu_rows, int64_t n_req, int64_t rows,
                           int64_t C, int64_t max_rows, const float *t_cur, const float *t_next, float eta,
                           void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOT_H */
