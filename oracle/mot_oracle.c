/*
 * CPU oracle for the Mixture-of-Transformers (MoT) token-routed projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * calls it.
 *
 * What it computes (plain definitions, fp64 accumulation, ascending k):
 *
 *  - Routing.  The RL-Kernel RFC page "[RFC][BAGEL-7B-MoT][CUDA/ROCm] WS1/WS2
 *    kernel roadmap and integration plan", section 1 (Motivation, item 1):
 *    one decoder holds two weight sets, and in each GEMM and norm a token
 *    row's set is given by a per-row index, not a learned router.  Here the
 *    index set is a byte per row: 0 = understanding set, 1 = generation set.
 *  - Routed GEMM (the "mot_routed_gemm" work item, same page, section 5):
 *    out[t,n] = bf16_rne( sum_k x[t,k] * W_{m(t)}[n,k] ), W stored [N,K].
 *  - Routed gate/up + SwiGLU (the "mot_swiglu_mlp" work item, section 5; the
 *    RL-Kernel MoE route/combine PR page gives the SwiGLU contract as gate_up
 *    GEMM, SwiGLU in fp32, one bf16 cast):  g and u are the routed GEMMs with
 *    the gate rows [0,F) and the up rows [F,2F) of the set's [2F,K] weight;
 *    act = g / (1 + exp(-g)) * u, then one bf16 rounding.
 *  - Routed fused add-RMSNorm (the "mot_fused_add_rmsnorm" work item,
 *    section 5; the MoE PR page's RMSNorm commits fix the convention: every
 *    multiply in fp32, one trailing cast, fixed reduction per row):
 *    h = bf16_rne(x + r) (the new residual), rstd = 1/sqrt(mean_k(h^2)+eps),
 *    y = bf16_rne(h * rstd * w_{m(t)}).
 *  - Routed backward (the RFC page, section 1: Phase A trains only the
 *    generation expert, and the frozen understanding operators still need
 *    dX for their rows):  dX[t,k] = bf16_rne( sum_n dY[t,n] * W_{m(t)}[n,k] )
 *    and the generation set's weight gradient
 *    dW[n,k] = bf16_rne( sum over rows t with m(t) = keep of dY[t,n] * X[t,k] ),
 *    rows in ascending order (the MoE route/combine PR page folds weight
 *    gradients over rows in ascending order).
 *  - Routed per-head QK RMSNorm and rotary embedding (the "mot_qk_norm_rope"
 *    work item; the RFC page's reference hazards: QK norm in fp32, then the
 *    rotation and Q/K in bf16): see mot_oracle_qk_norm_rope.  Its bf16
 *    roundings are part of the definition, so it rounds where the page does.
 *  - Shared joint attention (the "gen_joint_attention" work item, same page,
 *    section 5): softmax(q k^T / sqrt(D)) v over the pack's tokens of both
 *    modalities, not routed, with grouped kv heads and an optional causal
 *    mask aligned at the bottom-right corner (the page's reference hazards:
 *    a cached prefill needs that alignment).  See mot_oracle_attention.
 *
 * Every floating-point step is done in fp64 and rounded to bf16 exactly once,
 * directly from fp64 (no fp32 step), so the oracle is the exact result up to
 * fp64 rounding.  The GPU path computes in fp32 and is compared within a
 * tolerance; bitwise claims are only made GPU-against-GPU.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- bf16 encode / decode, written from the format's definition ---------- */

/* bf16 is the upper half of an IEEE binary32: 1 sign, 8 exponent, 7 fraction
 * bits.  Decoding is exact. */
static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double to the nearest bf16, ties to even, directly (no binary32
 * intermediate).  bf16 has 8 significant bits; the smallest subnormal is
 * 2^-133 and the largest finite value is (2 - 2^-7) * 2^127. */
static uint16_t bf16_round(double v)
{
    if (isnan(v))
        return 0x7fc0;
    double a = fabs(v);
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7f80;
    int e;
    frexp(a, &e);                 /* a = f * 2^e, 0.5 <= f < 1 */
    int q = e - 8;                /* spacing of 8-significant-bit numbers */
    if (q < -133)
        q = -133;                 /* subnormal spacing */
    double scaled = ldexp(a, -q); /* exact: power-of-two scaling */
    double n = nearbyint(scaled); /* default mode: round half to even */
    double r = ldexp(n, q);
    if (r >= ldexp(1.0, 128))     /* rounded past the largest finite value */
        return sign | 0x7f80;
    float rf = (float)r;          /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

uint16_t mot_oracle_bf16_round(double v) { return bf16_round(v); }
double mot_oracle_bf16_value(uint16_t b) { return bf16_value(b); }

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int mot_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- routing plan -------------------------------------------------------- */

/* Stable partition of the rows by modality: perm[0..n_und) lists the rows
 * with modality 0 in ascending order, perm[n_und..T) the rows with modality 1
 * in ascending order.  Returns 0, or -1 if a byte is neither 0 nor 1 (then
 * nothing is written). */
int mot_oracle_routing_plan(const uint8_t *modality, int64_t T, int32_t *perm,
                            int32_t *n_und, int32_t *n_gen)
{
    int64_t nu = 0, ng = 0;
    for (int64_t t = 0; t < T; ++t) {
        if (modality[t] == 0)
            ++nu;
        else if (modality[t] == 1)
            ++ng;
        else
            return -1;
    }
    int64_t iu = 0, ig = nu;
    for (int64_t t = 0; t < T; ++t) {
        if (modality[t] == 0)
            perm[iu++] = (int32_t)t;
        else
            perm[ig++] = (int32_t)t;
    }
    *n_und = (int32_t)nu;
    *n_gen = (int32_t)ng;
    return 0;
}

/* ---- routed GEMM ----------------------------------------------------------- */

/* x: [T, ldx] bf16 (first K columns used); w_und, w_gen: [N, K] bf16.
 * ref (may be NULL): [T, N] fp64 exact-ish sums; out (may be NULL): [T, N]
 * bf16 = bf16_round(ref). */
void mot_oracle_routed_gemm(const uint16_t *x, int64_t ldx,
                            const uint16_t *w_und, const uint16_t *w_gen,
                            const uint8_t *modality,
                            int64_t T, int64_t K, int64_t N,
                            double *ref, uint16_t *out, int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *w = modality[t] ? w_gen : w_und;
        const uint16_t *xr = x + t * ldx;
        for (int64_t n = 0; n < N; ++n) {
            const uint16_t *wr = w + n * K;
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += bf16_value(xr[k]) * bf16_value(wr[k]);
            if (ref)
                ref[t * N + n] = s;
            if (out)
                out[t * N + n] = bf16_round(s);
        }
    }
}

/* ---- routed backward ---------------------------------------------------------- */

/* dy [T, N] (row stride N), w_und / w_gen [N, K]: the forward's weights.
 * ref (may be NULL): [T, K] fp64; out (may be NULL): [T, K] bf16. */
void mot_oracle_routed_gemm_dx(const uint16_t *dy, const uint16_t *w_und, const uint16_t *w_gen,
                               const uint8_t *modality, int64_t T, int64_t N, int64_t K,
                               double *ref, uint16_t *out, int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *w = modality[t] ? w_gen : w_und;
        const uint16_t *gr = dy + t * N;
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t n = 0; n < N; ++n)
                s += bf16_value(gr[n]) * bf16_value(w[n * K + k]);
            if (ref)
                ref[t * K + k] = s;
            if (out)
                out[t * K + k] = bf16_round(s);
        }
    }
}

/* dy [T, N], x [T, K]: dW[n, k] over the rows whose modality byte is `keep`,
 * ascending t.  ref (may be NULL): [N, K] fp64; out (may be NULL): [N, K] bf16. */
void mot_oracle_grad_w(const uint16_t *dy, const uint16_t *x, const uint8_t *modality, int keep,
                       int64_t T, int64_t N, int64_t K, double *ref, uint16_t *out, int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            double s = 0.0;
            for (int64_t t = 0; t < T; ++t)
                if (modality[t] == keep)
                    s += bf16_value(dy[t * N + n]) * bf16_value(x[t * K + k]);
            if (ref)
                ref[n * K + k] = s;
            if (out)
                out[n * K + k] = bf16_round(s);
        }
    }
}

/* ---- routed gate/up GEMM + SwiGLU ------------------------------------------ */

/* w_und, w_gen: [2F, K] bf16, rows [0,F) gate and [F,2F) up.
 * ref (may be NULL): [T, F] fp64 silu(g)*u; out (may be NULL): [T, F] bf16. */
void mot_oracle_routed_gemm_swiglu(const uint16_t *x, int64_t ldx,
                                   const uint16_t *w_und, const uint16_t *w_gen,
                                   const uint8_t *modality,
                                   int64_t T, int64_t K, int64_t F,
                                   double *ref, uint16_t *out, int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *w = modality[t] ? w_gen : w_und;
        const uint16_t *xr = x + t * ldx;
        for (int64_t j = 0; j < F; ++j) {
            const uint16_t *wg = w + j * K;
            const uint16_t *wu = w + (F + j) * K;
            double g = 0.0, u = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = bf16_value(xr[k]);
                g += xv * bf16_value(wg[k]);
                u += xv * bf16_value(wu[k]);
            }
            double a = g / (1.0 + exp(-g)) * u;
            if (ref)
                ref[t * F + j] = a;
            if (out)
                out[t * F + j] = bf16_round(a);
        }
    }
}

/* ---- routed fused add-RMSNorm ------------------------------------------------ */

/* x: [T, H] bf16; r: [T, H] bf16 residual or NULL (then h = x).
 * h_out (may be NULL): [T, H] bf16 new residual; rstd (may be NULL): [T] fp64;
 * ref (may be NULL): [T, H] fp64; out (may be NULL): [T, H] bf16. */
void mot_oracle_fused_add_rmsnorm(const uint16_t *x, const uint16_t *r,
                                  const uint16_t *w_und, const uint16_t *w_gen,
                                  const uint8_t *modality, float eps,
                                  int64_t T, int64_t H,
                                  uint16_t *h_out, double *rstd,
                                  double *ref, uint16_t *out, int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *w = modality[t] ? w_gen : w_und;
        double ss = 0.0;
        for (int64_t k = 0; k < H; ++k) {
            double hv = bf16_value(x[t * H + k]);
            if (r)
                hv = bf16_value(bf16_round(hv + bf16_value(r[t * H + k])));
            ss += hv * hv;
        }
        double rs = 1.0 / sqrt(ss / (double)H + (double)eps);
        if (rstd)
            rstd[t] = rs;
        for (int64_t k = 0; k < H; ++k) {
            uint16_t hb = x[t * H + k];
            if (r)
                hb = bf16_round(bf16_value(hb) + bf16_value(r[t * H + k]));
            if (h_out)
                h_out[t * H + k] = hb;
            double y = bf16_value(hb) * rs * bf16_value(w[k]);
            if (ref)
                ref[t * H + k] = y;
            if (out)
                out[t * H + k] = bf16_round(y);
        }
    }
}

/* The second half of the routed RMSNorm for a given rstd: the A operand of
 * the GEMM's routed-RMSNorm prologue ("fused routed RMSNorm-prologue" of
 * the routed projection; the convention of the MoE PR page's RMSNorm
 * commits: the weight multiply in full precision, one trailing cast).
 * h: [T, H] bf16; rstd: [T] (an fp32 value, passed as a double);
 * ref (may be NULL): [T, H] fp64 h * rstd * w_{m(t)}; out (may be NULL):
 * [T, H] bf16 = bf16_round(ref).  (The product of a bf16, an fp32 and a bf16
 * value has at most 40 significant bits, so ref is exact.) */
void mot_oracle_rmsnorm_apply(const uint16_t *h, const double *rstd,
                              const uint16_t *w_und, const uint16_t *w_gen,
                              const uint8_t *modality, int64_t T, int64_t H,
                              double *ref, uint16_t *out, int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *w = modality[t] ? w_gen : w_und;
        for (int64_t k = 0; k < H; ++k) {
            double y = bf16_value(h[t * H + k]) * rstd[t] * bf16_value(w[k]);
            if (ref)
                ref[t * H + k] = y;
            if (out)
                out[t * H + k] = bf16_round(y);
        }
    }
}

/* ---- routed per-head QK RMSNorm, then rotary position embedding -------------- */

/* The "mot_qk_norm_rope" work item of the RFC page (section 5), with the
 * order the page's reference hazards fix: the QK norm in fp32, then the
 * rotation and Q/K in bf16.  Per row t (weight set m = modality[t]) and per
 * head of 128 columns (q heads at [0, 128*hq), k heads after them):
 *   rstd = 1/sqrt(mean_j(x_j^2) + eps),  y_j = bf16_rne(x_j * rstd * w_m[j])
 *   (the set's q or k norm weight, one cast as in the layer norm), then with
 *   c_i, s_i the bf16 table entries of the row's position (i = j mod 64) and
 *   the rotate-half pairing (j, j+64):
 *     out_j    = bf16(bf16(y_j * c_j)      + bf16(-y_{j+64} * s_j))   j < 64
 *     out_j+64 = bf16(bf16(y_{j+64} * c_j) + bf16( y_j * s_j))
 *   each bf16() one round-to-nearest-even of the exact value.
 * qkv, out: [T][ld] bf16 (out starts as a copy: other columns, and rows with
 * an invalid modality byte or position, keep their input bytes).  ref (may
 * be NULL): [T][ld] fp64, the exact sum before the last rounding (the input
 * value where copied).  cos_t, sin_t: [n_pos][64] bf16.  Returns 0, or the
 * largest error code seen: 6 (modality byte outside {0,1}), 7 (position
 * outside [0, n_pos)). */
int mot_oracle_qk_norm_rope(const uint16_t *qkv, int64_t ld, int64_t T, int64_t hq, int64_t hk,
                            const uint8_t *modality, const uint16_t *qw_und, const uint16_t *qw_gen,
                            const uint16_t *kw_und, const uint16_t *kw_gen, const int32_t *positions,
                            const uint16_t *cos_t, const uint16_t *sin_t, int64_t n_pos, float eps,
                            uint16_t *out, double *ref, int nthreads)
{
    int err = 0;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 4) reduction(max : err)
    for (int64_t t = 0; t < T; ++t) {
        const uint16_t *row = qkv + t * ld;
        for (int64_t c = 0; c < ld; ++c) {
            out[t * ld + c] = row[c];
            if (ref)
                ref[t * ld + c] = bf16_value(row[c]);
        }
        int e = 0;
        if (modality[t] > 1)
            e = 6;
        if (positions[t] < 0 || positions[t] >= n_pos)
            e = 7;
        if (e) {
            if (e > err)
                err = e;
            continue;
        }
        const int m = modality[t];
        const uint16_t *cs = cos_t + (int64_t)positions[t] * 64, *sn = sin_t + (int64_t)positions[t] * 64;
        for (int64_t h = 0; h < hq + hk; ++h) {
            const uint16_t *w = h < hq ? (m ? qw_gen : qw_und) : (m ? kw_gen : kw_und);
            const uint16_t *x = row + h * 128;
            double ss = 0.0;
            for (int j = 0; j < 128; ++j)
                ss += bf16_value(x[j]) * bf16_value(x[j]);
            const double rs = 1.0 / sqrt(ss / 128.0 + (double)eps);
            double y[128];
            for (int j = 0; j < 128; ++j)
                y[j] = bf16_value(bf16_round(bf16_value(x[j]) * rs * bf16_value(w[j])));
            for (int j = 0; j < 64; ++j) {
                const double c = bf16_value(cs[j]), s = bf16_value(sn[j]);
                const double lo = bf16_value(bf16_round(y[j] * c)) + bf16_value(bf16_round(-y[j + 64] * s));
                const double hi = bf16_value(bf16_round(y[j + 64] * c)) + bf16_value(bf16_round(y[j] * s));
                const int64_t o = t * ld + h * 128 + j;
                out[o] = bf16_round(lo);
                out[o + 64] = bf16_round(hi);
                if (ref) {
                    ref[o] = lo;
                    ref[o + 64] = hi;
                }
            }
        }
    }
    return err;
}

/* ---- shared joint attention ---------------------------------------------- */

/* Attention of query row i, q head h (kv head g = h / (hq / hkv); the heads'
 * columns are [h*D, (h+1)*D) of q and [g*D, (g+1)*D) of k and v):
 *   s_j = (sum_d q[i][h*D+d] * k[j][g*D+d]) / sqrt(D)   for each visible key j,
 *   out[i][h*D+d] = sum_j (exp(s_j - max s) / sum_j' exp(s_j' - max s)) * v[j][g*D+d].
 * Visible keys: every j < Tk when causal == 0; when causal == 1, the mask is
 * aligned at the bottom-right corner: query i sees keys j <= i + (Tk - Tq)
 * (so with Tq == Tk it is the usual causal mask, and the last query sees
 * every key).  A query that sees no key gets zeros.  fp64 throughout, one
 * bf16 rounding of the result.
 * rows (may be NULL = rows 0..nrows-1): the query rows to compute; ref and
 * out (either may be NULL) are [nrows][hq*D]. */
void mot_oracle_attention(const uint16_t *q, int64_t ldq, int64_t Tq,
                          const uint16_t *k, int64_t ldk, const uint16_t *v, int64_t ldv, int64_t Tk,
                          int64_t hq, int64_t hkv, int64_t D, int causal,
                          const int64_t *rows, int64_t nrows, double *ref, uint16_t *out, int nthreads)
{
    set_threads(nthreads);
    const double scale = 1.0 / sqrt((double)D);
    const int64_t group = hq / hkv;
    const int64_t width = hq * D;
#pragma omp parallel
    {
        double *p = (double *)malloc((size_t)(Tk > 0 ? Tk : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t r = 0; r < nrows; ++r) {
            for (int64_t h = 0; h < hq; ++h) {
                const int64_t i = rows ? rows[r] : r;
                const int64_t g = h / group;
                int64_t last = causal ? i + (Tk - Tq) : Tk - 1;
                if (last > Tk - 1)
                    last = Tk - 1;
                const uint16_t *qi = q + i * ldq + h * D;
                double mx = -INFINITY;
                for (int64_t j = 0; j <= last; ++j) {
                    const uint16_t *kj = k + j * ldk + g * D;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d)
                        dot += bf16_value(qi[d]) * bf16_value(kj[d]);
                    p[j] = dot * scale;
                    if (p[j] > mx)
                        mx = p[j];
                }
                double den = 0.0;
                for (int64_t j = 0; j <= last; ++j) {
                    p[j] = exp(p[j] - mx);
                    den += p[j];
                }
                for (int64_t d = 0; d < D; ++d) {
                    double num = 0.0;
                    for (int64_t j = 0; j <= last; ++j)
                        num += p[j] * bf16_value(v[j * ldv + g * D + d]);
                    const double val = last >= 0 ? num / den : 0.0;
                    if (ref)
                        ref[r * width + h * D + d] = val;
                    if (out)
                        out[r * width + h * D + d] = bf16_round(val);
                }
            }
        }
        free(p);
    }
}
