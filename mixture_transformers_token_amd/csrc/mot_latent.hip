// Latent-step kernels (gfx950): the three-branch renormalised CFG combine and
// the flow SDE step with its log-probability, the "cfg_combine_renorm" and
// "flow_sde_step_logp" work items of the RL-Kernel RFC page "[RFC][BAGEL-
// 7B-MoT][CUDA/ROCm] WS1/WS2 kernel roadmap and integration plan" (section
// 5).  The page gives their rules, not their formulas (section 1, item 3;
// section 3, its rules for BAGEL): at most three branches and two guidance
// scales, guidance only inside a window of t tested in fp32, a clamped
// rescale by a ratio of norms taken for each request alone; the step and its
// log-probability in fp32, sigma equal to t, a step down in t (positive dt),
// and the log-probability added up over the request's latent elements in an
// order fixed in advance.  The formulas are the library's readings
// of that contract (mot.h states them); the SDE is the Euler-Maruyama step of
// rectified flow's reverse SDE as published with Flow-GRPO.
//
// Layout: velocities, latents and noise are fp32 [rows][C], packed by request
// (request b owns rows [cu[b], cu[b+1])).  Work is cut into chunks of
// kChunkRows rows of one request; chunk j of request b always covers the same
// rows of that request, whatever the other requests, and its threads sum in
// one fixed order, so a request's results do not depend on the pack.  A
// request-wide sum (a norm, the log-probability's quadratic term) is the
// ascending sum of its chunks' partial sums, read from the workspace by every
// consumer in the same order.  No atomics take part in any result.
//
// Built with -ffp-contract=off: every multiply and add rounds where written.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mot_internal.h"

namespace mot {
namespace {

constexpr int kLThreads = 256;
constexpr int kChunkRows = 64;
constexpr int kErrSeqlensL = 8;   // MOT_ERR_SEQLENS
constexpr int kErrSchedule = 11;  // MOT_ERR_SCHEDULE
constexpr float kHalfLog2Pi = 0.918938533204672742f;  // log(2 pi) / 2, rounded once to fp32

// Row ranges (cu[0] = 0, non-decreasing, cu[n] = rows, no request over
// max_rows rows) and, for the SDE, the schedule (0 < t <= 1, 0 <= t_next < t)
// or, for the CFG, finite t.  One workgroup; writes the error word.
__global__ void __launch_bounds__(kLThreads)
latent_check_kernel(const int32_t *cu, int n, int64_t rows, int64_t max_rows, const float *t_cur,
                    const float *t_next, int sde, int32_t *err) {
    __shared__ int bad_rows, bad_sched;
    if (threadIdx.x == 0) {
        bad_rows = (cu[0] != 0 || (int64_t)cu[n] != rows) ? 1 : 0;
        bad_sched = 0;
    }
    __syncthreads();
    for (int b = (int)threadIdx.x; b < n; b += kLThreads) {
        const int64_t len = (int64_t)cu[b + 1] - cu[b];
        if (len < 0 || len > max_rows) bad_rows = 1;  // benign race: every writer stores 1
        const float t = t_cur[b];
        if (sde) {
            const float tn = t_next[b];
            if (!(t > 0.0f && t <= 1.0f && tn >= 0.0f && tn < t)) bad_sched = 1;
        } else if (!isfinite(t)) {
            bad_sched = 1;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) *err = bad_rows ? kErrSeqlensL : bad_sched ? kErrSchedule : 0;
}

// Workgroup sum of one value per thread in a fixed tree: an xor-butterfly
// within each wave, then the four wave sums in ascending wave order.
__device__ __forceinline__ float block_sum(float v, float *s_red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off, 64);
    const int wave = (int)threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s_red[wave] = v;
    __syncthreads();
    return ((s_red[0] + s_red[1]) + s_red[2]) + s_red[3];
}

struct CfgArgs {
    const float *vc, *vt, *vi;  // [rows][C]; vi == nullptr: two branches
    float *out;
    const int32_t *cu;
    int n, C, nchunk;            // requests, channels, chunk slots per request
    const float *t;
    float s_text, s_img, t_lo, t_hi, rmin;
    int type;                    // 0 none, 1 global (per request), 2 channel (per row)
    float *part;                 // [n][nchunk][2]: sum v_c^2, sum g^2 of each chunk
    const int32_t *err;
};

__device__ __forceinline__ float4 ld4(const float *p) { return *(const float4 *)p; }

// the guided velocity of four elements
__device__ __forceinline__ float4 guided(const CfgArgs &a, int64_t off, float4 &c) {
    c = ld4(a.vc + off);
    const float4 u = ld4(a.vt + off);
    float4 g;
    g.x = u.x + a.s_text * (c.x - u.x);
    g.y = u.y + a.s_text * (c.y - u.y);
    g.z = u.z + a.s_text * (c.z - u.z);
    g.w = u.w + a.s_text * (c.w - u.w);
    if (a.vi != nullptr) {
        const float4 w = ld4(a.vi + off);
        g.x = w.x + a.s_img * (g.x - w.x);
        g.y = w.y + a.s_img * (g.y - w.y);
        g.z = w.z + a.s_img * (g.z - w.z);
        g.w = w.w + a.s_img * (g.w - w.w);
    }
    return g;
}

__device__ __forceinline__ float renorm_ratio(float ssc, float ssg, float rmin) {
    if (ssg == 0.0f) return 1.0f;
    return fminf(1.0f, fmaxf(rmin, sqrtf(ssc) / sqrtf(ssg)));
}

__device__ __forceinline__ bool in_window(const CfgArgs &a, float t) { return a.t_lo < t && t <= a.t_hi; }

// Pass 1 of the global renorm: per chunk, the sums of squares of v_c and of
// the guided velocity (thread i takes the chunk's float4 groups i, i+256,
// ... in ascending order; then the workgroup tree).
__global__ void __launch_bounds__(kLThreads) cfg_partial_kernel(CfgArgs a) {
    __shared__ float s_red[4];
    if (__builtin_amdgcn_readfirstlane(*(volatile const int32_t *)a.err) != 0) return;
    const int b = (int)blockIdx.x / a.nchunk, j = (int)blockIdx.x % a.nchunk;
    const int64_t r0 = a.cu[b], r1 = a.cu[b + 1];
    const int64_t c0 = r0 + (int64_t)j * kChunkRows;
    if (c0 >= r1 || !in_window(a, a.t[b])) return;
    const int64_t ce = min(c0 + kChunkRows, r1);
    const int64_t e0 = c0 * a.C, e1 = ce * a.C;
    float ssc = 0.0f, ssg = 0.0f;
    for (int64_t e = e0 + 4 * (int64_t)threadIdx.x; e < e1; e += 4 * kLThreads) {
        float4 c;
        const float4 g = guided(a, e, c);
        ssc = ssc + c.x * c.x;
        ssc = ssc + c.y * c.y;
        ssc = ssc + c.z * c.z;
        ssc = ssc + c.w * c.w;
        ssg = ssg + g.x * g.x;
        ssg = ssg + g.y * g.y;
        ssg = ssg + g.z * g.z;
        ssg = ssg + g.w * g.w;
    }
    ssc = block_sum(ssc, s_red);
    ssg = block_sum(ssg, s_red);
    if (threadIdx.x == 0) {
        a.part[((int64_t)b * a.nchunk + j) * 2 + 0] = ssc;
        a.part[((int64_t)b * a.nchunk + j) * 2 + 1] = ssg;
    }
}

// Pass 2: the guided velocity again (same arithmetic), scaled by the
// request's ratio (global: from the chunks' sums, added in ascending chunk
// order; channel: per row, over its C channels, by one wave per row), or
// v_c outside the window.
__global__ void __launch_bounds__(kLThreads) cfg_apply_kernel(CfgArgs a) {
    __shared__ float s_red[4];
    if (__builtin_amdgcn_readfirstlane(*(volatile const int32_t *)a.err) != 0) return;
    const int b = (int)blockIdx.x / a.nchunk, j = (int)blockIdx.x % a.nchunk;
    const int64_t r0 = a.cu[b], r1 = a.cu[b + 1];
    const int64_t c0 = r0 + (int64_t)j * kChunkRows;
    if (c0 >= r1) return;
    const int64_t ce = min(c0 + kChunkRows, r1);
    const int C = a.C;
    if (!in_window(a, a.t[b])) {
        for (int64_t e = c0 * C + 4 * (int64_t)threadIdx.x; e < ce * C; e += 4 * kLThreads)
            *(float4 *)(a.out + e) = ld4(a.vc + e);
        return;
    }
    if (a.type == 2) {
        // channel renorm: wave w takes rows c0 + w, c0 + w + 4, ...; lane l
        // sums the row's float4 groups l, l+64, ... in order, then the
        // wave's butterfly
        const int lane = (int)threadIdx.x & 63, wave = (int)threadIdx.x >> 6;
        for (int64_t r = c0 + wave; r < ce; r += 4) {
            float ssc = 0.0f, ssg = 0.0f;
            for (int k = 4 * lane; k < C; k += 256) {
                float4 c;
                const float4 g = guided(a, r * C + k, c);
                ssc = ssc + c.x * c.x;
                ssc = ssc + c.y * c.y;
                ssc = ssc + c.z * c.z;
                ssc = ssc + c.w * c.w;
                ssg = ssg + g.x * g.x;
                ssg = ssg + g.y * g.y;
                ssg = ssg + g.z * g.z;
                ssg = ssg + g.w * g.w;
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                ssc = ssc + __shfl_xor(ssc, off, 64);
                ssg = ssg + __shfl_xor(ssg, off, 64);
            }
            const float rr = renorm_ratio(ssc, ssg, a.rmin);
            for (int k = 4 * lane; k < C; k += 256) {
                float4 c;
                float4 g = guided(a, r * C + k, c);
                g.x = g.x * rr;
                g.y = g.y * rr;
                g.z = g.z * rr;
                g.w = g.w * rr;
                *(float4 *)(a.out + r * C + k) = g;
            }
        }
        return;
    }
    float rr = 1.0f;
    if (a.type == 1) {
        const int nch = (int)((r1 - r0 + kChunkRows - 1) / kChunkRows);
        float ssc = 0.0f, ssg = 0.0f;
        for (int q = 0; q < nch; ++q) {
            ssc = ssc + a.part[((int64_t)b * a.nchunk + q) * 2 + 0];
            ssg = ssg + a.part[((int64_t)b * a.nchunk + q) * 2 + 1];
        }
        rr = renorm_ratio(ssc, ssg, a.rmin);
    }
    for (int64_t e = c0 * C + 4 * (int64_t)threadIdx.x; e < ce * C; e += 4 * kLThreads) {
        float4 c;
        float4 g = guided(a, e, c);
        if (a.type == 1) {
            g.x = g.x * rr;
            g.y = g.y * rr;
            g.z = g.z * rr;
            g.w = g.w * rr;
        }
        *(float4 *)(a.out + e) = g;
    }
}

struct SdeArgs {
    const float *x, *v, *noise, *xn_in;  // noise != nullptr: sample; else evaluate xn_in
    float *xn_out, *logp;
    const int32_t *cu;
    int n, C, nchunk;
    const float *t_cur, *t_next;
    float eta;
    float *part;  // [n][nchunk]: sum of (x_next - mu)^2 of each chunk
    const int32_t *err;
};

// Per-request constants of the step: dt, the drift factor k = s^2 / (2 t),
// 1 - t and the standard deviation s sqrt(dt), in fp32.
struct SdeStep {
    float dt, k, omt, sd;
};

__device__ __forceinline__ SdeStep sde_step(const SdeArgs &a, int b) {
    const float t = a.t_cur[b], tn = a.t_next[b];
    SdeStep st;
    st.dt = t - tn;
    const float den = 1.0f - (t < 1.0f ? t : tn);
    const float s = a.eta * sqrtf(t / den);
    st.k = (s * s) / (2.0f * t);
    st.omt = 1.0f - t;
    st.sd = s * sqrtf(st.dt);
    return st;
}

__device__ __forceinline__ float sde_mu(const SdeStep &st, float x, float v) {
    return x - st.dt * (v + st.k * (x + st.omt * v));
}

// The step on a chunk: the mean, the sample (sampling mode) and the chunk's
// sum of squared deviations of x_next from the mean (thread i takes float4
// groups i, i+256, ... in order; then the workgroup tree).
__global__ void __launch_bounds__(kLThreads) sde_step_kernel(SdeArgs a) {
    __shared__ float s_red[4];
    if (__builtin_amdgcn_readfirstlane(*(volatile const int32_t *)a.err) != 0) return;
    const int b = (int)blockIdx.x / a.nchunk, j = (int)blockIdx.x % a.nchunk;
    const int64_t r0 = a.cu[b], r1 = a.cu[b + 1];
    const int64_t c0 = r0 + (int64_t)j * kChunkRows;
    if (c0 >= r1) return;
    const int64_t ce = min(c0 + kChunkRows, r1);
    const SdeStep st = sde_step(a, b);
    float q = 0.0f;
    for (int64_t e = c0 * a.C + 4 * (int64_t)threadIdx.x; e < ce * a.C; e += 4 * kLThreads) {
        const float4 x = ld4(a.x + e), v = ld4(a.v + e);
        const float m[4] = {sde_mu(st, x.x, v.x), sde_mu(st, x.y, v.y), sde_mu(st, x.z, v.z), sde_mu(st, x.w, v.w)};
        float xn[4];
        if (a.noise != nullptr) {
            const float4 z = ld4(a.noise + e);
            xn[0] = m[0] + st.sd * z.x;
            xn[1] = m[1] + st.sd * z.y;
            xn[2] = m[2] + st.sd * z.z;
            xn[3] = m[3] + st.sd * z.w;
            *(float4 *)(a.xn_out + e) = make_float4(xn[0], xn[1], xn[2], xn[3]);
        } else {
            const float4 y = ld4(a.xn_in + e);
            xn[0] = y.x;
            xn[1] = y.y;
            xn[2] = y.z;
            xn[3] = y.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float d = xn[i] - m[i];
            q = q + d * d;
        }
    }
    q = block_sum(q, s_red);
    if (threadIdx.x == 0) a.part[(int64_t)b * a.nchunk + j] = q;
}

// logp of each request: its chunks' sums in ascending order, then
// -q / (2 sd^2) - n (log(sd) + log(2 pi) / 2) with n = rows * C elements.
__global__ void __launch_bounds__(kLThreads) sde_logp_kernel(SdeArgs a) {
    if (__builtin_amdgcn_readfirstlane(*(volatile const int32_t *)a.err) != 0) return;
    const int b = (int)(blockIdx.x * kLThreads + threadIdx.x);
    if (b >= a.n) return;
    const int64_t rows_b = (int64_t)a.cu[b + 1] - a.cu[b];
    const int nch = (int)((rows_b + kChunkRows - 1) / kChunkRows);
    float q = 0.0f;
    for (int j = 0; j < nch; ++j) q = q + a.part[(int64_t)b * a.nchunk + j];
    const SdeStep st = sde_step(a, b);
    const float ne = (float)(rows_b * a.C);
    a.logp[b] = -(q / (2.0f * (st.sd * st.sd))) - ne * (logf(st.sd) + kHalfLog2Pi);
}

}  // namespace

int latent_chunks(int64_t max_rows) { return (int)((max_rows + kChunkRows - 1) / kChunkRows); }

hipError_t launch_cfg_combine(const float *vc, const float *vt, const float *vi, float *out, const int32_t *cu,
                              int n, int64_t rows, int C, int64_t max_rows, const float *t, float s_text, float s_img,
                              float t_lo, float t_hi, float rmin, int type, int32_t *err, float *part,
                              hipStream_t stream) {
    hipLaunchKernelGGL(latent_check_kernel, dim3(1), dim3(kLThreads), 0, stream, cu, n, rows, max_rows, t,
                       (const float *)nullptr, 0, err);
    CfgArgs a{vc, vt, vi, out, cu, n, C, latent_chunks(max_rows), t, s_text, s_img, t_lo, t_hi, rmin, type, part, err};
    const dim3 grid((unsigned)((int64_t)n * a.nchunk));
    if (type == 1) hipLaunchKernelGGL(cfg_partial_kernel, grid, dim3(kLThreads), 0, stream, a);
    hipLaunchKernelGGL(cfg_apply_kernel, grid, dim3(kLThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_sde_step(const float *x, const float *v, const float *noise, const float *xn_in, float *xn_out,
                           float *logp, const int32_t *cu, int n, int64_t rows, int C, int64_t max_rows,
                           const float *t_cur, const float *t_next, float eta, int32_t *err, float *part,
                           hipStream_t stream) {
    hipLaunchKernelGGL(latent_check_kernel, dim3(1), dim3(kLThreads), 0, stream, cu, n, rows, max_rows, t_cur,
                       t_next, 1, err);
    SdeArgs a{x, v, noise, xn_in, xn_out, logp, cu, n, C, latent_chunks(max_rows), t_cur, t_next, eta, part, err};
    hipLaunchKernelGGL(sde_step_kernel, dim3((unsigned)((int64_t)n * a.nchunk)), dim3(kLThreads), 0, stream, a);
    hipLaunchKernelGGL(sde_logp_kernel, dim3((unsigned)((n + kLThreads - 1) / kLThreads)), dim3(kLThreads), 0, stream,
                       a);
    return hipGetLastError();
}

}  // namespace mot
