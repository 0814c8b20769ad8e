// Shared joint attention (gfx950): the attention that the two weight sets
// share.  The RL-Kernel RFC page "[RFC][BAGEL-7B-MoT][CUDA/ROCm] WS1/WS2
// kernel roadmap and integration plan" lists it as the "gen_joint_attention"
// work item (section 5); its reference hazards (section 2) note that a
// cached prefill needs a causal mask aligned at the bottom-right corner, and
// its numerical contract (section 3) rules out split-KV and unordered merges.
//
// out[i][h] = softmax_j(q_i . k_j / sqrt(128)) v_j over the keys j that query
// i sees: all Tk keys, or with the causal mask j <= i + (Tk - Tq).  q head h
// reads kv head h / (hq / hkv).  Head dimension 128.
//
// Workgroup: 4 waves, 128 query rows of one q head (32 per wave).  Keys go in
// blocks of 64, from key 0 upwards, one block at a time through LDS; each
// query keeps an online softmax (running max and sum, in fp32) and its fp32
// output accumulators.  No block is split across workgroups, so every output
// element sees one accumulation order, fixed by the key blocks -- which start
// at key 0 whatever the pack -- and the row's bytes do not depend on the
// other queries of the pack.  Blocks past a query's last visible key (the
// workgroup runs to its last query's) change nothing: their scores are -inf,
// so the rescale factor is exactly 1 and the weights exactly 0.
//
// MFMA (v_mfma_f32_32x32x16_bf16, D[i][j] = sum_k a_i[k] b_j[k], lane l
// holding a_i, b_j for i, j = l & 31 at k = 8 (l >> 5) + 0..7, and D[i][j]
// for j = l & 31, i = 8 (r >> 2) + 4 (l >> 5) + (r & 3) in register r):
//   scores  S^T[key][q] = sum_d K[key][d] Q[q][d]       (a = K row, b = Q row)
//   output  O^T[d][q]   = sum_key V^T[d][key] P[q][key]  (a = V^T row, b = P)
// so a lane holds its query's scores for 16 of each 32 keys, and its half-
// wave partner (lane ^ 32) the other 16; the P operand is the lane's own
// scores in register order, and the V^T operand lists the same keys in the
// same slots (keys 4h..4h+3, then 8+4h..8+4h+3 of each 16).  V is staged as
// it lies in memory, one key per LDS row, and the V^T operand comes from
// two transposing LDS reads (ds_read_b64_tr_b16: within each 16-lane group,
// element e of lane 4a+b is element b of the 4-value chunk that lane 4e+a
// addresses), so no transposed copy of V is made.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mot_internal.h"

namespace mot {
namespace {

typedef __bf16 at_bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 at_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float at_f32x2_t __attribute__((ext_vector_type(2)));
typedef float at_f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t at_u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t at_u32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t at_rsrc_t;

constexpr int kD = 128;            // head dimension
constexpr int kBQ = 128;           // query rows per workgroup
constexpr int kBK = 64;            // keys per block
constexpr int kKRow = kD * 2 + 16;   // bytes per staged K row (16 bytes of padding)
// bytes per staged V row (one key): no padding; its eight 32-byte granules
// are permuted by the row's index mod 4 (v_swz), so that the transposing
// reads of four consecutive keys by 16 lanes, and of the two 16-column halves
// by 32 lanes, fall on distinct banks
constexpr int kVRow = kD * 2;
constexpr int kThreads = 256;
// LDS fragments kept this many MFMAs ahead of the MFMAs that use them
// (scores: K fragments, one read each; output: V^T fragments, two
// transposing reads each).  The compiler's own order ran them one or two
// ahead; six K and ten V^T fragments measured fastest (same bytes).
constexpr int KPF = 6, VPF = 10;
constexpr float kLazy = 8.0f;        // log2 headroom of the softmax reference max

// Raw buffer over [base, base + bytes): a load whose per-lane offset lies
// past the end reads zeros (the wave-uniform offset is not range-checked).
__device__ __forceinline__ at_rsrc_t at_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// {x of lane l, x of lane l ^ 32} in every lane (v_permlane32_swap), lower
// half's value first
__device__ __forceinline__ void at_halves(float x, float &lo, float &hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}

// granule permutation of staged V row r: granule g is stored at g ^ v_swz(r)
// (0, 5, 2, 7 for r mod 4 = 0..3: distinct mod 4, and with their neighbours
// g ^ 1 they cover all eight granules)
__device__ __forceinline__ int v_swz(int r) { return ((r & 1) ? 5 : 0) ^ (r & 2); }

typedef short at_i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) at_i16x4_t lds_i16x4_t;

// max(a, b, c) and max(a, b) of finite or infinite scores in one instruction
// each (written out: the compiler's fmaxf first quiets every input with a
// v_max x, x of its own, which doubles the instruction count of a max tree)
__device__ __forceinline__ float at_max3(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}
__device__ __forceinline__ float at_max2(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// fp32 -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t at_pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((at_f32x2_t){lo, hi}, at_bf16x2_t));
}

__global__ void __launch_bounds__(kThreads, 2) attention_kernel(AttnArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t ks[kBK * kKRow];
    __shared__ __attribute__((aligned(16))) uint8_t vs[kBK * kVRow];

    const int tid = (int)threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int lq = lane & 31, hh = lane >> 5;
    // Sequence of this workgroup: one sequence, or (packed sequences) the
    // block's share of nqb query blocks x hq heads of sequence b, whose rows
    // are [cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]).
    int64_t Tq = a.Tq, Tk = a.Tk, qs = 0, ks0 = 0;
    unsigned rem = blockIdx.x;
    if (a.cu_q) {
        if (__builtin_amdgcn_readfirstlane(*(volatile const int32_t *)a.err) != 0) return;  // lengths invalid
        const int b = (int)(blockIdx.x / (unsigned)(a.nqb * a.hq));
        rem = blockIdx.x % (unsigned)(a.nqb * a.hq);
        qs = a.cu_q[b];
        Tq = a.cu_q[b + 1] - qs;
        ks0 = a.cu_k[b];
        Tk = a.cu_k[b + 1] - ks0;
    }
    // heads vary fastest and the query blocks run from the last one down, so
    // that under the causal mask the longest workgroups start first
    const int nqb = a.cu_q ? a.nqb : (int)((Tq + kBQ - 1) / kBQ);
    const int h = (int)(rem % (unsigned)a.hq);
    const int kvh = h / (a.hq / a.hkv);
    const int64_t q0 = (int64_t)(nqb - 1 - (int)(rem / (unsigned)a.hq)) * kBQ;
    if (q0 >= Tq) return;  // (packed sequences shorter than the longest)
    const int64_t qrow = q0 + wave * 32 + lq;
    const int64_t shift = Tk - Tq;  // bottom-right alignment of the causal mask
    const uint16_t *qbase = a.q + qs * a.ldq;
    const uint16_t *kbase0 = a.k + ks0 * a.ldk;
    const uint16_t *vbase0 = a.v + ks0 * a.ldv;
    uint16_t *obase = a.out + qs * a.ldo;

    // this query's last visible key, and the keys the workgroup needs
    int64_t last = a.causal ? qrow + shift : Tk - 1;
    if (last > Tk - 1) last = Tk - 1;
    // the wave's smallest last visible key: blocks up to it need no mask
    int64_t wlast = a.causal ? q0 + wave * 32 + shift : Tk - 1;
    if (wlast > Tk - 1) wlast = Tk - 1;
    const int64_t qlast = (q0 + kBQ - 1 < Tq - 1) ? q0 + kBQ - 1 : Tq - 1;
    int64_t kend = a.causal ? qlast + shift + 1 : Tk;
    if (kend > Tk) kend = Tk;
    const int nkb = kend > 0 ? (int)((kend + kBK - 1) / kBK) : 0;

    // Q fragments: row qrow (clamped; rows past Tq are never stored), columns
    // h*128 + 16 s + 8 hh .. +8
    at_bf16x8_t qf[8];
    {
        const int64_t qr = qrow < Tq ? qrow : Tq - 1;
        const uint16_t *qp = qbase + qr * a.ldq + h * kD + 8 * hh;
#pragma unroll
        for (int s = 0; s < 8; ++s) qf[s] = *(const at_bf16x8_t *)(qp + 16 * s);
    }

    // staging: 1024 16-byte chunks of K and of V (64 key rows x 16 each)
    // per block, four of each per thread, through raw buffers with 32-bit
    // offsets.  A chunk's whole offset (block row and key row) is the
    // per-lane offset: only that part of a buffer address is checked against
    // the buffer's size (the wave-uniform offset is not), so the rows of a
    // last, partial block that lie past key Tk - 1 start at or beyond the
    // buffer's end and read zeros instead of memory past the K and V views
    // (zero V rows keep the masked keys' products exactly 0).
    const at_rsrc_t kres =
        at_rsrc(kbase0 + kvh * kD, Tk > 0 ? (uint32_t)(((Tk - 1) * a.ldk + (a.hkv - kvh) * kD) * 2) : 0u);
    const at_rsrc_t vres =
        at_rsrc(vbase0 + kvh * kD, Tk > 0 ? (uint32_t)(((Tk - 1) * a.ldv + (a.hkv - kvh) * kD) * 2) : 0u);
    uint32_t koff[4], voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int idx = tid + kThreads * i;
        koff[i] = (uint32_t)(idx >> 4) * (uint32_t)a.ldk * 2u + (uint32_t)(idx & 15) * 16u;
        voff[i] = (uint32_t)(idx >> 4) * (uint32_t)a.ldv * 2u + (uint32_t)(idx & 15) * 16u;
    }
    at_u32x4_t kr[4], vr[4];
    auto load_block = [&](int kb) {
        const uint32_t kblk = (uint32_t)kb * kBK * (uint32_t)a.ldk * 2u;
        const uint32_t vblk = (uint32_t)kb * kBK * (uint32_t)a.ldv * 2u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            kr[i] = __builtin_amdgcn_raw_buffer_load_b128(kres, (int)(koff[i] + kblk), 0, 0);
            vr[i] = __builtin_amdgcn_raw_buffer_load_b128(vres, (int)(voff[i] + vblk), 0, 0);
        }
    };
    auto store_block = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + kThreads * i;
            const int r = idx >> 4, c = idx & 15;  // key row, 16-byte chunk
            *(at_u32x4_t *)(ks + r * kKRow + c * 16) = kr[i];
            *(at_u32x4_t *)(vs + r * kVRow + (((c >> 1) ^ v_swz(r)) << 5) + ((c & 1) << 4)) = vr[i];
        }
    };
    // V^T fragment addresses: lane l (16-lane group position L = l & 15)
    // addresses key row 4 (l >> 5) + (L >> 2) of each 8-key group and the
    // four values d = 32 dt + 16 ((l >> 4) & 1) + 4 (L & 3) + 0..3, so that it
    // receives d = 32 dt + (l & 31) for four consecutive keys
    uint32_t vrd[4];
    {
        const int L = lane & 15;
        const int r = 4 * hh + (L >> 2);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            vrd[dt] = (uint32_t)(r * kVRow + (((2 * dt + ((lane >> 4) & 1)) ^ v_swz(r)) << 5) + 8 * (L & 3));
    }

    at_f32x16_t oacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) oacc[t] = (at_f32x16_t){};
    // running max of the raw scores; the weights are 2^(c (s - m)) with the
    // constant c = log2(e)/sqrt(128) rounded once to fp32 (v_exp_f32)
    float m_run = -INFINITY, l_run = 0.0f;
    const float scale = a.scale_log2e;

    if (nkb > 0) load_block(0);
    for (int kb = 0; kb < nkb; ++kb) {
        __syncthreads();  // the previous block's LDS reads are done
        store_block();
        __syncthreads();
        if (kb + 1 < nkb) load_block(kb + 1);

        // scores of keys kb*64 + [0, 64)
        // (the two tiles' chains alternate, so no MFMA waits on the one
        // just issued; each tile's k order is unchanged)
        // The MFMA stretches run at raised wave priority: the two waves that
        // share a SIMD then drift out of phase, one issuing MFMAs while the
        // other does its softmax arithmetic (measured 4-7% faster, same
        // bytes).
        __builtin_amdgcn_s_setprio(1);
        at_f32x16_t sacc[2] = {(at_f32x16_t){}, (at_f32x16_t){}};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                const at_bf16x8_t kf = *(const at_bf16x8_t *)(ks + (kt * 32 + lq) * kKRow + 16 * hh + 32 * s);
                sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kt], 0, 0, 0);
            }
        }
        // K fragment reads KPF ahead of the score MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, KPF, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i + KPF < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        // mask (only where the block reaches past the wave's first row's
        // last visible key), block maximum of the raw scores
        if ((int64_t)kb * kBK + kBK - 1 > wlast) {
            const int rel = (int)(last - (int64_t)kb * kBK);  // last visible key, block-relative
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kt * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
                    if (key > rel) sacc[kt][r] = -INFINITY;
                }
            }
        }
        // the lane's 32 scores by a three-input tree (16 instructions; the
        // maximum does not depend on the grouping), then the two half-waves
        float mx;
        {
            float v32[32], w12[12], x4[4];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                v32[r] = sacc[0][r];
                v32[16 + r] = sacc[1][r];
            }
#pragma unroll
            for (int i = 0; i < 10; ++i) w12[i] = at_max3(v32[3 * i], v32[3 * i + 1], v32[3 * i + 2]);
            w12[10] = v32[30];
            w12[11] = v32[31];
#pragma unroll
            for (int i = 0; i < 4; ++i) x4[i] = at_max3(w12[3 * i], w12[3 * i + 1], w12[3 * i + 2]);
            const float lane_max = at_max2(at_max3(x4[0], x4[1], x4[2]), x4[3]);
            float mlo, mhi;
            at_halves(lane_max, mlo, mhi);
            mx = at_max2(mlo, mhi);
        }
        float t16[16];
        // The reference max moves only when a score exceeds it by more than
        // kLazy / c (weights then stay below 2^kLazy, far inside fp32 and
        // bf16 range): most blocks keep it, so the output needs no rescale.
        // The rule looks at the row's own scores only.
        // (no key seen yet: m_run = -inf makes d +inf or NaN, so the max is taken)
        const float d = (mx - m_run) * scale;
        const float m_new = d <= kLazy ? m_run : mx;
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;  // no key seen yet: weights 0
        // weight = 2^(s c - m c), c = log2(e)/sqrt(128): one fma per score
        const float mc = m_use * scale;
        // exactly 1 while the running max holds (blocks past a row's last
        // visible key then leave its state bit for bit as it was)
        const float alpha = m_run == m_use ? 1.0f : __builtin_amdgcn_exp2f(__builtin_fmaf(m_run, scale, -mc));
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], scale, -mc));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) t16[r] = sacc[0][r] + sacc[1][r];
#pragma unroll
        for (int w = 8; w >= 1; w >>= 1) {
#pragma unroll
            for (int r = 0; r < w; ++r) t16[r] = t16[r] + t16[r + w];
        }
        float slo, shi;
        at_halves(t16[0], slo, shi);
        const float psum = slo + shi;  // same operands, same order, in both halves
        l_run = l_run * alpha + psum;
        m_run = m_new;
        // alpha is exactly 1 while the running max holds: skip the rescale
        // when it holds for the whole wave (same bytes either way)
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int t = 0; t < 4; ++t) oacc[t] *= alpha;
        }

        // P as bf16 operands: k-step s2 covers registers 8 (s2 & 1) .. +8 of
        // score tile s2 >> 1
        at_bf16x8_t pf[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int kt = s2 >> 1, r0 = 8 * (s2 & 1);
            const at_u32x4_t pk = {at_pack2(sacc[kt][r0 + 0], sacc[kt][r0 + 1]),
                                   at_pack2(sacc[kt][r0 + 2], sacc[kt][r0 + 3]),
                                   at_pack2(sacc[kt][r0 + 4], sacc[kt][r0 + 5]),
                                   at_pack2(sacc[kt][r0 + 6], sacc[kt][r0 + 7])};
            pf[s2] = __builtin_bit_cast(at_bf16x8_t, pk);
        }
        __builtin_amdgcn_s_setprio(1);
        // O^T += V^T P^T, keys in ascending 16-key steps (the four output
        // tiles' chains alternate)
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                // keys 16 s2 + 4 hh + 0..3, then 16 s2 + 8 + 4 hh + 0..3
                const at_u32x2_t lo = __builtin_bit_cast(
                    at_u32x2_t,
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vs + vrd[dt] + s2 * 16 * kVRow)));
                const at_u32x2_t hi = __builtin_bit_cast(
                    at_u32x2_t,
                    __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(vs + vrd[dt] + (s2 * 16 + 8) * kVRow)));
                const at_u32x4_t vv = {lo.x, lo.y, hi.x, hi.y};
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(at_bf16x8_t, vv), pf[s2],
                                                                   oacc[dt], 0, 0, 0);
            }
        }
        // (two transposing reads per V^T fragment)
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * VPF, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (i + VPF < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    }

    if (qrow >= Tq) return;
    uint16_t *op = obase + qrow * a.ldo + h * kD + 4 * hh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = l_run > 0.0f ? oacc[dt][4 * j + e] / l_run : 0.0f;
            *(at_u32x2_t *)(op + dt * 32 + 8 * j) = (at_u32x2_t){at_pack2(v[0], v[1]), at_pack2(v[2], v[3])};
        }
    }
}

// Checks the packed sequences' cumulative lengths and writes the error word
// (0, or kErrSeqlens): cu_q and cu_k start at 0, never decrease, end at Tq
// and Tk, and no sequence has more than max_q rows.  One workgroup.
constexpr int kErrSeqlens = 8;  // MOT_ERR_SEQLENS

__global__ void __launch_bounds__(256) seqlens_check_kernel(const int32_t *cu_q, const int32_t *cu_k, int n,
                                                            int64_t Tq, int64_t Tk, int64_t max_q, int32_t *err) {
    __shared__ int bad;
    if (threadIdx.x == 0) bad = (cu_q[0] != 0 || cu_k[0] != 0 || cu_q[n] != Tq || cu_k[n] != Tk) ? 1 : 0;
    __syncthreads();
    for (int b = (int)threadIdx.x; b < n; b += (int)blockDim.x) {
        const int64_t lq = (int64_t)cu_q[b + 1] - cu_q[b], lk = (int64_t)cu_k[b + 1] - cu_k[b];
        if (lq < 0 || lk < 0 || lq > max_q) atomicOr(&bad, 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) *err = bad ? kErrSeqlens : 0;
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, hipStream_t stream) {
    const int64_t nqb = a.cu_q ? a.nqb : (a.Tq + kBQ - 1) / kBQ;
    const int64_t nseq = a.cu_q ? a.nseq : 1;
    const dim3 grid((unsigned)(nseq * a.hq * nqb));
    hipLaunchKernelGGL(attention_kernel, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_seqlens_check(const int32_t *cu_q, const int32_t *cu_k, int n, int64_t Tq, int64_t Tk,
                                int64_t max_q, int32_t *err, hipStream_t stream) {
    hipLaunchKernelGGL(seqlens_check_kernel, dim3(1), dim3(256), 0, stream, cu_q, cu_k, n, Tq, Tk, max_q, err);
    return hipGetLastError();
}

}  // namespace mot
