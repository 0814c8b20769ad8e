// HIP kernels of the MoT token-routed projection for gfx950 (MI355X).
//
//  * plan_kernel   -- the routing plan: stable partition of the pack's rows by
//                     modality byte (the per-set segment list), for packs
//                     larger than the GEMM kernels build in-kernel.
//  * gemm_kernel   -- persistent routed GEMM  y = A * W_set^T on bf16 MFMA
//                     with fp32 accumulation (256x256 tiles on a five-slot
//                     LDS ring, 128x128 tiles for the rest); in-kernel
//                     segment list; optional routed-RMSNorm prologue on the A
//                     operand; optional SwiGLU epilogue (gate/up pairs).
//  * skinny_kernel -- the same GEMM for packs of at most 128 rows, spread
//                     over one workgroup per 32 output columns, all four
//                     waves streaming weights (weight-bound).
//  * norm_kernel   -- routed fused add-RMSNorm.
//  * qk_norm_rope_kernel -- routed per-head QK RMSNorm, then the bf16 rotary
//                     embedding, in place on the QKV rows.
//  * transpose_kernel -- bf16 transpose (operands of the routed backward).
//
// Numerical contract (RL-Kernel RFC page "[RFC][BAGEL-7B-MoT] WS1/WS2 kernel
// roadmap", section 3): one fixed fp32 accumulation order per output element,
// no split-K, no atomics, no fast math, casts only where declared.  A row's
// bytes depend only on its own data: the GEMM's per-element k order is fixed
// (one MFMA instruction, k ascending in 16-wide steps) whatever the tile shape,
// the tile's position in the grid or the pack's composition.
//
// Built with -ffp-contract=off: every fp32 multiply and add in the epilogues
// and the norm rounds where the source says so.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "mot_internal.h"

namespace mot {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kErrModality = 6;  // MOT_ERR_MODALITY
constexpr int kErrPlan = 9;      // MOT_ERR_PLAN

// ---- bf16 helpers (format definition: upper 16 bits of an IEEE binary32) ----

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest, ties to even: gfx950's v_cvt_pk_bf16_f32
// (two values per instruction; a NaN comes out as a quiet NaN).  Every
// rounding to bf16 in this library goes through it.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ---- per-head QK RMSNorm + rotary helpers (standalone kernel and fused epilogue) ----

constexpr int kErrPosition = 7;  // MOT_ERR_POSITION
constexpr int kQkChunks = 2;     // 4-head chunks per wave (8 heads)

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_at(const u32x4_t &v, int e) {
    return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
}

// The value v holds in lane (i + N) mod 16 of this lane's 16-lane row (a DPP
// row rotation: no LDS round trip).
template <int N>
__device__ __forceinline__ uint32_t row_rot(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x120 + N, 0xf, 0xf, false);
}

// One head of one row, as 16 lanes hold it (lane gi of the group: elements
// 8 gi .. 8 gi + 7 in v; the groups are DPP rows): the head's RMSNorm (sum of
// squares per lane in element order, then the xor-butterfly over the group:
// one fixed tree), y = bf16((x * rstd) * w), then the rotate-half rotation
// with the partner 64 columns away in lane gi ^ 8.  The butterfly's partners
// come from row rotations by 8, 4, 2, 1: once a value is the same in lanes
// i and i ^ 8 (and i ^ 4 ...), lane (i + 4) mod 16 holds the value of lane
// i ^ 4, and so on, so each lane adds exactly the xor partner's value (the
// same sums, bit for bit, as an exchange by lane xor).  `live` lanes hold a
// real head; every lane of the wave must call it with all lanes active.
// Shared by the standalone kernel and the QKV GEMM's fused epilogue, so both
// give the same bytes.
__device__ __forceinline__ u32x4_t qk_head(const u32x4_t &v, bool live, int gi, float eps, const u32x4_t &wv,
                                           const u32x4_t &cv, const u32x4_t &sv) {
    float ss = 0.0f;
    if (live) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = bf16_at(v, e);
            ss = e == 0 ? x * x : ss + x * x;
        }
    }
    ss += __uint_as_float(row_rot<8>(__float_as_uint(ss)));
    ss += __uint_as_float(row_rot<4>(__float_as_uint(ss)));
    ss += __uint_as_float(row_rot<2>(__float_as_uint(ss)));
    ss += __uint_as_float(row_rot<1>(__float_as_uint(ss)));
    const float rstd = 1.0f / sqrtf(ss / 128.0f + eps);
    u32x4_t y;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        y[e] = pack2(bf16_lo(v[e]) * rstd * bf16_lo(wv[e]), bf16_hi(v[e]) * rstd * bf16_hi(wv[e]));
    u32x4_t z;
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = row_rot<8>(y[e]);
    // out = bf16(bf16(y c) + bf16(sg (y' s))), sg = -1 in the first half of
    // the head (y c - y' s), +1 in the second.  The sign goes into the sine's
    // sign bits (negating a factor negates the product exactly, zeros
    // included), each pair of roundings is one packed conversion, and the
    // sum is rounded once by the final pack (rounding a bf16 value again
    // leaves it as it is): the same bits, fewer instructions.
    const uint32_t sflip = gi < 8 ? 0x80008000u : 0u;
    u32x4_t o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t c = pack2(bf16_lo(y[e]) * bf16_lo(cv[e]), bf16_hi(y[e]) * bf16_hi(cv[e]));
        const uint32_t sw = sv[e] ^ sflip;
        const uint32_t t = pack2(bf16_lo(z[e]) * bf16_lo(sw), bf16_hi(z[e]) * bf16_hi(sw));
        o[e] = pack2(bf16_lo(c) + bf16_lo(t), bf16_hi(c) + bf16_hi(t));
    }
    return o;
}

// ============================================================================
// Routing plan
// ============================================================================

// One workgroup of 1024 threads walks the pack in chunks of 16 rows per
// thread.  Pass 1 counts the und rows and checks the bytes; pass 2 writes
// each row's position: und rows at [0, n_und) and gen rows at [n_und, T), both
// in ascending row order (an exclusive scan of per-thread counts).
constexpr int kPlanThreads = 1024;
constexpr int kPlanPerThread = 16;

__device__ __forceinline__ int block_exclusive_scan(int v, int *s_wave, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    if (lane == 63) s_wave[wave] = inc;
    __syncthreads();
    int wave_base = 0, sum = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
        int t = s_wave[w];
        if (w < wave) wave_base += t;
        sum += t;
    }
    __syncthreads();
    total = sum;
    return wave_base + inc - v;
}

__global__ void __launch_bounds__(kPlanThreads)
plan_kernel(const uint8_t *__restrict__ modality, int T, int32_t *__restrict__ hdr,
            int32_t *__restrict__ perm) {
    __shared__ int s_wave[kPlanThreads / 64];
    const int chunk = kPlanThreads * kPlanPerThread;
    // pass 1: count und rows, detect invalid bytes
    int n_und = 0, bad = 0;
    for (int base = 0; base < T; base += chunk) {
        const int r0 = base + threadIdx.x * kPlanPerThread;
        int cu = 0;
        for (int i = 0; i < kPlanPerThread; ++i) {
            const int r = r0 + i;
            if (r < T) {
                const uint8_t m = modality[r];
                cu += (m == 0);
                bad |= (m > 1);
            }
        }
        int tot;
        (void)block_exclusive_scan(cu, s_wave, tot);
        n_und += tot;
    }
    bad = __syncthreads_or(bad);
    if (bad) {
        if (threadIdx.x == 0) {
            hdr[0] = kErrModality;
            hdr[1] = 0;
            hdr[2] = 0;
            hdr[3] = T;
        }
        return;
    }
    // pass 2: positions
    int und_base = 0, gen_base = n_und;
    for (int base = 0; base < T; base += chunk) {
        const int r0 = base + threadIdx.x * kPlanPerThread;
        uint32_t mask = 0;  // bit i: row r0+i is gen
        int cu = 0, cnt = 0;
        for (int i = 0; i < kPlanPerThread; ++i) {
            const int r = r0 + i;
            if (r < T) {
                const uint8_t m = modality[r];
                mask |= uint32_t(m) << i;
                cu += (m == 0);
                ++cnt;
            }
        }
        int tot_u, tot_all;
        const int pu = block_exclusive_scan(cu, s_wave, tot_u);
        const int pa = block_exclusive_scan(cnt, s_wave, tot_all);
        int iu = und_base + pu;
        int ig = gen_base + (pa - pu);
        for (int i = 0; i < cnt; ++i) {
            if ((mask >> i) & 1u)
                perm[ig++] = r0 + i;
            else
                perm[iu++] = r0 + i;
        }
        und_base += tot_u;
        gen_base += tot_all - tot_u;
    }
    if (threadIdx.x == 0) {
        hdr[0] = 0;
        hdr[1] = n_und;
        hdr[2] = T - n_und;
        hdr[3] = T;
    }
}

// ============================================================================
// Modality bytes from the two index sets
// ============================================================================
//
// The pack's rows come as two index lists (understanding rows, generation
// rows).  Every row must be in exactly one list, once.  Per row, a word of
// the workspace counts the row's appearances in its low 30 bits (at most
// n_und + n_gen = T <= 2^24, so it never carries) and every generation-list
// appearance also adds 2^30; the adds are integer adds, so the result does
// not depend on their order.  A count of exactly 1 gives the row's byte: 0,
// or 1 when that one appearance was in the generation list.  Any other
// count (a row in neither list, in both, or twice in one) gives 0xFF, an
// invalid byte, and raises MOT_ERR_INDEX_SET (a routed call on those bytes
// then writes nothing).  An index outside [0, T) raises the same error.

constexpr int kErrIndexSet = 10;  // MOT_ERR_INDEX_SET
constexpr uint32_t kGenFlag = 1u << 30;
constexpr uint32_t kCountMask = kGenFlag - 1u;

__global__ void __launch_bounds__(256)
index_clear_kernel(uint32_t *__restrict__ cnt, int T, int32_t *__restrict__ err) {
    const int stride = (int)(gridDim.x * blockDim.x);
    for (int t = (int)(blockIdx.x * blockDim.x + threadIdx.x); t < T; t += stride) cnt[t] = 0u;
    if (blockIdx.x == 0 && threadIdx.x == 0) *err = 0;
}

__global__ void __launch_bounds__(256)
index_count_kernel(const int32_t *__restrict__ und_idx, int n_und, const int32_t *__restrict__ gen_idx,
                   int n_gen, uint32_t *__restrict__ cnt, int T, int32_t *__restrict__ err) {
    const int stride = (int)(gridDim.x * blockDim.x);
    bool bad = false;
    for (int i = (int)(blockIdx.x * blockDim.x + threadIdx.x); i < n_und + n_gen; i += stride) {
        const bool is_gen = i >= n_und;
        const int r = is_gen ? gen_idx[i - n_und] : und_idx[i];
        if (r < 0 || r >= T) {
            bad = true;
            continue;
        }
        atomicAdd(cnt + r, is_gen ? kGenFlag + 1u : 1u);
    }
    if (bad) atomicMax(err, kErrIndexSet);
}

__global__ void __launch_bounds__(256)
index_finish_kernel(const uint32_t *__restrict__ cnt, int T, uint8_t *__restrict__ modality,
                    int32_t *__restrict__ err) {
    const int stride = (int)(gridDim.x * blockDim.x);
    bool bad = false;
    for (int t = (int)(blockIdx.x * blockDim.x + threadIdx.x); t < T; t += stride) {
        const uint32_t c = cnt[t];
        const uint8_t m = (c & kCountMask) == 1u ? (uint8_t)(c >> 30) : (uint8_t)0xFF;
        bad |= m == 0xFF;
        modality[t] = m;
    }
    if (bad) atomicMax(err, kErrIndexSet);
}

// ============================================================================
// Routed GEMM
// ============================================================================
//
// Orientation: the MFMA computes D[n][m] = sum_k W[n][k] * A[m][k] over a
// 32 (weight rows) x 32 (token rows) block with v_mfma_f32_32x32x16_bf16 --
// the only MFMA instruction used anywhere, so every output element sees the
// same k-step sequence (ascending, 16 per step) whatever the tile shape, the
// tile's place in the schedule or the pack's composition.
//
// Workgroup: 256 threads = 4 waves in a 2 (tokens) x 2 (weights) grid.  A
// tile is BM token rows of ONE weight set (a slice of that set's segment
// list) by BN weight rows.  Two tile shapes share one launch: 256x256 "big"
// tiles (two LDS stages of 64 KiB) fill whole rounds of the machine, and
// 128x128 "small" tiles (four stages of 32 KiB) cover what is left: the
// partial row blocks of each set and, split in quarters, the big tiles that
// would open a mostly idle extra round.  No tile splits K: each output
// element has one writer and one accumulation order.  The kernel is
// persistent: at most one workgroup per CU walks the tile list in rounds,
// and every workgroup derives the same list from the pack's set sizes.
//
// Pipeline: LDS stages of 64 k-columns (one 128-byte row piece per operand
// row, so every direct global->LDS 16-byte buffer load moves whole cache
// lines).  A stage is consumed in four 16-wide k-steps; each k-step's MFMAs
// run while the next k-step's fragments are read.  One barrier per stage,
// placed before its last k-step: there the next stage must have landed, the
// stage just read is free, and the last k-step's MFMAs cover both the first
// fragment reads of the next stage and the refill of the freed stage NS
// stages ahead.
//
// LDS rows are 128 bytes (64 bf16).  The 16-byte chunk c of staged row r is
// stored at chunk position c ^ swz(r), swz(r) = ((r >> 1) ^ ((r & 1) << 2)) & 7,
// which keeps any 8 or 16 consecutive rows read at one k-chunk on distinct
// LDS banks.
//
// Gathered rows: the A-operand row of tile slot i is the i-th row of the
// tile's slice of the segment list; slots past the slice's end load row 0 and
// are never stored.

constexpr int kBK = 64;          // k per stage
constexpr int kRowBytes = 128;   // kBK bf16
constexpr int kThreads = 256;

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

constexpr int kBigM = 256, kBigN = 256, kSmallM = 128, kSmallN = 128;
// Wide-round big tiles: 256 token rows x 224 weight rows (four waves of 64 x
// 224), for plain GEMMs whose weight rows split into 224-row tiles that fill
// whole rounds better than 256-row ones (O and down at N = 3584: 16 x 16 =
// 256 tiles at T = 4096, one per CU, against 16 x 14 = 224).
constexpr int kWideN = 224;
// Short big tiles: 192 token rows x 256 weight rows (four waves of 96 x 128),
// in the same instantiation, for packs whose 192-row blocks fill whole rounds
// better (O and down on a generation step's 3072 latent rows: 16 x 14 = 224
// tiles of 48 MFMA blocks, against 12 x 16 = 192 wide tiles of 56).
constexpr int kShortM = 192;
constexpr int kNarrowN = 64;  // weight rows of the narrow tiles (mid-size packs)
constexpr int kPartialBigRows = 160;    // rows from which a partial row block is a big tile
constexpr int kPartialShortRows = 120;  // the same for 192-row blocks

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Shape of the big tiles of a plain GEMM's schedule (U und and G gen rows,
// wrows weight rows, grid workgroups, small tiles of sn weight rows).
// Besides 256 x 256 the candidates are 256 x 224 (allow_wide, weight rows a
// multiple of 224) and 192 x 256 (allow_short), which always run whole.
// Each is priced at its rounds of big tiles (a partial round counted whole)
// times the tile's area; a candidate must fill more than half of the grid
// and leave the small tiles of its partial row blocks room in the idle
// workgroups of its last round (two each).  Short tiles must also beat
// 256 x 256 priced as the schedule runs it: a partial round at most half
// full as rounds of quarters, each a third of a big tile's time (the QKV
// projection at T = 4096: one round and a quarter round, where short tiles
// would need two rounds).  The cheapest wins; ties keep 256 x 256.  Shared
// by the kernels' schedule and the host's choice of instantiation.
__host__ __device__ inline void big_shape(int U, int G, int wrows, int grid, int sn, bool allow_wide,
                                          bool allow_short, int &bm, int &bn) {
    auto up = [](int a, int b) { return (a + b - 1) / b; };
    auto blocks = [](int n, int b, int partial) { return n / b + (n % b >= partial ? 1 : 0); };
    auto small_tiles = [&](int bu, int bg, int b) {
        const int ru = bu * b < U ? bu * b : U, rg = bg * b < G ? bg * b : G;
        return (up(U - ru, kSmallM) + up(G - rg, kSmallM)) * up(wrows, sn);
    };
    const int bu = blocks(U, kBigM, kPartialBigRows), bg = blocks(G, kBigM, kPartialBigRows);
    bm = kBigM;
    bn = kBigN;
    // costs in 64 bits: rounds times a tile's area overflows 32 bits for
    // the largest packs
    const int64_t area = (int64_t)kBigM * kBigN;
    int64_t best = up((bu + bg) * up(wrows, kBigN), grid) * area;
    if (allow_wide && wrows % kWideN == 0) {
        const int nw = (bu + bg) * (wrows / kWideN);
        const int rw = up(nw, grid);
        if (2 * nw > grid && rw * (int64_t)kBigM * kWideN < best && small_tiles(bu, bg, kBigM) <= 2 * (rw * grid - nw)) {
            best = rw * (int64_t)kBigM * kWideN;
            bn = kWideN;
        }
    }
    if (allow_short) {
        const int nn = (bu + bg) * up(wrows, kBigN), left = nn % grid;
        int64_t base = up(nn, grid) * area;
        if (2 * nn <= grid)
            base = up(4 * nn, grid) * area / 3;
        else if (nn > grid && left > 0 && 2 * left <= grid)
            base = (nn / grid) * area + up(4 * left, grid) * area / 3;
        const int su = blocks(U, kShortM, kPartialShortRows), sg = blocks(G, kShortM, kPartialShortRows);
        const int nsh = (su + sg) * up(wrows, kBigN);
        const int rs = up(nsh, grid);
        if (2 * nsh > grid && rs * (int64_t)kShortM * kBigN < (best < base ? best : base) &&
            small_tiles(su, sg, kShortM) <= 2 * (rs * grid - nsh)) {
            bm = kShortM;
            bn = kBigN;
        }
    }
}

struct Tile {
    int set;    // 0 = und, 1 = gen
    int first;  // offset of the tile's first row in the segment list
    int count;  // valid token rows
    int wrow0;  // first weight row of the tile (tile-local W row space)
    bool big;
};

// Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
// that each XCD receives a contiguous range of tile ids (tiles that share
// operands share that XCD's L2).
__device__ __forceinline__ int xcd_remap(int id, int total) {
    const int per = total >> 3, rem = total & 7;
    const int xcd = id & 7, local = id >> 3;
    return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + local;
}

// The tile list, computed identically by every workgroup from the set sizes:
// [nkeep big tiles][4*nleft quarter tiles][small tiles of the rows past the
// big row blocks].  mode 0: big tiles (full row blocks, and a partial one of
// at least kPartialBigRows rows) for whole rounds, small for the rest;
// mode 1: big tiles only; mode 2: small tiles only.
struct Schedule {
    int U, G;
    int bm;        // big tiles' token rows: kBigM, or kShortM
    int bn;        // big tiles' weight rows: kBigN, or kWideN
    int nwt, nws;  // weight tiles of bn and of sn rows
    int sn;        // small tiles' weight rows: 128, or 64 (narrow mode)
    int bu, nbr;   // big row blocks: und, und + gen
    int nkeep;     // big tiles run as such
    int nleft;     // big tiles run as four small tiles each
    int ru, rg;    // first row (within its set) of the small row blocks
    int su, sg;    // small row blocks of each set
    int ntiles;
};

// allow_wide: 256 x 224 big tiles where the cost model prefers them;
// short: 192 x 256 big tiles always (the host launched the short-tile
// instantiation because the cost model prefers them for the pack's size).
__device__ __forceinline__ Schedule make_schedule(int U, int G, int wrows, int grid, int mode,
                                                   int sn = kSmallN, bool allow_wide = false,
                                                   bool short_tiles = false) {
    Schedule s;
    s.sn = sn;
    s.U = U;
    s.G = G;
    s.bm = kBigM;
    s.bn = kBigN;
    s.nws = cdiv(wrows, sn);
    if (mode == 0 && short_tiles)
        s.bm = kShortM;
    else if (mode == 0 && allow_wide)
        big_shape(U, G, wrows, grid, sn, true, false, s.bm, s.bn);
    s.nwt = cdiv(wrows, s.bn);
    if (mode == 2) {
        s.bu = s.nbr = 0;
    } else if (mode == 1) {
        s.bu = cdiv(U, kBigM);
        s.nbr = s.bu + cdiv(G, kBigM);
    } else {
        // a set's partial row block runs as a big tile when it is mostly
        // full (its 128 x 128 tiles would be as padded and less efficient)
        const int partial = s.bm == kShortM ? kPartialShortRows : kPartialBigRows;
        s.bu = U / s.bm + (U % s.bm >= partial ? 1 : 0);
        s.nbr = s.bu + G / s.bm + (G % s.bm >= partial ? 1 : 0);
    }
    const int nbig = s.nbr * s.nwt;
    if (s.bn == kWideN || s.bm == kShortM) {
        s.nkeep = nbig;
    } else if (mode == 0 && 2 * nbig <= grid) {
        // big tiles would leave at least half of the machine idle through a
        // whole big-tile time: their quarters (at most two rounds of small
        // tiles, each about a third of a big tile's time) finish sooner
        s.nkeep = 0;
    } else if (mode == 0 && nbig >= grid) {
        // whole rounds as big tiles; a partial last round stays big when it
        // fills more than half of the grid (its quarters would take more
        // than two rounds of small tiles, each over a third of a big tile's
        // time), else it runs as quarters
        const int left = nbig % grid;
        s.nkeep = 2 * left > grid ? nbig : nbig - left;
    } else {
        s.nkeep = nbig;
    }
    s.nleft = nbig - s.nkeep;
    s.ru = min(s.bu * s.bm, U);
    s.rg = min((s.nbr - s.bu) * s.bm, G);
    s.su = cdiv(U - s.ru, kSmallM);
    s.sg = cdiv(G - s.rg, kSmallM);
    s.ntiles = s.nkeep + 4 * s.nleft + (s.su + s.sg) * s.nws;
    return s;
}

// Big tile b: 256-row block mb of the concatenated blocks [und..., gen...] by
// weight tile nb, ordered in groups of 4 weight tiles, all row blocks of a
// group before the next group (consecutive tiles share A rows or weight
// rows).  An XCD's 32 consecutive tiles then cover 8 row blocks by 4 weight
// tiles, fewer distinct operand panels than the row-grouped order gave with
// 18 weight tiles (the QKV projection), so more of its operand reads hit the
// XCD's L2: about 1% faster on the QKV, O, down and gate/up GEMMs.
__device__ __forceinline__ void big_tile(const Schedule &s, int b, int &mb, int &nb) {
    constexpr int GN = 4;
    const int height = GN * s.nbr;
    const int g = b / height;
    const int first_n = g * GN;
    const int gn = min(s.nwt - first_n, GN);
    const int in = b - g * height;
    mb = in / gn;
    nb = first_n + in % gn;
}

__device__ __forceinline__ void block_rows(const Schedule &s, int mb, Tile &ti) {
    if (mb < s.bu) {
        ti.set = 0;
        ti.first = mb * s.bm;
        ti.count = min(s.bm, s.U - ti.first);
    } else {
        const int off = (mb - s.bu) * s.bm;
        ti.set = 1;
        ti.first = s.U + off;
        ti.count = min(s.bm, s.G - off);
    }
}

__device__ __forceinline__ Tile tile_of(const Schedule &s, int t) {
    Tile ti;
    if (t < s.nkeep) {
        int mb, nb;
        big_tile(s, t, mb, nb);
        block_rows(s, mb, ti);
        ti.wrow0 = nb * s.bn;
        ti.big = true;
        return ti;
    }
    ti.big = false;
    const int q = t - s.nkeep;
    if (q < 4 * s.nleft) {
        // quarter (q & 3) of a big tile that would have opened an extra round
        int mb, nb;
        big_tile(s, s.nkeep + (q >> 2), mb, nb);
        block_rows(s, mb, ti);
        const int off = ((q >> 1) & 1) * kSmallM;
        ti.first += off;
        ti.count = min(kSmallM, ti.count - off);
        ti.wrow0 = nb * kBigN + (q & 1) * kSmallN;
    } else {
        // 128-row slices of the rows past the big row blocks of each set
        const int q2 = q - 4 * s.nleft;
        const int sm = q2 / s.nws, n = q2 % s.nws;
        if (sm < s.su) {
            const int r0 = s.ru + sm * kSmallM;
            ti.set = 0;
            ti.first = r0;
            ti.count = min(kSmallM, s.U - r0);
        } else {
            const int r0 = s.rg + (sm - s.su) * kSmallM;
            ti.set = 1;
            ti.first = s.U + r0;
            ti.count = min(kSmallM, s.G - r0);
        }
        ti.wrow0 = n * s.sn;
    }
    return ti;
}

// ---- in-kernel segment list ------------------------------------------------
//
// For packs of up to kInlineRouteMaxT rows every workgroup reads the modality
// bytes itself, once: thread i owns rows p*4096 + 16i .. +15 of each pass p
// and keeps one bit per row (und, gen) in registers.  Per tile, an exclusive
// scan of the per-thread counts gives the rank of each row among its set's
// rows (stable partition, ascending row order), and the rows of the tile's
// slice are written to LDS.  Integer work only.

constexpr int kRouteRows = 16;                     // rows per thread per pass
constexpr int kRoutePass = kThreads * kRouteRows;  // rows per pass
constexpr int kRoutePasses = 2;                    // 32 bits per thread and set
static_assert(kRoutePass * kRoutePasses == kInlineRouteMaxT, "in-kernel segment list size");

// Exclusive scan of v over the workgroup (thread order); total to every thread.
__device__ __forceinline__ int block_excl_scan(int v, int *s_red, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(inc, d, 64);
        if (lane >= d) inc += o;
    }
    if (lane == 63) s_red[wave] = inc;
    __syncthreads();
    int base = 0, sum = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
        const int t = s_red[w];
        if (w < wave) base += t;
        sum += t;
    }
    __syncthreads();
    total = sum;
    return base + inc - v;
}

struct RouteBits {
    uint32_t bits[2];  // [set]: bit 16p + i <=> row p*kRoutePass + 16*tid + i is in the set
    uint32_t ubase;    // rank among the und rows of this thread's first row of pass 0 (low
                       // half) and pass 1 (high half); its gen rank is the rows before it
                       // minus this (every byte is valid whenever ranks are used)
};

// Reads the pack's modality bytes once (all loads issued before any is
// used); returns true if some byte is neither 0 nor 1.  U = und rows.  The
// ranks of this thread's rows among each set's rows come from one pair of
// workgroup scans here, so that a tile's rows need no scan later.
__device__ bool route_count(const uint8_t *__restrict__ mod, int T, int *s_red, int &U, RouteBits &rb) {
    uint32_t v[kRoutePasses * kRouteRows];
    if ((reinterpret_cast<uintptr_t>(mod) & 15u) == 0 && T >= kRouteRows) {
        // 16 bytes per pass and thread in one load (the last full 16-byte
        // piece of the pack for a thread past its end: masked below)
#pragma unroll
        for (int p = 0; p < kRoutePasses; ++p) {
            const int r0 = min(p * kRoutePass + (int)threadIdx.x * kRouteRows, (T & ~(kRouteRows - 1)) - kRouteRows);
            const uint4 q = *(const uint4 *)(mod + r0);
            const int sh = p * kRoutePass + (int)threadIdx.x * kRouteRows - r0;  // 0 unless clamped
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < kRouteRows; ++i) v[p * kRouteRows + i] = (w[i >> 2] >> (8 * (i & 3))) & 0xffu;
            if (sh != 0) {
                // rows past the last full piece: byte loads
#pragma unroll
                for (int i = 0; i < kRouteRows; ++i) {
                    const int r = p * kRoutePass + (int)threadIdx.x * kRouteRows + i;
                    v[p * kRouteRows + i] = mod[min(r, T - 1)];
                }
            }
        }
    } else {
#pragma unroll
        for (int p = 0; p < kRoutePasses; ++p)
#pragma unroll
            for (int i = 0; i < kRouteRows; ++i) {
                const int r = p * kRoutePass + (int)threadIdx.x * kRouteRows + i;
                v[p * kRouteRows + i] = mod[min(r, T - 1)];
            }
    }
    uint32_t und = 0, gen = 0, bad = 0;
#pragma unroll
    for (int p = 0; p < kRoutePasses; ++p)
#pragma unroll
        for (int i = 0; i < kRouteRows; ++i) {
            const int r = p * kRoutePass + (int)threadIdx.x * kRouteRows + i;
            const uint32_t m = v[p * kRouteRows + i];
            if (r < T) {
                und |= (uint32_t)(m == 0) << (16 * p + i);
                gen |= (uint32_t)(m == 1) << (16 * p + i);
                bad |= (m > 1);
            }
        }
    rb.bits[0] = und;
    rb.bits[1] = gen;
    // Per-pass und counts, two to a word (each total <= 4096 < 2^16:
    // kInlineRouteMaxT = 2 passes of 4096 rows), in one workgroup scan.  Each
    // wave's "some byte is invalid" flag goes beside the scan's per-wave sums
    // and is published by its first barrier.  A gen rank needs no scan of its
    // own: when every byte is valid, the rows before a thread's first row of
    // a pass are und or gen, so its gen rank is their number minus its und
    // rank.  No other LDS is used (the GEMM's stage arrays fill the LDS).
    const int cu = __popc(und & 0xffffu) | (__popc(und >> 16) << 16);
    const int nw = kThreads / 64;
    const bool wave_bad = __ballot(bad != 0) != 0;
    if ((threadIdx.x & 63) == 0) s_red[nw + (threadIdx.x >> 6)] = wave_bad ? 1 : 0;
    int tu;
    const int eu = block_excl_scan(cu, s_red, tu);
    const int tu0 = tu & 0xffff;
    rb.ubase = (uint32_t)(eu & 0xffff) | ((uint32_t)(tu0 + (eu >> 16)) << 16);
    U = tu0 + (tu >> 16);
    int any_bad = 0;
#pragma unroll
    for (int w = 0; w < nw; ++w) any_bad |= s_red[nw + w];
    return any_bad != 0;
}

// s_rows[i] = the row of rank f + i among the pack's rows of `set` (i < count),
// row 0 for the slots past count.  tid: the thread index.  No workgroup-wide step: each thread
// writes its own rows whose rank falls in the tile's window.
__device__ void route_gather(const RouteBits &rb, int T, int set, int f, int count, int bm, int32_t *s_rows,
                             int tid) {
    for (int i = count + tid; i < bm; i += kThreads) s_rows[i] = 0;
    const uint32_t all = set ? rb.bits[1] : rb.bits[0];
#pragma unroll
    for (int p = 0; p < kRoutePasses; ++p) {
        uint32_t mask = (all >> (16 * p)) & 0xffffu;
        const int r0 = p * kRoutePass + tid * kRouteRows;
        const int ub = (int)((rb.ubase >> (16 * p)) & 0xffffu);
        int rank = set ? min(r0, T) - ub : ub;
        if (rank >= f + count || rank + __popc(mask) <= f) continue;
        while (mask != 0 && rank < f + count) {
            const int i = __ffs(mask) - 1;
            mask &= mask - 1;
            if (rank >= f) s_rows[rank - f] = r0 + i;
            ++rank;
        }
    }
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

// Direct global->LDS 16-byte buffer load: lane L's 16 bytes land at
// lds + 16*L.  `voff` is the lane's byte offset (a row start plus a 16-byte
// chunk of the row's first 64 columns), `soff` the wave-uniform k offset
// (k-block * 128 bytes, below the row's K columns).  The GEMMs stage only
// valid rows (rows past a tile's end repeat a valid row, weight rows are
// clamped to the last one), so voff + soff always lies inside the operand;
// only voff is checked against the resource's size by the hardware, which
// is why the kernels never rely on that check.  Operands are limited to
// 4 GiB (32-bit offsets).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, gfx9 data format word

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcFlags);
}

__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff, uint8_t *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, (int)voff, (int)soff, 0, 0);
}

// s_waitcnt: vmcnt <= N and lgkmcnt == 0 (gfx9 encoding: vmcnt[3:0] and
// vmcnt[5:4] at bits 15:14, expcnt 6:4 = 7 (no wait), lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// ---- fused QK norm + rotary epilogue (QKV projection) ------------------------
//
// The "mot_qk_norm_rope" step (RL-Kernel RFC page, section 5) inside the QKV
// GEMM.  A head is 128 output columns, and both tile shapes that run it (256 x
// 256 and 128 x 128) start on a head boundary.  The tile's bf16 outputs (the
// plain GEMM's bytes) are staged in LDS one head at a time, the rotary table
// rows of the tile's positions are staged beside them by LDS-DMA, and each
// 16-lane group runs qk_head on one (row, head) exactly as the standalone
// kernel's groups hold it: the result is that kernel's, bit for bit.  Staged
// head rows are 256 bytes, their 16-byte chunks XOR-swizzled by the row.

constexpr int kQkRowBytes = 256;

__device__ __forceinline__ uint32_t qk_chunk_off(int r, int c) {
    return (uint32_t)(r * kQkRowBytes + ((c ^ (r & 15)) << 4));
}

// Row r = thread i of the tile (one row per thread: tiles have at most 256
// rows): its output row and its position, loaded before the tile's main loop
// so that their latency hides under it (two registers through the loop).
// i is the thread index the tile loop made opaque, so that no address
// derived from it is hoisted out of that loop (and spilled).
struct QkRow {
    int row;  // output row (0 for the slots past the tile's rows)
    int pos;  // position
};

__device__ __forceinline__ QkRow qk_row_load(const GemmArgs &a, const Tile &ti, const int32_t *s_rows, int bm,
                                             int i) {
    QkRow q{0, 0};
    if (i < bm) q.row = s_rows[i];
    if (i < ti.count) q.pos = a.positions[q.row];
    return q;
}

// After the main loop: the row list and the positions into LDS (p_rows: -1
// for a position outside the table, which raises MOT_ERR_POSITION; the row
// keeps the GEMM's bytes).
__device__ __forceinline__ void qk_row_store(const GemmArgs &a, const Tile &ti, const QkRow &q, int32_t *s_rows,
                                             int32_t *p_rows, int bm, int i) {
    if (i < bm) {
        int p = q.pos;
        if (i < ti.count && (p < 0 || p >= a.n_pos)) {
            atomicMax(a.hdr_out, kErrPosition);
            p = -1;
        }
        s_rows[i] = q.row;
        p_rows[i] = i < ti.count ? p : 0;
    }
}

// The rotary table rows (128 bytes of cos into cs, of sin into sn) of the
// tile's rows, by LDS-DMA: each instruction fills eight rows.  A bad or
// padding row reads table row 0 (its result is not stored).
template <int BM>
__device__ __forceinline__ void qk_tables(const GemmArgs &a, const int32_t *p_rows, uint8_t *cs, uint8_t *sn,
                                          int wave, int lane) {
    const rsrc_t cr = make_rsrc(a.cos_t, (uint32_t)a.n_pos * 128u);
    const rsrc_t sr = make_rsrc(a.sin_t, (uint32_t)a.n_pos * 128u);
#pragma unroll
    for (int r0 = wave * 8; r0 < BM; r0 += 32) {
        const int p = max(p_rows[r0 + (lane >> 3)], 0);
        const uint32_t off = (uint32_t)p * 128u + (uint32_t)(lane & 7) * 16u;
        dma16(cr, off, 0, cs + r0 * 128);
        dma16(sr, off, 0, sn + r0 * 128);
    }
}

// A wave's MI x MJ accumulator blocks as bf16 into a head's staging rows:
// token row row0 + 32 j + (lane & 31), head column col0 + 32 i + 8 q +
// 4 (lane >> 5) .. +3 (the plain epilogue's rounding of the same values).
template <int MI, int MJ>
__device__ __forceinline__ void qk_stage(const f32x16_t (&acc)[MI][MJ], uint8_t *st, int row0, int col0, int lane) {
    const int rsel = lane & 31, khalf = lane >> 5;
#pragma unroll
    for (int j = 0; j < MJ; ++j)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = row0 + 32 * j + rsel;
                const int c = col0 + 32 * i + 8 * q + 4 * khalf;
                const u32x2_t pk = {pack2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                    pack2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
                *(lds_u32x2 *)((lds_u8 *)st + qk_chunk_off(r, c >> 3) + (c & 7) * 2) = pk;
            }
}

// One staged head (tile rows [0, BM): rows below 128 in st_lo, the rest in
// st_hi; output columns col0 .. col0 + 127): group g of the wave takes rows
// 4 wave + g, + 16, ...  Heads past the q and k heads (v) are stored as they
// are.
template <int BM>
__device__ __forceinline__ void qk_head_rows(const GemmArgs &a, const Tile &ti, int col0, const uint8_t *st_lo,
                                             const uint8_t *st_hi, const uint8_t *cs, const uint8_t *sn,
                                             const int32_t *s_rows, const int32_t *p_rows, int wave, int lane) {
    if (col0 >= a.N) return;  // uniform
    const int gi = lane & 15, g = lane >> 4;
    const int hg = col0 >> 7;
    const bool qk = hg < a.qk_heads;
    const uint16_t *w = hg < a.qk_hq ? (ti.set ? a.qw_gen : a.qw_und) : (ti.set ? a.kw_gen : a.kw_und);
    u32x4_t wv = {0u, 0u, 0u, 0u};
    if (qk) wv = *(const u32x4_t *)(w + 8 * gi);
    const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
    const uint32_t ldy_bytes = (uint32_t)a.ldy * 2u;
    const bool col_ok = col0 + 8 * gi < a.N;  // (a last head may end at a 64-column edge)
    // four rows per group at a time (r, r + 16, r + 32, r + 48): their LDS
    // reads are issued together and their arithmetic interleaves
    constexpr int U = BM > 128 ? 2 : 4;
    static_assert(BM % (16 * U) == 0, "rows per pass");
    for (int r0 = wave * 4 + g; r0 < BM; r0 += 16 * U) {
        u32x4_t v[U], cv[U], sv[U], o[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + 16 * u;
            const uint8_t *st = (BM > 128 && r >= 128) ? st_hi : st_lo;
            v[u] = *(const lds_u32x4 *)((const lds_u8 *)st + qk_chunk_off(r & 127, gi));
            cv[u] = *(const lds_u32x4 *)((const lds_u8 *)cs + r * 128 + (gi & 7) * 16);
            sv[u] = *(const lds_u32x4 *)((const lds_u8 *)sn + r * 128 + (gi & 7) * 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) o[u] = qk_head(v[u], true, gi, a.qk_eps, wv, cv[u], sv[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = r0 + 16 * u;
            if (r < ti.count && col_ok) {
                const u32x4_t out = (qk && p_rows[r] >= 0) ? o[u] : v[u];
                __builtin_amdgcn_raw_buffer_store_b128(out, yr,
                                                       (uint32_t)s_rows[r] * ldy_bytes + (uint32_t)(col0 + 8 * gi) * 2u,
                                                       0, 0);
            }
        }
    }
}

// Rows per epilogue pass: the largest multiple of 32 that divides the wave's
// rows and whose padded rows fit one 32 KiB LDS array.
constexpr int ep_rows(int wm, int rs) {
    int best = 32;
    for (int r = 32; r <= wm; r += 32)
        if (wm % r == 0 && r * rs <= 32768) best = r;
    return best;
}

// Cache policy of the staged (full-row-segment) output stores: system scope
// (written through, no dirty lines left in L2 at the end of the kernel);
// measured faster than the default for the end-of-tile store burst.
constexpr int kStoreAux = 0x11;

// Staged epilogue of one wave's WM x WN accumulator block.  Lane holds, for
// token row m = lane&31 of each 32x32 block, the weight rows
// 8*(e/4) + 4*(lane>>5) + (e&3), e = 0..15: four consecutive output columns
// per register quad.  The bf16 results (SwiGLU: act of each gate/up pair) go
// through a wave-private LDS region (rows padded by 16 bytes) so that every
// global store writes whole 16-byte chunks of contiguous row segments.  The
// caller has synchronised the workgroup after the main loop.  SEQ (big
// tiles, whose accumulators fill the register file): passes of 32 rows, one
// 32 x 32 block at a time (a scheduling barrier after each block's LDS
// writes), so that the accumulators are not all copied out to VGPRs first,
// and at most eight row read-backs at a time.
template <int WM, int WN, int MI, int MJ, bool SWIGLU, bool SEQ = false>
__device__ __forceinline__ void epilogue_staged(const GemmArgs &a, const Tile &ti, f32x16_t (&acc)[MI][MJ],
                                                lds_u8 *const eb, const int32_t *s_rows, int lane, int wm,
                                                int wn) {
    constexpr int BN = 2 * WN;
    const int rsel = lane & 31, khalf = lane >> 5;
    constexpr int OC = SWIGLU ? WN / 2 : WN;  // output columns per wave
    constexpr int OI = OC / 32;               // output column blocks
    constexpr int RS = OC * 2 + 16;           // LDS row stride, bytes
    constexpr int RH = SEQ ? 32 : ep_rows(WM, RS);  // rows per pass
    constexpr int LPR = OC / 8;               // lanes holding a row's 16-byte pieces
    constexpr int LPP = LPR <= 8 ? 8 : LPR <= 16 ? 16 : 32;  // lanes per row (a power of two)
    constexpr int RPI = 64 / LPP;             // rows per store instruction
    static_assert(RH % 32 == 0 && WM % RH == 0 && LPR <= LPP && RH % RPI == 0, "epilogue");
    // (lanes LPR..LPP-1 of a row, if any, read padding or the next row and store nothing)
    static_assert((RH - RPI + 63 / LPP) * RS + LPP * 16 <= 32768, "epilogue read-back stays in the array");
    const int col0 = SWIGLU ? ti.wrow0 / 2 + wn * (BN / 4) : ti.wrow0 + wn * WN;
    // one LDS base per lane for the writes and one for the read-back; the
    // rest are immediate offsets
    lds_u8 *const wp = eb + rsel * RS + khalf * 8;
    lds_u8 *const rp = eb + (lane / LPP) * RS + (lane % LPP) * 16;
    const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
    const uint32_t ldy_bytes = (uint32_t)a.ldy * 2u;
    const int col = col0 + (lane % LPP) * 8;
    const bool col_ok = lane % LPP < LPR && col < a.N;
#pragma unroll
    for (int jp = 0; jp < MJ; jp += RH / 32) {
#pragma unroll
        for (int jj = 0; jj < RH / 32; ++jj) {
            const int j = jp + jj;
#pragma unroll
            for (int i = 0; i < OI; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (SWIGLU) {
                            const float g = acc[i][j][4 * q + e];
                            const float u = acc[i + MI / 2][j][4 * q + e];
                            v[e] = (g / (1.0f + expf(-g))) * u;
                        } else {
                            v[e] = acc[i][j][4 * q + e];
                        }
                    }
                    const u32x2_t pk = {pack2(v[0], v[1]), pack2(v[2], v[3])};
                    *(lds_u32x2 *)(wp + jj * 32 * RS + (i * 32 + q * 8) * 2) = pk;
                }
                if constexpr (SEQ) __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int r = 0; r < RH; r += RPI) {
            const u32x4_t v = *(const lds_u32x4 *)(rp + r * RS);
            const int mloc = wm * WM + jp * 32 + r + lane / LPP;
            if (col_ok && mloc < ti.count)
                __builtin_amdgcn_raw_buffer_store_b128(
                    v, yr,
                    (uint32_t)s_rows[mloc] * ldy_bytes + (uint32_t)col * 2u, 0, kStoreAux);
            // (at most eight read-backs in flight: not all of a pass's rows
            // are loaded into VGPRs before the first store)
            if constexpr (SEQ)
                if ((r / RPI) % 8 == 7) __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// One tile of BM x BN.  The stage arrays are distinct LDS objects so that
// the compiler can tell the stage being filled by DMA from the stage being
// read, and does not make the reads wait for the in-flight loads.
//
// NS pipeline stages; stage s stages its A rows at xb[s] and its W rows at
// wb[s] (BM and BN rows of 128 bytes).  Every stage issues exactly one
// refill (re-reading the final k-block when it runs past the end), so the
// number of DMA instructions in flight is a compile-time constant.
// s_rows (the tile's A rows) is filled and published by the caller.
template <int BM, int BN, int NS, bool SWIGLU, bool PRO, bool QK = false>
__device__ __forceinline__ void run_tile(const GemmArgs &a, const Tile &ti, uint8_t *const (&xb)[NS],
                                         uint8_t *const (&wb)[NS], lds_u8 *const eb,
                                         const int32_t *s_rows, uint16_t *s_nw, const int tid,
                                         int32_t *qk_p = nullptr) {
    static_assert(!QK || (BM == 128 && BN == 128 && NS >= 2 && !SWIGLU && !PRO),
                  "fused QK epilogue: plain 128 x 128 tiles");
    constexpr int WM = BM / 2, WN = BN / 2;   // wave tile: tokens x weight rows
    constexpr int MJ = WM / 32, MI = WN / 32; // MFMA blocks per wave
    constexpr int NM = MI * MJ;               // MFMAs per k-step
    constexpr int XL = BM / 32;               // A-tile DMA instructions per wave per stage
    constexpr int WL = BN / 32;               // W-tile DMA instructions per wave per stage
    constexpr int PER_STAGE = XL + WL;
    static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
    static_assert(!SWIGLU || MI % 2 == 0, "SwiGLU pairs gate and up blocks");
    static_assert(PER_STAGE * (NS - 1) < 64, "vmcnt range");

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int K = a.K;
    const int nk = K / kBK;

    if constexpr (PRO) {
        const uint16_t *nw = ti.set ? a.nw_gen : a.nw_und;
        for (int i = tid * 8; i < K; i += kThreads * 8)
            *(uint4 *)(s_nw + i) = *(const uint4 *)(nw + i);
        __syncthreads();
    }

    const rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    const rsrc_t wr = make_rsrc(ti.set ? a.w_gen : a.w_und, a.w_bytes);

    // Per-lane byte offsets of this wave's DMA instructions: instruction j
    // fills staged rows R0 .. R0+7 (R0 = wave*(rows/4) + 8j); LDS position
    // lane&7 of row R0 + (lane>>3) receives global chunk (lane&7) ^ swz(row).
    uint32_t xoff[XL], woff[WL];
#pragma unroll
    for (int j = 0; j < XL; ++j) {
        const int r = wave * (BM / 4) + j * 8 + (lane >> 3);
        xoff[j] = (uint32_t)s_rows[r] * (uint32_t)(a.ldx * 2) + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    }
#pragma unroll
    for (int j = 0; j < WL; ++j) {
        const int r = wave * (BN / 4) + j * 8 + (lane >> 3);
        int wrow;
        if constexpr (SWIGLU) {
            const int half = r / (BN / 2), q = r % (BN / 2);
            int col = ti.wrow0 / 2 + half * (BN / 4) + (q % (BN / 4));
            col = min(col, a.N - 1);
            wrow = (q < BN / 4) ? col : a.N + col;
        } else {
            wrow = min(ti.wrow0 + r, a.N - 1);
        }
        woff[j] = (uint32_t)wrow * (uint32_t)(K * 2) + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    }

    // DMA of k-block kt into stage slot s: instructions [lo, hi) of the
    // stage's XL A-row and WL W-row instructions.
    auto issue = [&](int kt, int s, int lo, int hi) {
#pragma unroll
        for (int j = 0; j < XL + WL; ++j) {
            if (j < lo || j >= hi) continue;
            if (j < XL)
                dma16(xr, xoff[j], (uint32_t)kt * kRowBytes, xb[s] + (wave * (BM / 4) + j * 8) * kRowBytes);
            else
                dma16(wr, woff[j - XL], (uint32_t)kt * kRowBytes,
                      wb[s] + (wave * (BN / 4) + (j - XL) * 8) * kRowBytes);
        }
    };
    auto issue_all = [&](int kt, int s) { issue(kt, s, 0, PER_STAGE); };

    QkRow qkr{0, 0};
    if constexpr (QK) {
        if (ti.wrow0 < a.qk_heads * 128) qkr = qk_row_load(a, ti, s_rows, BM, tid);
    }

    float rs[MJ];
    if constexpr (PRO) {
#pragma unroll
        for (int j = 0; j < MJ; ++j) rs[j] = a.rstd[s_rows[wm * WM + j * 32 + (lane & 31)]];
    }

    f32x16_t acc[MI][MJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < MJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int rsel = lane & 31;   // row within a 32-row fragment
    const int khalf = lane >> 5;  // which 8-wide half of a 16-wide k step
    const int lsw = swz(lane & 15);
    // LDS byte offsets (within a stage) of this lane's fragment row at each of
    // the four k-steps; blocks of 32 rows are immediate offsets from these.
    uint32_t xq[4], wq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t pos = (uint32_t)(((2 * q + khalf) ^ lsw) * 16);
        xq[q] = (uint32_t)((wm * WM + rsel) * kRowBytes) + pos;
        wq[q] = (uint32_t)((wn * WN + rsel) * kRowBytes) + pos;
    }

    // Fragments of k-step q (16 k) of staged k-block kt.
    // Reads are emitted in the order the MFMAs (i-major) first need them:
    // fa[0], fb[0..MJ), then fa[1..MI).
    auto load_frags = [&](int s, int kt, int q, bf16x8_t (&fa)[MI], bf16x8_t (&fb)[MJ]) {
        const uint8_t *xs = xb[s], *ws = wb[s];
        fa[0] = *(const bf16x8_t *)(ws + wq[q]);
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
            if constexpr (PRO) {
                const uint4 v = *(const uint4 *)(xs + xq[q] + j * 32 * kRowBytes);
                const uint4 nwv = *(const uint4 *)(s_nw + kt * kBK + q * 16 + khalf * 8);
                const uint32_t in[4] = {v.x, v.y, v.z, v.w};
                const uint32_t wv[4] = {nwv.x, nwv.y, nwv.z, nwv.w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float lo = (bf16_to_f32(in[e] & 0xffffu) * rs[j]) * bf16_to_f32(wv[e] & 0xffffu);
                    const float hi = (bf16_to_f32(in[e] >> 16) * rs[j]) * bf16_to_f32(wv[e] >> 16);
                    o[e] = pack2(lo, hi);
                }
                const uint4 ov = {o[0], o[1], o[2], o[3]};
                fb[j] = __builtin_bit_cast(bf16x8_t, ov);
            } else {
                fb[j] = *(const bf16x8_t *)(xs + xq[q] + j * 32 * kRowBytes);
            }
        }
#pragma unroll
        for (int i = 1; i < MI; ++i)
            fa[i] = *(const bf16x8_t *)(ws + wq[q] + i * 32 * kRowBytes);
    };
    auto mfmas = [&](const bf16x8_t (&fa)[MI], const bf16x8_t (&fb)[MJ]) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < MJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };
    // Issue the next k-step's fragment reads over the first MFMAs of this
    // k-step (one read per MFMA), leaving the rest of the k-step to cover
    // their latency.
    // (with fewer MFMAs than reads, as in 128x64 tiles, the last reads go
    // without an MFMA of their own)
    auto interleave_reads = [&]() {
#pragma unroll
        for (int i = 0; i < MI + MJ; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
            if (i < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        }
        if constexpr (NM > MI + MJ)
            __builtin_amdgcn_sched_group_barrier(0x008, NM - (MI + MJ), 0);
    };
    // The refill of a freed stage is issued in two halves: H instructions
    // over the last k-step of the stage, the rest over the first k-step of
    // the next one, each spread evenly over that k-step's MFMAs together with
    // the fragment reads.
    constexpr int H = PER_STAGE / 2;
    auto interleave_reads_dma = [&](auto nd_c) {
        constexpr int ND = decltype(nd_c)::value;
        constexpr int DQ = ND / NM, DR = ND % NM;
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if (i < MI + MJ) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            if (i < DR)
                __builtin_amdgcn_sched_group_barrier(0x020, DQ + 1, 0);  // VMEM (DMA)
            else if (DQ > 0)
                __builtin_amdgcn_sched_group_barrier(0x020, DQ, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        }
    };

    bf16x8_t fa0[MI], fb0[MJ], fa1[MI], fb1[MJ];

    // Stage kt sits in slot s = kt % NS; stages kt+1 .. kt+NS-1 are in flight.
    // Once every wave has finished reading slot s it is refilled with k-block
    // kt+NS.  On entry fa0/fb0 hold the fragments of k-step 0 of stage kt.
    auto stage = [&](int kt, int s) {
        const int nxt = (s + 1) % NS, prv = (s + NS - 1) % NS;
        // second half of the refill the previous stage started (slot prv,
        // k-block kt-1+NS; in the first stage a harmless repeat of the
        // prologue's load of that slot)
        load_frags(s, kt, 1, fa1, fb1);
        issue(min(kt - 1 + NS, nk - 1), prv, H, PER_STAGE);
        mfmas(fa0, fb0);
        interleave_reads_dma(std::integral_constant<int, PER_STAGE - H>{});
        __builtin_amdgcn_sched_barrier(0);
        load_frags(s, kt, 2, fa0, fb0);
        mfmas(fa1, fb1);
        interleave_reads();
        __builtin_amdgcn_sched_barrier(0);
        load_frags(s, kt, 3, fa1, fb1);
        mfmas(fa0, fb0);
        interleave_reads();
        __builtin_amdgcn_sched_barrier(0);
        // all reads of slot s are issued; stage kt+1 must have landed (the
        // NS-2 younger stages may still be in flight)
        wait_vm_lgkm0<PER_STAGE * (NS - 2)>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // No branch around MFMAs (it would make the accumulators change
        // registers): past the end the refill re-reads the final k-block (in
        // bounds) into a slot nobody reads again, and the first fragments of
        // a stage that does not exist are read from a stale, in-bounds slot.
        load_frags(nxt, min(kt + 1, nk - 1), 0, fa0, fb0);
        issue(min(kt + NS, nk - 1), s, 0, H);
        mfmas(fa1, fb1);
        interleave_reads_dma(std::integral_constant<int, H>{});
        __builtin_amdgcn_sched_barrier(0);
    };

#pragma unroll
    for (int s = 0; s < NS; ++s) issue_all(min(s, nk - 1), s);
    wait_vm_lgkm0<PER_STAGE * (NS - 1)>();
    __builtin_amdgcn_s_barrier();
    load_frags(0, 0, 0, fa0, fb0);

    // The k loop is unrolled by NS so that every LDS access names one stage
    // array; the stages left over run after the loop.
    int kt = 0;
    for (; kt + NS - 1 < nk; kt += NS) {
#pragma unroll
        for (int s = 0; s < NS; ++s) stage(kt + s, s);
    }
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (kt + s < nk) stage(kt + s, s);
    wait_vm_lgkm0<0>();  // no DMA may still be writing LDS when the tile ends

    // Epilogue.
    __syncthreads();  // every wave is done reading the last stage
    if constexpr (QK) {
        if (ti.wrow0 < a.qk_heads * 128) {
            // the tile is one head: staged in array 0, the rotary rows in
            // array 1 (cos, then sin)
            qk_row_store(a, ti, qkr, const_cast<int32_t *>(s_rows), qk_p, BM, tid);
            __syncthreads();
            qk_tables<BM>(a, qk_p, xb[1], xb[1] + BM * 128, wave, lane);
            qk_stage<MI, MJ>(acc, xb[0], wm * WM, wn * WN, lane);
            wait_vm_lgkm0<0>();
            __syncthreads();
            qk_head_rows<BM>(a, ti, ti.wrow0, xb[0], xb[0], xb[1], xb[1] + BM * 128, s_rows, qk_p, wave, lane);
            return;
        }
    }
    epilogue_staged<WM, WN, MI, MJ, SWIGLU>(a, ti, acc, eb, s_rows, lane, wm, wn);
}

// Big tile (256 x 256) without the prologue, on a ring of five 32 KiB LDS
// slots (all of the LDS).  Each slot holds one operand of one stage (256 rows
// of a 64-wide k-block): the A rows of stage j sit in slot (2j) % 5 and its
// W rows in slot (2j+1) % 5.  Once stage j has been read, its two slots take
// the W rows of stage j+2 and the A rows of stage j+3, so the A rows are
// requested about five k-steps and the W rows about two and a half k-steps
// before they are read, and the refill is spread evenly: four DMA
// instructions per wave in every k-step.
//   k-step 0: second half of W(j+1)    k-step 1: first half of A(j+2)
//   k-step 2: second half of A(j+2)    barrier
//   k-step 3: first half of W(j+2)
// At the barrier of stage j, A(j+1) and W(j+1) must have landed; only the
// eight instructions of A(j+2) may still be in flight.
// The row list lives in slot 4 until the prologue's barrier: each lane
// takes its DMA offsets and the token rows of its four output rows from it
// first.  Epilogue of the 256 x 256 bf16 tiles: the row list, which the ring
// overwrote, is rebuilt in slot 4 from those rows, and each wave writes its
// results through its own array (epilogue_staged), so that every store
// instruction covers whole 256-byte (SwiGLU: 128-byte) row segments.  The
// accumulators' own layout gives 16 contiguous bytes per row and store
// instruction, which takes the memory system about twice as long to absorb
// when every workgroup stores its tile at the same time.  fp32 output and
// 224-row tiles store straight from the accumulators.
// TOK: token-major operands (the weight gradient): the contraction runs over
// token rows, both operands are read as they lie in memory ([token][column],
// a.x = dY with pitch a.ldx, the weight side = X with pitch a.ldw), and the
// tile's rows are the output rows of the x side (its row list the identity).
// A stage slot then holds 64 token rows of 256 columns (512 bytes each, their
// 32-byte granules permuted by the row index mod 4: granule g at
// g ^ tok_swz(r)), filled by LDS-DMA two token rows per instruction, and a
// fragment (eight consecutive tokens of one column) is two transposing reads
// (ds_read_b64_tr_b16: within each 16-lane group, element e of lane 4a+b is
// element b of the 4-value chunk that lane 4e+a addresses).  The k order and
// the MFMA operands are those of the same product on transposed copies.
// Weight-side token rows whose modality byte is not a.keep, and rows past
// a.t_tok, read as zeros (out-of-range buffer offsets).
__device__ __forceinline__ int tok_swz(int r) { return ((r & 1) ? 5 : 0) ^ (r & 2); }
constexpr int kTokRowBytes = 2 * kBigN;  // 256 bf16 columns

// WTOK: only the weight side is contraction-major: W [contraction][ldw]
// (the forward's [N][K] weights read as they lie, for dX = dY W: the
// contraction runs over W's rows), staged and read as TOK stages it; the x
// side is the routed token rows as usual.  All W rows count.
template <bool SWIGLU, bool F32 = false, bool QK = false, int BN = kBigN, int BM = kBigM, bool TOK = false,
          bool WTOK = false>
__device__ __forceinline__ void run_big5(const GemmArgs &a, const Tile &ti, uint8_t *const (&hs)[5],
                                         const int32_t *s_rows, const int tid, lds_u8 *const eb,
                                         int32_t *qk_p = nullptr) {
    static_assert(!(SWIGLU && F32), "fp32 output: plain GEMM only");
    static_assert(!TOK || (!SWIGLU && !QK && BN == kBigN && BM == kBigM), "token-major operands: plain 256 x 256");
    static_assert(!WTOK || (!TOK && !SWIGLU && !QK && !F32 && BN == kBigN && BM == kBigM),
                  "contraction-major weights: plain bf16 256 x 256");
    static_assert(!QK || (!SWIGLU && !F32), "fused QK epilogue: plain bf16 GEMM only");
    constexpr uint32_t kOutBytes = F32 ? 4u : 2u;  // bytes per output element
    static_assert(BN == kBigN || (BN == kWideN && !SWIGLU && !F32 && !QK), "wide tiles: plain bf16 GEMM only");
    static_assert(BM == kBigM || (BM == kShortM && BN == kBigN && !SWIGLU && !F32 && !QK),
                  "short tiles: plain bf16 GEMM only");
    // 256 x 256: waves in a 2 x 2 grid of 128 x 128; 192 x 256: a 2 x 2 grid
    // of 96 x 128; 256 x 224: four waves of 64 token rows x all 224 weight
    // rows
    constexpr int WAVES_N = BN == kBigN ? 2 : 1;
    constexpr int WM = BM / (4 / WAVES_N), WN = BN / WAVES_N;
    constexpr int MJ = WM / 32, MI = WN / 32;
    constexpr int NM = MI * MJ;
    constexpr int XL = BM / 32, WL = BN / 32;  // DMA instructions per wave per operand and stage
    constexpr int HX = XL / 2, HW = WL / 2;
    static_assert((XL == 8 && ((WL == 8 && NM == 16) || (WL == 7 && NM == 14))) ||
                      (XL == 6 && WL == 8 && NM == 12),
                  "big tile");
    constexpr int DL = XL > WL ? XL : WL;

    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = WAVES_N == 2 ? wave >> 1 : wave, wn = WAVES_N == 2 ? (wave & 1) : 0;
    const int K = a.K;
    const int nk = K / kBK;

    const rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    const rsrc_t wr = make_rsrc(ti.set ? a.w_gen : a.w_und, a.w_bytes);

    uint32_t xoff[XL], woff[WL];
    if constexpr (TOK) {
        // instruction j: token row r = 16 wave + 2 j + (lane >> 5) of the
        // stage; the lane's 16-byte position p = lane & 31 holds the row's
        // chunk p ^ 2 tok_swz(r), columns ti.first (x) or ti.wrow0 (w) +
        // 8 (p ^ 2 tok_swz(r))
#pragma unroll
        for (int j = 0; j < XL; ++j) {
            const int r = wave * 16 + 2 * j + (lane >> 5);
            const uint32_t c = (uint32_t)((lane & 31) ^ (tok_swz(r) << 1));
            xoff[j] = (uint32_t)r * (uint32_t)(a.ldx * 2) + ((uint32_t)ti.first + 8u * c) * 2u;
            woff[j] = (uint32_t)r * (uint32_t)(a.ldw * 2) + ((uint32_t)ti.wrow0 + 8u * c) * 2u;
        }
    } else {
#pragma unroll
    for (int j = 0; j < XL; ++j) {
        const int r = wave * (BM / 4) + j * 8 + (lane >> 3);
        xoff[j] = (uint32_t)s_rows[r] * (uint32_t)(a.ldx * 2) + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    }
#pragma unroll
    for (int j = 0; j < WL; ++j) {
        if constexpr (WTOK) {
            // as TOK's weight side: W row r of the stage, chunk position
            // lane & 31, columns ti.wrow0 + 8 (p ^ 2 tok_swz(r))
            const int r = wave * 16 + 2 * j + (lane >> 5);
            const uint32_t c = (uint32_t)((lane & 31) ^ (tok_swz(r) << 1));
            woff[j] = (uint32_t)r * (uint32_t)(a.ldw * 2) + ((uint32_t)ti.wrow0 + 8u * c) * 2u;
            continue;
        }
        const int r = wave * (BN / 4) + j * 8 + (lane >> 3);
        int wrow;
        if constexpr (SWIGLU) {
            const int half = r / (BN / 2), q = r % (BN / 2);
            int col = ti.wrow0 / 2 + half * (BN / 4) + (q % (BN / 4));
            col = min(col, a.N - 1);
            wrow = (q < BN / 4) ? col : a.N + col;
        } else {
            wrow = min(ti.wrow0 + r, a.N - 1);
        }
        woff[j] = (uint32_t)wrow * (uint32_t)(K * 2) + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    }
    }
    // TOK: the weight-side rows' modality bytes, one 16-row group per wave
    // and stage (lane l reads row 16 wave + (l & 15) of the stage): loaded at
    // the start of a stage for the stage two ahead, turned into a row mask
    // (bit q: row 16 wave + q is kept) after that stage's barrier, by which
    // the load has landed (the DMA issued after it is what remains in flight)
    const rsrc_t mr = make_rsrc(a.modality, TOK ? (uint32_t)a.t_tok : 0u);
    uint32_t tflag = 0;
    uint32_t tmask = 0;
    auto flag_load = [&](int kb) {
        if constexpr (TOK)
            tflag = __builtin_amdgcn_raw_buffer_load_b8(
                mr, (int)((uint32_t)kb * kBK + (uint32_t)(wave * 16 + (lane & 15))), 0, 0);
    };
    auto flag_mask = [&]() {
        if constexpr (TOK)
            tmask = (uint32_t)__builtin_amdgcn_ballot_w64(tflag == (uint32_t)a.keep) & 0xffffu;
    };
    // the fused QK epilogue's row and position (the ring overwrites the
    // row list during the main loop)
    QkRow qkr{0, 0};
    if constexpr (QK) {
        if (ti.wrow0 < a.qk_heads * 128) qkr = qk_row_load(a, ti, s_rows, BM, tid);
    }
    // token rows of this lane's four output rows, -1 past the tile's rows
    const int rsel = lane & 31;
    const int khalf = lane >> 5;
    int32_t yrow[MJ];
#pragma unroll
    for (int j = 0; j < MJ; ++j) {
        const int mloc = wm * WM + j * 32 + rsel;
        yrow[j] = mloc < ti.count ? s_rows[mloc] : -1;
    }

    // operand o (0 = A, 1 = W) of k-block kb into slot s, instructions [lo, hi)
    auto issue = [&](int o, int kb, int s, int lo, int hi) {
        if constexpr (TOK) {
            const uint32_t tb = (uint32_t)kb * kBK;  // first token row of the stage
#pragma unroll
            for (int j = 0; j < DL; ++j) {
                if (j < lo || j >= hi) continue;
                uint8_t *dst = hs[s] + (wave * 16 + 2 * j) * kTokRowBytes;
                if (o == 0) {
                    dma16(xr, xoff[j] + tb * (uint32_t)(a.ldx * 2), 0, dst);
                } else {
                    // a dropped row reads an offset past the buffer's end
                    // (zeros; the extents stay below 2^32 - 256)
                    const bool kept = (tmask >> (2 * j + (lane >> 5))) & 1u;
                    dma16(wr, kept ? woff[j] + tb * (uint32_t)(a.ldw * 2) : 0xffffff00u, 0, dst);
                }
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < DL; ++j) {
            if (j < lo || j >= hi) continue;
            if (WTOK && o == 1) {
                dma16(wr, woff[j] + (uint32_t)kb * kBK * (uint32_t)(a.ldw * 2), 0,
                      hs[s] + (wave * 16 + 2 * j) * kTokRowBytes);
                continue;
            }
            if (o == 0) {
                if (j < XL)
                    dma16(xr, xoff[j], (uint32_t)kb * kRowBytes, hs[s] + (wave * (BM / 4) + j * 8) * kRowBytes);
            } else {
                if (j < WL)
                    dma16(wr, woff[j], (uint32_t)kb * kRowBytes, hs[s] + (wave * (BN / 4) + j * 8) * kRowBytes);
            }
        }
    };

    f32x16_t acc[MI][MJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < MJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int lsw = swz(lane & 15);
    uint32_t xq[4], wq[4];
    if constexpr (TOK) {
        // 32-column block cb of the tile: lane l (L = l & 15) addresses token
        // row 8 (l >> 5) + (L >> 2) (+ 16 q, + 4 for the second half) and the
        // four columns 32 cb + 16 ((l >> 4) & 1) + 4 (L & 3), and receives
        // column 32 cb + (l & 31) of four consecutive token rows
        const int L = lane & 15;
        const int tr = 8 * khalf + (L >> 2);
        const int gs = ((lane >> 4) & 1) ^ tok_swz(tr);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t base = (uint32_t)(tr * kTokRowBytes + 8 * (L & 3));
            xq[q] = base + (uint32_t)(((2 * (wm * MJ + q)) ^ gs) << 5);
            wq[q] = base + (uint32_t)(((2 * (wn * MI + q)) ^ gs) << 5);
        }
    } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const uint32_t pos = (uint32_t)(((2 * q + khalf) ^ lsw) * 16);
        xq[q] = (uint32_t)((wm * WM + rsel) * kRowBytes) + pos;
        if constexpr (WTOK) {
            // (as TOK's: q indexes the wave's 32-column block of W)
            const int L = lane & 15;
            const int tr = 8 * khalf + (L >> 2);
            const int gs = ((lane >> 4) & 1) ^ tok_swz(tr);
            wq[q] = (uint32_t)(tr * kTokRowBytes + 8 * (L & 3)) + (uint32_t)(((2 * (wn * MI + q)) ^ gs) << 5);
        } else {
            wq[q] = (uint32_t)((wn * WN + rsel) * kRowBytes) + pos;
        }
    }
    }
    // TOK: eight consecutive token rows of one column block (xq / wq index
    // the block, q the 16-row k-step)
    auto tok_frag = [&](const uint8_t *sl, uint32_t off, int q) -> bf16x8_t {
        typedef short i16x4_t __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
        const u32x2_t lo = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(sl + off + q * 16 * kTokRowBytes)));
        const u32x2_t hi = __builtin_bit_cast(
            u32x2_t,
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(sl + off + (q * 16 + 4) * kTokRowBytes)));
        return __builtin_bit_cast(bf16x8_t, (u32x4_t){lo.x, lo.y, hi.x, hi.y});
    };
    // fragments of k-step q of the stage whose A rows are in slot sa and W rows in sw
    auto load_frags = [&](int sa, int sw, int q, bf16x8_t (&fa)[MI], bf16x8_t (&fb)[MJ]) {
        const uint8_t *xs = hs[sa], *ws = hs[sw];
        if constexpr (TOK) {
            static_assert(!TOK || (MI == 4 && MJ == 4), "token-major tiles: 4 x 4 blocks per wave");
            fa[0] = tok_frag(ws, wq[0], q);
#pragma unroll
            for (int j = 0; j < MJ; ++j) fb[j] = tok_frag(xs, xq[j], q);
#pragma unroll
            for (int i = 1; i < MI; ++i) fa[i] = tok_frag(ws, wq[i], q);
            return;
        }
        if constexpr (WTOK) {
            static_assert(!WTOK || MI == 4, "contraction-major weights: 4 column blocks per wave");
            fa[0] = tok_frag(ws, wq[0], q);
#pragma unroll
            for (int j = 0; j < MJ; ++j) fb[j] = *(const bf16x8_t *)(xs + xq[q] + j * 32 * kRowBytes);
#pragma unroll
            for (int i = 1; i < MI; ++i) fa[i] = tok_frag(ws, wq[i], q);
            return;
        }
        fa[0] = *(const bf16x8_t *)(ws + wq[q]);
#pragma unroll
        for (int j = 0; j < MJ; ++j) fb[j] = *(const bf16x8_t *)(xs + xq[q] + j * 32 * kRowBytes);
#pragma unroll
        for (int i = 1; i < MI; ++i) fa[i] = *(const bf16x8_t *)(ws + wq[q] + i * 32 * kRowBytes);
    };
    auto mfmas = [&](const bf16x8_t (&fa)[MI], const bf16x8_t (&fb)[MJ]) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < MJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    };
    // one k-step: the next fragment reads over the first MFMAs, four DMA
    // instructions spread over all of them
    auto interleave = [&]() {
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            if (WTOK ? i < 2 * MI + MJ : i < MI + MJ)
                __builtin_amdgcn_sched_group_barrier(0x100, TOK ? 2 : 1, 0);  // DS read
            if (i % 4 == 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM (DMA)
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  // MFMA
        }
    };

    bf16x8_t fa0[MI], fb0[MJ], fa1[MI], fb1[MJ];

    // Stage kt with jm = kt % 5 (a compile-time slot pattern).  On entry
    // fa0/fb0 hold the fragments of its k-step 0.
    auto stage = [&](auto jm_c, int kt) {
        constexpr int jm = decltype(jm_c)::value;
        constexpr int sa = (2 * jm) % 5, sw = (2 * jm + 1) % 5;            // this stage
        constexpr int na = (2 * jm + 2) % 5, nw = (2 * jm + 3) % 5;        // next stage
        constexpr int a2 = (2 * jm + 4) % 5, w2 = (2 * jm + 5) % 5;        // A(j+2), W(j+2)
        flag_load(min(kt + 2, nk - 1));             // TOK: modality of stage j+2
        load_frags(sa, sw, 1, fa1, fb1);
        issue(1, min(kt + 1, nk - 1), nw, HW, WL);  // W(j+1), second half
        mfmas(fa0, fb0);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        load_frags(sa, sw, 2, fa0, fb0);
        issue(0, min(kt + 2, nk - 1), a2, 0, HX);   // A(j+2), first half
        mfmas(fa1, fb1);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        load_frags(sa, sw, 3, fa1, fb1);
        issue(0, min(kt + 2, nk - 1), a2, HX, XL);  // A(j+2), second half
        mfmas(fa0, fb0);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        // slot reads of this stage are done; A(j+1), W(j+1) have landed
        wait_vm_lgkm0<XL>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        flag_mask();
        // Past the end the refills re-read the final k-block into freed
        // slots, and the first fragments of a stage that does not exist are
        // read from a stale, in-bounds slot.
        load_frags(na, nw, 0, fa0, fb0);
        issue(1, min(kt + 2, nk - 1), w2, 0, HW);   // W(j+2), first half
        mfmas(fa1, fb1);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
    };

    // prologue: A0, W0, A1, W1 into slots 0..3 (slot 4 holds the row list
    // until every wave has passed the barrier below)
    if constexpr (TOK) {
        flag_load(0);
        wait_vm_lgkm0<0>();
        flag_mask();
    }
    issue(0, 0, 0, 0, XL);
    issue(1, 0, 1, 0, WL);
    if constexpr (TOK) {
        flag_load(min(1, nk - 1));
        wait_vm_lgkm0<0>();
        flag_mask();
    }
    issue(0, min(1, nk - 1), 2, 0, XL);
    issue(1, min(1, nk - 1), 3, 0, WL);
    wait_vm_lgkm0<XL + WL>();
    __builtin_amdgcn_s_barrier();
    load_frags(0, 1, 0, fa0, fb0);

    int kt = 0;
    for (; kt + 4 < nk; kt += 5) {
        stage(std::integral_constant<int, 0>{}, kt);
        stage(std::integral_constant<int, 1>{}, kt + 1);
        stage(std::integral_constant<int, 2>{}, kt + 2);
        stage(std::integral_constant<int, 3>{}, kt + 3);
        stage(std::integral_constant<int, 4>{}, kt + 4);
    }
    if (kt < nk) stage(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 < nk) stage(std::integral_constant<int, 1>{}, kt + 1);
    if (kt + 2 < nk) stage(std::integral_constant<int, 2>{}, kt + 2);
    if (kt + 3 < nk) stage(std::integral_constant<int, 3>{}, kt + 3);
    wait_vm_lgkm0<0>();  // no DMA may still be writing LDS when the tile ends

    if constexpr (QK) {
        if (ti.wrow0 < a.qk_heads * 128) {
            // Two heads per tile, one after the other: the head of the waves
            // with wn = h is staged in slots 0 (rows 0-127) and 1 (rows
            // 128-255); the rotary rows go to slots 2 (cos) and 3 (sin); the
            // row list, which the ring overwrote, is rebuilt in slot 4.
            __syncthreads();  // every wave is done with the ring
            qk_row_store(a, ti, qkr, const_cast<int32_t *>(s_rows), qk_p, BM, tid);
            __syncthreads();
            qk_tables<BM>(a, qk_p, hs[2], hs[3], wave, lane);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (wn == h) qk_stage<MI, MJ>(acc, wm ? hs[1] : hs[0], 0, 0, lane);
                wait_vm_lgkm0<0>();
                __syncthreads();
                qk_head_rows<BM>(a, ti, ti.wrow0 + 128 * h, hs[0], hs[1], hs[2], hs[3], s_rows, qk_p, wave, lane);
                __syncthreads();  // the staging slots are read before the next head overwrites them
            }
            return;
        }
    }

    if constexpr (!F32) {
        int32_t *const rows = const_cast<int32_t *>(s_rows);
        __syncthreads();  // every wave is done with the ring
        if (wn == 0 && khalf == 0) {
#pragma unroll
            for (int j = 0; j < MJ; ++j) rows[wm * WM + j * 32 + rsel] = yrow[j];
        }
        __syncthreads();
        // (the lane index made opaque: the epilogue's LDS and column
        // offsets are then computed here, not before the main loop, where
        // they would be kept, or spilled, through it)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        epilogue_staged<WM, WN, MI, MJ, SWIGLU, true>(a, ti, acc, eb, rows, ln, wm, wn);
        return;
    }

    // Epilogue: lane holds, for token row m = lane&31 of each block, four
    // consecutive output columns per register quad (SwiGLU: the act of each
    // gate/up pair).
    {
        const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
        constexpr int OI = SWIGLU ? MI / 2 : MI;
        const int col0 = SWIGLU ? ti.wrow0 / 2 + wn * (BN / 4) : ti.wrow0 + wn * WN;
#pragma unroll
        for (int j = 0; j < MJ; ++j) {
            if (yrow[j] < 0) continue;
            const uint32_t yoff = (uint32_t)yrow[j] * (uint32_t)a.ldy * kOutBytes;  // below 4 GiB
#pragma unroll
            for (int i = 0; i < OI; ++i) {
                const int n0 = col0 + i * 32;
                if (n0 >= a.N) continue;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if constexpr (SWIGLU) {
                            const float g = acc[i][j][4 * q + e];
                            const float u = acc[i + MI / 2][j][4 * q + e];
                            v[e] = (g / (1.0f + expf(-g))) * u;
                        } else {
                            v[e] = acc[i][j][4 * q + e];
                        }
                    }
                    if constexpr (F32) {
                        // the fp32 accumulators themselves: 16 bytes per store
                        const u32x4_t pk = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                            __float_as_uint(v[3])};
                        __builtin_amdgcn_raw_buffer_store_b128(
                            pk, yr, yoff + (uint32_t)(n0 + q * 8 + khalf * 4) * 4u, 0, 0);
                    } else {
                        const u32x2_t pk = {pack2(v[0], v[1]), pack2(v[2], v[3])};
                        __builtin_amdgcn_raw_buffer_store_b64(
                            pk, yr, yoff + (uint32_t)(n0 + q * 8 + khalf * 4) * 2u, 0, 0);
                    }
                }
            }
        }
    }
}

// Norm weights of the prologue, staged in LDS (only the prologue variants
// reserve this space).
template <bool PRO>
__device__ __forceinline__ uint16_t *prologue_nw_lds() {
    if constexpr (PRO) {
        __shared__ __attribute__((aligned(16))) uint16_t s_nw[kMaxPrologueK];
        return s_nw;
    } else {
        return nullptr;
    }
}

// INLINE: the workgroups build the segment list from the modality bytes
// (and publish it to the workspace); otherwise they read the plan that
// plan_kernel wrote.
//
// LDS: four 32 KiB arrays and a fifth that is a 32 KiB stage slot without
// the prologue (the big tiles' five-slot ring; the row list and the scan
// scratch then live in it outside the main loop) and 2 KiB with it (row
// list and scan scratch; the prologue's big tiles run two stages of A in
// array 0 or 2 and W in array 1 or 3, and its norm weights take 16 KiB).
// Small tiles run four stages, one array each.
// WIDE: the schedule may pick 256 x 224 big tiles (plain GEMMs whose weight
// rows are a multiple of 224); SHORT: its big tiles are 192 x 256.
// Separate instantiations, so that the other GEMMs keep their register
// allocation (a kernel with the 192-row and the 256-row paths spills).
template <bool SWIGLU, bool PRO, bool INLINE, bool NARROW = false, bool F32 = false, bool QK = false,
          bool WIDE = false, bool SHORT = false, bool WTOK = false>
__global__ void __launch_bounds__(kThreads, 1)
gemm_kernel(GemmArgs a) {
    static_assert(!NARROW || (!SWIGLU && !PRO), "narrow tiles: plain GEMM only");
    static_assert(!F32 || (!SWIGLU && !PRO && !NARROW), "fp32 output: plain GEMM, big tiles only");
    static_assert(!QK || (!SWIGLU && !PRO && !NARROW && !F32), "fused QK epilogue: plain bf16 GEMM only");
    static_assert(!WIDE || (!SWIGLU && !PRO && !NARROW && !F32 && !QK), "wide tiles: plain bf16 GEMM only");
    static_assert(!SHORT || (!SWIGLU && !PRO && !NARROW && !F32 && !QK && !WIDE), "short tiles: plain bf16 GEMM only");
    static_assert(!WTOK || (!SWIGLU && !PRO && !NARROW && !F32 && !QK && !WIDE && !SHORT),
                  "contraction-major weights: plain bf16 GEMM, big tiles only (mode 1)");
    constexpr int kArrayBytes = kBigM * kRowBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kArrayBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kArrayBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[kArrayBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[kArrayBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds4[PRO ? 2048 : kArrayBytes];
    int32_t *const s_rows = (int32_t *)lds4;            // kBigM entries
    int *const s_red = (int *)(lds4 + kBigM * 4);       // block-scan scratch
    int32_t *const qk_p = QK ? (int32_t *)(lds4 + 2048) : nullptr;  // fused QK epilogue: row positions
    uint16_t *const s_nw = prologue_nw_lds<PRO>();

    const int T = (int)a.T;
    int U, G;
    RouteBits rb;
    if constexpr (INLINE) {
        const bool bad = route_count(a.modality, T, s_red, U, rb);
        // the count is the same in every lane (an LDS reduction); say so, so
        // that everything derived from it (tile, weight set, buffer
        // resources) stays in scalar registers
        U = __builtin_amdgcn_readfirstlane(U);
        G = T - U;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            // (with the fused QK epilogue the word is cleared before the
            // launch and other workgroups may raise position errors in it)
            if constexpr (QK) {
                if (bad) atomicMax(a.hdr_out, kErrModality);
            } else {
                a.hdr_out[0] = bad ? kErrModality : 0;
            }
            a.hdr_out[1] = bad ? 0 : U;
            a.hdr_out[2] = bad ? 0 : G;
            a.hdr_out[3] = T;
        }
        if (bad) return;  // the pack holds an invalid byte: write nothing
    } else {
        const int32_t *hdr = a.hdr;
        const int e0 = hdr[0];
        U = hdr[1];
        G = hdr[2];
        // A plan whose error word is set makes every workgroup exit (the word
        // already reports why).  A plan that does not describe exactly T rows
        // (a stale plan, or one of another pack, passed with
        // MOT_FLAG_PLAN_READY) fails closed too: nothing is written and
        // workgroup 0 raises MOT_ERR_PLAN in the error word, after every
        // workgroup has read the header (the others see the same header, so
        // they exit as well).
        // (with the fused QK epilogue another workgroup may already have
        // raised a position error; only the plan's own error stops the call)
        if (QK ? e0 == kErrModality : e0 != 0) return;
        if (hdr[3] != T || U < 0 || G < 0 || U + G != T) {
            if (blockIdx.x == 0 && threadIdx.x == 0) a.hdr_out[0] = kErrPlan;
            return;
        }
    }
    // per-wave epilogue staging: array `wave` of the first four
    const int wave_id = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    lds_u8 *const eb = (lds_u8 *)(wave_id == 0 ? lds0 : wave_id == 1 ? lds1 : wave_id == 2 ? lds2 : lds3);
    const int grid = (int)gridDim.x;
    // fp32 output runs 256 x 256 tiles only (mode 1: every row block,
    // partial ones included, is a big tile; no small tiles)
    const Schedule sc = NARROW ? make_schedule(U, G, a.wrows, grid, 2, kNarrowN)
                               : make_schedule(U, G, a.wrows, grid, F32 ? 1 : a.tile_mode, kSmallN, WIDE, SHORT);
    // Static assignment.  Big tiles go round-robin (whole rounds, or one
    // partial round); small tiles (about a quarter of a big tile's work each)
    // go first to the workgroups that hold no big tile, up to four each, then
    // round-robin over all workgroups.
    const int w = xcd_remap((int)blockIdx.x, grid);
    const int nsm = sc.ntiles - sc.nkeep;
    // workgroups w < fill run one big tile more than the others (the last,
    // partial round); the others are idle then and take small tiles first
    const int fill = sc.nkeep % grid;
    const int idle = fill > 0 ? grid - fill : (sc.nkeep == 0 ? grid : 0);
    const int cap = min(nsm, 4 * idle);
    const int n_big = w < sc.nkeep ? cdiv(sc.nkeep - w, grid) : 0;
    const int n_idle = (idle > 0 && w >= fill && w - fill < cap) ? cdiv(cap - (w - fill), idle) : 0;
    // Round-robin small tiles that fit in one round go in chunks of eight
    // consecutive tiles (two neighbouring big tiles' quarters, or neighbours
    // in a row block: they share operand panels) dealt to the XCDs in turn.
    // Contiguous ranges per XCD would crowd such a round onto the first few
    // XCDs, whose L2s and fabric links then carry all of its operand traffic
    // (QKV at T=4096: 164 small tiles on five XCDs; dealt out, 3% faster;
    // chunks of eight fetch less than chunks of four in the same time).
    int wsm = w;
    if ((grid & 63) == 0 && nsm - cap <= grid) {
        const int id = (int)blockIdx.x, local = id >> 3;
        wsm = (local >> 3) * 64 + (id & 7) * 8 + (local & 7);
    }
    const int n_rr = cap + wsm < nsm ? cdiv(nsm - cap - wsm, grid) : 0;
    for (int it = 0; it < n_big + n_idle + n_rr; ++it) {
        int t;
        if (it < n_big)
            t = w + it * grid;
        else if (it < n_big + n_idle)
            t = sc.nkeep + (w - fill) + (it - n_big) * idle;
        else
            t = sc.nkeep + cap + wsm + (it - n_big - n_idle) * grid;
        const Tile ti = tile_of(sc, t);
        if (ti.count <= 0 || ti.wrow0 >= a.wrows) continue;  // uniform: nothing to compute
        const int bm = ti.big ? sc.bm : kSmallM;
        // The thread index, made opaque per tile: per-lane offsets are then
        // recomputed in each tile instead of being hoisted out of this loop
        // and spilled (a spill reload waits on vmcnt, i.e. on in-flight DMA).
        int tid = (int)threadIdx.x;
        asm volatile("" : "+v"(tid));
        __syncthreads();  // every wave is done with the previous tile's LDS
        // the tile's rows into s_rows
        if constexpr (INLINE) {
            // (the route words made opaque per tile as well: the ranks
            // derived from them are then not hoisted out of this loop, where
            // they would be kept, or spilled, through the whole tile)
            RouteBits rt = rb;
            if constexpr (!PRO) asm volatile("" : "+v"(rt.bits[0]), "+v"(rt.bits[1]), "+v"(rt.ubase));
            route_gather(rt, T, ti.set, ti.first - (ti.set ? U : 0), ti.count, bm, s_rows,
                         PRO ? (int)threadIdx.x : tid);
        } else {
            for (int i = threadIdx.x; i < bm; i += kThreads)
                s_rows[i] = i < ti.count ? min(max(a.perm[ti.first + i], 0), T - 1) : 0;
        }
        __syncthreads();
        if constexpr (INLINE) {
            // the tiles of weight rows [0, ...) cover every row once: they
            // publish the segment list
            if (ti.wrow0 == 0)
                for (int i = threadIdx.x; i < ti.count; i += kThreads) a.perm_out[ti.first + i] = s_rows[i];
        }
        if constexpr (NARROW) {
            // 128 x 64 tiles only (mode 2): twice the small tiles, for packs
            // whose 128 x 128 tiles would leave most CUs idle
            constexpr int kHalf = kSmallM * kRowBytes;
            uint8_t *const xb[4] = {lds0, lds1, lds2, lds3};
            uint8_t *const wb[4] = {lds0 + kHalf, lds1 + kHalf, lds2 + kHalf, lds3 + kHalf};
            run_tile<kSmallM, kNarrowN, 4, false, false>(a, ti, xb, wb, eb, s_rows, s_nw, tid);
        } else if (ti.big) {
            if constexpr (PRO) {
                uint8_t *const xb[2] = {lds0, lds2}, *const wb[2] = {lds1, lds3};
                run_tile<kBigM, kBigN, 2, SWIGLU, PRO>(a, ti, xb, wb, eb, s_rows, s_nw, tid);
            } else {
                uint8_t *const hs[5] = {lds0, lds1, lds2, lds3, lds4};
                if constexpr (WIDE) {
                    if (sc.bn == kWideN)
                        run_big5<false, false, false, kWideN>(a, ti, hs, s_rows, tid, eb, qk_p);
                    else
                        run_big5<false, false, false>(a, ti, hs, s_rows, tid, eb, qk_p);
                } else if constexpr (SHORT) {
                    run_big5<false, false, false, kBigN, kShortM>(a, ti, hs, s_rows, tid, eb, qk_p);
                } else if constexpr (WTOK) {
                    run_big5<false, false, false, kBigN, kBigM, false, true>(a, ti, hs, s_rows, tid, eb);
                } else {
                    run_big5<SWIGLU, F32, QK>(a, ti, hs, s_rows, tid, eb, qk_p);
                }
            }
        } else if constexpr (!F32 && !WTOK) {  // (mode 1 schedules no small tiles)
            constexpr int kHalf = kSmallM * kRowBytes;
            uint8_t *const xb[4] = {lds0, lds1, lds2, lds3};
            uint8_t *const wb[4] = {lds0 + kHalf, lds1 + kHalf, lds2 + kHalf, lds3 + kHalf};
            run_tile<kSmallM, kSmallN, 4, SWIGLU, PRO, QK>(a, ti, xb, wb, eb, s_rows, s_nw, tid, qk_p);
        }
    }
}

// ============================================================================
// Weight gradient over token-major operands
// ============================================================================
//
// dW_set[n][k] = sum over the pack's rows t of that set of dY[t][n] X[t][k]:
// one 256 x 256 output tile per workgroup (n rows from dY's columns, k
// columns from X's), the contraction over all token rows in blocks of 64
// (the rows of the other set read as zeros), fp32 accumulation in ascending
// 16-row MFMA steps, stored as bf16 (one rounding) or as the fp32 sums.  The
// big-tile ring with token-major staging (run_big5<..., TOK>): the operands
// are read where they lie, with no transposed copies.  Tiles are numbered
// in groups of four k tiles over all n tiles (as the GEMM's big tiles), and
// the XCD remap gives each XCD a contiguous range of them.
template <bool F32>
__global__ void __launch_bounds__(kThreads, 1) grad_w_kernel(GemmArgs a) {
    constexpr int kArrayBytes = kBigM * kRowBytes;
    __shared__ __attribute__((aligned(1024))) uint8_t lds0[kArrayBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds1[kArrayBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds2[kArrayBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds3[kArrayBytes];
    __shared__ __attribute__((aligned(1024))) uint8_t lds4[kArrayBytes];
    int32_t *const s_rows = (int32_t *)lds4;
    const int grid = (int)gridDim.x;
    const int t = xcd_remap((int)blockIdx.x, grid);
    const int nmb = cdiv((int)a.T, kBigM), nwt = cdiv(a.wrows, kBigN);
    constexpr int GN = 4;
    const int g = t / (GN * nmb);
    const int gn = min(nwt - g * GN, GN);
    const int in = t - g * GN * nmb;
    Tile ti;
    ti.set = 0;
    ti.first = (in / gn) * kBigM;
    ti.count = min(kBigM, (int)a.T - ti.first);
    ti.wrow0 = (g * GN + in % gn) * kBigN;
    ti.big = true;
    if (ti.count <= 0 || ti.wrow0 >= a.wrows) return;  // uniform (grid = whole tiles)
    for (int i = (int)threadIdx.x; i < kBigM; i += kThreads) s_rows[i] = ti.first + i;
    const int wave_id = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    lds_u8 *const eb = (lds_u8 *)(wave_id == 0 ? lds0 : wave_id == 1 ? lds1 : wave_id == 2 ? lds2 : lds3);
    uint8_t *const hs[5] = {lds0, lds1, lds2, lds3, lds4};
    __syncthreads();
    run_big5<false, F32, false, kBigN, kBigM, true>(a, ti, hs, s_rows, (int)threadIdx.x, eb);
}

// ============================================================================
// Routed fused add-RMSNorm
// ============================================================================
//
// One wave per row, four rows per workgroup.  Lane L owns the 8-element
// chunks L, L+64, L+128, ... of the row.  The sum of squares is taken per lane
// over its chunks in ascending order (elements ascending within a chunk), then
// combined across the wave with a fixed xor-butterfly -- a tree fixed by H
// alone, so a row's rstd and outputs do not depend on T or on the row's
// position in the pack.

template <int CPL>  // chunks per lane; 0 = generic (re-reads h from memory)
__global__ void __launch_bounds__(256)
norm_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ residual,
            const uint16_t *__restrict__ w_und, const uint16_t *__restrict__ w_gen,
            const uint8_t *__restrict__ modality, float eps, uint16_t *__restrict__ out,
            float *__restrict__ rstd_out, int T, int H, int32_t *__restrict__ err_word) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const uint8_t m = modality[t];
    if (m > 1) {
        if (err_word != nullptr && lane == 0) *err_word = kErrModality;
        return;
    }
    const int nchunk = H >> 3;
    const uint16_t *xr = x + (int64_t)t * H;
    uint16_t *rr = residual ? residual + (int64_t)t * H : nullptr;
    const uint16_t *w = m ? w_gen : w_und;

    constexpr int NC = CPL > 0 ? CPL : 1;
    uint4 hv[NC];
    float ss = 0.0f;
    auto make_h = [&](int c) -> uint4 {
        uint4 xv = *(const uint4 *)(xr + c * 8);
        if (rr == nullptr) return xv;
        uint4 rv = *(const uint4 *)(rr + c * 8);
        uint32_t xa[4] = {xv.x, xv.y, xv.z, xv.w}, ra[4] = {rv.x, rv.y, rv.z, rv.w}, o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = bf16_to_f32(xa[e] & 0xffffu) + bf16_to_f32(ra[e] & 0xffffu);
            const float hi = bf16_to_f32(xa[e] >> 16) + bf16_to_f32(ra[e] >> 16);
            o[e] = pack2(lo, hi);
        }
        return uint4{o[0], o[1], o[2], o[3]};
    };
    auto sumsq = [&](uint4 v) {
        uint32_t va[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float lo = bf16_to_f32(va[e] & 0xffffu);
            const float hi = bf16_to_f32(va[e] >> 16);
            ss = ss + lo * lo;
            ss = ss + hi * hi;
        }
    };

    if constexpr (CPL > 0) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            if (c < nchunk) {
                hv[i] = make_h(c);
                sumsq(hv[i]);
            }
        }
    } else {
        for (int c = lane; c < nchunk; c += 64) sumsq(make_h(c));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) ss = ss + __shfl_xor(ss, d, 64);

    const float rstd = 1.0f / sqrtf(ss / (float)H + eps);
    if (rstd_out != nullptr && lane == 0) rstd_out[t] = rstd;

    auto emit = [&](int c, uint4 h) {
        if (rr != nullptr) *(uint4 *)(rr + c * 8) = h;
        if (out != nullptr) {
            uint4 wv = *(const uint4 *)(w + c * 8);
            uint32_t ha[4] = {h.x, h.y, h.z, h.w}, wa[4] = {wv.x, wv.y, wv.z, wv.w}, o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = (bf16_to_f32(ha[e] & 0xffffu) * rstd) * bf16_to_f32(wa[e] & 0xffffu);
                const float hi = (bf16_to_f32(ha[e] >> 16) * rstd) * bf16_to_f32(wa[e] >> 16);
                o[e] = pack2(lo, hi);
            }
            *(uint4 *)(out + (int64_t)t * H + c * 8) = uint4{o[0], o[1], o[2], o[3]};
        }
    };
    if constexpr (CPL > 0) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            if (c < nchunk) emit(c, hv[i]);
        }
    } else {
        // generic path: h must be recomputed before the residual is overwritten
        for (int c = lane; c < nchunk; c += 64) emit(c, make_h(c));
    }
}

// ============================================================================
// Routed GEMM for small packs (weight-bound)
// ============================================================================
//
// A pack of at most kSkinnyMaxT rows reads far more weight bytes than it
// computes on, so the work is spread over as many CUs as the weights allow:
// workgroup b takes weight set b / nblk and the 32 output columns (32 weight
// rows; SwiGLU: 32 gate and the matching 32 up rows) of block b % nblk, for
// all of that set's rows.  Stage j (64 k of the set's XG*8 A rows and of the
// weight rows) sits in LDS slot j % S; all four waves load a share of every
// stage, and one barrier per stage both publishes a stage and frees the slot
// whose fragments were read before it.  Wave i < MJ runs the MFMA chain of
// token rows [32i, 32i+32), reading each stage's fragments one stage ahead
// so that the LDS latency hides under the MFMAs.  The chain is the one of the
// big and small tiles (v_mfma_f32_32x32x16_bf16, D[n][m] = sum_k W[n][k]
// A[m][k], k ascending), so every output element gets the same bytes; its
// K/16 dependent MFMAs (44 cycles each when dependent, measured), not the
// weight loads, set the kernel's time.  Only the pack's A row groups are
// loaded (XG groups of 8: 1 to 16, so up to four compute waves); a fragment
// of an unloaded row reads other bytes of the same slot, which only reach
// output rows that are never stored.  With XG of 12 or 16 a workgroup's ring
// fills most of the LDS, so a pack holding both sets (twice as many
// workgroups as weight blocks) runs its extra workgroups in a second wave
// of the grid; packs of one set, the usual case (a prompt, a decode batch),
// use one workgroup per CU.

constexpr int kSkThreads = 256;
constexpr int kSkLdsBytes = 152 * 1024;  // ring budget
// Ring depth: measured best at 6 stages of one 64-wide k-block (deeper
// rings, and two-block stages, measured equal or slower).  The loads are not what bounds this
// kernel (four waves stream the weights at HBM rate with 8 DMA in flight
// each); the chain is: every output element takes K/16 dependent MFMAs.  A
// shallower ring leaves LDS for a second workgroup per CU (packs that hold
// both sets launch more workgroups than there are CUs).
constexpr int kSkMaxStages = 6;

template <int MI, int XG, int KSUB_>
struct SkinnyCfg {
    static constexpr int KSUB = KSUB_;                          // 64-wide k-blocks per stage
    static constexpr int JMAX = XG >= 8 ? XG / 4 : 1;           // row blocks of 32
    static constexpr int AB = XG * 8 * kRowBytes;               // A rows' bytes of a k-block
    static constexpr int SUB = AB + MI * 32 * kRowBytes;        // + the weight rows
    static constexpr int SLOT = KSUB * SUB;
    static constexpr int XW = XG >= 4 ? XG / 4 : 1;             // A DMA per k-block, waves that load A
    static constexpr int CMAX = (MI + XW) * KSUB;               // most DMA per wave and stage
    static constexpr int S0 = kSkLdsBytes / SLOT;
    static constexpr int S1 = 63 / CMAX + 1;                    // (S - 1) * CMAX <= 63
    static constexpr int S2 = S0 < S1 ? S0 : S1;
    static constexpr int S = S2 < kSkMaxStages ? S2 : kSkMaxStages;  // stages in the ring
    static_assert(SUB >= JMAX * 32 * kRowBytes, "fragment reads stay in the k-block");
    static_assert(S >= 3, "ring depth");
};

// Slot I of a ring of SLOT-byte stages: a distinct LDS object per slot, so
// that the compiler sees that DMA into one slot never aliases reads of
// another and waits only where the code says so.
template <int I, int SLOT>
__device__ __forceinline__ uint8_t *sk_slot() {
    __shared__ __attribute__((aligned(1024))) uint8_t buf[SLOT];
    return buf;
}
template <int SLOT, int... I>
__device__ __forceinline__ void sk_slots(uint8_t *(&sl)[sizeof...(I)], std::integer_sequence<int, I...>) {
    ((sl[I] = sk_slot<I, SLOT>()), ...);
}

template <bool SWIGLU, int XG, int KS>
__device__ __forceinline__ void skinny_tile(const GemmArgs &a, int set, int blk, int count,
                                            uint8_t *const (&sl)[SkinnyCfg<SWIGLU ? 2 : 1, XG, KS>::S],
                                            const int32_t *s_rows, const int wave, const int lane) {
    constexpr int MI = SWIGLU ? 2 : 1;
    using C = SkinnyCfg<MI, XG, KS>;
    constexpr int S = C::S, AB = C::AB, XW = C::XW, KSUB = C::KSUB, SUB = C::SUB;
    const int K = a.K;
    const int nk = K / kBK / KSUB;  // stages (the launch makes KSUB divide K / 64)
    const rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    const rsrc_t wr = make_rsrc(set ? a.w_gen : a.w_und, a.w_bytes);
    // this wave's DMA of a stage: A groups wave + 4g (g < XW; with XG < 4
    // only waves 0 .. XG-1 load one), weight groups wave + 4i (i < MI)
    const bool loads_a = XG >= 4 || wave < XG;
    uint32_t xoff[XW], woff[MI];
#pragma unroll
    for (int g = 0; g < XW; ++g) {
        const int r = (wave + 4 * g) * 8 + (lane >> 3);
        xoff[g] = (uint32_t)s_rows[r] * (uint32_t)(a.ldx * 2) + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int r = (wave + 4 * i) * 8 + (lane >> 3);  // staged W row: [0,32) gate (or plain), [32,64) up
        const int wrow = SWIGLU ? (r < 32 ? blk * 32 + r : a.N + blk * 32 + (r - 32)) : blk * 32 + r;
        woff[i] = (uint32_t)wrow * (uint32_t)(K * 2) + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    }
    auto issue = [&](int kt, int s) {
#pragma unroll
        for (int u = 0; u < KSUB; ++u) {
            const uint32_t koff = (uint32_t)(kt * KSUB + u) * kRowBytes;
            if (loads_a) {
#pragma unroll
                for (int g = 0; g < XW; ++g)
                    dma16(xr, xoff[g], koff, sl[s] + u * SUB + (wave + 4 * g) * 8 * kRowBytes);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
                dma16(wr, woff[i], koff, sl[s] + u * SUB + AB + (wave + 4 * i) * 8 * kRowBytes);
        }
    };
    // a stage has landed for this wave once at most Y younger stages are in
    // flight (counts differ between waves that load A and those that do
    // not, each a wave-uniform branch)
    auto wait_stage = [&](auto y_c) {
        constexpr int Y = decltype(y_c)::value;
        if constexpr (XG >= 4) {
            wait_vm_lgkm0<Y * (MI + XW) * KSUB>();
        } else {
            if (loads_a)
                wait_vm_lgkm0<Y * (MI + 1) * KSUB>();
            else
                wait_vm_lgkm0<Y * MI * KSUB>();
        }
    };

    const int mj = (count + 31) / 32;
    const bool computes = wave < mj;
    f32x16_t acc[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
    const int rsel = lane & 31, khalf = lane >> 5;
    const int lsw = swz(lane & 15);
    const int arow = wave * 32 + rsel;  // this wave's token row of the slot (compute waves)

    // Fragments are read one stage ahead, so that the LDS latency hides
    // under the MFMAs: iteration kt waits for stage kt+1, passes the barrier
    // (which also tells every wave that stage kt's slot, read in the
    // previous iteration, is free), refills that slot with k-block kt+S (the
    // final k-block again past the end, into a slot that is not read again),
    // reads stage kt+1's fragments and runs stage kt's four k-steps.
    constexpr int NQ = 4 * KSUB;  // k-steps of 16 per stage, ascending
    bf16x8_t fa0[NQ][MI], fb0[NQ], fa1[NQ][MI], fb1[NQ];
    auto read_stage = [&](int s, bf16x8_t (&fa)[NQ][MI], bf16x8_t (&fb)[NQ]) {
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            const int u = t / 4, q = t % 4;
            const uint32_t pos = (uint32_t)(((2 * q + khalf) ^ lsw) * 16);
#pragma unroll
            for (int i = 0; i < MI; ++i)
                fa[t][i] = *(const bf16x8_t *)(sl[s] + u * SUB + AB + (i * 32 + rsel) * kRowBytes + pos);
            fb[t] = *(const bf16x8_t *)(sl[s] + u * SUB + arow * kRowBytes + pos);
        }
    };
    auto mfma_stage = [&](const bf16x8_t (&fa)[NQ][MI], const bf16x8_t (&fb)[NQ]) {
#pragma unroll
        for (int t = 0; t < NQ; ++t)
#pragma unroll
            for (int i = 0; i < MI; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[t][i], fb[t], acc[i], 0, 0, 0);
    };
    // stage kt sits in slot s; its fragments are in (fa0, fb0) when the
    // parity p is 0, else in (fa1, fb1)
    auto stage = [&](int kt, int s, auto p_c) {
        wait_stage(std::integral_constant<int, S - 2>{});
        __builtin_amdgcn_s_barrier();
        issue(min(kt + S, nk - 1), s);
        if (computes) {
            if constexpr (decltype(p_c)::value == 0) {
                read_stage((s + 1) % S, fa1, fb1);
                mfma_stage(fa0, fb0);
            } else {
                read_stage((s + 1) % S, fa0, fb0);
                mfma_stage(fa1, fb1);
            }
        }
    };
#pragma unroll
    for (int s = 0; s < S; ++s) issue(min(s, nk - 1), s);
    wait_stage(std::integral_constant<int, S - 1>{});
    __builtin_amdgcn_s_barrier();
    if (computes) read_stage(0, fa0, fb0);
    // unrolled by 2S so that both the slot and the register parity of every
    // stage are compile-time constants
    int kt = 0;
    for (; kt + 2 * S - 1 < nk; kt += 2 * S) {
#pragma unroll
        for (int s = 0; s < 2 * S; ++s) {
            if (s % 2 == 0)
                stage(kt + s, s % S, std::integral_constant<int, 0>{});
            else
                stage(kt + s, s % S, std::integral_constant<int, 1>{});
        }
    }
#pragma unroll
    for (int s = 0; s < 2 * S - 1; ++s) {
        if (kt + s < nk) {
            if (s % 2 == 0)
                stage(kt + s, s % S, std::integral_constant<int, 0>{});
            else
                stage(kt + s, s % S, std::integral_constant<int, 1>{});
        }
    }
    wait_vm_lgkm0<0>();  // no DMA may still be writing LDS when the workgroup ends
    if (!computes) return;

    const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
    const int col0 = blk * 32;
    const int mloc = wave * 32 + rsel;
    if (mloc >= count) return;
    const uint32_t yrow = (uint32_t)s_rows[mloc] * (uint32_t)a.ldy * 2u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (SWIGLU) {
                const float g = acc[0][4 * q + e];
                const float u = acc[1][4 * q + e];
                v[e] = (g / (1.0f + expf(-g))) * u;
            } else {
                v[e] = acc[0][4 * q + e];
            }
        }
        const u32x2_t pk = {pack2(v[0], v[1]), pack2(v[2], v[3])};
        __builtin_amdgcn_raw_buffer_store_b64(pk, yr, yrow + (uint32_t)(col0 + q * 8 + khalf * 4) * 2u, 0, 0);
    }
}

// skinny_tile for a plain GEMM whose workgroup takes two adjacent 32-row
// weight blocks (64 output columns; blk counts them in 64s) and the rows the
// caller gives it (at most 64): the same stages, fragments and MFMA chain per
// output element.  A separate function, so that the other instantiations'
// code is not touched.
template <int XG, int KS>
__device__ __forceinline__ void skinny_pair_tile(const GemmArgs &a, int set, int blk, int count,
                                                 uint8_t *const (&sl)[SkinnyCfg<2, XG, KS>::S],
                                                 const int32_t *s_rows, const int wave, const int lane) {
    constexpr bool SWIGLU = false;
    constexpr int MI = 2;
    using C = SkinnyCfg<MI, XG, KS>;
    constexpr int S = C::S, AB = C::AB, XW = C::XW, KSUB = C::KSUB, SUB = C::SUB;
    const int K = a.K;
    const int nk = K / kBK / KSUB;  // stages (the launch makes KSUB divide K / 64)
    const rsrc_t xr = make_rsrc(a.x, a.x_bytes);
    const rsrc_t wr = make_rsrc(set ? a.w_gen : a.w_und, a.w_bytes);
    // this wave's DMA of a stage: A groups wave + 4g (g < XW; with XG < 4
    // only waves 0 .. XG-1 load one), weight groups wave + 4i (i < MI)
    const bool loads_a = XG >= 4 || wave < XG;
    uint32_t xoff[XW], woff[MI];
#pragma unroll
    for (int g = 0; g < XW; ++g) {
        const int r = (wave + 4 * g) * 8 + (lane >> 3);
        xoff[g] = (uint32_t)s_rows[r] * (uint32_t)(a.ldx * 2) + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int r = (wave + 4 * i) * 8 + (lane >> 3);  // staged W row: [0,32) gate (or plain), [32,64) up
        const int wrow = blk * 64 + r;
        woff[i] = (uint32_t)wrow * (uint32_t)(K * 2) + (uint32_t)(((lane & 7) ^ swz(r)) * 16);
    }
    auto issue = [&](int kt, int s) {
#pragma unroll
        for (int u = 0; u < KSUB; ++u) {
            const uint32_t koff = (uint32_t)(kt * KSUB + u) * kRowBytes;
            if (loads_a) {
#pragma unroll
                for (int g = 0; g < XW; ++g)
                    dma16(xr, xoff[g], koff, sl[s] + u * SUB + (wave + 4 * g) * 8 * kRowBytes);
            }
#pragma unroll
            for (int i = 0; i < MI; ++i)
                dma16(wr, woff[i], koff, sl[s] + u * SUB + AB + (wave + 4 * i) * 8 * kRowBytes);
        }
    };
    // a stage has landed for this wave once at most Y younger stages are in
    // flight (counts differ between waves that load A and those that do
    // not, each a wave-uniform branch)
    auto wait_stage = [&](auto y_c) {
        constexpr int Y = decltype(y_c)::value;
        if constexpr (XG >= 4) {
            wait_vm_lgkm0<Y * (MI + XW) * KSUB>();
        } else {
            if (loads_a)
                wait_vm_lgkm0<Y * (MI + 1) * KSUB>();
            else
                wait_vm_lgkm0<Y * MI * KSUB>();
        }
    };

    const int mj = (count + 31) / 32;
    const bool computes = wave < mj;
    f32x16_t acc[MI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
    const int rsel = lane & 31, khalf = lane >> 5;
    const int lsw = swz(lane & 15);
    const int arow = wave * 32 + rsel;  // this wave's token row of the slot (compute waves)

    // Fragments are read one stage ahead, so that the LDS latency hides
    // under the MFMAs: iteration kt waits for stage kt+1, passes the barrier
    // (which also tells every wave that stage kt's slot, read in the
    // previous iteration, is free), refills that slot with k-block kt+S (the
    // final k-block again past the end, into a slot that is not read again),
    // reads stage kt+1's fragments and runs stage kt's four k-steps.
    constexpr int NQ = 4 * KSUB;  // k-steps of 16 per stage, ascending
    bf16x8_t fa0[NQ][MI], fb0[NQ], fa1[NQ][MI], fb1[NQ];
    auto read_stage = [&](int s, bf16x8_t (&fa)[NQ][MI], bf16x8_t (&fb)[NQ]) {
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            const int u = t / 4, q = t % 4;
            const uint32_t pos = (uint32_t)(((2 * q + khalf) ^ lsw) * 16);
#pragma unroll
            for (int i = 0; i < MI; ++i)
                fa[t][i] = *(const bf16x8_t *)(sl[s] + u * SUB + AB + (i * 32 + rsel) * kRowBytes + pos);
            fb[t] = *(const bf16x8_t *)(sl[s] + u * SUB + arow * kRowBytes + pos);
        }
    };
    auto mfma_stage = [&](const bf16x8_t (&fa)[NQ][MI], const bf16x8_t (&fb)[NQ]) {
#pragma unroll
        for (int t = 0; t < NQ; ++t)
#pragma unroll
            for (int i = 0; i < MI; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[t][i], fb[t], acc[i], 0, 0, 0);
    };
    // stage kt sits in slot s; its fragments are in (fa0, fb0) when the
    // parity p is 0, else in (fa1, fb1)
    auto stage = [&](int kt, int s, auto p_c) {
        wait_stage(std::integral_constant<int, S - 2>{});
        __builtin_amdgcn_s_barrier();
        issue(min(kt + S, nk - 1), s);
        if (computes) {
            if constexpr (decltype(p_c)::value == 0) {
                read_stage((s + 1) % S, fa1, fb1);
                mfma_stage(fa0, fb0);
            } else {
                read_stage((s + 1) % S, fa0, fb0);
                mfma_stage(fa1, fb1);
            }
        }
    };
#pragma unroll
    for (int s = 0; s < S; ++s) issue(min(s, nk - 1), s);
    wait_stage(std::integral_constant<int, S - 1>{});
    __builtin_amdgcn_s_barrier();
    if (computes) read_stage(0, fa0, fb0);
    // unrolled by 2S so that both the slot and the register parity of every
    // stage are compile-time constants
    int kt = 0;
    for (; kt + 2 * S - 1 < nk; kt += 2 * S) {
#pragma unroll
        for (int s = 0; s < 2 * S; ++s) {
            if (s % 2 == 0)
                stage(kt + s, s % S, std::integral_constant<int, 0>{});
            else
                stage(kt + s, s % S, std::integral_constant<int, 1>{});
        }
    }
#pragma unroll
    for (int s = 0; s < 2 * S - 1; ++s) {
        if (kt + s < nk) {
            if (s % 2 == 0)
                stage(kt + s, s % S, std::integral_constant<int, 0>{});
            else
                stage(kt + s, s % S, std::integral_constant<int, 1>{});
        }
    }
    wait_vm_lgkm0<0>();  // no DMA may still be writing LDS when the workgroup ends
    if (!computes) return;

    const rsrc_t yr = make_rsrc(a.y, a.y_bytes);
    const int col0 = blk * 64;
    const int mloc = wave * 32 + rsel;
    if (mloc >= count) return;
    const uint32_t yrow = (uint32_t)s_rows[mloc] * (uint32_t)a.ldy * 2u;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x2_t pk = {pack2(acc[i][4 * q], acc[i][4 * q + 1]), pack2(acc[i][4 * q + 2], acc[i][4 * q + 3])};
            __builtin_amdgcn_raw_buffer_store_b64(pk, yr, yrow + (uint32_t)(col0 + 32 * i + q * 8 + khalf * 4) * 2u, 0,
                                                  0);
        }
}


// nblk: output column blocks of 32 (N / 32, or F / 32 for SwiGLU); XG: A row
// groups of 8 staged per k-block (at least the pack's rows / 8); KS: k-blocks
// of 64 per stage (dividing K / 64).  Builds the
// pack's segment list itself (every wave from the same ballots: lane l owns
// row l); workgroup 0 publishes it (and the error word) to the workspace
// unless the caller passed a ready plan.
// nblk: output column blocks of 32 (N / 32, or F / 32 for SwiGLU); XG: A row
// groups of 8 staged per k-block (at least the pack's rows / 8); KS: k-blocks
// of 64 per stage (dividing K / 64).  Builds the pack's segment list itself
// (every wave from the same ballots: lane l owns rows l and, for packs of more
// than 64 rows, l + 64); workgroup 0 publishes it (and the error word) to the
// workspace unless the caller passed a ready plan.
template <bool SWIGLU, int XG, int KS>
__global__ void __launch_bounds__(kSkThreads)
skinny_kernel(GemmArgs a, int nblk, int publish) {
    using C = SkinnyCfg<SWIGLU ? 2 : 1, XG, KS>;
    constexpr int RW = XG > 8 ? 2 : 1;  // rows per lane
    __shared__ int32_t s_rows[64 * RW];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int T = (int)a.T;
    const int set = (int)blockIdx.x / nblk, blk = (int)blockIdx.x % nblk;
    uint32_t m[RW];
    uint64_t und[RW], gen[RW], bad = 0;
    int U = 0;
#pragma unroll
    for (int h = 0; h < RW; ++h) {
        const int r = lane + 64 * h;
        m[h] = r < T ? (uint32_t)a.modality[r] : 0u;
        bad |= __ballot(r < T && m[h] > 1);
        und[h] = __ballot(r < T && m[h] == 0);
        gen[h] = __ballot(r < T && m[h] == 1);
        U += __popcll(und[h]);
    }
    const uint64_t below = (1ull << lane) - 1;
    if (publish && blockIdx.x == 0 && wave == 0) {
        if (lane == 0) {
            a.hdr_out[0] = bad ? kErrModality : 0;
            a.hdr_out[1] = bad ? 0 : U;
            a.hdr_out[2] = bad ? 0 : T - U;
            a.hdr_out[3] = T;
        }
        if (!bad) {
            int base_u = 0, base_g = U;
#pragma unroll
            for (int h = 0; h < RW; ++h) {
                const int r = lane + 64 * h;
                if (r < T) {
                    const uint64_t mine = m[h] ? gen[h] : und[h];
                    a.perm_out[(m[h] ? base_g : base_u) + __popcll(mine & below)] = r;
                }
                base_u += __popcll(und[h]);
                base_g += __popcll(gen[h]);
            }
        }
    }
    if (bad) {
        // the pack holds an invalid byte: write nothing (all waves), and
        // raise the error word also when a ready plan was passed
        if (!publish && blockIdx.x == 0 && threadIdx.x == 0) a.hdr_out[0] = kErrModality;
        return;
    }
    int count = 0, first = -1;
#pragma unroll
    for (int h = 0; h < RW; ++h) {
        const uint64_t mine = set ? gen[h] : und[h];
        if (first < 0 && mine) first = 64 * h + __ffsll((unsigned long long)mine) - 1;
        count += __popcll(mine);
    }
    if (count == 0) return;  // all waves
    if (wave == 0) {
        int base = 0;
#pragma unroll
        for (int h = 0; h < RW; ++h) {
            const uint64_t mine = set ? gen[h] : und[h];
            if ((mine >> lane) & 1ull) s_rows[base + __popcll(mine & below)] = lane + 64 * h;
            base += __popcll(mine);
        }
#pragma unroll
        for (int h = 0; h < RW; ++h)
            if (lane + 64 * h >= count) s_rows[lane + 64 * h] = first;  // padding: a row of the set
    }
    __syncthreads();
    uint8_t *sl[C::S];
    sk_slots<C::SLOT>(sl, std::make_integer_sequence<int, C::S>{});
    skinny_tile<SWIGLU, XG, KS>(a, set, blk, count, sl, s_rows, wave, lane);
}

// Plain GEMM packs of up to two halves of HR = 8 XG rows (HR = 64: packs of
// 33-128 rows; HR = 128: 129-256).  The 64 output columns of block j have
// four workgroup slots; each set takes c of them in turn (und first):
//   - more than HR rows: c = 2, slot h runs the HR-row half h of the set's
//     rows (in ascending order) by all 64 columns;
//   - at most HR rows, the other set empty: c = 2, slot h runs all of them
//     by the 32 columns of block 2j + h;
//   - at most HR rows, the other set not empty: c = 1, all of them by all
//     64 columns, when the grid (2 nblk) is larger than the CU count
//     (`spread` = 0); else c = 2 as for a lone set;
//   - more than HR rows, the other set empty, `spread` = 1: c = 4, slot p
//     runs half p / 2 of the rows by the 32 columns of block 2j + p % 2;
//   - no rows: c = 0;
// and slots past both sets' share exit.  A mixed pack of many blocks then
// keeps at most three workgroups per block busy (one wave of the grid on
// 256 CUs where four per block, at one workgroup per CU, took two), one of
// few blocks keeps every CU it can busy, and a workgroup
// stages HR A rows and 64 weight rows per k-block instead of all the rows
// and 32.  Every output element keeps its MFMA chain in every case.  nblk =
// N / 32 (even: N is a multiple of 64); the grid is 2 nblk.  Segment list
// and error word as skinny_kernel.
template <int XG, int KS, int RW>
__global__ void __launch_bounds__(kSkThreads)
skinny_pair_kernel(GemmArgs a, int nblk, int publish, int spread) {
    using C = SkinnyCfg<2, XG, KS>;
    constexpr int HR = XG * 8;  // rows of a half
    static_assert(64 * RW == 2 * HR, "a pack of up to two halves, RW rows per lane");
    __shared__ int32_t s_rows[HR];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int T = (int)a.T;
    // slot-major: the busy slots (the low ones) are consecutive workgroups,
    // spread evenly over the XCDs and their shader engines, and a block's
    // slots sit nblk / 2 apart (one XCD, one L2 for its weight rows, when
    // that is a multiple of 8).  Slots interleaved with the block index at a
    // stride of 8 ran packs of one set at half the busy CUs' count per
    // engine and left a second wave: 17.9 -> 30.2 us at T = 100.
    const int npair = nblk >> 1;
    const int slot = (int)blockIdx.x / npair, blk = (int)blockIdx.x % npair;
    uint32_t m[RW];
    uint64_t und[RW], gen[RW], bad = 0;
    int U = 0;
#pragma unroll
    for (int h = 0; h < RW; ++h) {
        const int r = lane + 64 * h;
        m[h] = r < T ? (uint32_t)a.modality[r] : 0u;
        bad |= __ballot(r < T && m[h] > 1);
        und[h] = __ballot(r < T && m[h] == 0);
        gen[h] = __ballot(r < T && m[h] == 1);
        U += __popcll(und[h]);
    }
    const uint64_t below = (1ull << lane) - 1;
    if (publish && blockIdx.x == 0 && wave == 0) {
        if (lane == 0) {
            a.hdr_out[0] = bad ? kErrModality : 0;
            a.hdr_out[1] = bad ? 0 : U;
            a.hdr_out[2] = bad ? 0 : T - U;
            a.hdr_out[3] = T;
        }
        if (!bad) {
            int base_u = 0, base_g = U;
#pragma unroll
            for (int h = 0; h < RW; ++h) {
                const int r = lane + 64 * h;
                if (r < T) {
                    const uint64_t mine = m[h] ? gen[h] : und[h];
                    a.perm_out[(m[h] ? base_g : base_u) + __popcll(mine & below)] = r;
                }
                base_u += __popcll(und[h]);
                base_g += __popcll(gen[h]);
            }
        }
    }
    if (bad) {
        // the pack holds an invalid byte: write nothing (all waves), and
        // raise the error word also when a ready plan was passed
        if (!publish && blockIdx.x == 0 && threadIdx.x == 0) a.hdr_out[0] = kErrModality;
        return;
    }
    if (!publish && T > 128) {
        // above 128 rows a ready plan is checked as the tiled kernel checks
        // it (the segment list itself is still rebuilt from the bytes): a
        // plan whose error word is set, or whose header does not describe T
        // rows, makes every workgroup exit, and workgroup 0 raises
        // MOT_ERR_PLAN for the latter (a workgroup that reads the header
        // after that write sees the error word and exits too)
        const int e0 = a.hdr[0], pu = a.hdr[1], pg = a.hdr[2];
        if (e0 != 0) return;
        if (a.hdr[3] != T || pu < 0 || pg < 0 || pu + pg != T) {
            if (blockIdx.x == 0 && threadIdx.x == 0) a.hdr_out[0] = kErrPlan;
            return;
        }
    }
    const int G = T - U;
    const int c0 = U == 0 ? 0 : (spread && G == 0 && U > HR) ? 4 : (U > HR || G == 0 || spread) ? 2 : 1;
    const int c1 = G == 0 ? 0 : (spread && U == 0 && G > HR) ? 4 : (G > HR || U == 0 || spread) ? 2 : 1;
    if (slot >= c0 + c1) return;  // all waves
    const int set = slot < c0 ? 0 : 1;
    const int part = slot < c0 ? slot : slot - c0;
    const int total = set ? G : U;
    const int cs = set ? c1 : c0;
    const bool split = cs == 4 || (total <= HR && cs == 2);  // one 32-column block each
    const int half = cs == 4 ? part >> 1 : part;
    const int col = cs == 4 ? part & 1 : part;               // 32-column block 2 blk + col (split)
    const int lo = total > HR ? HR * half : 0;               // first sorted row of this workgroup
    const int count = min(total - lo, HR);                    // > 0
    if (wave == 0) {
        int base = 0;
#pragma unroll
        for (int h = 0; h < RW; ++h) {
            const uint64_t mine = set ? gen[h] : und[h];
            const int p = base + __popcll(mine & below);
            if (((mine >> lane) & 1ull) && p >= lo && p < lo + HR) s_rows[p - lo] = lane + 64 * h;
            base += __popcll(mine);
        }
    }
    __syncthreads();
    for (int i = (int)threadIdx.x; i < HR; i += kSkThreads)
        if (i >= count) s_rows[i] = s_rows[0];  // padding: a row of the half
    __syncthreads();
    // one ring serves both tiles: the 32-column stages fit in the slots
    static_assert(SkinnyCfg<1, XG, KS>::S == C::S && SkinnyCfg<1, XG, KS>::SLOT <= C::SLOT, "shared ring");
    uint8_t *sl[C::S];
    sk_slots<C::SLOT>(sl, std::make_integer_sequence<int, C::S>{});
    if (split)
        skinny_tile<false, XG, KS>(a, set, 2 * blk + col, count, sl, s_rows, wave, lane);
    else
        skinny_pair_tile<XG, KS>(a, set, blk, count, sl, s_rows, wave, lane);
}

// ============================================================================
// Routed per-head QK RMSNorm, then the rotary embedding (in place)
// ============================================================================
//
// The "mot_qk_norm_rope" work item (RL-Kernel RFC page, section 5), in the
// order the page's reference hazards fix: the QK norm in fp32, then the
// rotation with Q/K in bf16.  One wave per row and group of eight heads; a
// group of 16 lanes covers one head of 128 columns (lane i of the group holds
// elements 8i .. 8i+7), so one 16-byte load per lane covers four heads, and
// the wave issues its data loads together with those of the row's modality
// byte and position.  Each element's rotate-half partner (64
// columns away) sits in lane i ^ 8 of the same group.  The head's sum of
// squares is taken per lane over its 8 elements in order, then by an
// xor-butterfly over the group's 16 lanes: one fixed tree.  y = bf16((x *
// rstd) * w_set) as in the layer norm; then out = bf16(bf16(y * c) -+
// bf16(y' * s)), where every product of two bf16 values is exact in fp32
// before its rounding.  Rows whose modality byte or position is invalid keep
// their bytes and raise the error word (atomic maximum, so the larger code
// wins whatever the order).

__global__ void set_word_kernel(int32_t *p, int32_t v) {
    if (threadIdx.x == 0) *p = v;
}

__global__ void copy_word_kernel(const int32_t *src, int32_t *dst) {
    if (threadIdx.x == 0) *dst = *src;
}

__global__ void __launch_bounds__(256) qk_norm_rope_kernel(QkArgs a) {
    if (a.after_gemm && __builtin_amdgcn_readfirstlane(*(volatile const int32_t *)a.err) != 0) return;
    const int lane = threadIdx.x & 63;
    const int gi = lane & 15, grp = lane >> 4;  // lane in its 16-lane group, group = head within a chunk
    const int H = a.hq + a.hk;
    const int nch = (H + 3) / 4;                           // 4-head chunks per row
    const int G = (nch + kQkChunks - 1) / kQkChunks;       // waves per row
    const int64_t total = a.T * (int64_t)G;
    for (int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); w < total; w += (int64_t)gridDim.x * 4) {
        const int64_t t = w / G;
        const int c0 = (int)(w - t * G) * kQkChunks;
        uint16_t *const row = a.qkv + t * a.ld;
        // the row's data first (in bounds whatever the row's byte), so that
        // its loads overlap those of the modality byte and the position
        u32x4_t v[kQkChunks];
#pragma unroll
        for (int c = 0; c < kQkChunks; ++c) {
            const int h = 4 * (c0 + c) + grp;
            if (c0 + c < nch && h < H) v[c] = *(const u32x4_t *)(row + (int64_t)h * 128 + 8 * gi);
        }
        const uint32_t m = a.modality[t];
        const int p = a.positions[t];
        const bool bad_pos = p < 0 || p >= a.n_pos;
        if (m > 1 || bad_pos) {
            if (lane == 0 && c0 == 0) atomicMax(a.err, bad_pos ? kErrPosition : kErrModality);
            continue;
        }
        const int64_t ti = (int64_t)p * 64 + 8 * (gi & 7);
        const u32x4_t cv = *(const u32x4_t *)(a.cos_t + ti), sv = *(const u32x4_t *)(a.sin_t + ti);
        const u32x4_t wq = *(const u32x4_t *)((m ? a.qw_gen : a.qw_und) + 8 * gi);
        const u32x4_t wk = *(const u32x4_t *)((m ? a.kw_gen : a.kw_und) + 8 * gi);
#pragma unroll
        for (int c = 0; c < kQkChunks; ++c) {
            if (c0 + c >= nch) break;  // wave-uniform
            const int h = 4 * (c0 + c) + grp;
            const bool live = h < H;
            const u32x4_t o = qk_head(v[c], live, gi, a.eps, h < a.hq ? wq : wk, cv, sv);
            if (live) *(u32x4_t *)(row + (int64_t)h * 128 + 8 * gi) = o;
        }
    }
}

// ============================================================================
// Transpose (backward operands)
// ============================================================================
//
// out[c][r] = in[r][c] for r < rows, c < cols; zero where the row's modality
// byte differs from `keep` (when a modality array is given) and for
// rows <= r < rows_pad.  64x64 tiles through LDS: 16-byte row-contiguous reads
// and writes.  Pure data movement (no arithmetic), so the bytes are exact.

constexpr int kTrTile = 64;

__global__ void __launch_bounds__(256)
transpose_kernel(const uint16_t *__restrict__ in, int64_t ld_in, int rows, int cols,
                 const uint8_t *__restrict__ modality, int keep, uint16_t *__restrict__ out,
                 int64_t ld_out, int rows_pad) {
    __shared__ uint16_t tile[kTrTile][kTrTile + 8];  // +8: 16-byte aligned rows, fewer bank conflicts
    const int r0 = blockIdx.x * kTrTile, c0 = blockIdx.y * kTrTile;
    const int tid = threadIdx.x;
    // read: thread -> (row r0 + tid/8 + 32*pass, 8 columns at c0 + 8*(tid%8))
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int lr = tid / 8 + 32 * pass, lc = 8 * (tid % 8);
        const int r = r0 + lr, c = c0 + lc;
        uint16_t v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (r < rows && (modality == nullptr || (int)modality[r] == keep)) {
            if (c + 8 <= cols) {
                const uint4 q = *(const uint4 *)(in + (int64_t)r * ld_in + c);
                const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = (uint16_t)(w[e] & 0xffffu);
                    v[2 * e + 1] = (uint16_t)(w[e] >> 16);
                }
            } else {
                for (int e = 0; e < 8 && c + e < cols; ++e) v[e] = in[(int64_t)r * ld_in + c + e];
            }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[lr][lc + e] = v[e];
    }
    __syncthreads();
    // write: thread -> (out row c0 + tid/8 + 32*pass, 8 out columns r0 + 8*(tid%8))
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int lc = tid / 8 + 32 * pass, lr = 8 * (tid % 8);
        const int c = c0 + lc, r = r0 + lr;
        if (c >= cols || r >= rows_pad) continue;
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = tile[lr + e][lc];
        uint16_t *dst = out + (int64_t)c * ld_out + r;
        if (r + 8 <= rows_pad) {
            const uint4 q = {v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                             v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16)};
            *(uint4 *)dst = q;
        } else {
            for (int e = 0; e < 8 && r + e < rows_pad; ++e) dst[e] = v[e];
        }
    }
}

}  // namespace

// ============================================================================
// Launchers
// ============================================================================

hipError_t launch_index_sets(const int32_t *und_idx, int64_t n_und, const int32_t *gen_idx, int64_t n_gen,
                             uint8_t *modality, int64_t T, int32_t *err, uint32_t *cnt, hipStream_t stream) {
    const auto blocks = [](int64_t n) { return dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 4096))); };
    hipLaunchKernelGGL(index_clear_kernel, blocks(T), dim3(256), 0, stream, cnt, (int)T, err);
    if (n_und + n_gen > 0)
        hipLaunchKernelGGL(index_count_kernel, blocks(n_und + n_gen), dim3(256), 0, stream, und_idx, (int)n_und,
                           gen_idx, (int)n_gen, cnt, (int)T, err);
    hipLaunchKernelGGL(index_finish_kernel, blocks(T), dim3(256), 0, stream, (const uint32_t *)cnt, (int)T,
                       modality, err);
    return hipGetLastError();
}

hipError_t launch_plan(const uint8_t *modality, int64_t T, int32_t *hdr, int32_t *perm,
                       hipStream_t stream) {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, modality, (int)T,
                       hdr, perm);
    return hipGetLastError();
}

hipError_t launch_gemm_wtok(const GemmArgs &a, bool inline_route, hipStream_t stream) {
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (ncu <= 0) ncu = 1;
    // mode 1: at most (row blocks of T, plus one for the two sets' partial
    // blocks) x weight tiles big tiles
    const int64_t tiles = ((a.T + kBigM - 1) / kBigM + 1) * ((a.wrows + kBigN - 1) / kBigN);
    const int grid = (int)(tiles < ncu ? tiles : ncu);
    if (grid <= 0) return hipSuccess;
    if (inline_route)
        hipLaunchKernelGGL((gemm_kernel<false, false, true, false, false, false, false, false, true>), dim3(grid),
                           dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_kernel<false, false, false, false, false, false, false, false, true>),
                           dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_grad_w(const GemmArgs &a, hipStream_t stream) {
    const int64_t tiles = (a.T + kBigM - 1) / kBigM * ((a.wrows + kBigN - 1) / kBigN);
    if (tiles <= 0) return hipSuccess;
    if (a.out_f32)
        hipLaunchKernelGGL(grad_w_kernel<true>, dim3((unsigned)tiles), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(grad_w_kernel<false>, dim3((unsigned)tiles), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

namespace {
hipError_t launch_gemm_f32(const GemmArgs &a, bool inline_route, int grid, hipStream_t stream) {
    if (inline_route)
        hipLaunchKernelGGL((gemm_kernel<false, false, true, false, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_kernel<false, false, false, false, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_gemm_narrow(const GemmArgs &a, bool inline_route, int grid, hipStream_t stream) {
    if (inline_route)
        hipLaunchKernelGGL((gemm_kernel<false, false, true, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_kernel<false, false, false, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_gemm_qk(const GemmArgs &a, bool inline_route, int grid, hipStream_t stream) {
    if (inline_route)
        hipLaunchKernelGGL((gemm_kernel<false, false, true, false, false, true>), dim3(grid), dim3(kThreads), 0, stream,
                           a);
    else
        hipLaunchKernelGGL((gemm_kernel<false, false, false, false, false, true>), dim3(grid), dim3(kThreads), 0,
                           stream, a);
    return hipGetLastError();
}

template <bool SWIGLU, bool PRO>
hipError_t launch_gemm_t(const GemmArgs &a, bool inline_route, int grid, hipStream_t stream) {
    if constexpr (!SWIGLU && !PRO) {
        // The host does not know the pack's split into the two sets before
        // an in-kernel segment list is built: it picks the instantiation from
        // the cost model with every row in one set.  The short-tile kernel
        // then runs 192-row big tiles for the real split (same bytes as any
        // other shape); the wide-tile kernel chooses between 256 x 224 and
        // 256 x 256 for it.
        int bm = kBigM, bn = kBigN;
        if (a.tile_mode == 0 && a.T <= (1 << 30))
            big_shape(0, (int)a.T, (int)a.wrows, grid, kSmallN, true, true, bm, bn);
        if (a.tile_mode == 0 && bm == kShortM) {
            if (inline_route)
                hipLaunchKernelGGL((gemm_kernel<false, false, true, false, false, false, false, true>), dim3(grid),
                                   dim3(kThreads), 0, stream, a);
            else
                hipLaunchKernelGGL((gemm_kernel<false, false, false, false, false, false, false, true>), dim3(grid),
                                   dim3(kThreads), 0, stream, a);
            return hipGetLastError();
        }
        if (a.tile_mode == 0 && a.wrows % kWideN == 0) {
            if (inline_route)
                hipLaunchKernelGGL((gemm_kernel<false, false, true, false, false, false, true>), dim3(grid),
                                   dim3(kThreads), 0, stream, a);
            else
                hipLaunchKernelGGL((gemm_kernel<false, false, false, false, false, false, true>), dim3(grid),
                                   dim3(kThreads), 0, stream, a);
            return hipGetLastError();
        }
    }
    if (inline_route)
        hipLaunchKernelGGL((gemm_kernel<SWIGLU, PRO, true>), dim3(grid), dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((gemm_kernel<SWIGLU, PRO, false>), dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}
}  // namespace

// Upper bound of the tile list's length for any split of T rows into the two
// sets (at most one workgroup per CU is launched; a shorter list leaves the
// rest of the grid idle).
int64_t gemm_tile_bound(int64_t T, int64_t wrows, int ncu) {
    const int64_t nwt = (wrows + kBigN - 1) / kBigN, nws = (wrows + kSmallN - 1) / kSmallN;
    const int64_t small_only = ((T + kSmallM - 1) / kSmallM + 1) * nws;
    const int64_t big_first = (T / kBigM) * nwt + 4 * (int64_t)ncu + 4 * nws;
    return small_only > big_first ? small_only : big_first;
}

// 1 when the paired small-pack grid (2 nblk workgroups) fits the device's
// CUs: every non-empty set then takes two slots per column block.
int skinny_spread(int nblk) {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    return 2 * nblk <= ncu ? 1 : 0;
}

hipError_t launch_gemm(const GemmArgs &a, bool swiglu, bool inline_route, hipStream_t stream) {
    if (a.out_f32) {
        // fp32 output: 256 x 256 tiles for every row block, one workgroup per CU
        int dev = 0, ncu = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        if (ncu <= 0) ncu = 1;
        const int64_t tiles = ((a.T + kBigM - 1) / kBigM + 1) * ((a.wrows + kBigN - 1) / kBigN);
        return launch_gemm_f32(a, inline_route, (int)(tiles < ncu ? tiles : ncu), stream);
    }
    if (a.T <= kSkinnyMaxT && a.rstd == nullptr && a.tile_mode == 0 && a.qk_heads == 0) {
        // small pack: weight-bound path, one workgroup per 32 output columns
        // and set; XG = A row groups of 8 that cover the pack
        const int nblk = a.N / 32;
        const int pub = inline_route ? 1 : 0;
        const dim3 grid(2 * nblk), block(kSkThreads);
        if (swiglu) {
            if (a.T <= 8)
                hipLaunchKernelGGL((skinny_kernel<true, 1, 1>), grid, block, 0, stream, a, nblk, pub);
            else if (a.T <= 32)
                hipLaunchKernelGGL((skinny_kernel<true, 4, 1>), grid, block, 0, stream, a, nblk, pub);
            else if (a.T <= 64)
                hipLaunchKernelGGL((skinny_kernel<true, 8, 1>), grid, block, 0, stream, a, nblk, pub);
            else if (a.T <= 96)
                hipLaunchKernelGGL((skinny_kernel<true, 12, 1>), grid, block, 0, stream, a, nblk, pub);
            else
                hipLaunchKernelGGL((skinny_kernel<true, 16, 1>), grid, block, 0, stream, a, nblk, pub);
        } else {
            // packs of up to 8 rows measured faster with four A groups (all
            // four waves loading A) than with one
            if (a.T <= 32)
                hipLaunchKernelGGL((skinny_kernel<false, 4, 1>), grid, block, 0, stream, a, nblk, pub);
            else
                // 33-128 rows: halves of each set's rows by 64 output columns
                hipLaunchKernelGGL((skinny_pair_kernel<8, 1, 2>), grid, block, 0, stream, a, nblk, pub,
                                   skinny_spread(nblk));
        }
        return hipGetLastError();
    }
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (ncu <= 0) ncu = 1;
    const bool pro = a.rstd != nullptr;
    if (!swiglu && !pro && a.T <= 2 * kSkinnyMaxT && a.tile_mode == 0 && a.qk_heads == 0) {
        // 129-256 rows: halves of 128 of each set's rows by 64 output columns
        const int nblk = a.N / 32;
        hipLaunchKernelGGL((skinny_pair_kernel<16, 1, 4>), dim3(2 * nblk), dim3(kSkThreads), 0, stream, a, nblk,
                           inline_route ? 1 : 0, skinny_spread(nblk));
        return hipGetLastError();
    }
    // mid-size pack: when every 128-row block of both sets times 64-row
    // weight blocks fits one tile per CU, 128 x 64 tiles put twice as many
    // CUs to work on the weight stream as 128 x 128 ones
    const int64_t narrow_tiles = ((a.T + kSmallM - 1) / kSmallM + 1) * ((a.wrows + kNarrowN - 1) / kNarrowN);
    if (!swiglu && !pro && a.qk_heads == 0 && a.tile_mode == 0 && narrow_tiles <= ncu)
        return launch_gemm_narrow(a, inline_route, (int)narrow_tiles, stream);
    const int64_t bound = gemm_tile_bound(a.T, a.wrows, ncu);
    const int grid = (int)(bound < ncu ? bound : ncu);
    if (grid <= 0) return hipSuccess;
    if (a.qk_heads > 0) return launch_gemm_qk(a, inline_route, grid, stream);
    if (swiglu)
        return pro ? launch_gemm_t<true, true>(a, inline_route, grid, stream)
                   : launch_gemm_t<true, false>(a, inline_route, grid, stream);
    return pro ? launch_gemm_t<false, true>(a, inline_route, grid, stream)
               : launch_gemm_t<false, false>(a, inline_route, grid, stream);
}

hipError_t launch_set_word(int32_t *dst, int32_t v, hipStream_t stream) {
    hipLaunchKernelGGL(set_word_kernel, dim3(1), dim3(64), 0, stream, dst, v);
    return hipGetLastError();
}

hipError_t launch_copy_word(const int32_t *src, int32_t *dst, hipStream_t stream) {
    hipLaunchKernelGGL(copy_word_kernel, dim3(1), dim3(64), 0, stream, src, dst);
    return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const QkArgs &a, hipStream_t stream) {
    if (!a.after_gemm) hipLaunchKernelGGL(set_word_kernel, dim3(1), dim3(64), 0, stream, a.err, 0);
    const int64_t G = ((a.hq + a.hk + 3) / 4 + kQkChunks - 1) / kQkChunks;  // waves per row
    int64_t blocks = (a.T * G + 3) / 4;
    if (blocks > (1 << 20)) blocks = 1 << 20;  // the kernel strides over the rest
    if (blocks > 0)
        hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t *in, int64_t ld_in, int64_t rows, int64_t cols,
                            const uint8_t *modality, int keep, uint16_t *out, int64_t ld_out,
                            int64_t rows_pad, hipStream_t stream) {
    const dim3 grid((unsigned)((rows_pad + kTrTile - 1) / kTrTile), (unsigned)((cols + kTrTile - 1) / kTrTile));
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, stream, in, ld_in, (int)rows, (int)cols, modality,
                       keep, out, ld_out, (int)rows_pad);
    return hipGetLastError();
}

hipError_t launch_norm(const uint16_t *x, uint16_t *residual, const uint16_t *w_und,
                       const uint16_t *w_gen, const uint8_t *modality, float eps, uint16_t *out,
                       float *rstd_out, int64_t T, int H, int32_t *err_word,
                       hipStream_t stream) {
    const dim3 grid((unsigned)((T + 3) / 4)), block(256);
    const int cpl = (H / 8 + 63) / 64;
#define MOT_NORM_CASE(C)                                                                       \
    case C:                                                                                    \
        hipLaunchKernelGGL(norm_kernel<C>, grid, block, 0, stream, x, residual, w_und, w_gen,  \
                           modality, eps, out, rstd_out, (int)T, H, err_word);                 \
        break;
    switch (cpl) {
        MOT_NORM_CASE(1)
        MOT_NORM_CASE(2)
        MOT_NORM_CASE(3)
        MOT_NORM_CASE(4)
        MOT_NORM_CASE(5)
        MOT_NORM_CASE(6)
        MOT_NORM_CASE(7)
        MOT_NORM_CASE(8)
    default:
        hipLaunchKernelGGL(norm_kernel<0>, grid, block, 0, stream, x, residual, w_und, w_gen,
                           modality, eps, out, rstd_out, (int)T, H, err_word);
    }
#undef MOT_NORM_CASE
    return hipGetLastError();
}

}  // namespace mot
