"""Bitwise batch invariance on the GPU (raw-bit identity, +0/-0 distinct).

An output row's bytes may not change with the other rows packed beside it
(RL-Kernel RFC page "[RFC][BAGEL-7B-MoT] WS1/WS2 kernel roadmap", section 1),
and a routed row counts only with both weight sets exercised and a test of
mixed-modality packs (section 6).  The sweep follows the
batch-invariance workload: a fixed 1024-row probe block (77 und then 947 gen
rows, so both sets are probed) repacked with 0, 1, 512 and 3072 other rows at
gen fractions 0%, one token, 50% and 100%, each pack row-permuted with three
seeds; the probe rows must be bitwise equal to the probe-only pack in
identity order.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_transformers_token_amd as mot
import workloads as W
from helpers import dev, raw_equal

pytestmark = pytest.mark.gpu

K, N = W.HIDDEN, W.QKV_DIM


@pytest.fixture(scope="module")
def qkv_setup():
    probe_m = W.pattern(1024)
    x_probe = W.normal_bf16((1024, K), W.seed_of(3, 1))
    x_fill = W.normal_bf16((3072, K), W.seed_of(3, 2))
    wu = dev(W.normal_bf16((N, K), W.seed_of(3, 3), 0.02))
    wg = dev(W.normal_bf16((N, K), W.seed_of(3, 4), 0.02))
    ref = mot.routed_gemm(dev(x_probe), wu, wg, dev(torch.from_numpy(probe_m)))
    torch.cuda.synchronize()
    return dict(probe_m=probe_m, x_probe=x_probe, x_fill=x_fill, wu=wu, wg=wg, ref=ref)


def _fill_modality(n, frac):
    if n == 0:
        return np.zeros(0, np.uint8)
    if frac == "0%":
        return np.zeros(n, np.uint8)
    if frac == "1 token":
        m = np.zeros(n, np.uint8)
        m[n // 2] = 1
        return m
    if frac == "50%":
        m = np.zeros(n, np.uint8)
        m[np.random.default_rng(n).permutation(n)[: n // 2]] = 1
        return m
    return np.ones(n, np.uint8)


PACKS = [(0, "0%")] + [(1, "0%"), (1, "1 token")] + \
        [(n, f) for n in (512, 3072) for f in ("0%", "1 token", "50%", "100%")]


@pytest.mark.parametrize("n,frac", PACKS)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_probe_rows_bitwise_invariant(qkv_setup, n, frac, seed):
    s = qkv_setup
    fm = _fill_modality(n, frac)
    x = torch.cat([s["x_probe"], s["x_fill"][:n]])
    m = np.concatenate([s["probe_m"], fm])
    T = x.shape[0]
    perm = W.permutation(T, 100 + seed).numpy()
    y = mot.routed_gemm(dev(x[perm]), s["wu"], s["wg"], dev(torch.from_numpy(m[perm])))
    pos = np.empty(T, np.int64)
    pos[perm] = np.arange(T)
    got = y[torch.from_numpy(pos[:1024]).cuda()]
    torch.cuda.synchronize()
    assert raw_equal(got, s["ref"]), f"probe rows changed in pack n={n} frac={frac} seed={seed}"


def test_relabel_invariance(qkv_setup):
    s = qkv_setup
    m = s["probe_m"]
    y = mot.routed_gemm(dev(s["x_probe"]), s["wg"], s["wu"], dev(torch.from_numpy(1 - m)))
    assert raw_equal(y, s["ref"])


def test_repeatable_and_strided_output(qkv_setup):
    s = qkv_setup
    md = dev(torch.from_numpy(s["probe_m"]))
    xd = dev(s["x_probe"])
    for _ in range(3):
        assert raw_equal(mot.routed_gemm(xd, s["wu"], s["wg"], md), s["ref"])
    big = torch.zeros((1024, N + 64), dtype=torch.bfloat16, device="cuda")
    mot.routed_gemm(xd, s["wu"], s["wg"], md, out=big[:, 32:32 + N])
    assert raw_equal(big[:, 32:32 + N].contiguous(), s["ref"])


@pytest.mark.parametrize("n_und,n_gen,N", [(0, 3072, 8448), (100, 2972, 8448), (0, 3072, 4352)])
def test_partial_round_of_big_tiles_gives_the_same_bytes(n_und, n_gen, N):
    """A last round of big tiles more than half full runs as big tiles (12 x
    33 = 396 tiles: 140 in the second round), with the partial row blocks'
    small tiles on the workgroups idle in it; N = 4352 (12 x 17 = 204, under
    one round) as a reference.  Bytes equal those of forced tile shapes."""
    T = n_und + n_gen
    m = np.concatenate([np.zeros(n_und, np.uint8), np.ones(n_gen, np.uint8)])
    m = m[W.permutation(T, 6).numpy()].copy()
    x = dev(W.normal_bf16((T, 128), 940))
    wu = dev(W.normal_bf16((N, 128), 941, 0.02))
    wg = dev(W.normal_bf16((N, 128), 942, 0.02))
    md = dev(torch.from_numpy(m))
    auto = mot.routed_gemm(x, wu, wg, md)
    for tile in ("256x256", "128x128"):
        forced = mot.routed_gemm(x, wu, wg, md, tile=tile)
        torch.cuda.synchronize()
        assert raw_equal(auto, forced), tile


@pytest.mark.parametrize("n_und,n_gen,N", [(1024, 3072, 3584), (512, 2048, 3584), (1024, 3072, 448)])
def test_wide_tiles_give_the_bytes_of_the_other_shapes(n_und, n_gen, N):
    """Packs whose weight rows split into 224-row tiles that fill the rounds
    better (O and down at N = 3584 on a pack of whole 256-row blocks: 256
    tiles of 256 x 224 in one round, or a partial round of 160) run the wide
    tiles; their bytes equal those of forced 256 x 256 and 128 x 128 tiles.
    N = 448 is a shape the wide tiles do not take (too few tiles)."""
    T = n_und + n_gen
    m = np.concatenate([np.zeros(n_und, np.uint8), np.ones(n_gen, np.uint8)])
    m = m[W.permutation(T, 5).numpy()].copy()
    x = dev(W.normal_bf16((T, 512), 930))
    wu = dev(W.normal_bf16((N, 512), 931, 0.02))
    wg = dev(W.normal_bf16((N, 512), 932, 0.02))
    md = dev(torch.from_numpy(m))
    auto = mot.routed_gemm(x, wu, wg, md)
    ws = mot.routing_plan(md)
    ready = mot.routed_gemm(x, wu, wg, md, workspace=ws, plan_ready=True)
    for tile in ("256x256", "128x128"):
        forced = mot.routed_gemm(x, wu, wg, md, tile=tile)
        torch.cuda.synchronize()
        assert raw_equal(auto, forced), tile
    assert raw_equal(auto, ready)


@pytest.mark.parametrize("n_und,n_gen,N", [(0, 3072, 3584), (100, 2972, 3584), (0, 3072, 1024)])
def test_short_tiles_give_the_bytes_of_the_other_shapes(n_und, n_gen, N):
    """A pack whose 192-row blocks fill the rounds better (O and down on a
    generation step's 3072 latent rows: 16 x 14 = 224 tiles of 192 x 256,
    against 192 of 256 x 224) runs the short-tile kernel, also when some rows
    belong to the other set (the host chooses from the pack's size alone);
    bytes equal those of forced 256 x 256 and 128 x 128 tiles, with the
    in-kernel segment list and with a ready plan.  N = 1024 is a shape the
    short tiles do not take (too few tiles)."""
    T = n_und + n_gen
    m = np.concatenate([np.zeros(n_und, np.uint8), np.ones(n_gen, np.uint8)])
    m = m[W.permutation(T, 7).numpy()].copy()
    x = dev(W.normal_bf16((T, 512), 950))
    wu = dev(W.normal_bf16((N, 512), 951, 0.02))
    wg = dev(W.normal_bf16((N, 512), 952, 0.02))
    md = dev(torch.from_numpy(m))
    auto = mot.routed_gemm(x, wu, wg, md)
    ws = mot.routing_plan(md)
    ready = mot.routed_gemm(x, wu, wg, md, workspace=ws, plan_ready=True)
    for tile in ("256x256", "128x128"):
        forced = mot.routed_gemm(x, wu, wg, md, tile=tile)
        torch.cuda.synchronize()
        assert raw_equal(auto, forced), tile
    assert raw_equal(auto, ready)


@pytest.mark.parametrize("tile", ["256x256", "128x128"])
def test_tile_shape_does_not_change_bytes(qkv_setup, tile):
    """Every tile shape runs the same per-element k order: forcing one shape
    gives the bytes of the library's own choice."""
    s = qkv_setup
    md = dev(torch.from_numpy(s["probe_m"]))
    y = mot.routed_gemm(dev(s["x_probe"]), s["wu"], s["wg"], md, tile=tile)
    assert raw_equal(y, s["ref"])


@pytest.mark.parametrize("T", [1, 7, 32, 33, 64, 65, 96, 97, 128, 129])
def test_small_packs_match_large_pack_bytes(qkv_setup, T):
    """Packs of up to 128 rows run the weight-bound small-pack kernel (8, 12
    or 16 row groups; 129 rows the tiled kernel): each row's bytes equal
    those of the 1024-row pack."""
    s = qkv_setup
    rows = np.random.default_rng(T).permutation(1024)[:T]
    y = mot.routed_gemm(dev(s["x_probe"][rows]), s["wu"], s["wg"],
                        dev(torch.from_numpy(s["probe_m"][rows].copy())))
    assert raw_equal(y, s["ref"][torch.from_numpy(rows).cuda()])


@pytest.mark.parametrize("T,N,n_und", [(100, 192, 70), (120, 64, 30), (128, 256, 64), (128, 128, 65),
                                       (97, 4608, 97), (256, 192, 128), (256, 128, 129), (200, 4608, 200),
                                       (129, 64, 0), (160, 320, 31), (48, 192, 24), (33, 64, 0),
                                       (64, 4608, 1), (77, 128, 40), (150, 4608, 140), (64, 3584, 32),
                                       (256, 3584, 100), (100, 3584, 100), (256, 3584, 0), (65, 192, 0)])
def test_small_packs_paired_columns(T, N, n_und):
    """Packs of 33-128 (129-256) rows: a set of more than 64 (128) rows is
    split in halves of 64 (128) over workgroups of 64 output columns, a
    smaller set over workgroups of 32 columns.  The bytes of forced 128 x 128
    tiles, for sets just over, at and under a half, and an empty set."""
    m = np.zeros(T, np.uint8)
    m[n_und:] = 1
    m = m[np.random.default_rng(T + N).permutation(T)]
    x = dev(W.normal_bf16((T, 512), 960 + T))
    wu = dev(W.normal_bf16((N, 512), 961, 0.02))
    wg = dev(W.normal_bf16((N, 512), 962, 0.02))
    md = dev(torch.from_numpy(m))
    small = mot.routed_gemm(x, wu, wg, md)
    tiled = mot.routed_gemm(x, wu, wg, md, tile="128x128")
    assert raw_equal(small, tiled)


def test_mixed_equals_per_set_dense(qkv_setup):
    """Mixed pack == each set's rows run as a single-set pack (gathered)."""
    s = qkv_setup
    m = s["probe_m"]
    for setv, w in ((0, s["wu"]), (1, s["wg"])):
        rows = np.nonzero(m == setv)[0]
        xs = dev(s["x_probe"][rows])
        y = mot.routed_gemm(xs, w, w, dev(torch.full((rows.size,), setv, dtype=torch.uint8)))
        assert raw_equal(y, s["ref"][torch.from_numpy(rows).cuda()])


def test_prologue_fused_equals_unfused():
    """Routed-RMSNorm prologue inside the GEMM == norm kernel output fed to
    the plain GEMM, bit for bit (QKV and SwiGLU)."""
    T = 1101
    m = W.pattern(T)
    md = dev(torch.from_numpy(m))
    x, r = W.residual_inputs(T, K, base=70)
    nwu, nwg = (dev(t) for t in W.norm_weights(K, base=70))
    res = dev(r)
    y_norm, rstd = mot.fused_add_rmsnorm(dev(x), res, nwu, nwg, md)
    wu = dev(W.normal_bf16((N, K), 71, 0.02))
    wg = dev(W.normal_bf16((N, K), 72, 0.02))
    unfused = mot.routed_gemm(y_norm, wu, wg, md)
    fused = mot.routed_gemm(res, wu, wg, md, norm=(rstd, nwu, nwg))
    assert raw_equal(fused, unfused)
    F = 256
    gu_u = dev(W.normal_bf16((2 * F, K), 73, 0.02))
    gu_g = dev(W.normal_bf16((2 * F, K), 74, 0.02))
    a1 = mot.routed_gemm_swiglu(y_norm, gu_u, gu_g, md)
    a2 = mot.routed_gemm_swiglu(res, gu_u, gu_g, md, norm=(rstd, nwu, nwg))
    assert raw_equal(a1, a2)


def test_norm_rows_invariant():
    T, H = 4096, K
    m = W.pattern(T)
    x, r = W.residual_inputs(T, H, base=75)
    nwu, nwg = (dev(t) for t in W.norm_weights(H, base=75))
    full, rstd = mot.fused_add_rmsnorm(dev(x), dev(r), nwu, nwg, dev(torch.from_numpy(m)))
    perm = W.permutation(T, 5).numpy()[:300]
    part, rstd_p = mot.fused_add_rmsnorm(dev(x[perm]), dev(r[perm]), nwu, nwg,
                                         dev(torch.from_numpy(m[perm])))
    idx = torch.from_numpy(perm).cuda()
    assert raw_equal(part, full[idx])
    assert torch.equal(rstd_p.view(torch.int32), rstd[idx].view(torch.int32))


def test_plan_ready_reuses_the_plan(qkv_setup):
    s = qkv_setup
    md = dev(torch.from_numpy(s["probe_m"]))
    ws = mot.routing_plan(md)
    y = mot.routed_gemm(dev(s["x_probe"]), s["wu"], s["wg"], md, workspace=ws, plan_ready=True)
    assert raw_equal(y, s["ref"])


@pytest.mark.parametrize("T,N", [(65, 4608), (200, 4608), (256, 4608), (300, 192), (1025, 320)])
def test_narrow_tiles_match_wide_tile_bytes(T, N):
    """Mid-size packs whose 128-row blocks times 64-row weight blocks fit one
    tile per CU run 128 x 64 tiles; their bytes equal those of the 128 x 128
    tiles (forced with a tile flag) row for row."""
    m = W.pattern(T)
    m[::3] = 1 - m[::3]
    x = dev(W.normal_bf16((T, 512), 980 + T))
    wu = dev(W.normal_bf16((N, 512), 981, 0.02))
    wg = dev(W.normal_bf16((N, 512), 982, 0.02))
    md = dev(torch.from_numpy(m))
    auto = mot.routed_gemm(x, wu, wg, md)
    wide = mot.routed_gemm(x, wu, wg, md, tile="128x128")
    assert raw_equal(auto, wide)



@pytest.mark.parametrize("T,N", [(256, 4608), (160, 4480), (129, 64), (200, 192)])
def test_narrow_tiles_one_set(T, N):
    """Mid-size packs of one set, whose tiles are dealt to the XCDs by
    weight tile (weight tile counts that are and are not multiples of 8,
    and a single weight tile): the bytes of 128 x 128 tiles."""
    m = np.ones(T, np.uint8)
    x = dev(W.normal_bf16((T, 512), 985 + T))
    wu = dev(W.normal_bf16((N, 512), 986, 0.02))
    wg = dev(W.normal_bf16((N, 512), 987, 0.02))
    md = dev(torch.from_numpy(m))
    auto = mot.routed_gemm(x, wu, wg, md)
    wide = mot.routed_gemm(x, wu, wg, md, tile="128x128")
    assert raw_equal(auto, wide)


@pytest.mark.parametrize("T,K,N,n_und", [(40, 64, 128, 20), (150, 64, 192, 150), (256, 18944, 3584, 100),
                                         (100, 18944, 3584, 0), (33, 3584, 64, 32)])
def test_small_packs_paired_strides_and_depths(T, K, N, n_und):
    """Packs of 33-256 rows at the shortest contraction (one k-block) and at
    the down projection's (296 k-blocks), reading x and writing y through
    row strides wider than the rows: the bytes of forced 128 x 128 tiles on
    contiguous copies, and the columns past N of y's rows left as they were."""
    m = np.zeros(T, np.uint8)
    m[n_und:] = 1
    m = m[np.random.default_rng(T + K).permutation(T)]
    xb = dev(W.normal_bf16((T, K + 64), 970 + T))
    x = xb[:, :K]
    wu = dev(W.normal_bf16((N, K), 971, 0.02))
    wg = dev(W.normal_bf16((N, K), 972, 0.02))
    md = dev(torch.from_numpy(m))
    yb = torch.full((T, N + 128), 3.0, dtype=torch.bfloat16, device="cuda")
    mot.routed_gemm(x, wu, wg, md, out=yb[:, :N])
    tiled = mot.routed_gemm(x.contiguous(), wu, wg, md, tile="128x128")
    assert raw_equal(yb[:, :N].contiguous(), tiled)
    assert torch.all(yb[:, N:] == 3.0)


@pytest.mark.parametrize("T", [40, 100, 200])
def test_plan_ready_small_and_mid_packs(T):
    """A ready plan reused by the small-pack and the 128 x 64 tile paths
    gives the bytes of the in-kernel segment list."""
    m = W.pattern(T)
    m[::4] = 1 - m[::4]
    x = dev(W.normal_bf16((T, 512), 990 + T))
    wu = dev(W.normal_bf16((4608, 512), 991, 0.02))
    wg = dev(W.normal_bf16((4608, 512), 992, 0.02))
    md = dev(torch.from_numpy(m))
    inline = mot.routed_gemm(x, wu, wg, md)
    ws = mot.routing_plan(md)
    ready = mot.routed_gemm(x, wu, wg, md, workspace=ws, plan_ready=True)
    assert raw_equal(ready, inline)


# ---- the same sweep on the MLP's routed GEMMs --------------------------------

@pytest.fixture(scope="module")
def mlp_setup():
    """BAGEL MLP weights at full size: gate/up K=3584 -> 2 x 18944 (SwiGLU)
    and down K=18944 -> 3584; probe and filler rows for both."""
    gu_u, gu_g, dn_u, dn_g = (dev(t) for t in W.mlp_weights(base=7))
    probe_m = W.pattern(1024)
    xg_probe = W.normal_bf16((1024, K), W.seed_of(7, 20))
    xg_fill = W.normal_bf16((3072, K), W.seed_of(7, 21))
    xd_probe = W.normal_bf16((1024, W.FFN), W.seed_of(7, 22))
    xd_fill = W.normal_bf16((3072, W.FFN), W.seed_of(7, 23))
    md = dev(torch.from_numpy(probe_m))
    ref_g = mot.routed_gemm_swiglu(dev(xg_probe), gu_u, gu_g, md)
    ref_d = mot.routed_gemm(dev(xd_probe), dn_u, dn_g, md)
    torch.cuda.synchronize()
    return dict(probe_m=probe_m, swiglu=(xg_probe, xg_fill, lambda x, m: mot.routed_gemm_swiglu(x, gu_u, gu_g, m),
                                         ref_g),
                down=(xd_probe, xd_fill, lambda x, m: mot.routed_gemm(x, dn_u, dn_g, m), ref_d))


# a subset of the QKV sweep's packs: the probe alone, one extra row of each
# set, and 512 / 3072 extra rows at 0%, 50% and 100% gen, permuted
MLP_PACKS = [(0, "0%"), (1, "0%"), (1, "1 token"), (512, "50%"), (3072, "0%"), (3072, "50%"), (3072, "100%")]


@pytest.mark.parametrize("op", ["swiglu", "down"])
@pytest.mark.parametrize("n,frac", MLP_PACKS)
def test_mlp_probe_rows_bitwise_invariant(mlp_setup, op, n, frac):
    s = mlp_setup
    x_probe, x_fill, run, ref = s[op]
    fm = _fill_modality(n, frac)
    x = torch.cat([x_probe, x_fill[:n]])
    m = np.concatenate([s["probe_m"], fm])
    T = x.shape[0]
    perm = W.permutation(T, 300 + n).numpy()
    y = run(dev(x[perm]), dev(torch.from_numpy(m[perm])))
    pos = np.empty(T, np.int64)
    pos[perm] = np.arange(T)
    got = y[torch.from_numpy(pos[:1024]).cuda()]
    torch.cuda.synchronize()
    assert raw_equal(got, ref), f"{op}: probe rows changed in pack n={n} frac={frac}"


@pytest.mark.parametrize("op", ["swiglu", "down"])
def test_mlp_small_packs_match_large_pack_bytes(mlp_setup, op):
    """Packs of 1, 33, 64, 100 and 128 rows (the small-pack kernel) give each
    row the bytes it has in the 1024-row pack, for the MLP shapes too."""
    s = mlp_setup
    x_probe, _, run, ref = s[op]
    for T in (1, 33, 64, 100, 128):
        rows = np.random.default_rng(50 + T).permutation(1024)[:T]
        y = run(dev(x_probe[rows]), dev(torch.from_numpy(s["probe_m"][rows].copy())))
        assert raw_equal(y, ref[torch.from_numpy(rows).cuda()]), (op, T)
