"""Pins of the CPU oracle against things other than itself.

Every check here is independent of the oracle's own code: exact integer /
rational arithmetic written in this file, library routines (torch fp64
matmul, torch silu), closed forms, brute force on tiny shapes, and structural
invariants of the routing definition (RL-Kernel RFC page "[RFC][BAGEL-7B-MoT]
WS1/WS2 kernel roadmap", section 1: a per-row index, not a router, gives each
row its weight set, and an output row's bytes may not change with the other
rows of the pack).

The mutation tests at the end plant typical mistakes (swapped weight sets, a
dropped k term, a transposed operand, a wrong SiLU sign, a norm without the
mean) on the CPU and show that the pins catch them.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- an independent bf16 rounding, by exact rational arithmetic ---------------

def rne_bf16_exact(v) -> int:
    """Nearest bf16 (ties to even) of an exact rational or float, computed with
    integers only: find the binade, scale to an integer significand grid and
    round half to even by comparing remainders."""
    q = Fraction(v)
    if q == 0:
        return 0x8000 if (isinstance(v, float) and math.copysign(1.0, v) < 0) else 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    step_exp = max(e - 7, -133)           # spacing of the bf16 grid at a
    scaled = a / (Fraction(2) ** step_exp)
    n, rem = divmod(scaled.numerator, scaled.denominator)
    twice = 2 * rem
    if twice > scaled.denominator or (twice == scaled.denominator and n % 2 == 1):
        n += 1
    val = Fraction(n) * Fraction(2) ** step_exp
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    f = np.float32(float(val))             # exact: val has <= 8 significant bits
    return sign | int(f.view(np.uint32) >> 16)


def test_rounding_helper_against_torch_on_fp32_exact_values():
    # For values exactly representable in fp32, torch's fp32->bf16 cast is RNE:
    # a library special case that pins the helper above.
    g = torch.Generator().manual_seed(5)
    v = torch.randn(4000, generator=g) * torch.exp2(torch.randint(-140, 120, (4000,), generator=g).float())
    v = torch.cat([v, torch.tensor([1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 2.0**-133, 2.0**-134,
                                    3 * 2.0**-135, 3.3895313892515355e38, 3.3961775292304957e38, 0.0])])
    want = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for x, wv in zip(v.tolist(), want.tolist()):
        assert rne_bf16_exact(float(np.float32(x))) == wv, x


def test_oracle_bf16_round_matches_exact_rounding():
    rng = np.random.default_rng(1)
    vals = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 127, 3000)))
    # ties and near-ties at several binades, subnormals, overflow boundary
    for e in (-133, -130, -126, -20, 0, 7, 100, 126):
        for k in range(0, 40):
            base = 2.0 ** e
            vals += [base * (1 + k / 256), base * (1 + k / 256) + base * 2**-30,
                     base * (1 + k / 256) - base * 2**-30]
    vals += [2.0**-134, 2.0**-134 * 1.0000001, 2.0**-135, 3.3961775292304957e38, 3.3961775292304955e38,
             1e300, -1e300, 0.0, -0.0]
    for v in vals:
        assert oracle.bf16_round(v) == rne_bf16_exact(v), v


def test_bf16_decode_is_exact():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (b & 0x7F80) != 0x7F80
    got = oracle.bf16_to_f64(b[finite])
    want = torch.from_numpy(b[finite].view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(got, want)
    # the C decoder agrees with the numpy decoder on a spread of patterns
    for v in (0x0000, 0x0001, 0x3F80, 0xBF80, 0x7F7F, 0x8001, 0x4049):
        assert oracle.bf16_value(v) == oracle.bf16_to_f64(np.array([v], np.uint16))[0]


# ---- routed GEMM -------------------------------------------------------------

def _dense(x, w):
    return (torch.from_numpy(oracle.bf16_to_f64(x)) @ torch.from_numpy(oracle.bf16_to_f64(w)).T).numpy()


def test_tiny_brute_force_every_element():
    """Tiny case (T=64, K=256, N=384, 24 und + 40 gen rows): every fp64 sum is
    within the sequential-summation bound of the exact sum (math.fsum of the
    exact bf16 x bf16 products), and every bf16 output is the exactly rounded
    exact sum."""
    x, wu, wg, m = W.tiny()
    X, WU, WG = W.bits(x), W.bits(wu), W.bits(wg)
    ref, out = oracle.routed_gemm(X, WU, WG, m)
    xd = oracle.bf16_to_f64(X)
    wud, wgd = oracle.bf16_to_f64(WU), oracle.bf16_to_f64(WG)
    K = X.shape[1]
    for t in range(X.shape[0]):
        w = wgd if m[t] else wud
        P = xd[t][None, :] * w            # exact: 8x8-bit significands
        for n in range(w.shape[0]):
            p = P[n]
            s = math.fsum(p)
            bound = K * 2.0**-53 * float(np.abs(p).sum())
            assert abs(ref[t, n] - s) <= bound
            exact = sum((Fraction(v) for v in p), Fraction(0)) if _near_tie(s) else s
            assert out[t, n] == rne_bf16_exact(exact), (t, n)


def _near_tie(s: float) -> bool:
    if s == 0.0:
        return False
    e = math.frexp(abs(s))[1] - 1
    step = 2.0 ** max(e - 7, -133)
    r = abs(s) / step
    return abs(r - math.floor(r) - 0.5) < 1e-6


@pytest.mark.parametrize("which", [W.UND, W.GEN])
def test_single_set_pack_is_plain_gemm(which):
    """All-und pack == torch fp64 matmul with W_und (and gen with W_gen)."""
    T, K, N = 96, 320, 192
    x, wu, wg, _ = W.gemm_case(T, K, N, np.zeros(T, np.uint8), base=3)
    m = np.full(T, which, np.uint8)
    ref, out = oracle.routed_gemm(W.bits(x), W.bits(wu), W.bits(wg), m)
    want = _dense(W.bits(x), W.bits(wg if which else wu))
    assert np.max(np.abs(ref - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_mixed_pack_is_per_row_gemm():
    """A mixed pack equals the per-set dense GEMMs of the gathered rows,
    scattered back to their positions."""
    T, K, N = 200, 256, 128
    m = np.random.default_rng(7).integers(0, 2, T).astype(np.uint8)
    x, wu, wg, _ = W.gemm_case(T, K, N, m, base=4)
    X = W.bits(x)
    ref, _ = oracle.routed_gemm(X, W.bits(wu), W.bits(wg), m)
    want = np.empty_like(ref)
    for s, w in ((0, wu), (1, wg)):
        rows = np.nonzero(m == s)[0]
        want[rows] = _dense(X[rows], W.bits(w))
    assert np.max(np.abs(ref - want)) <= 1e-12 * np.max(np.abs(want))


def test_permutation_equivariance_and_relabel():
    T, K, N = 150, 192, 64
    m = W.pattern(T)
    x, wu, wg, _ = W.gemm_case(T, K, N, m, base=5)
    X, WU, WG = W.bits(x), W.bits(wu), W.bits(wg)
    _, out = oracle.routed_gemm(X, WU, WG, m)
    p = np.random.default_rng(2).permutation(T)
    _, outp = oracle.routed_gemm(X[p], WU, WG, m[p])
    assert np.array_equal(outp, out[p])
    _, outr = oracle.routed_gemm(X, WG, WU, (1 - m).astype(np.uint8))
    assert np.array_equal(outr, out)
    # a row computed alone equals the row inside the pack
    _, one = oracle.routed_gemm(X[7:8], WU, WG, m[7:8])
    assert np.array_equal(one[0], out[7])


def test_leading_dimension():
    T, K, N = 40, 128, 64
    m = W.pattern(T)
    x, wu, wg, _ = W.gemm_case(T, 2 * K, N, m, base=6)
    X = W.bits(x)
    wu2, wg2 = W.bits(wu)[:, :K].copy(), W.bits(wg)[:, :K].copy()
    ref_slice, _ = oracle.routed_gemm(X[:, :K].copy(), wu2, wg2, m)
    # strided view through the C entry point: x rows of length 2K, first K used
    L = oracle.lib()
    ref = np.empty((T, N))
    L.mot_oracle_routed_gemm(oracle._p(X), 2 * K, oracle._p(wu2), oracle._p(wg2), oracle._p(m),
                             T, K, N, oracle._p(ref), None, 0)
    assert np.array_equal(ref, ref_slice)


# ---- SwiGLU ------------------------------------------------------------------

def test_swiglu_matches_torch_silu_fp64():
    T, K, F = 48, 256, 96
    m = W.pattern(T)
    x, _, _, _ = W.gemm_case(T, K, 8, m, base=7)
    wu = W.normal_bf16((2 * F, K), 71, 0.05)
    wg = W.normal_bf16((2 * F, K), 72, 0.05)
    X, WU, WG = W.bits(x), W.bits(wu), W.bits(wg)
    ref, out = oracle.routed_gemm_swiglu(X, WU, WG, m)
    want = np.empty((T, F))
    for s, w in ((0, WU), (1, WG)):
        rows = np.nonzero(m == s)[0]
        gu = torch.from_numpy(_dense(X[rows], w))
        want[rows] = (torch.nn.functional.silu(gu[:, :F]) * gu[:, F:]).numpy()
    assert np.max(np.abs(ref - want)) <= 1e-12 * np.max(np.abs(want))
    assert all(out[i, j] == rne_bf16_exact(float(ref[i, j])) for i in range(0, T, 5) for j in range(F))


def test_swiglu_closed_forms():
    K, F = 64, 4
    # g = 0 exactly (gate rows zero) -> act = 0 for any u
    x = np.full((2, K), 0x3F80, np.uint16)                      # x = 1
    w = np.zeros((2 * F, K), np.uint16)
    w[F:] = 0x3F80                                              # u = K
    ref, out = oracle.routed_gemm_swiglu(x, w, w, np.array([0, 1], np.uint8))
    assert np.all(ref == 0.0) and np.all((out & 0x7FFF) == 0)
    # g large: silu(g) = g up to exp(-g); g = 64 (all ones), u = 2 -> act = 128
    w2 = np.full((2 * F, K), 0x3F80, np.uint16)
    w2[F:] = 0x0000
    w2[F:, 0] = 0x4000                                          # u = 2*x0 = 2
    ref, out = oracle.routed_gemm_swiglu(x, w2, w2, np.array([1, 0], np.uint8))
    assert np.allclose(ref, 128.0, rtol=1e-20, atol=128 * 64 * math.exp(-64))
    assert np.all(out == 0x4300)                                # bf16(128)
    # g very negative: silu -> -0-ish tiny, act finite and ~0
    w3 = np.full((2 * F, K), 0xBF80, np.uint16)                 # g = -64
    ref, _ = oracle.routed_gemm_swiglu(x, w3, w3, np.array([0, 0], np.uint8))
    assert np.all(np.abs(ref) < 1e-20)


# ---- fused add-RMSNorm -------------------------------------------------------

def test_rmsnorm_textbook_special_case():
    """w = 1 and no residual: the textbook x / sqrt(mean(x^2) + eps), by torch
    fp64; the routing then cannot matter."""
    T, H = 33, 3584
    x = W.normal_bf16((T, H), 81)
    ones = np.full(H, 0x3F80, np.uint16)
    m = W.pattern(T)
    r = oracle.fused_add_rmsnorm(W.bits(x), None, ones, ones, m, eps=1e-6)
    xd = x.double()
    want = (xd / torch.sqrt((xd * xd).mean(-1, keepdim=True) + float(np.float32(1e-6)))).numpy()
    assert np.max(np.abs(r["ref"] - want)) <= 1e-14
    assert np.array_equal(r["h"], W.bits(x))


def test_rmsnorm_constant_row_closed_form():
    H = 256
    c = 0x4040                                                  # 3.0
    x = np.full((2, H), c, np.uint16)
    wu = np.full(H, 0x3F80, np.uint16)                          # 1.0
    wg = np.full(H, 0x4000, np.uint16)                          # 2.0
    eps = 0.5
    r = oracle.fused_add_rmsnorm(x, None, wu, wg, np.array([0, 1], np.uint8), eps=eps)
    y0 = 3.0 / math.sqrt(9.0 + eps)
    assert np.allclose(r["ref"][0], y0, rtol=1e-15) and np.allclose(r["ref"][1], 2 * y0, rtol=1e-15)
    assert np.allclose(r["rstd"], 1 / math.sqrt(9.5), rtol=1e-15)


def test_fused_add_residual_is_exactly_rounded_sum():
    T, H = 16, 512
    x, res = W.residual_inputs(T, H, base=9)
    wu, wg = W.norm_weights(H, base=9)
    m = W.pattern(T)
    r = oracle.fused_add_rmsnorm(W.bits(x), W.bits(res), W.bits(wu), W.bits(wg), m)
    xd, rd = oracle.bf16_to_f64(W.bits(x)), oracle.bf16_to_f64(W.bits(res))
    for t in range(T):
        for k in range(0, H, 7):
            assert r["h"][t, k] == rne_bf16_exact(Fraction(float(xd[t, k])) + Fraction(float(rd[t, k])))
    # normalising the rounded sum equals the fused result (fused == add, store, norm)
    r2 = oracle.fused_add_rmsnorm(r["h"], None, W.bits(wu), W.bits(wg), m)
    assert np.array_equal(r2["out"], r["out"]) and np.array_equal(r2["ref"], r["ref"])


def test_rmsnorm_routing_rows_independent():
    T, H = 20, 384
    x = W.normal_bf16((T, H), 91)
    wu, wg = W.norm_weights(H, base=10)
    m = W.pattern(T)
    full = oracle.fused_add_rmsnorm(W.bits(x), None, W.bits(wu), W.bits(wg), m)["out"]
    for t in (0, 5, 19):
        one = oracle.fused_add_rmsnorm(W.bits(x)[t:t + 1], None, W.bits(wu), W.bits(wg), m[t:t + 1])["out"]
        assert np.array_equal(one[0], full[t])
    # the weight applied is the row's own set
    xd = oracle.bf16_to_f64(W.bits(x))
    for t in range(T):
        wv = oracle.bf16_to_f64(W.bits(wg if m[t] else wu))
        rs = 1 / math.sqrt(float(np.mean(xd[t] ** 2)) + float(np.float32(1e-6)))
        assert np.allclose(oracle.bf16_to_f64(full[t]), xd[t] * rs * wv, rtol=2**-8, atol=0)


# ---- routing plan ------------------------------------------------------------

def test_routing_plan_is_stable_partition():
    for T, seed in ((0, 0), (1, 1), (77, 2), (4096, 3)):
        m = np.random.default_rng(seed).integers(0, 2, T).astype(np.uint8)
        perm, nu, ng = oracle.routing_plan(m)
        want = np.argsort(m, kind="stable")
        assert np.array_equal(perm, want) and nu == int((m == 0).sum()) and ng == T - nu
    bad = np.array([0, 1, 2, 0], np.uint8)
    assert oracle.routing_plan(bad) is None


# ---- the hand-worked examples in tests/golden ---------------------------------

def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_golden_hand_worked_gemm():
    g = _load("routed_gemm_worked_example.json")
    x = np.array(g["x_bits"], np.uint16)
    ref, out = oracle.routed_gemm(x, np.array(g["w_und_bits"], np.uint16),
                                  np.array(g["w_gen_bits"], np.uint16), np.array(g["modality"], np.uint8))
    assert ref.tolist() == g["expected_sum"]
    assert out.tolist() == g["expected_bits"]


def test_golden_hand_worked_norm():
    g = _load("rmsnorm_worked_example.json")
    r = oracle.fused_add_rmsnorm(np.array(g["x_bits"], np.uint16), np.array(g["r_bits"], np.uint16),
                                 np.array(g["w_und_bits"], np.uint16), np.array(g["w_gen_bits"], np.uint16),
                                 np.array(g["modality"], np.uint8), eps=g["eps"])
    assert r["h"].tolist() == g["expected_h_bits"]
    assert r["out"].tolist() == g["expected_bits"]


# ---- planted mistakes: the pins must catch them ---------------------------------

def _pin_dense(out_ref, X, WU, WG, m):
    want = np.empty_like(out_ref)
    for s, w in ((0, WU), (1, WG)):
        rows = np.nonzero(m == s)[0]
        if rows.size:
            want[rows] = _dense(X[rows], w)
    return np.max(np.abs(out_ref - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_pins_catch_planted_gemm_mistakes():
    T, K, N = 64, 128, 128
    m = W.tiny_modality()
    x, wu, wg, _ = W.gemm_case(T, K, N, m, base=11)
    X, WU, WG = W.bits(x), W.bits(wu), W.bits(wg)
    good, _ = oracle.routed_gemm(X, WU, WG, m)
    assert _pin_dense(good, X, WU, WG, m)
    swapped, _ = oracle.routed_gemm(X, WG, WU, m)               # sets swapped
    assert not _pin_dense(swapped, X, WU, WG, m)
    dropped, _ = oracle.routed_gemm(X[:, :K - 1].copy(), WU[:, :K - 1].copy(), WG[:, :K - 1].copy(), m)
    assert not _pin_dense(dropped, X, WU, WG, m)                 # last k term dropped
    transposed, _ = oracle.routed_gemm(X, WU.reshape(K, N).T.copy(), WG.reshape(K, N).T.copy(), m)
    assert not _pin_dense(transposed, X, WU, WG, m)              # operand read transposed
    one_set, _ = oracle.routed_gemm(X, WU, WU, m)               # routing ignored
    assert not _pin_dense(one_set, X, WU, WG, m)


def test_pins_catch_planted_swiglu_and_norm_mistakes():
    T, K, F = 16, 64, 32
    m = W.pattern(T)
    x = W.normal_bf16((T, K), 12)
    w = W.normal_bf16((2 * F, K), 13, 0.1)
    X, Wb = W.bits(x), W.bits(w)
    ref, _ = oracle.routed_gemm_swiglu(X, Wb, Wb, m)
    gu = torch.from_numpy(_dense(X, Wb))
    g, u = gu[:, :F], gu[:, F:]
    good = (torch.nn.functional.silu(g) * u).numpy()
    assert np.allclose(ref, good, rtol=1e-12, atol=1e-14)
    for wrong in ((g * torch.sigmoid(-g) * u), (torch.nn.functional.silu(u) * g), (g * u)):
        assert not np.allclose(ref, wrong.numpy(), rtol=1e-6, atol=1e-9)
    H = 128
    xn = W.normal_bf16((4, H), 14)
    ones = np.full(H, 0x3F80, np.uint16)
    r = oracle.fused_add_rmsnorm(W.bits(xn), None, ones, ones, W.pattern(4))
    xd = xn.double()
    sum_not_mean = (xd / torch.sqrt((xd * xd).sum(-1, keepdim=True) + 1e-6)).numpy()
    no_eps_sqrt = (xd / (xd * xd).mean(-1, keepdim=True)).numpy()
    assert not np.allclose(r["ref"], sum_not_mean, rtol=1e-6)
    assert not np.allclose(r["ref"], no_eps_sqrt, rtol=1e-6)


# ---- routed backward: dX = dY W_{m(t)} and the gen set's dW ------------------

def _bf(shape, seed, std=1.0):
    return W.bits(W.normal_bf16(shape, seed, std))


def test_backward_tiny_brute_force():
    """Every dX and dW element against math.fsum of the exact products (each
    bf16 x bf16 product is exact in fp64), and the bf16 outputs against the
    exactly rounded sum."""
    T, N, K = 9, 40, 24
    m = np.array([0, 1, 1, 0, 1, 0, 0, 1, 1], np.uint8)
    dy, wu, wg, x = _bf((T, N), 701), _bf((N, K), 702, 0.05), _bf((N, K), 703, 0.05), _bf((T, K), 704)
    d, w_u, w_g, xv = (oracle.bf16_to_f64(a) for a in (dy, wu, wg, x))
    ref, out = oracle.routed_gemm_dx(dy, wu, wg, m)
    for t in range(T):
        w = w_g if m[t] else w_u
        for k in range(K):
            exact = math.fsum(float(d[t, n]) * float(w[n, k]) for n in range(N))
            assert abs(ref[t, k] - exact) <= N * 2.0 ** -52 * math.fsum(abs(d[t, n] * w[n, k]) for n in range(N))
            assert out[t, k] == rne_bf16_exact(exact)
    gref, gout = oracle.grad_w(dy, x, m, keep=1)
    for n in range(N):
        for k in range(K):
            exact = math.fsum(float(d[t, n]) * float(xv[t, k]) for t in range(T) if m[t] == 1)
            assert abs(gref[n, k] - exact) <= T * 2.0 ** -52 * (1 + abs(exact) * 4)
            assert gout[n, k] == rne_bf16_exact(exact)


def test_backward_matches_torch_fp64():
    """Single-set packs: dX is dY @ W; dW over the gen rows is
    dY[gen]^T @ X[gen] (torch fp64 matmul)."""
    T, N, K = 70, 128, 96
    m = (np.arange(T) % 3 == 0).astype(np.uint8)
    dy, wu, wg, x = _bf((T, N), 711), _bf((N, K), 712, 0.05), _bf((N, K), 713, 0.05), _bf((T, K), 714)
    tdy, twu, twg, tx = (torch.from_numpy(oracle.bf16_to_f64(a)) for a in (dy, wu, wg, x))
    ref, _ = oracle.routed_gemm_dx(dy, wu, wg, m)
    want = torch.where(torch.from_numpy(m).bool()[:, None], tdy @ twg, tdy @ twu).numpy()
    assert np.allclose(ref, want, rtol=1e-12, atol=1e-12)
    gen = torch.from_numpy(m).bool()
    gref, _ = oracle.grad_w(dy, x, m, keep=1)
    assert np.allclose(gref, (tdy[gen].T @ tx[gen]).numpy(), rtol=1e-12, atol=1e-12)
    uref, _ = oracle.grad_w(dy, x, m, keep=0)
    assert np.allclose(uref, (tdy[~gen].T @ tx[~gen]).numpy(), rtol=1e-12, atol=1e-12)


def test_backward_adjoint_identities():
    """dX is the adjoint of the forward routed GEMM: <dY, X W^T> = <dY W, X>
    for each row's own set; and <dW_gen, V> = sum over gen rows of
    <dY[t], X[t] V^T>, with the forward oracle on the right-hand side."""
    T, N, K = 33, 64, 80
    m = np.random.default_rng(5).integers(0, 2, T).astype(np.uint8)
    dy, wu, wg, x = _bf((T, N), 721), _bf((N, K), 722, 0.05), _bf((N, K), 723, 0.05), _bf((T, K), 724)
    fwd, _ = oracle.routed_gemm(x, wu, wg, m)           # X W^T per row, [T, N]
    dx, _ = oracle.routed_gemm_dx(dy, wu, wg, m)         # dY W per row, [T, K]
    lhs = float(np.sum(oracle.bf16_to_f64(dy) * fwd))
    rhs = float(np.sum(dx * oracle.bf16_to_f64(x)))
    assert abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs))
    v = _bf((N, K), 725, 0.05)
    gw, _ = oracle.grad_w(dy, x, m, keep=1)
    xv, _ = oracle.routed_gemm(x, v, v, m)              # X V^T, [T, N]
    lhs = float(np.sum(gw * oracle.bf16_to_f64(v)))
    rhs = float(np.sum((oracle.bf16_to_f64(dy) * xv)[m == 1]))
    assert abs(lhs - rhs) <= 1e-9 * (1 + abs(lhs))


def test_pins_catch_planted_backward_mistakes():
    """Plausible mistakes, planted here on the CPU, fail the torch pin: the
    other row's set, the transposed weight, und rows in the gen gradient."""
    T, N, K = 40, 64, 64
    m = (np.arange(T) % 2).astype(np.uint8)
    dy, wu, wg, x = _bf((T, N), 731), _bf((N, K), 732, 0.05), _bf((N, K), 733, 0.05), _bf((T, K), 734)
    tdy, twu, twg, tx = (torch.from_numpy(oracle.bf16_to_f64(a)) for a in (dy, wu, wg, x))
    good = torch.where(torch.from_numpy(m).bool()[:, None], tdy @ twg, tdy @ twu).numpy()
    swapped, _ = oracle.routed_gemm_dx(dy, wu, wg, 1 - m)
    assert not np.allclose(swapped, good, rtol=1e-6)
    transposed = torch.where(torch.from_numpy(m).bool()[:, None], tdy @ twg.T, tdy @ twu.T).numpy()
    assert not np.allclose(transposed, good, rtol=1e-6)
    all_rows = (tdy.T @ tx).numpy()
    gref, _ = oracle.grad_w(dy, x, m, keep=1)
    assert not np.allclose(gref, all_rows, rtol=1e-6)


# ---- routed per-head QK RMSNorm + rotary embedding -----------------------------

def _qk_case(T, hq, hk, ld, base, n_pos=97):
    qkv = _bf((T, ld), W.seed_of(base, 1), 1.2)
    m = (np.arange(T) % 3 == 0).astype(np.uint8)
    qn, kn = W.qk_norm_weights(base)
    cos_t, sin_t, pos = W.rope_inputs(T, n_pos, base)
    return qkv, m, qn, kn, cos_t, sin_t, pos.numpy()


def _oracle_qk(qkv, hq, hk, m, qn, kn, cos_t, sin_t, pos, eps=1e-6):
    return oracle.qk_norm_rope(qkv, hq, hk, m, tuple(W.bits(t) for t in qn), tuple(W.bits(t) for t in kn),
                               pos, W.bits(cos_t), W.bits(sin_t), eps)


def _torch_qk(qkv, hq, hk, m, qn, kn, cos_t, sin_t, pos, eps=1e-6, pair=64, weights_of_k=None,
              swap_tables=False, whole_row=False, cast_first=False):
    """The op from library routines: torch's fp64 rms_norm with the row's
    set's weight, rounded to bf16, then the rotate-half rotation in torch's
    own bf16 arithmetic (each product and the sum rounded).  The keyword
    arguments plant plausible mistakes."""
    F = torch.nn.functional
    x = torch.from_numpy(oracle.bf16_to_f64(qkv))
    out = W.from_bits(qkv).clone()
    gen = torch.from_numpy(m.astype(bool))[:, None]
    c, s = (cos_t, sin_t) if not swap_tables else (sin_t, cos_t)
    c2 = torch.cat((c[pos], c[pos]), 1)
    s2 = torch.cat((s[pos], s[pos]), 1)
    for h in range(hq + hk):
        xs = x[:, h * 128:(h + 1) * 128]
        wu, wg = qn if (h < hq or weights_of_k == "q") else kn
        if whole_row:
            rs = torch.rsqrt(x[:, :128 * (hq + hk)].pow(2).mean(1, keepdim=True) + eps)
            yu, yg = xs * rs * wu.double(), xs * rs * wg.double()
        elif cast_first:
            n = F.rms_norm(xs, (128,), eps=eps).to(torch.bfloat16)
            yu, yg = n * wu, n * wg
        else:
            yu = F.rms_norm(xs, (128,), weight=wu.double(), eps=eps)
            yg = F.rms_norm(xs, (128,), weight=wg.double(), eps=eps)
        y = torch.where(gen, yg, yu).to(torch.bfloat16)
        rh = torch.cat((-y[:, pair:], y[:, :pair]), 1)
        out[:, h * 128:(h + 1) * 128] = y * c2 + rh * s2
    return W.bits(out)


def test_qk_norm_rope_matches_torch():
    """Both sets, 3 q and 2 k heads, extra columns past the heads: the oracle
    equals the op built from torch's rms_norm and bf16 arithmetic bit for bit,
    and leaves the other columns alone."""
    T, hq, hk, ld = 40, 3, 2, 5 * 128 + 64
    case = _qk_case(T, hq, hk, ld, base=801)
    ref, out, err = _oracle_qk(*case[:1], hq, hk, *case[1:])
    assert err == 0
    want = _torch_qk(case[0], hq, hk, *case[1:])
    assert np.array_equal(out, want)
    assert np.array_equal(out[:, 5 * 128:], case[0][:, 5 * 128:])
    # ref is the exact sum of two bf16 values, rounded once to give out
    assert np.array_equal(np.array([oracle.bf16_round(v) for v in ref[:3].ravel()], np.uint16).reshape(3, ld),
                          out[:3])


def test_qk_norm_rope_special_angles():
    """cos 1, sin 0: the per-head RMSNorm alone (torch's fp64 rms_norm, one
    rounding).  cos 0, sin 1: exactly the rotate-half of that.  cos -1, sin 0:
    exactly its negation."""
    T, hq, hk, ld = 12, 2, 1, 3 * 128
    qkv, m, qn, kn, _, _, pos = _qk_case(T, hq, hk, ld, base=802, n_pos=5)
    one, zero = torch.ones((5, 64), dtype=torch.bfloat16), torch.zeros((5, 64), dtype=torch.bfloat16)
    _, y, err = _oracle_qk(qkv, hq, hk, m, qn, kn, one, zero, pos)
    assert err == 0
    x = torch.from_numpy(oracle.bf16_to_f64(qkv))
    for h in range(hq + hk):
        wu, wg = qn if h < hq else kn
        xs = x[:, h * 128:(h + 1) * 128]
        F = torch.nn.functional
        want = torch.where(torch.from_numpy(m.astype(bool))[:, None],
                           F.rms_norm(xs, (128,), weight=wg.double(), eps=1e-6),
                           F.rms_norm(xs, (128,), weight=wu.double(), eps=1e-6)).to(torch.bfloat16)
        assert np.array_equal(y[:, h * 128:(h + 1) * 128], W.bits(want))
    _, r, _ = _oracle_qk(qkv, hq, hk, m, qn, kn, zero, one, pos)
    _, neg, _ = _oracle_qk(qkv, hq, hk, m, qn, kn, -one, zero, pos)
    for h in range(hq + hk):
        yh, rh, nh = (a[:, h * 128:(h + 1) * 128] for a in (y, r, neg))
        assert np.array_equal(rh[:, :64], yh[:, 64:] ^ np.uint16(0x8000))
        assert np.array_equal(rh[:, 64:], yh[:, :64])
        assert np.array_equal(nh, yh ^ np.uint16(0x8000))


def test_qk_norm_rope_errors_and_relabel():
    """Rows with a modality byte outside {0,1} or a position outside the
    table keep their bytes and set the error (7 wins over 6); swapping the
    sets' weights and flipping the bytes gives the same output."""
    T, hq, hk, ld = 10, 1, 1, 2 * 128
    qkv, m, qn, kn, c, s, pos = _qk_case(T, hq, hk, ld, base=803, n_pos=11)
    _, good, err = _oracle_qk(qkv, hq, hk, m, qn, kn, c, s, pos)
    assert err == 0
    _, flip, _ = _oracle_qk(qkv, hq, hk, 1 - m, (qn[1], qn[0]), (kn[1], kn[0]), c, s, pos)
    assert np.array_equal(flip, good)
    bm = m.copy()
    bm[3] = 2
    _, o, err = _oracle_qk(qkv, hq, hk, bm, qn, kn, c, s, pos)
    assert err == 6 and np.array_equal(o[3], qkv[3]) and np.array_equal(np.delete(o, 3, 0), np.delete(good, 3, 0))
    bp = pos.copy()
    bp[5], bp[6] = 11, -1
    _, o, err = _oracle_qk(qkv, hq, hk, bm, qn, kn, c, s, bp)
    assert err == 7 and all(np.array_equal(o[i], qkv[i]) for i in (3, 5, 6))


def test_pins_catch_planted_qk_mistakes():
    """Plausible mistakes, planted in the torch pin on the CPU, change the
    result: a wrong rotation pair, cos and sin swapped, k heads normalized
    with the q weights, one norm over all heads, the cast-first norm."""
    T, hq, hk, ld = 24, 2, 2, 4 * 128
    case = _qk_case(T, hq, hk, ld, base=804)
    _, out, _ = _oracle_qk(*case[:1], hq, hk, *case[1:])
    for kw in (dict(pair=63), dict(swap_tables=True), dict(weights_of_k="q"), dict(whole_row=True),
               dict(cast_first=True)):
        assert not np.array_equal(_torch_qk(case[0], hq, hk, *case[1:], **kw), out), kw


# ---- shared joint attention ------------------------------------------------------


def _attn_case(Tq, Tk, hq, hkv, base, extra=64, q_std=1.0):
    D = 128
    q = _bf((Tq, hq * D + extra), W.seed_of(base, 1), q_std)
    k = _bf((Tk, hkv * D + extra), W.seed_of(base, 2))
    v = _bf((Tk, hkv * D + extra), W.seed_of(base, 3))
    return q, k, v


def _torch_attention(q, k, v, hq, hkv, causal, align="bottom_right", kv_map="group", scale=True):
    """The op from library routines: torch's fp64 scaled_dot_product_attention
    with an explicit boolean mask and the kv heads repeated per group.  The
    keyword arguments plant plausible mistakes."""
    D = 128
    Tq, Tk = q.shape[0], k.shape[0]
    Q = torch.from_numpy(oracle.bf16_to_f64(q[:, :hq * D])).view(Tq, hq, D).transpose(0, 1)
    K = torch.from_numpy(oracle.bf16_to_f64(k[:, :hkv * D])).view(Tk, hkv, D).transpose(0, 1)
    V = torch.from_numpy(oracle.bf16_to_f64(v[:, :hkv * D])).view(Tk, hkv, D).transpose(0, 1)
    idx = torch.arange(hq) // (hq // hkv) if kv_map == "group" else torch.arange(hq) % hkv
    K, V = K[idx], V[idx]
    i = torch.arange(Tq)[:, None]
    j = torch.arange(Tk)[None, :]
    if not causal:
        mask = torch.ones((Tq, Tk), dtype=torch.bool)
    elif align == "bottom_right":
        mask = j <= i + (Tk - Tq)
    else:
        mask = j <= i
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask,
                                                           scale=None if scale else 1.0)
    return out.transpose(0, 1).reshape(Tq, hq * D).numpy()


@pytest.mark.parametrize("Tq,Tk,causal", [(37, 90, True), (50, 50, True), (50, 50, False), (1, 64, True),
                                          (70, 33, False)])
def test_attention_matches_torch_sdpa(Tq, Tk, causal):
    """Grouped heads (4 q, 2 kv), extra columns past the heads, a cached
    prefix (Tk > Tq): the oracle equals torch's fp64 attention to rounding,
    and its bf16 output is the RNE rounding of its fp64 result."""
    q, k, v = _attn_case(Tq, Tk, 4, 2, base=900 + Tq)
    ref, out = oracle.attention(q, k, v, 4, 2, causal)
    want = _torch_attention(q, k, v, 4, 2, causal)
    assert np.abs(ref - want).max() <= 1e-12
    rows = [0, Tq - 1]
    for r in rows:
        for c in (0, 129, 511):
            assert out[r, c] == oracle.bf16_round(ref[r, c])


def test_attention_closed_forms():
    """q = 0: uniform weights, so each row is the mean of the V rows it sees.
    The first row of a square causal pack sees key 0 only: V's row 0 exactly.
    Rows that see no key (Tq > Tk, causal) are zero.  A key whose score
    dwarfs the others takes all the weight."""
    D = 128
    Tq, Tk = 6, 9
    q = np.zeros((Tq, 2 * D), np.uint16)
    k = _bf((Tk, D), 911)
    v = _bf((Tk, D), 912)
    ref, _ = oracle.attention(q, k, v, 2, 1, True)
    V = oracle.bf16_to_f64(v)
    for i in range(Tq):
        want = V[:i + Tk - Tq + 1].mean(0)
        assert np.abs(ref[i, :D] - want).max() <= 1e-14 and np.abs(ref[i, D:] - want).max() <= 1e-14
    q2, k2, v2 = _attn_case(8, 8, 1, 1, base=913)
    _, out2 = oracle.attention(q2, k2, v2, 1, 1, True)
    assert np.array_equal(out2[0], v2[0, :D])
    # Tq = 5 queries over 3 keys, bottom-right: rows 0 and 1 see nothing
    q3, k3, v3 = _attn_case(5, 3, 1, 1, base=914)
    ref3, out3 = oracle.attention(q3, k3, v3, 1, 1, True)
    assert not ref3[:2].any() and not out3[:2].any()
    assert np.array_equal(out3[2], v3[0, :D])
    # dominance: the query is 8x key 1 and keys 0 and 2 are zero, so key 1's
    # score exceeds theirs by about 90 and their weights are below 1e-38
    K4 = torch.from_numpy(oracle.bf16_to_f64(k3[:, :D]))
    qd = np.zeros((1, D), np.uint16)
    qd[0] = W.bits((8 * K4[1]).to(torch.bfloat16)[None])[0]
    kb = k3.copy()
    kb[0, :D] = 0
    kb[2, :D] = 0
    refd, _ = oracle.attention(qd, kb, v3, 1, 1, False)
    assert np.abs(refd[0] - oracle.bf16_to_f64(v3[1, :D])).max() <= 1e-9


def test_pins_catch_planted_attention_mistakes():
    """Plausible mistakes, planted in the torch pin on the CPU, move it far
    from the oracle: a top-left aligned causal mask, kv heads taken round
    robin instead of in groups, no 1/sqrt(D) scale, no mask at all."""
    q, k, v = _attn_case(24, 56, 4, 2, base=920)
    ref, _ = oracle.attention(q, k, v, 4, 2, True)
    assert np.abs(ref - _torch_attention(q, k, v, 4, 2, True)).max() <= 1e-12
    for kw in (dict(align="top_left"), dict(kv_map="round_robin"), dict(scale=False)):
        assert np.abs(ref - _torch_attention(q, k, v, 4, 2, True, **kw)).max() > 1e-2, kw
    assert np.abs(ref - _torch_attention(q, k, v, 4, 2, False)).max() > 1e-2


# ---- packed sequences (attention over several requests in one pack) ---------

def _torch_attention_packed(q, k, v, cu_q, cu_k, hq, hkv, causal, keys_by="cu_k", align="per_seq"):
    """The packed op as ONE torch fp64 attention over the whole pack with a
    block-diagonal mask: query row i of sequence b sees key j of sequence b
    (and, causal, j - cu_k[b] <= (i - cu_q[b]) + Lk - Lq).  Rows that see no
    key are zero.  keys_by / align plant mistakes: keys cut by the query
    offsets, or the causal mask aligned at the whole pack's corner."""
    D = 128
    Tq, Tk = q.shape[0], k.shape[0]
    Q = torch.from_numpy(oracle.bf16_to_f64(q[:, :hq * D])).view(Tq, hq, D).transpose(0, 1)
    K = torch.from_numpy(oracle.bf16_to_f64(k[:, :hkv * D])).view(Tk, hkv, D).transpose(0, 1)
    V = torch.from_numpy(oracle.bf16_to_f64(v[:, :hkv * D])).view(Tk, hkv, D).transpose(0, 1)
    idx = torch.arange(hq) // (hq // hkv)
    K, V = K[idx], V[idx]
    ck = list(cu_q) if keys_by == "cu_q" else list(cu_k)
    mask = torch.zeros((Tq, Tk), dtype=torch.bool)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(ck[b]), int(ck[b + 1])
        for i in range(q0, q1):
            for j in range(k0, min(k1, Tk)):
                if not causal:
                    ok = True
                elif align == "per_seq":
                    ok = (j - k0) <= (i - q0) + (k1 - k0) - (q1 - q0)
                else:
                    ok = j <= i + (Tk - Tq)
                mask[i, j] = ok
    out = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
    out = out.transpose(0, 1).reshape(Tq, hq * D)
    seen = mask.any(1)
    out[~seen] = 0.0
    return out.numpy()


# ragged requests: one empty, one with more keys than rows (a cached prefix),
# one with more rows than keys (its first rows see nothing when causal)
_PACKS = [([0, 17, 17, 40, 71, 72], [0, 30, 31, 40, 90, 92]),
          ([0, 64, 130], [0, 64, 129])]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("pack", range(len(_PACKS)))
def test_attention_varlen_matches_block_diagonal_torch(pack, causal):
    cu_q, cu_k = _PACKS[pack]
    q, k, v = _attn_case(cu_q[-1], cu_k[-1], 4, 2, base=930 + pack)
    ref, out = oracle.attention_varlen(q, k, v, cu_q, cu_k, 4, 2, causal)
    want = _torch_attention_packed(q, k, v, cu_q, cu_k, 4, 2, causal)
    assert np.abs(ref - want).max() <= 1e-12
    for r in (0, cu_q[-1] - 1):
        for c in (0, 300):
            assert out[r, c] == oracle.bf16_round(ref[r, c])


def _varlen_mutant(q, k, v, cu_q, cu_k, hq, hkv, causal, mistake):
    """oracle.attention_varlen with a planted mistake, on the CPU."""
    ref = np.zeros((q.shape[0], hq * 128))
    for b in range(len(cu_q) - 1):
        q0, q1 = cu_q[b], cu_q[b + 1]
        k0, k1 = (cu_q[b], cu_q[b + 1]) if mistake == "keys_by_cu_q" else (cu_k[b], cu_k[b + 1])
        if mistake == "keys_from_zero":
            k0 = 0
        if q1 == q0:
            continue
        r, _ = oracle.attention(q[q0:q1], k[k0:k1], v[k0:k1], hq, hkv, causal)
        ref[q0:q1] = r
    return ref


def test_pins_catch_planted_varlen_mistakes():
    cu_q, cu_k = _PACKS[0]
    q, k, v = _attn_case(cu_q[-1], cu_k[-1], 4, 2, base=940)
    want = _torch_attention_packed(q, k, v, cu_q, cu_k, 4, 2, True)
    assert np.abs(_varlen_mutant(q, k, v, cu_q, cu_k, 4, 2, True, None) - want).max() <= 1e-12
    for mistake in ("keys_by_cu_q", "keys_from_zero"):
        assert np.abs(_varlen_mutant(q, k, v, cu_q, cu_k, 4, 2, True, mistake) - want).max() > 1e-2, mistake
    # the pin itself tells the per-sequence alignment from the pack's corner
    assert np.abs(_torch_attention_packed(q, k, v, cu_q, cu_k, 4, 2, True, align="pack") - want).max() > 1e-2


# ---- the gate's metrics and the bf16 step distance ----------------------------

def _all_finite_bf16():
    """Every finite bf16 pattern, and its rank among the distinct finite
    values in increasing order (+0 and -0 share a rank)."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f64(pats)
    fin = np.isfinite(vals)
    pats, vals = pats[fin], vals[fin]
    distinct = np.unique(vals)
    rank = np.searchsorted(distinct, vals)
    return pats, vals, dict(zip(pats.tolist(), rank.tolist()))


def test_ulp_distance_is_rank_difference():
    """The bf16 step distance equals the difference of the two values' ranks
    among all distinct finite bf16 values -- checked on the sign boundary,
    the subnormals, the largest values and random pairs."""
    pats, _, rank = _all_finite_bf16()
    rng = np.random.default_rng(3)
    edge = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x807F, 0x8080, 0x3F80, 0xBF80,
                     0x7F7F, 0xFF7F, 0x7F7E, 0x3F7F], np.uint16)
    a = np.concatenate([np.repeat(edge, edge.size), rng.choice(pats, 20000)])
    b = np.concatenate([np.tile(edge, edge.size), rng.choice(pats, 20000)])
    want = np.abs(np.array([rank[x] for x in a.tolist()]) - np.array([rank[x] for x in b.tolist()]))
    assert np.array_equal(oracle.ulp_distance(a, b), want)
    # a count of raw patterns, without the sign handling, is wrong across zero
    raw = np.abs(a.astype(np.int64) - b.astype(np.int64))
    assert not np.array_equal(raw, want)


def test_gate_metrics_hand_worked():
    """A hand-worked case: ref = (3, -4, 0, 0.5); got = bf16 (3, -4.03125,
    0.0078125, 0.5).  Differences (0, -1/32, 1/128, 0): max-abs 1/32,
    ||d|| = sqrt(1/1024 + 1/16384) = sqrt(17)/128, ||ref|| = sqrt(25.25),
    elementwise excess max(|d| - (2e-2 + 1.6e-2|ref|)) over (-0.068,
    -0.05275, -0.0121875, -0.028) at the third entry: 1/128 - 2e-2; bf16 step
    distance to RNE(ref): 0, 1, 0x3C00 patterns up from 0 (1/128 = 2^-7:
    biased exponent 120, so 120*128 = 15360), 0."""
    ref = np.array([3.0, -4.0, 0.0, 0.5])
    got = np.array([0x4040, 0xC081, 0x3C00, 0x3F00], np.uint16)
    assert list(oracle.bf16_to_f64(got)) == [3.0, -4.03125, 0.0078125, 0.5]
    m = oracle.gate_metrics(got, ref)
    assert m["max_abs"] == 1 / 32
    assert math.isclose(m["rel_fro"], math.sqrt(17) / 128 / math.sqrt(25.25), rel_tol=1e-14)
    assert math.isclose(m["elem_excess"], 1 / 128 - 2e-2, rel_tol=1e-14)
    assert m["max_ref"] == 4.0
    assert m["max_ulp_to_rne"] == 15360


def test_gate_metrics_against_fsum_and_planted_mistakes():
    """The metrics against a plain re-derivation with math.fsum on random
    data, and two plausible mistakes that the re-derivation tells apart:
    the Frobenius error relative to the GPU result's norm instead of the
    reference's, and the max-abs error taken without the absolute value."""
    rng = np.random.default_rng(11)
    ref = rng.standard_normal(500) * 3
    got = np.array([oracle.bf16_round(v + 0.01 * rng.standard_normal()) for v in ref], np.uint16)
    g = oracle.bf16_to_f64(got)
    d = [gi - ri for gi, ri in zip(g.tolist(), ref.tolist())]
    want_rel = math.sqrt(math.fsum(x * x for x in d)) / math.sqrt(math.fsum(x * x for x in ref.tolist()))
    want_max = max(abs(x) for x in d)
    want_exc = max(abs(x) - (2e-2 + 1.6e-2 * abs(r)) for x, r in zip(d, ref.tolist()))
    m = oracle.gate_metrics(got, ref)
    assert math.isclose(m["rel_fro"], want_rel, rel_tol=1e-12)
    assert m["max_abs"] == want_max and math.isclose(m["elem_excess"], want_exc, rel_tol=1e-12, abs_tol=1e-15)
    wrong_rel = math.sqrt(math.fsum(x * x for x in d)) / math.sqrt(math.fsum(x * x for x in g.tolist()))
    assert not math.isclose(wrong_rel, want_rel, rel_tol=1e-9)
    assert max(d) != want_max or min(d) > -want_max


# ---- modality bytes from the two index sets -----------------------------------

def test_index_sets_brute_force():
    """Every way of listing the rows of a pack of up to 3 rows, each row
    placed 0, 1 or 2 times in each list (plus an out-of-range index): the
    byte is 0 or 1 exactly for the rows listed once overall, and the error
    is raised exactly when some row is not, or an index is out of range."""
    import itertools
    for T in range(0, 4):
        for placing in itertools.product(range(9), repeat=T):
            und, gen = [], []
            for r, p in enumerate(placing):
                und += [r] * (p % 3)
                gen += [r] * (p // 3)
            for extra in ((), (T,)):
                m, err = oracle.modality_from_index_sets(np.array(und, np.int64),
                                                         np.array(gen + list(extra), np.int64), T)
                ok = True
                for r, p in enumerate(placing):
                    nu, ng = p % 3, p // 3
                    if nu + ng == 1:
                        assert m[r] == (1 if ng else 0)
                    else:
                        assert m[r] == 0xFF
                        ok = False
                assert (err == 0) == (ok and not extra)


def test_index_sets_round_trip_to_the_segment_list():
    """For a valid split the bytes are the pack's modality, and the routing
    plan of those bytes lists each index set in ascending order."""
    m0 = W.pattern(2202)
    rng = np.random.default_rng(4)
    und = rng.permutation(np.flatnonzero(m0 == 0))
    gen = rng.permutation(np.flatnonzero(m0 == 1))
    m, err = oracle.modality_from_index_sets(und, gen, m0.size)
    assert err == 0 and np.array_equal(m, m0)
    perm, nu, ng = oracle.routing_plan(m)
    assert np.array_equal(perm, np.concatenate([np.sort(und), np.sort(gen)])) and (nu, ng) == (und.size, gen.size)


def test_rmsnorm_apply_exact_by_rationals():
    """The norm application for a given fp32 rstd, element by element
    against exact rational arithmetic: ref == h * rstd * w_{m(t)} exactly, and
    out is its correct bf16 rounding; rows pick their own set's weights."""
    T, H = 6, 64
    m = np.array([0, 1, 1, 0, 1, 0], np.uint8)
    h = W.bits(W.normal_bf16((T, H), 960))
    wu, wg = (W.bits(t) for t in W.norm_weights(H, base=96))
    rstd = np.float32(np.random.default_rng(9).uniform(0.5, 2.0, T))
    ref, out = oracle.rmsnorm_apply(h, rstd, wu, wg, m)
    hv, wuv, wgv = oracle.bf16_to_f64(h), oracle.bf16_to_f64(wu), oracle.bf16_to_f64(wg)
    for t in range(T):
        w = wgv if m[t] else wuv
        for k in range(H):
            q = Fraction(float(hv[t, k])) * Fraction(float(rstd[t])) * Fraction(float(w[k]))
            assert Fraction(float(ref[t, k])) == q
            assert out[t, k] == rne_bf16_exact(q)
    # with rstd from the norm itself (rounded to fp32) it reproduces the
    # norm's outputs but for the few elements the fp32 rounding of rstd moves
    full = oracle.fused_add_rmsnorm(h, None, wu, wg, m)
    _, out2 = oracle.rmsnorm_apply(h, np.float32(full["rstd"]), wu, wg, m)
    assert (out2 == full["out"]).mean() >= 0.99
