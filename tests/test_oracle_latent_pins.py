"""Pins of the oracle's latent-step functions (three-branch renormalised CFG
and the flow SDE step with its log-probability) against things other than
themselves: closed forms on inputs built so the answer is known, library
routines (scipy's normal log-density, numpy's norm), the straight-line path
of rectified flow (which fixes the timestep scaling and the sign of dt, as
the RL-Kernel RFC page asks to test explicitly, section 6), request
independence (the page's section 3: renormalisation is per request), and
planted mistakes, on the CPU, that the pins catch."""
from __future__ import annotations

import math

import numpy as np
import pytest
import scipy.stats

import oracle

G, CH = oracle.RENORM_GLOBAL, oracle.RENORM_CHANNEL


def _f32(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


# ---- CFG combine + renorm ------------------------------------------------------

def test_cfg_outside_window_is_the_conditional_velocity():
    """t outside (t_lo, t_hi] leaves the conditional branch untouched; the
    window's ends are compared on fp32 t: t == t_lo is outside, t == t_hi
    inside."""
    vc, vt, vi = _f32((20, 8), 1), _f32((20, 8), 2), _f32((20, 8), 3)
    cu = [0, 5, 12, 20]
    lo, hi = np.float32(0.1), np.float32(0.9)
    t = np.array([lo, np.nextafter(hi, np.float32(2)), hi], np.float32)
    out = oracle.cfg_combine_renorm(vc, vt, vi, cu, t, 4.0, 2.0, lo, hi, 0.0, G)
    assert np.array_equal(out[:12], vc[:12].astype(np.float64))
    assert not np.allclose(out[12:], vc[12:])


def test_cfg_unit_scales_and_min_one():
    vc, vt, vi = _f32((16, 8), 4), _f32((16, 8), 5), _f32((16, 8), 6)
    cu, t = [0, 16], np.float32([0.5])
    out = oracle.cfg_combine_renorm(vc, vt, vi, cu, t, 1.0, 1.0, 0.0, 1.0, 0.0, G)
    assert np.array_equal(out, vc.astype(np.float64))
    # renorm_min = 1 clamps the ratio to 1: the plain guided velocity
    g = vi.astype(np.float64) + 2.0 * (vt + 3.0 * (vc.astype(np.float64) - vt) - vi)
    out = oracle.cfg_combine_renorm(vc, vt, vi, cu, t, 3.0, 2.0, 0.0, 1.0, 1.0, G)
    assert np.abs(out - g).max() <= 1e-12


@pytest.mark.parametrize("s,rmin,factor", [(4.0, 0.0, 1.0), (4.0, 0.5, 2.0), (0.5, 0.0, 0.5)])
def test_cfg_renorm_closed_form(s, rmin, factor):
    """v_tu = 0: the guided velocity is s v_c, its norm s ||v_c||, the ratio
    clamp(1/s, min, 1); the output is v_c scaled by s * ratio."""
    vc = _f32((30, 16), 7)
    zero = np.zeros_like(vc)
    out = oracle.cfg_combine_renorm(vc, zero, None, [0, 30], np.float32([0.5]), s, 1.0, 0.0, 1.0, rmin, G)
    assert np.abs(out - factor * vc).max() <= 1e-12 * np.abs(vc).max()


def test_cfg_three_branch_roles_hand_worked():
    """One element per branch, integers: v_c = 5, v_tu = 1, v_iu = -2,
    s_text = 3, s_img = 2: g1 = 1 + 3 (5 - 1) = 13, g = -2 + 2 (13 + 2) = 28;
    no renorm.  With the two unconditional branches swapped: g1 = -2 + 3*7 =
    19, g = 1 + 2*18 = 37."""
    one = lambda v: np.array([[v]], np.float32)
    out = oracle.cfg_combine_renorm(one(5), one(1), one(-2), [0, 1], np.float32([0.5]), 3, 2, 0, 1, 0,
                                    oracle.RENORM_NONE)
    assert out[0, 0] == 28.0
    out = oracle.cfg_combine_renorm(one(5), one(-2), one(1), [0, 1], np.float32([0.5]), 3, 2, 0, 1, 0,
                                    oracle.RENORM_NONE)
    assert out[0, 0] == 37.0


def test_cfg_channel_versus_global_renorm():
    """Row 0 has v_tu = 0 (ratio 1/s on its own), row 1 has v_tu = v_c (its
    guided velocity is v_c, ratio 1).  Per-row (channel) renorm gives v_c in
    both rows; the request-wide ratio is ||v_c|| / ||(s v_c0, v_c1)||."""
    s = 3.0
    vc = np.array([[3, 4], [6, 8]], np.float32)        # row norms 5 and 10
    vt = np.array([[0, 0], [6, 8]], np.float32)
    cu, t = [0, 2], np.float32([0.5])
    ch = oracle.cfg_combine_renorm(vc, vt, None, cu, t, s, 1.0, 0.0, 1.0, 0.0, CH)
    assert np.abs(ch - vc).max() <= 1e-12
    gl = oracle.cfg_combine_renorm(vc, vt, None, cu, t, s, 1.0, 0.0, 1.0, 0.0, G)
    r = math.sqrt(25 + 100) / math.sqrt(225 + 100)
    want = np.array([[9, 12], [6, 8]], np.float64) * r
    assert np.abs(gl - want).max() <= 1e-12


def _batch_coupled_mutant(vc, vt, cu, s):
    """A planted mistake: one renorm ratio over the whole packed batch."""
    g = vt.astype(np.float64) + s * (vc.astype(np.float64) - vt)
    r = min(1.0, np.linalg.norm(vc.astype(np.float64)) / np.linalg.norm(g))
    return g * r


def test_cfg_requests_are_independent_and_pins_catch_batch_coupling():
    """A request's output does not depend on the other requests of the pack
    (renormalisation is per request); a batch-coupled renorm does."""
    vc, vt = _f32((40, 8), 8), _f32((40, 8), 9, 0.3)
    vc[25:] *= 4.0                              # requests of different scale
    cu = [0, 25, 40]
    t = np.float32([0.5, 0.5])
    both = oracle.cfg_combine_renorm(vc, vt, None, cu, t, 4.0, 1.0, 0.0, 1.0, 0.0, G)
    alone = oracle.cfg_combine_renorm(vc[:25], vt[:25], None, [0, 25], t[:1], 4.0, 1.0, 0.0, 1.0, 0.0, G)
    assert np.array_equal(both[:25], alone)
    assert np.abs(_batch_coupled_mutant(vc, vt, cu, 4.0)[:25] - alone).max() > 1e-3


def test_cfg_scale_equivariance_and_norms():
    """Doubling every input (exact in fp32) doubles the output exactly; the
    fsum norms agree with numpy's."""
    vc, vt, vi = _f32((33, 8), 10), _f32((33, 8), 11), _f32((33, 8), 12)
    cu, t = [0, 10, 33], np.float32([0.3, 0.7])
    a = oracle.cfg_combine_renorm(vc, vt, vi, cu, t, 4.0, 1.5, 0.0, 1.0, 0.2, G)
    b = oracle.cfg_combine_renorm(2 * vc, 2 * vt, 2 * vi, cu, t, 4.0, 1.5, 0.0, 1.0, 0.2, G)
    assert np.array_equal(2 * a, b)
    c = oracle.cfg_combine_renorm(vc, vt, vi, cu, t, 4.0, 1.5, 0.0, 1.0, 0.0, oracle.RENORM_NONE)
    for r0, r1 in ((0, 10), (10, 33)):
        ratio = min(1.0, max(float(np.float32(0.2)), np.linalg.norm(vc[r0:r1].astype(np.float64)) / np.linalg.norm(c[r0:r1])))
        assert np.abs(a[r0:r1] - ratio * c[r0:r1]).max() <= 1e-12


# ---- flow SDE step and log-probability ----------------------------------------

def _straight_line(t, n=64, seed=20):
    """A point mass at x0: on the straight path x_t = (1 - t) x0 + t eps the
    velocity dx/dt is eps - x0 at every t."""
    x0 = _f32((1, n), seed).astype(np.float64)
    eps = _f32((1, n), seed + 1).astype(np.float64)
    x = ((1 - t) * x0 + t * eps).astype(np.float32)
    v = (eps - x0).astype(np.float32)
    return x0, eps, x, v


@pytest.mark.parametrize("t,tn", [(1.0, 0.98), (0.6, 0.4), (0.05, 0.0), (1.0, 0.0)])
def test_sde_deterministic_limit_follows_the_path(t, tn):
    """With a vanishing noise level the step is the Euler step of the flow
    ODE, which lands on the straight path at t_next: this fixes the timestep
    scaling (x_t = (1 - t) x0 + t eps, sigma = t) and the sign of dt > 0."""
    x0, eps, x, v = _straight_line(t)
    mu, _, _ = oracle.flow_sde_step_logp(x, v, [0, 1], np.float32([t]), np.float32([tn]), 1e-9,
                                         noise=np.zeros_like(x))
    xx, vv = x.astype(np.float64), v.astype(np.float64)
    want = xx - (np.float32(t) - np.float32(tn)) * vv   # x - dt v with the fp32 inputs
    assert np.abs(mu - want).max() <= 1e-9
    path = (1 - tn) * x0 + tn * eps
    assert np.abs(mu - path).max() <= 1e-5           # fp32 rounding of x and v only


@pytest.mark.parametrize("t,tn,eta", [(0.6, 0.4, 0.7), (0.3, 0.25, 1.0), (1.0, 0.9, 0.5)])
def test_sde_drift_correction_closed_form(t, tn, eta):
    """On the straight path x + (1 - t) v = eps, so the mean is the ODE step
    minus dt s^2 / (2 t) eps."""
    x0, eps, x, v = _straight_line(t, seed=30)
    mu, _, _ = oracle.flow_sde_step_logp(x, v, [0, 1], np.float32([t]), np.float32([tn]), eta,
                                         noise=np.zeros_like(x))
    xx, vv = x.astype(np.float64), v.astype(np.float64)
    tf, tnf = float(np.float32(t)), float(np.float32(tn))
    dt = tf - tnf
    s = oracle.sde_scale(t, tn, eta)
    e = xx + (1 - tf) * vv                  # = eps up to the fp32 rounding of x and v
    assert np.abs(e - eps).max() <= 1e-6
    assert np.abs(mu - (xx - dt * vv - dt * s * s / (2 * tf) * e)).max() <= 1e-12


def test_sde_scale_closed_forms():
    """eta sqrt(t / (1 - t)) on exact fp32 inputs (eta's fp32 value), with
    1 - t_next in the denominator at the first step t = 1."""
    e8, e3 = float(np.float32(0.8)), float(np.float32(0.3))
    assert oracle.sde_scale(0.5, 0.4, 0.8) == pytest.approx(e8, rel=1e-15)
    assert oracle.sde_scale(0.75, 0.5, 1.0) == pytest.approx(math.sqrt(3), rel=1e-15)
    assert oracle.sde_scale(1.0, 0.5, 1.0) == pytest.approx(math.sqrt(2), rel=1e-15)   # first step
    assert oracle.sde_scale(1.0, 0.0, 0.3) == pytest.approx(e3, rel=1e-15)             # single step


def test_sde_logp_is_the_gaussian_density_sum():
    """logp of a given x_next equals scipy's normal log-density of each
    element around the mean with standard deviation s sqrt(dt), summed; in
    sampling mode it is the closed form -|noise|^2 / 2 - n log(s sqrt(dt)) -
    n log(2 pi) / 2."""
    x, v = _f32((30, 16), 40), _f32((30, 16), 41)
    xn_in = _f32((30, 16), 42)
    cu = [0, 12, 30]
    tc, tn = np.float32([0.8, 0.3]), np.float32([0.7, 0.1])
    mu, _, logp = oracle.flow_sde_step_logp(x, v, cu, tc, tn, 0.9, x_next=xn_in)
    for b in range(2):
        r0, r1 = cu[b], cu[b + 1]
        std = oracle.sde_scale(tc[b], tn[b], 0.9) * math.sqrt(float(tc[b]) - float(tn[b]))
        want = scipy.stats.norm.logpdf(xn_in[r0:r1].astype(np.float64), loc=mu[r0:r1], scale=std).sum()
        assert logp[b] == pytest.approx(want, rel=1e-12)
    noise = _f32((30, 16), 43)
    _, xs, logp_s = oracle.flow_sde_step_logp(x, v, cu, tc, tn, 0.9, noise=noise)
    for b in range(2):
        r0, r1 = cu[b], cu[b + 1]
        std = oracle.sde_scale(tc[b], tn[b], 0.9) * math.sqrt(float(tc[b]) - float(tn[b]))
        nb = noise[r0:r1].astype(np.float64)
        want = -0.5 * (nb * nb).sum() - nb.size * (math.log(std) + 0.5 * math.log(2 * math.pi))
        assert logp_s[b] == pytest.approx(want, rel=1e-12)
        assert np.abs(xs[r0:r1] - (mu[r0:r1] + std * nb)).max() <= 1e-12


def test_sde_requests_are_independent():
    x, v, noise = _f32((50, 8), 50), _f32((50, 8), 51), _f32((50, 8), 52)
    cu = [0, 20, 50]
    tc, tn = np.float32([0.5, 0.9]), np.float32([0.4, 0.8])
    _, xs, lp = oracle.flow_sde_step_logp(x, v, cu, tc, tn, 0.7, noise=noise)
    _, xs1, lp1 = oracle.flow_sde_step_logp(x[20:], v[20:], [0, 30], tc[1:], tn[1:], 0.7, noise=noise[20:])
    assert np.array_equal(xs[20:], xs1) and lp[1] == lp1[0]


def _sde_mutant(x, v, t, tn, eta, noise, mistake):
    """The oracle's step with a planted mistake, on the CPU."""
    xx, vv = x.astype(np.float64), v.astype(np.float64)
    dt = float(np.float32(t)) - float(np.float32(tn))
    tf = float(np.float32(t))
    s = oracle.sde_scale(t, tn, eta)
    if mistake == "dt_sign":
        return xx + dt * (vv + s * s / (2 * tf) * (xx + (1 - tf) * vv))
    if mistake == "one_plus_t":
        return xx - dt * (vv + s * s / (2 * tf) * (xx + (1 + tf) * vv))
    if mistake == "no_half":
        return xx - dt * (vv + s * s / tf * (xx + (1 - tf) * vv))
    raise ValueError(mistake)


def test_pins_catch_planted_sde_mistakes():
    t, tn = 0.6, 0.4
    x0, eps, x, v = _straight_line(t, seed=60)
    path = (1 - tn) * x0 + tn * eps
    # the deterministic-limit pin catches the sign of dt
    assert np.abs(_sde_mutant(x, v, t, tn, 1e-9, None, "dt_sign") - path).max() > 1e-2
    # the drift-correction pin catches a wrong factor
    dt, tf = float(np.float32(t)) - float(np.float32(tn)), float(np.float32(t))
    s = oracle.sde_scale(t, tn, 0.8)
    xx, vv = x.astype(np.float64), v.astype(np.float64)
    want = xx - dt * vv - dt * s * s / (2 * tf) * (xx + (1 - tf) * vv)
    for mistake in ("one_plus_t", "no_half"):
        assert np.abs(_sde_mutant(x, v, t, tn, 0.8, None, mistake) - want).max() > 1e-3, mistake
    # the density pin catches a mean over the elements instead of a sum
    xn = _f32((1, 64), 61)
    _, _, lp = oracle.flow_sde_step_logp(x, v, [0, 1], np.float32([t]), np.float32([tn]), 0.8, x_next=xn)
    mu, _, _ = oracle.flow_sde_step_logp(x, v, [0, 1], np.float32([t]), np.float32([tn]), 0.8, x_next=xn)
    dens = scipy.stats.norm.logpdf(xn.astype(np.float64), loc=mu, scale=s * math.sqrt(dt))
    assert lp[0] == pytest.approx(dens.sum(), rel=1e-12) and abs(dens.mean() - lp[0]) > 1.0
