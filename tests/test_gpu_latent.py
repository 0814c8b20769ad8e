"""GPU parity of the latent step (the renormalised CFG combine and the flow
SDE step with its log-probability) against the oracle, through the C ABI,
plus the properties the RL-Kernel RFC page asks for (section 3): results per
request that do not depend on the pack, the first step t = 1 and the last step
t -> 0 as separate cases, and a sampling call whose log-probability equals the
evaluation of its own sample bit for bit (rollout and training agree).

Floating-point bars are derived from the fp32 arithmetic of each output
(below); the oracle is fp64."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import mixture_transformers_token_amd as mot
import oracle

pytestmark = pytest.mark.gpu

U = 2.0 ** -24       # fp32 unit roundoff
C = 64               # BAGEL latent channels per token (16 channels, 2 x 2 patches)
DEPTH = 96           # longest chain of fp32 additions in any sum here (per-thread run,
                     # butterfly, wave order and chunk order), with margin


def _f32(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * scale).numpy()


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _d(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()


# a batch of step-batched requests: a 512x512 image (1024 latent rows), a
# smaller one, an empty request, a single row
LENGTHS = [1024, 300, 0, 1]


# ---- CFG combine ----------------------------------------------------------------

def _cfg_case(lengths, seed, three=True):
    rows = int(sum(lengths))
    vc = _f32((rows, C), seed)
    vt = _f32((rows, C), seed + 1, 0.8)
    vi = _f32((rows, C), seed + 2, 0.9) if three else None
    return vc, vt, vi


def _cfg_bound(vc, vt, vi, s1, s2, ref, renorm):
    """Elementwise bound of |fp32 out - exact out|: the guided velocity's fp32
    ops (a few roundings of terms no larger than M), the ratio's sums (at
    most DEPTH roundings each), square roots, the divide and the last
    product."""
    a = lambda z: np.abs(z.astype(np.float64))
    M = a(vt) + abs(s1) * (a(vc) + a(vt))
    if vi is not None:
        M = a(vi) + abs(s2) * (M + a(vi))
    rel_r = (2 * DEPTH + 8) * U if renorm != "none" else 0.0
    return 8 * U * M + np.abs(ref) * (rel_r + U) + 1e-30


@pytest.mark.parametrize("renorm", ["global", "channel", "none"])
@pytest.mark.parametrize("three", [True, False])
def test_cfg_against_oracle(renorm, three):
    vc, vt, vi = _cfg_case(LENGTHS, 10 + three, three)
    cu = _cu(LENGTHS)
    t = np.float32([0.5, 0.95, 0.3, 0.7])
    s1, s2, lo, hi, rmin = 4.0, 1.5, 0.0, 0.9, 0.2   # request 1 is outside the window
    out, ws = mot.cfg_combine_renorm(_d(vc), _d(vt), _d(vi), _d(cu), max(LENGTHS), _d(t), s1, s2, lo, hi, rmin, renorm)
    assert mot.read_device_error(ws) == 0
    got = out.cpu().numpy().astype(np.float64)
    kind = {"none": oracle.RENORM_NONE, "global": oracle.RENORM_GLOBAL, "channel": oracle.RENORM_CHANNEL}[renorm]
    ref = oracle.cfg_combine_renorm(vc, vt, vi, cu, t, s1, s2, lo, hi, rmin, kind)
    bound = _cfg_bound(vc, vt, vi, s1, s2, ref, renorm)
    assert np.all(np.abs(got - ref) <= bound), float(np.max(np.abs(got - ref) / bound))
    # outside the window: the conditional branch's bytes
    r0, r1 = cu[1], cu[2]
    assert np.array_equal(out.cpu().numpy()[r0:r1].view(np.uint32), vc[r0:r1].view(np.uint32))


def test_cfg_window_ends_and_closed_form():
    """t == t_lo is outside the window, t == t_hi inside; with v_tu = 0 and
    one branch pair the global renorm returns v_c up to rounding."""
    lengths = [256, 256]
    vc = _f32((512, C), 20)
    zero = np.zeros_like(vc)
    cu = _cu(lengths)
    lo, hi = np.float32(0.25), np.float32(0.75)
    t = np.array([lo, hi], np.float32)
    out, ws = mot.cfg_combine_renorm(_d(vc), _d(zero), None, _d(cu), 256, _d(t), 4.0, 1.0, lo, hi, 0.0, "global")
    got = out.cpu().numpy()
    assert mot.read_device_error(ws) == 0
    assert np.array_equal(got[:256].view(np.uint32), vc[:256].view(np.uint32))
    assert np.abs(got[256:] - vc[256:]).max() <= (2 * DEPTH + 16) * U * np.abs(vc[256:]).max()


@pytest.mark.parametrize("renorm", ["global", "channel"])
def test_cfg_request_bytes_do_not_depend_on_the_pack(renorm):
    """Renormalisation is per request: a request's bytes alone equal its
    bytes inside a pack of other requests of different scale."""
    vc, vt, vi = _cfg_case(LENGTHS, 30)
    vc[1024:] *= 8.0
    cu = _cu(LENGTHS)
    t = np.float32([0.5, 0.5, 0.5, 0.5])
    full, _ = mot.cfg_combine_renorm(_d(vc), _d(vt), _d(vi), _d(cu), 1024, _d(t), 4.0, 1.5, 0.0, 1.0, 0.1, renorm)
    alone, _ = mot.cfg_combine_renorm(_d(vc[:1024]), _d(vt[:1024]), _d(vi[:1024]), _d(_cu([1024])), 1024, _d(t[:1]),
                                      4.0, 1.5, 0.0, 1.0, 0.1, renorm)
    torch.cuda.synchronize()
    assert torch.equal(full[:1024].view(torch.int32), alone.view(torch.int32))


# ---- flow SDE step and log-probability -----------------------------------------

def _sde_case(lengths, seed):
    rows = int(sum(lengths))
    return _f32((rows, C), seed), _f32((rows, C), seed + 1), _f32((rows, C), seed + 2)


def _sde_bounds(x, v, z, cu, tc, tn, eta, mu, xn, sample):
    """Elementwise bounds of the fp32 mean and sample, and per-request bounds
    of the fp32 logp, from the roundings of each fp32 operation (a factor 2
    of margin on each)."""
    a = lambda q: np.abs(q.astype(np.float64))
    b_mu = np.zeros_like(mu)
    b_xn = np.zeros_like(mu)
    b_lp = np.zeros(len(cu) - 1)
    for b in range(len(cu) - 1):
        r0, r1 = cu[b], cu[b + 1]
        t, tnx = float(tc[b]), float(tn[b])
        dt = t - tnx
        s = oracle.sde_scale(t, tnx, eta)
        k = s * s / (2 * t)
        sd = s * math.sqrt(dt)
        b_mu[r0:r1] = 32 * U * (a(x[r0:r1]) + dt * (a(v[r0:r1]) + k * (a(x[r0:r1]) + a(v[r0:r1]))))
        if sample:
            b_xn[r0:r1] = b_mu[r0:r1] + 16 * U * (np.abs(xn[r0:r1]) + sd * a(z[r0:r1]))
        n = (r1 - r0) * C
        if n == 0:
            continue
        d = xn[r0:r1] - mu[r0:r1]
        bd = b_xn[r0:r1] + b_mu[r0:r1] + U * np.abs(d) + U * np.abs(xn[r0:r1])
        q = float((d * d).sum())
        dq = float((2 * np.abs(d) * bd + bd * bd).sum()) + DEPTH * U * q
        b_lp[b] = 2 * (dq / (2 * sd * sd) + q / (2 * sd * sd) * 16 * U
                       + n * (16 * U + U * abs(math.log(sd) + 1.0)) + 4 * U * abs(q / (2 * sd * sd))
                       + 4 * U * n * abs(math.log(sd) + 1.0))
    return b_mu, b_xn, b_lp


SCHEDULES = {
    "middle": (np.float32([0.6, 0.5, 0.5, 0.3]), np.float32([0.55, 0.45, 0.4, 0.2])),
    "first_step": (np.float32([1.0, 1.0, 1.0, 1.0]), np.float32([0.98, 0.9, 0.5, 0.98])),
    "last_step": (np.float32([0.02, 0.05, 0.05, 0.1]), np.float32([0.0, 0.0, 0.0, 0.0])),
    "mixed": (np.float32([1.0, 0.5, 0.7, 0.02]), np.float32([0.98, 0.45, 0.6, 0.0])),
}


@pytest.mark.parametrize("sched", sorted(SCHEDULES))
def test_sde_sample_against_oracle(sched):
    x, v, z = _sde_case(LENGTHS, 40)
    cu = _cu(LENGTHS)
    tc, tn = SCHEDULES[sched]
    eta = 0.7
    xn, logp, ws = mot.flow_sde_step_logp(_d(x), _d(v), _d(cu), max(LENGTHS), _d(tc), _d(tn), eta, noise=_d(z))
    assert mot.read_device_error(ws) == 0
    mu, xn_ref, lp_ref = oracle.flow_sde_step_logp(x, v, cu, tc, tn, eta, noise=z)
    b_mu, b_xn, b_lp = _sde_bounds(x, v, z, cu, tc, tn, eta, mu, xn_ref, True)
    got = xn.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - xn_ref) <= b_xn + 1e-30), float(np.max(np.abs(got - xn_ref) / (b_xn + 1e-30)))
    lp = logp.cpu().numpy().astype(np.float64)
    for b in range(len(LENGTHS)):
        if LENGTHS[b] == 0:
            assert lp[b] == 0.0 or abs(lp[b]) <= 1e-30
            continue
        assert abs(lp[b] - lp_ref[b]) <= b_lp[b], (sched, b, lp[b], lp_ref[b], b_lp[b])


@pytest.mark.parametrize("sched", ["middle", "first_step", "last_step"])
def test_sde_evaluate_against_oracle(sched):
    """Evaluation of a given x_next (the oracle's own sample of another
    noise, rounded to fp32: an input, not a GPU output)."""
    x, v, z = _sde_case(LENGTHS, 50)
    cu = _cu(LENGTHS)
    tc, tn = SCHEDULES[sched]
    eta = 1.0
    _, xs, _ = oracle.flow_sde_step_logp(x, v, cu, tc, tn, eta, noise=z)
    xin = xs.astype(np.float32)
    _, logp, ws = mot.flow_sde_step_logp(_d(x), _d(v), _d(cu), 1024, _d(tc), _d(tn), eta, x_next=_d(xin))
    assert mot.read_device_error(ws) == 0
    mu, _, lp_ref = oracle.flow_sde_step_logp(x, v, cu, tc, tn, eta, x_next=xin)
    _, _, b_lp = _sde_bounds(x, v, z, cu, tc, tn, eta, mu, xin.astype(np.float64), False)
    lp = logp.cpu().numpy().astype(np.float64)
    for b in range(len(LENGTHS)):
        if LENGTHS[b]:
            assert abs(lp[b] - lp_ref[b]) <= b_lp[b], (sched, b, lp[b], lp_ref[b], b_lp[b])


def test_sde_rollout_equals_training_bitwise_and_requests_independent():
    """The log-probability of a sampling call equals, bit for bit, the
    evaluation of its own sample; a request's sample and logp alone equal
    those inside the pack."""
    x, v, z = _sde_case(LENGTHS, 60)
    cu = _cu(LENGTHS)
    tc, tn = SCHEDULES["mixed"]
    xn, lp_s, _ = mot.flow_sde_step_logp(_d(x), _d(v), _d(cu), 1024, _d(tc), _d(tn), 0.9, noise=_d(z))
    _, lp_e, _ = mot.flow_sde_step_logp(_d(x), _d(v), _d(cu), 1024, _d(tc), _d(tn), 0.9, x_next=xn.clone())
    torch.cuda.synchronize()
    assert torch.equal(lp_s.view(torch.int32), lp_e.view(torch.int32))
    r0, r1 = cu[1], cu[2]
    xn1, lp1, _ = mot.flow_sde_step_logp(_d(x[r0:r1]), _d(v[r0:r1]), _d(_cu([r1 - r0])), 1024, _d(tc[1:2]),
                                         _d(tn[1:2]), 0.9, noise=_d(z[r0:r1]))
    torch.cuda.synchronize()
    assert torch.equal(xn[r0:r1].view(torch.int32), xn1.view(torch.int32))
    assert torch.equal(lp_s[1:2].view(torch.int32), lp1.view(torch.int32))


@pytest.mark.parametrize("bad", ["t_next_equal", "t_above_one", "t_zero", "cu_order", "cu_total"])
def test_latent_errors_write_nothing(bad):
    x, v, z = _sde_case([64, 64], 70)
    cu = _cu([64, 64])
    tc, tn = np.float32([0.5, 0.4]), np.float32([0.4, 0.3])
    if bad == "t_next_equal":
        tn[1] = tc[1]
    elif bad == "t_above_one":
        tc[0] = np.float32(1.0001)
    elif bad == "t_zero":
        tc[1], tn[1] = 0.0, 0.0
    elif bad == "cu_order":
        cu[1] = 100
        cu[2] = 90
    elif bad == "cu_total":
        cu[2] = 120
    out = torch.full((128, C), 7.0, device="cuda")
    logp = torch.full((2,), 7.0, device="cuda")
    _, _, ws = mot.flow_sde_step_logp(_d(x), _d(v), _d(cu), 128, _d(tc), _d(tn), 0.5, noise=_d(z), out=out,
                                      logp=logp)
    want = 8 if bad.startswith("cu") else 11
    assert mot.read_device_error(ws) == want
    assert torch.all(out == 7.0) and torch.all(logp == 7.0)
    vc = _d(x)
    o2 = torch.full((128, C), 7.0, device="cuda")
    tcfg = np.float32([0.5, np.inf]) if not bad.startswith("cu") else np.float32([0.5, 0.5])
    _, ws2 = mot.cfg_combine_renorm(vc, _d(v), None, _d(cu), 128, _d(tcfg), 3.0, 1.0, 0.0, 1.0, 0.0, "global",
                                    out=o2)
    assert mot.read_device_error(ws2) == want
    assert torch.all(o2 == 7.0)
