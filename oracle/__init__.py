"""CPU oracle for the MoT token-routed projection (ctypes over mot_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.

Every function takes and returns numpy arrays.  bf16 tensors travel as raw
uint16 bit patterns.  The C source cites, per function, the passage of the
pages it follows.  Pins against things other than itself live in
tests/test_oracle_pins.py.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mot_oracle.c")
_LIB = os.path.join(_HERE, "libmot_oracle.so")


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no fast math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            "-std=c11", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.mot_oracle_bf16_round.argtypes = [ctypes.c_double]
        L.mot_oracle_bf16_round.restype = ctypes.c_uint16
        L.mot_oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.mot_oracle_bf16_value.restype = ctypes.c_double
        L.mot_oracle_max_threads.restype = ctypes.c_int
        L.mot_oracle_routing_plan.argtypes = [P, I64, P, P, P]
        L.mot_oracle_routing_plan.restype = ctypes.c_int
        L.mot_oracle_routed_gemm.argtypes = [P, I64, P, P, P, I64, I64, I64, P, P, ctypes.c_int]
        L.mot_oracle_routed_gemm.restype = None
        L.mot_oracle_routed_gemm_swiglu.argtypes = [P, I64, P, P, P, I64, I64, I64, P, P, ctypes.c_int]
        L.mot_oracle_routed_gemm_dx.argtypes = [P, P, P, P, I64, I64, I64, P, P, ctypes.c_int]
        L.mot_oracle_routed_gemm_dx.restype = None
        L.mot_oracle_grad_w.argtypes = [P, P, P, ctypes.c_int, I64, I64, I64, P, P, ctypes.c_int]
        L.mot_oracle_grad_w.restype = None
        L.mot_oracle_routed_gemm_swiglu.restype = None
        L.mot_oracle_fused_add_rmsnorm.argtypes = [P, P, P, P, P, ctypes.c_float, I64, I64,
                                                   P, P, P, P, ctypes.c_int]
        L.mot_oracle_fused_add_rmsnorm.restype = None
        L.mot_oracle_rmsnorm_apply.argtypes = [P, P, P, P, P, I64, I64, P, P, ctypes.c_int]
        L.mot_oracle_rmsnorm_apply.restype = None
        L.mot_oracle_qk_norm_rope.argtypes = [P, I64, I64, I64, I64, P, P, P, P, P, P, P, P, I64,
                                              ctypes.c_float, P, P, ctypes.c_int]
        L.mot_oracle_qk_norm_rope.restype = ctypes.c_int
        L.mot_oracle_attention.argtypes = [P, I64, I64, P, I64, P, I64, I64, I64, I64, I64, ctypes.c_int,
                                           P, I64, P, P, ctypes.c_int]
        L.mot_oracle_attention.restype = None
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a, shape=None):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    if shape is not None:
        assert a.shape == shape, (a.shape, shape)
    return a


def max_threads() -> int:
    return int(lib().mot_oracle_max_threads())


def bf16_round(v: float) -> int:
    return int(lib().mot_oracle_bf16_round(float(v)))


def bf16_value(b: int) -> float:
    return float(lib().mot_oracle_bf16_value(int(b)))


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float64."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def routing_plan(modality: np.ndarray):
    """Returns (perm int32 [T], n_und, n_gen), or None for a bad modality byte."""
    m = np.ascontiguousarray(modality, dtype=np.uint8)
    perm = np.zeros(m.size, np.int32)
    nu = np.zeros(1, np.int32)
    ng = np.zeros(1, np.int32)
    rc = lib().mot_oracle_routing_plan(_p(m), m.size, _p(perm), _p(nu), _p(ng))
    if rc != 0:
        return None
    return perm, int(nu[0]), int(ng[0])


ERR_INDEX_SET = 10  # a row not in exactly one index set, or an index outside [0, T)


def modality_from_index_sets(und_idx, gen_idx, T):
    """Per-row modality bytes from the two index sets (RL-Kernel RFC page,
    section 1, item 1: each row's weight set is fixed by an index set).  A
    row listed exactly once, in the understanding list, gets 0; exactly once,
    in the generation list, 1; any other row (in neither list, in both, or
    twice in one) gets the invalid byte 0xFF and the call reports
    ERR_INDEX_SET, as does an index outside [0, T) (which marks no row).
    Plain loops over the lists.  Returns (modality uint8 [T], error)."""
    count = [0] * T
    in_gen = [False] * T
    err = 0
    for lst, is_gen in ((und_idx, False), (gen_idx, True)):
        for r in np.asarray(lst).tolist():
            if not 0 <= r < T:
                err = ERR_INDEX_SET
                continue
            count[r] += 1
            in_gen[r] = in_gen[r] or is_gen
    m = np.empty(T, np.uint8)
    for t in range(T):
        if count[t] == 1:
            m[t] = 1 if in_gen[t] else 0
        else:
            m[t] = 0xFF
            err = ERR_INDEX_SET
    return m, err


def routed_gemm(x, w_und, w_gen, modality, want_ref=True, want_out=True, threads=0):
    """x [T,K] uint16, w_* [N,K] uint16, modality [T] uint8 -> (ref f64 [T,N], out u16 [T,N])."""
    x = _u16(x)
    T, K = x.shape
    N = w_und.shape[0]
    wu = _u16(w_und, (N, K))
    wg = _u16(w_gen, (N, K))
    m = np.ascontiguousarray(modality, dtype=np.uint8)
    assert m.shape == (T,)
    ref = np.empty((T, N), np.float64) if want_ref else None
    out = np.empty((T, N), np.uint16) if want_out else None
    lib().mot_oracle_routed_gemm(_p(x), K, _p(wu), _p(wg), _p(m), T, K, N, _p(ref), _p(out), threads)
    return ref, out


def routed_gemm_dx(dy, w_und, w_gen, modality, threads=0):
    """dy [T,N] uint16, w_* [N,K] uint16 (forward weights) -> (ref f64 [T,K], out u16 [T,K]):
    dX[t] = dY[t] @ W_{modality[t]}."""
    dy = _u16(dy)
    T, N = dy.shape
    K = w_und.shape[1]
    wu = _u16(w_und, (N, K))
    wg = _u16(w_gen, (N, K))
    m = np.ascontiguousarray(modality, dtype=np.uint8)
    assert m.shape == (T,)
    ref = np.empty((T, K), np.float64)
    out = np.empty((T, K), np.uint16)
    lib().mot_oracle_routed_gemm_dx(_p(dy), _p(wu), _p(wg), _p(m), T, N, K, _p(ref), _p(out), threads)
    return ref, out


def grad_w(dy, x, modality, keep=1, threads=0):
    """dy [T,N], x [T,K] uint16 -> (ref f64 [N,K], out u16 [N,K]):
    dW = sum over rows with modality == keep of dY[t]^T X[t], ascending t."""
    dy = _u16(dy)
    T, N = dy.shape
    x = _u16(x, (T, x.shape[1]))
    K = x.shape[1]
    m = np.ascontiguousarray(modality, dtype=np.uint8)
    assert m.shape == (T,)
    ref = np.empty((N, K), np.float64)
    out = np.empty((N, K), np.uint16)
    lib().mot_oracle_grad_w(_p(dy), _p(x), _p(m), int(keep), T, N, K, _p(ref), _p(out), threads)
    return ref, out


def routed_gemm_swiglu(x, w_und, w_gen, modality, want_ref=True, want_out=True, threads=0):
    """w_* [2F,K] (gate rows then up rows) -> (ref f64 [T,F], out u16 [T,F])."""
    x = _u16(x)
    T, K = x.shape
    F2 = w_und.shape[0]
    assert F2 % 2 == 0
    F = F2 // 2
    wu = _u16(w_und, (F2, K))
    wg = _u16(w_gen, (F2, K))
    m = np.ascontiguousarray(modality, dtype=np.uint8)
    assert m.shape == (T,)
    ref = np.empty((T, F), np.float64) if want_ref else None
    out = np.empty((T, F), np.uint16) if want_out else None
    lib().mot_oracle_routed_gemm_swiglu(_p(x), K, _p(wu), _p(wg), _p(m), T, K, F, _p(ref), _p(out), threads)
    return ref, out


def fused_add_rmsnorm(x, r, w_und, w_gen, modality, eps=1e-6, threads=0):
    """x, r [T,H] uint16 (r may be None) -> dict(h u16, rstd f64, ref f64, out u16)."""
    x = _u16(x)
    T, H = x.shape
    rr = None if r is None else _u16(r, (T, H))
    wu = _u16(w_und, (H,))
    wg = _u16(w_gen, (H,))
    m = np.ascontiguousarray(modality, dtype=np.uint8)
    assert m.shape == (T,)
    h = np.empty((T, H), np.uint16)
    rstd = np.empty(T, np.float64)
    ref = np.empty((T, H), np.float64)
    out = np.empty((T, H), np.uint16)
    lib().mot_oracle_fused_add_rmsnorm(_p(x), _p(rr), _p(wu), _p(wg), _p(m), float(eps), T, H,
                                       _p(h), _p(rstd), _p(ref), _p(out), threads)
    return {"h": h, "rstd": rstd, "ref": ref, "out": out}


def rmsnorm_apply(h, rstd, w_und, w_gen, modality, threads=0):
    """The routed RMSNorm's output for a given per-row rstd (fp32 values):
    h [T,H] uint16, rstd [T] -> (ref f64 [T,H] = h*rstd*w_m exactly, out u16
    [T,H] = its bf16 rounding).  This is the A operand of the GEMM's
    routed-RMSNorm prologue."""
    h = _u16(h)
    T, H = h.shape
    rs = np.ascontiguousarray(np.asarray(rstd, np.float32).astype(np.float64))
    assert rs.shape == (T,)
    wu, wg = _u16(w_und, (H,)), _u16(w_gen, (H,))
    m = np.ascontiguousarray(modality, dtype=np.uint8)
    assert m.shape == (T,)
    ref = np.empty((T, H), np.float64)
    out = np.empty((T, H), np.uint16)
    lib().mot_oracle_rmsnorm_apply(_p(h), _p(rs), _p(wu), _p(wg), _p(m), T, H, _p(ref), _p(out), threads)
    return ref, out


def qk_norm_rope(qkv, n_q_heads, n_k_heads, modality, q_norm, k_norm, positions, cos_t, sin_t,
                 eps=1e-6, threads=0):
    """Routed per-head QK RMSNorm, then the bf16 rotary embedding (rotate-half
    pairs), on a [T, ld] bf16 copy of the QKV rows.  q_norm, k_norm: (und,
    gen) pairs of [128] bf16 weights; positions [T] int32; cos_t, sin_t
    [n_pos, 64] bf16.  Returns (ref fp64 [T, ld], out bf16 [T, ld], error)."""
    qkv = _u16(qkv)
    T, ld = qkv.shape
    m = np.ascontiguousarray(modality, dtype=np.uint8)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    qu, qg, ku, kg = (_u16(a) for a in (q_norm[0], q_norm[1], k_norm[0], k_norm[1]))
    ct, st = _u16(cos_t), _u16(sin_t)
    assert m.shape == (T,) and pos.shape == (T,) and ct.shape == st.shape and ct.shape[1] == 64
    assert 128 * (n_q_heads + n_k_heads) <= ld and all(a.shape == (128,) for a in (qu, qg, ku, kg))
    out = np.empty((T, ld), np.uint16)
    ref = np.empty((T, ld), np.float64)
    err = lib().mot_oracle_qk_norm_rope(_p(qkv), ld, T, n_q_heads, n_k_heads, _p(m), _p(qu), _p(qg), _p(ku),
                                        _p(kg), _p(pos), _p(ct), _p(st), ct.shape[0], eps, _p(out), _p(ref),
                                        threads)
    return ref, out, int(err)


def ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between two arrays of finite bf16 bit patterns."""
    def key(v):
        v = np.asarray(v, np.uint16).astype(np.int32)
        mag = v & 0x7FFF
        return np.where(v & 0x8000, -mag, mag)
    return np.abs(key(a) - key(b))


def gate_metrics(got_bits: np.ndarray, ref: np.ndarray) -> dict:
    """Tolerance metrics of a bf16 result against the unrounded fp64 oracle:
    max-abs error, relative Frobenius error, elementwise excess over the
    bf16 row of the tolerance contract (|d| <= 2e-2 + 1.6e-2*|ref|), and the
    largest bf16-step distance to the correctly rounded oracle."""
    got = bf16_to_f64(got_bits)
    d = got - ref
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d)) / nref if nref > 0 else float(np.linalg.norm(d))
    excess = float(np.max(np.abs(d) - (2e-2 + 1.6e-2 * np.abs(ref)))) if d.size else 0.0
    rne = np.vectorize(bf16_round, otypes=[np.uint16])(ref) if ref.size <= 4096 else None
    return {
        "max_abs": float(np.max(np.abs(d))) if d.size else 0.0,
        "rel_fro": rel,
        "elem_excess": excess,
        "max_ref": float(np.max(np.abs(ref))) if ref.size else 0.0,
        "max_ulp_to_rne": int(np.max(ulp_distance(got_bits, rne))) if rne is not None and rne.size else None,
    }


def attention(q, k, v, hq, hkv, causal, rows=None, head_dim=128, threads=0):
    """q [Tq, ldq], k [Tk, ldk], v [Tk, ldv] uint16 (the heads' columns first)
    -> (ref f64 [n, hq*D], out u16 [n, hq*D]) for the query rows `rows`
    (default: all): shared joint attention, bottom-right causal when causal."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    Tq, Tk = q.shape[0], k.shape[0]
    assert v.shape[0] == Tk and hq % hkv == 0
    assert q.shape[1] >= hq * head_dim and k.shape[1] >= hkv * head_dim and v.shape[1] >= hkv * head_dim
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = Tq if r is None else r.size
    ref = np.empty((n, hq * head_dim), np.float64)
    out = np.empty((n, hq * head_dim), np.uint16)
    if n:
        lib().mot_oracle_attention(_p(q), q.shape[1], Tq, _p(k), k.shape[1], _p(v), v.shape[1], Tk, hq, hkv,
                                   head_dim, int(causal), _p(r), n, _p(ref), _p(out), threads)
    return ref, out


def attention_varlen(q, k, v, cu_q, cu_k, hq, hkv, causal, head_dim=128, threads=0):
    """Packed sequences: sequence b is q rows [cu_q[b], cu_q[b+1]) over keys
    [cu_k[b], cu_k[b+1]), each by attention() -> (ref f64 [Tq, hq*D], out u16)."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    ref = np.zeros((q.shape[0], hq * head_dim), np.float64)
    out = np.zeros((q.shape[0], hq * head_dim), np.uint16)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0:
            continue
        r, o = attention(q[q0:q1], k[k0:k1], v[k0:k1], hq, hkv, causal, head_dim=head_dim, threads=threads)
        ref[q0:q1], out[q0:q1] = r, o
    return ref, out


# ---- latent step: three-branch renormalised CFG, and the flow SDE step -------
#
# The RL-Kernel RFC page lists both as work items ("cfg_combine_renorm" and
# "flow_sde_step_logp", section 5) and gives their rules, not their formulas
# (section 1, item 3; section 3, its rules for BAGEL): at most three branches
# and two guidance scales, guidance only inside a window of t, a rescale by a
# clamped ratio of norms taken for each request alone; the step and its
# log-probability in fp32, sigma equal to t, a step down in t (positive dt),
# and the log-probability added up over every latent element of a request.
# The formulas below are this project's readings of that contract; the SDE is
# the Euler-Maruyama step of the rectified flow's reverse SDE published with
# Flow-GRPO (arXiv 2505.05470, cited on the RFC page).  Plain fp64 per request.

RENORM_NONE, RENORM_GLOBAL, RENORM_CHANNEL = 0, 1, 2


def _f32(v):
    return float(np.float32(v))


def cfg_combine_renorm(v_cond, v_text_uncond, v_img_uncond, cu_rows, t, s_text, s_img, t_lo, t_hi,
                       renorm_min, renorm_type):
    """Guided velocity of each request b (rows [cu_rows[b], cu_rows[b+1])),
    inputs fp32 [R, C] (v_img_uncond None: two branches):
      inside the window t_lo < t[b] <= t_hi (fp32 comparisons):
        g = v_tu + s_text (v_c - v_tu);  three branches: g = v_iu + s_img (g - v_iu)
        global renorm: r = clamp(||v_c||_2 / ||g||_2, renorm_min, 1) over the
          request's elements (r = 1 when ||g|| = 0); out = r g
        channel renorm: the same ratio per row (over its C channels)
        none: out = g
      outside the window: out = v_c.
    Returns the fp64 result [R, C]."""
    vc = np.asarray(v_cond, np.float32).astype(np.float64)
    vt = np.asarray(v_text_uncond, np.float32).astype(np.float64)
    vi = None if v_img_uncond is None else np.asarray(v_img_uncond, np.float32).astype(np.float64)
    s1, s2, lo, hi, rmin = (_f32(a) for a in (s_text, s_img, t_lo, t_hi, renorm_min))
    out = np.zeros_like(vc)
    for b in range(len(cu_rows) - 1):
        r0, r1 = int(cu_rows[b]), int(cu_rows[b + 1])
        tb = _f32(t[b])
        if not (lo < tb <= hi):
            out[r0:r1] = vc[r0:r1]
            continue
        g = vt[r0:r1] + s1 * (vc[r0:r1] - vt[r0:r1])
        if vi is not None:
            g = vi[r0:r1] + s2 * (g - vi[r0:r1])
        if renorm_type == RENORM_GLOBAL:
            ng = math.sqrt(math.fsum((g * g).ravel().tolist()))
            nc = math.sqrt(math.fsum((vc[r0:r1] ** 2).ravel().tolist()))
            r = 1.0 if ng == 0.0 else min(1.0, max(rmin, nc / ng))
            out[r0:r1] = g * r
        elif renorm_type == RENORM_CHANNEL:
            for i in range(r1 - r0):
                ng = math.sqrt(math.fsum((g[i] * g[i]).tolist()))
                nc = math.sqrt(math.fsum((vc[r0 + i] ** 2).tolist()))
                r = 1.0 if ng == 0.0 else min(1.0, max(rmin, nc / ng))
                out[r0 + i] = g[i] * r
        else:
            out[r0:r1] = g
    return out


def sde_scale(t, t_next, eta):
    """Diffusion scale of the step from t to t_next: s = eta sqrt(t / (1 - t)),
    with 1 - t_next in the denominator at the first step t = 1."""
    t, tn, e = _f32(t), _f32(t_next), _f32(eta)
    den = 1.0 - (t if t < 1.0 else tn)
    return e * math.sqrt(t / den)


def flow_sde_step_logp(x, v, cu_rows, t_cur, t_next, eta, noise=None, x_next=None):
    """One step of request b from t = t_cur[b] down to t_next[b]
    (dt = t - t_next > 0), x_t = (1 - t) x_0 + t eps and v = dx/dt:
      s  = sde_scale(t, t_next, eta)
      mu = x - dt (v + s^2 / (2 t) (x + (1 - t) v))
      x_next = mu + s sqrt(dt) noise              (when noise is given)
      logp_b = sum over the request's elements of
               -(x_next - mu)^2 / (2 s^2 dt) - log(s sqrt(dt)) - log(2 pi) / 2
    x, v, noise, x_next: fp32 [R, C].  Returns (mu, x_next, logp) in fp64."""
    xx = np.asarray(x, np.float32).astype(np.float64)
    vv = np.asarray(v, np.float32).astype(np.float64)
    mu = np.zeros_like(xx)
    xn = np.zeros_like(xx)
    logp = np.zeros(len(cu_rows) - 1)
    for b in range(len(cu_rows) - 1):
        r0, r1 = int(cu_rows[b]), int(cu_rows[b + 1])
        t, tn = _f32(t_cur[b]), _f32(t_next[b])
        dt = t - tn
        s = sde_scale(t, tn, eta)
        m = xx[r0:r1] - dt * (vv[r0:r1] + (s * s / (2.0 * t)) * (xx[r0:r1] + (1.0 - t) * vv[r0:r1]))
        std = s * math.sqrt(dt)
        if noise is not None:
            xb = m + std * np.asarray(noise, np.float32)[r0:r1].astype(np.float64)
        else:
            xb = np.asarray(x_next, np.float32)[r0:r1].astype(np.float64)
        d = (xb - m).ravel().tolist()
        n = len(d)
        logp[b] = -math.fsum(di * di for di in d) / (2.0 * std * std) - n * (math.log(std) + 0.5 * math.log(2 * math.pi))
        mu[r0:r1], xn[r0:r1] = m, xb
    return mu, xn, logp
