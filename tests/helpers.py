"""Shared test helpers: device transfer, raw-bit views and the parity gate.

The parity gate compares a bf16 GPU result with the oracle's unrounded fp64
result: relative Frobenius error <= 5e-3 over the whole output (bf16
rounding alone contributes about 1.7e-3) and, element by element, max-abs
error <= 2e-2.  Where an exact value reaches 8 or more, a bf16 half-step
(1/32 there) exceeds 2e-2 even for a correctly rounded result, so for those
elements (and only those) the elementwise bf16 row of the tolerance
contract on the RL-Kernel MoE route/combine PR page applies instead:
|d| <= 2e-2 + 1.6e-2 |ref|.

Single operations are also held to a bound derived from their arithmetic,
element by element: the GPU rounds an fp32 result s to bf16 once, so
|got - ref| <= halfstep(got) + |s - ref|, where halfstep(got) is half the
bf16 spacing at got and |s - ref| is bounded by the fp32 arithmetic that
produced s.  For a GEMM of K terms that is K * 2^-23 * sum_k |a_k||w_k| (each
of at most K fp32 additions rounds by at most 2^-24 of a partial sum, which
never exceeds the sum of the products' magnitudes; the factor 2 covers any
rounding inside the matrix unit).  The sum of magnitudes is the oracle run on
the operands' absolute values (sign bits cleared).  Near zero, after
cancellation, this bound is set by the summands' size, not the result's.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

MAX_ABS = 2e-2
REL_FRO = 5e-3


def dev(t: torch.Tensor) -> torch.Tensor:
    return t.to("cuda")


def bits(t: torch.Tensor) -> np.ndarray:
    """uint16 view of a bf16 tensor (any device)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def halfstep(bits_: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at each finite bf16 value: 2^(e-8) in the binade
    [2^e, 2^(e+1)), 2^-134 for zero and the subnormals."""
    e = (np.asarray(bits_, np.uint16).astype(np.int32) >> 7) & 0xFF
    return np.where(e == 0, 2.0 ** -134, np.ldexp(1.0, e - 127 - 8))


def _abs_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16) & np.uint16(0x7FFF)).astype(np.uint16)


def gemm_bound(xb, wub, wgb, m) -> np.ndarray:
    """Per-element bound of |fp32 result - exact| for the routed GEMM of the
    oracle's arguments: K 2^-23 sum_k |x||w| (plus the oracle's own fp64
    rounding, K 2^-52 of the same sum)."""
    K = np.asarray(xb).shape[1]
    mag, _ = oracle.routed_gemm(_abs_bits(xb), _abs_bits(wub), _abs_bits(wgb), m, want_out=False)
    return K * (2.0 ** -23 + 2.0 ** -52) * mag


def swiglu_bound(xb, wub, wgb, m) -> np.ndarray:
    """Per-element bound of |fp32 act - exact act| for act = silu(g) u:
    with g, u the exact sums and Bg, Bu their GEMM bounds,
    |d act| <= 1.1 Bg |u| + |silu(g)| Bu + 1.1 Bg Bu (|silu'| <= 1.0999),
    plus 8 fp32 roundings of the epilogue (expf, the add, the divide, the
    product: at most 8 * 2^-24 relative)."""
    F = np.asarray(wub).shape[0] // 2
    g, _ = oracle.routed_gemm(xb, wub[:F], wgb[:F], m, want_out=False)
    u, _ = oracle.routed_gemm(xb, wub[F:], wgb[F:], m, want_out=False)
    bg = gemm_bound(xb, wub[:F], wgb[:F], m)
    bu = gemm_bound(xb, wub[F:], wgb[F:], m)
    silu = g / (1.0 + np.exp(-g))
    return 1.1 * bg * np.abs(u) + np.abs(silu) * bu + 1.1 * bg * bu + 8 * 2.0 ** -24 * np.abs(silu * u)


def norm_bound(ref: np.ndarray, H: int) -> np.ndarray:
    """Per-element bound for y = (h rstd) w with h exact: the fp32 sum of H
    squares (H roundings), the mean, eps, sqrt and reciprocal (4), and the
    two products (2): (H + 12) 2^-24 relative to the exact result."""
    return (H + 12) * 2.0 ** -24 * np.abs(ref)


def check_parity(got_bits: np.ndarray, ref: np.ndarray, rne_bits: np.ndarray, what: str,
                 one_step: bool = True, bound: np.ndarray | None = None):
    """The parity gate: relative Frobenius error over the whole output, and
    per element max-abs (where |ref| < 8) or the bf16 row (where |ref| >= 8).
    one_step (single ops) additionally requires |got - ref| <= halfstep(got)
    + bound element by element, with `bound` the fp32 arithmetic's error bound
    (gemm_bound, swiglu_bound, norm_bound); it does not apply to a chain
    where the oracle carries its own bf16 intermediates (a one-step
    difference in an intermediate propagates)."""
    m = oracle.gate_metrics(got_bits, ref)
    got = oracle.bf16_to_f64(got_bits)
    d = np.abs(got - ref)
    assert np.isfinite(got).all(), (what, "non-finite output")
    assert m["rel_fro"] <= REL_FRO, (what, m)
    big = np.abs(ref) >= 8.0
    allowed = np.where(big, MAX_ABS + 1.6e-2 * np.abs(ref), MAX_ABS)
    excess = d - allowed
    m["gate_excess"] = float(excess.max()) if excess.size else 0.0
    assert m["gate_excess"] <= 0.0, (what, m)
    if one_step:
        assert bound is not None, (what, "a single op needs its arithmetic's error bound")
        over = d - (halfstep(got_bits) + bound)
        m["bound_excess"] = float(over.max()) if over.size else 0.0
        assert m["bound_excess"] <= 0.0, (what, m, np.unravel_index(int(np.argmax(over)), over.shape))
    if rne_bits is not None and rne_bits.size:
        m["max_ulp_to_rne"] = int(oracle.ulp_distance(got_bits, rne_bits).max())
    return m


def raw_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Raw-bit identity: same dtype and shape, every bit pattern equal (so
    +0.0 and -0.0 differ), no NaN or Inf allowed."""
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    fa = a.float()
    if not torch.isfinite(fa).all() or not torch.isfinite(b.float()).all():
        return False
    ia = a.contiguous().view(torch.int16)
    ib = b.contiguous().view(torch.int16)
    return bool(torch.equal(ia, ib))
