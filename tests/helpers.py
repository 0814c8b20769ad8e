"""Shared test helpers: device transfer, raw-bit views and the parity gate.

The parity gate compares a bf16 GPU result with the oracle's unrounded fp64
result: max-abs error <= 2e-2 and relative Frobenius error <= 5e-3 (bf16
rounding alone contributes about 1.7e-3 to the latter).  Where the exact
values reach 8 and above, a bf16 half-step (1/32 there) exceeds 2e-2 even for
a correctly rounded result, so there the elementwise bf16 row of the
tolerance contract on the RL-Kernel MoE route/combine PR page applies
(|d| <= 2e-2 + 1.6e-2 |ref|), together with a distance of at most one bf16
step from the correctly rounded oracle value.

The one-step check is applied where |ref| >= 1/4 only: near zero, after
cancellation, the fp32 accumulation error is set by the size of the summands,
not of the result, and may reach a few bf16 steps of a tiny result while
staying far below the absolute gate.
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


def check_parity(got_bits: np.ndarray, ref: np.ndarray, rne_bits: np.ndarray, what: str,
                 one_step: bool = True):
    """The parity gate (max-abs / relative Frobenius, elementwise bf16 row
    where |ref| >= 8).  one_step additionally requires every output with
    |ref| >= 1/4 to be within one bf16 step of the correctly rounded oracle
    value; it applies to single ops, not to a chain where the oracle carries
    its own bf16 intermediates (a one-step difference in an intermediate
    propagates)."""
    m = oracle.gate_metrics(got_bits, ref)
    big = np.abs(ref) >= 0.25
    ulp = int(oracle.ulp_distance(got_bits[big], rne_bits[big]).max()) if big.any() else 0
    m["max_ulp_to_rne"] = ulp
    assert np.isfinite(oracle.bf16_to_f64(got_bits)).all(), (what, "non-finite output")
    assert m["rel_fro"] <= REL_FRO, (what, m)
    if m["max_ref"] < 8.0:
        assert m["max_abs"] <= MAX_ABS, (what, m)
    else:
        assert m["elem_excess"] <= 0.0, (what, m)
    if one_step:
        assert ulp <= 1, (what, m)
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
