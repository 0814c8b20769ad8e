"""GPU parity of the routed per-head QK RMSNorm + rotary embedding against
the CPU oracle (the "mot_qk_norm_rope" work item of the RFC page "[RFC]
[BAGEL-7B-MoT] WS1/WS2 kernel roadmap", section 5; order from its reference
hazards: QK norm in fp32, then the rotation with Q/K in bf16).

Every rounding after the norm is reproduced exactly on the GPU (products of
two bf16 values are exact in fp32), so outputs are the oracle's bf16 values
except where the fp32 norm product and the fp64 one land on different sides
of a bf16 rounding boundary.  The normalized value is a bf16 intermediate,
so such a one-step flip can move an output by two steps where the two
rotated products partly cancel: the gate is the usual one against the exact
last sum, as for a chain (no one-step check), plus a bit-exact share of at
least 99.9%.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_transformers_token_amd as mot
import oracle
import workloads as W
from helpers import bits, check_parity, dev, raw_equal

pytestmark = pytest.mark.gpu

HQ, HK, LD = 28, 4, 4608  # the BAGEL QKV row: 28 q heads, 4 k heads, then v


def _inputs(T, base, ld=LD, n_pos=512, std=1.2):
    qkv = W.normal_bf16((T, ld), W.seed_of(base, 1), std)
    m = W.pattern(T)
    m[::5] = 1 - m[::5]
    qn, kn = W.qk_norm_weights(base)
    cos_t, sin_t, pos = W.rope_inputs(T, n_pos, base)
    return qkv, m, qn, kn, cos_t, sin_t, pos


def _gpu(qkv, m, qn, kn, cos_t, sin_t, pos, hq=HQ, hk=HK, ws=None, ld_pad=0):
    T, ld = qkv.shape
    if ld_pad:
        big = torch.full((T, ld + ld_pad), 5.0, dtype=torch.bfloat16, device="cuda")
        big[:, :ld] = dev(qkv)
        q = big[:, :ld]
    else:
        big, q = None, dev(qkv).clone()
    ws = ws if ws is not None else mot.new_workspace(0, q.device)
    mot.qk_norm_rope(q, hq, hk, dev(torch.from_numpy(m)), tuple(dev(t) for t in qn), tuple(dev(t) for t in kn),
                     dev(pos), dev(cos_t), dev(sin_t), workspace=ws)
    err = mot.read_device_error(ws)
    if ld_pad:
        assert torch.all(big[:, ld:] == 5.0), "wrote past the row"
    return q, err


def _oracle(qkv, m, qn, kn, cos_t, sin_t, pos, hq=HQ, hk=HK, rows=None):
    sel = np.arange(qkv.shape[0]) if rows is None else rows
    return oracle.qk_norm_rope(W.bits(qkv)[sel], hq, hk, m[sel], tuple(W.bits(t) for t in qn),
                               tuple(W.bits(t) for t in kn), pos.numpy()[sel], W.bits(cos_t), W.bits(sin_t))


def _check(got_bits, ref, out, what, cols):
    m = check_parity(got_bits[:, :cols], ref[:, :cols], out[:, :cols], what, one_step=False)
    exact = float((got_bits[:, :cols] == out[:, :cols]).mean())
    assert exact >= 0.999, (what, exact, m)
    return exact


@pytest.mark.parametrize("T", [1, 5, 77, 333])
def test_small_packs(T):
    case = _inputs(T, base=900 + T)
    q, err = _gpu(*case, ld_pad=64)
    assert err == 0
    ref, out, oerr = _oracle(*case)
    assert oerr == 0
    got = bits(q)
    _check(got, ref, out, f"qk_norm_rope T={T}", 128 * (HQ + HK))
    # v columns are not touched
    assert np.array_equal(got[:, 128 * (HQ + HK):], W.bits(case[0])[:, 128 * (HQ + HK):])


def test_full_size_sampled():
    """The BAGEL QKV rows at T=4096 (3788 gen, 308 und), 4096 positions; rows
    are independent, so the oracle on a row sample is the exact restriction."""
    T = 4096
    case = _inputs(T, base=950, n_pos=4096)
    q, err = _gpu(*case)
    assert err == 0
    rows = W.sample_rows(case[1], 48, seed=3)
    ref, out, _ = _oracle(*case, rows=rows)
    _check(bits(q)[rows], ref, out, "qk_norm_rope T=4096 sampled", 128 * (HQ + HK))


def test_few_heads_and_errors():
    """3 q + 1 k heads in a wider row; a row with an invalid modality byte and
    one with a position past the table keep their bytes and raise the error
    word (position wins); the next clean call clears it."""
    T, hq, hk = 40, 3, 1
    qkv, m, qn, kn, c, s, pos = _inputs(T, base=960, ld=640, n_pos=64)
    q0, err = _gpu(qkv, m, qn, kn, c, s, pos, hq, hk)
    assert err == 0
    ref, out, _ = _oracle(qkv, m, qn, kn, c, s, pos, hq, hk)
    _check(bits(q0), ref, out, "qk_norm_rope 3+1 heads", 512)
    bm = m.copy()
    bm[7] = 3
    ws = mot.new_workspace(0, "cuda")
    q1, err = _gpu(qkv, bm, qn, kn, c, s, pos, hq, hk, ws=ws)
    assert err == 6
    keep = np.delete(np.arange(T), 7)
    assert raw_equal(q1[7].cpu(), qkv[7]) and raw_equal(q1[keep], q0[keep])
    bp = pos.clone()
    bp[9] = 64
    q2, err = _gpu(qkv, bm, qn, kn, c, s, bp, hq, hk, ws=ws)
    assert err == 7
    assert raw_equal(q2[9].cpu(), qkv[9])
    _, err = _gpu(qkv, m, qn, kn, c, s, pos, hq, hk, ws=ws)
    assert err == 0


def test_rows_batch_invariant():
    """A row's bytes do not depend on the pack around it."""
    probe = _inputs(100, base=970)
    ref, _ = _gpu(*probe)
    fill = _inputs(700, base=971)
    cat = [torch.cat([fill[i][:350], probe[i], fill[i][350:]]) if isinstance(probe[i], torch.Tensor) and i in (0, 6)
           else None for i in range(7)]
    m = np.concatenate([fill[1][:350], probe[1], fill[1][350:]])
    perm = W.permutation(800, 11).numpy()
    # the fill rows use the probe's tables and weights (positions index them)
    args = (cat[0][perm], m[perm], probe[2], probe[3], probe[4], probe[5], cat[6][perm] % 512)
    out, err = _gpu(*args)
    assert err == 0
    pos_of = np.empty(800, np.int64)
    pos_of[perm] = np.arange(800)
    got = out[torch.from_numpy(pos_of[350:450]).cuda()]
    assert raw_equal(got, ref)
