"""GPU parity of the shared joint attention (the RFC page's
"gen_joint_attention" work item: one attention over the pack's tokens of both
modalities, grouped kv heads, causal mask aligned at the bottom-right corner
for a cached prefill) against the CPU oracle, and its batch invariance.

Parity bar: the gate of the other parity tests (max-abs 2e-2, relative
Frobenius 5e-3) against the oracle's exact fp64 result.  The one-step check
does not apply: the kernel feeds the softmax weights to the second product
as bf16 (a declared cast), so its result is not the rounding of the exact
value; a per-element bound derived from that cast, the hardware exp2 and
the fp32 sums takes its place (test_attention_per_element_bound).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_transformers_token_amd as mot
import oracle
import workloads as W
from helpers import bits, check_parity, dev, halfstep

pytestmark = pytest.mark.gpu

D = 128


def _inputs(Tq, Tk, hq, hkv, base, extra=0):
    q = W.normal_bf16((Tq, hq * D + extra), W.seed_of(base, 1))
    k = W.normal_bf16((Tk, hkv * D + extra), W.seed_of(base, 2))
    v = W.normal_bf16((Tk, hkv * D + extra), W.seed_of(base, 3))
    return q, k, v


def _parity(q, k, v, hq, hkv, causal, what, rows=None, out=None):
    got = mot.joint_attention(dev(q) if not q.is_cuda else q, dev(k) if not k.is_cuda else k,
                              dev(v) if not v.is_cuda else v, hq, hkv, causal=causal, out=out)
    torch.cuda.synchronize()
    gb = bits(got)
    sel = np.arange(q.shape[0]) if rows is None else rows
    ref, rne = oracle.attention(W.bits(q.cpu()), W.bits(k.cpu()), W.bits(v.cpu()), hq, hkv, causal, rows=sel)
    check_parity(gb[sel][:, :hq * D], ref, rne, what, one_step=False)
    return got


@pytest.mark.parametrize("Tq,Tk,hq,hkv,causal", [
    (1, 1, 1, 1, True), (37, 90, 4, 2, True), (128, 128, 2, 1, True), (128, 128, 2, 1, False),
    (200, 333, 7, 1, True), (300, 300, 4, 4, False), (129, 700, 4, 2, True), (65, 64, 2, 2, False)])
def test_attention_small(Tq, Tk, hq, hkv, causal):
    q, k, v = _inputs(Tq, Tk, hq, hkv, base=1000 + Tq + Tk, extra=64)
    _parity(q, k, v, hq, hkv, causal, f"attn Tq={Tq} Tk={Tk} hq={hq} hkv={hkv} causal={causal}")


@pytest.mark.parametrize("Tq,Tk,hq,hkv,causal", [(300, 300, 4, 2, True), (256, 700, 4, 2, False),
                                                  (3, 1101, 28, 4, False)])
def test_attention_per_element_bound(Tq, Tk, hq, hkv, causal):
    """Every output element within a bound derived from the kernel's
    arithmetic (R31), against the oracle's exact fp64 attention:
      |got - exact| <= halfstep(got) + A (2^-8 + (Tk + 160) 2^-23 + 2 ds / sqrt(128))
    with A = sum_j w_j |v_j| (the oracle run on v with its sign bits
    cleared): the bf16 rounding of each weight (at most 2^-8 relative), the
    hardware exp2 and the fp32 argument, rescales and sums over the keys
    (each at most 2^-23 relative per step, Tk + 160 steps), and the score
    error ds <= 128 2^-23 max_j |q|.|k_j| of the fp32 dot products, which
    moves a weight by ds / sqrt(128) relative (numerator and denominator)."""
    q, k, v = _inputs(Tq, Tk, hq, hkv, base=1050 + Tq)
    got = mot.joint_attention(dev(q), dev(k), dev(v), hq, hkv, causal=causal)
    torch.cuda.synchronize()
    gb = bits(got)[:, :hq * D]
    qb, kb, vb = W.bits(q), W.bits(k), W.bits(v)
    ref, _ = oracle.attention(qb, kb, vb, hq, hkv, causal)
    A, _ = oracle.attention(qb, kb, vb & np.uint16(0x7FFF), hq, hkv, causal)
    qa = np.abs(oracle.bf16_to_f64(qb)).reshape(Tq, hq, D)
    ka = np.abs(oracle.bf16_to_f64(kb)).reshape(Tk, hkv, D)
    ds = np.empty((Tq, hq))
    for h in range(hq):
        ds[:, h] = 128 * 2.0 ** -23 * (qa[:, h] @ ka[:, h // (hq // hkv)].T).max(axis=1)
    rel = 2.0 ** -8 + (Tk + 160) * 2.0 ** -23 + 2 * ds / np.sqrt(128.0)
    bound = halfstep(gb) + A * np.repeat(rel, D, axis=1)
    g = oracle.bf16_to_f64(gb)
    excess = np.abs(g - ref) - bound
    assert excess.max() <= 0, (float(excess.max()), np.unravel_index(int(np.argmax(excess)), excess.shape))


def test_attention_rows_without_keys():
    """Tq > Tk with the bottom-right causal mask: the first Tq - Tk rows see
    no key and are zero; the rest match the oracle."""
    q, k, v = _inputs(333, 200, 2, 1, base=1010)
    got = _parity(q, k, v, 2, 1, True, "attn Tq>Tk")
    assert not bits(got)[:133].any()


def test_attention_no_keys():
    q = W.normal_bf16((70, 256), 1011)
    k = torch.empty((0, 128), dtype=torch.bfloat16)
    out = mot.joint_attention(dev(q), dev(k), dev(k), 2, 1, causal=False)
    torch.cuda.synchronize()
    assert not bits(out).any()
    e = mot.joint_attention(dev(q[:0]), dev(k), dev(k), 2, 1)
    assert tuple(e.shape) == (0, 256)


def test_attention_qkv_layout_sampled():
    """The BAGEL layer's shape: 28 q heads and 4 kv heads of 128 read from one
    [4096, 4608] QKV buffer (q, k, v as column ranges), causal over the
    4096-row pack, 40 sampled rows checked against the oracle."""
    T = 4096
    qkv = W.normal_bf16((T, W.QKV_DIM), 1012)
    qkv_d = dev(qkv)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, 127, 128, T - 1],
                                     np.random.default_rng(15).integers(0, T, 33)]))
    got = mot.joint_attention(qkv_d[:, :W.Q_DIM], qkv_d[:, W.Q_DIM:W.Q_DIM + W.KV_DIM],
                              qkv_d[:, W.Q_DIM + W.KV_DIM:], W.N_Q_HEADS, W.N_K_HEADS, causal=True)
    torch.cuda.synchronize()
    qb = W.bits(qkv)
    ref, rne = oracle.attention(qb[:, :W.Q_DIM], qb[:, W.Q_DIM:W.Q_DIM + W.KV_DIM], qb[:, W.Q_DIM + W.KV_DIM:],
                                W.N_Q_HEADS, W.N_K_HEADS, True, rows=rows)
    check_parity(bits(got)[rows], ref, rne, "attn QKV T=4096", one_step=False)


def test_attention_cached_prefill_sampled():
    """A cached prefill: 1000 new rows over 4096 keys (3096 cached), the mask
    aligned at the bottom-right corner; sampled rows."""
    q, k, v = _inputs(1000, 4096, W.N_Q_HEADS, W.N_K_HEADS, base=1013)
    rows = np.unique(np.concatenate([[0, 999], np.random.default_rng(16).integers(0, 1000, 14)]))
    _parity(q, k, v, W.N_Q_HEADS, W.N_K_HEADS, True, "attn prefill 1000/4096", rows=rows)


def test_attention_rows_batch_invariant():
    """A row's bytes depend only on its q row and the keys it sees: the last
    300 rows of a 1000-row causal pack, run as a pack of their own over the
    same keys (the bottom-right alignment keeps what each row sees), give the
    same bytes; without the mask, permuting the rows permutes the output
    rows bit for bit."""
    q, k, v = _inputs(1000, 1500, 4, 2, base=1014)
    qd, kd, vd = dev(q), dev(k), dev(v)
    full = mot.joint_attention(qd, kd, vd, 4, 2, causal=True)
    tail = mot.joint_attention(qd[700:].contiguous(), kd, vd, 4, 2, causal=True)
    torch.cuda.synchronize()
    assert np.array_equal(bits(full)[700:], bits(tail))
    perm = W.permutation(1000, 17).to("cuda")
    a = mot.joint_attention(qd, kd, vd, 4, 2, causal=False)
    b = mot.joint_attention(qd[perm].contiguous(), kd, vd, 4, 2, causal=False)
    torch.cuda.synchronize()
    assert np.array_equal(bits(a)[perm.cpu().numpy()], bits(b))


# ---- packed sequences ------------------------------------------------------------


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_varlen_small(causal):
    """Five packed sequences of ragged lengths (one with no rows, one with
    more keys than rows, one with more rows than keys): each row matches the
    oracle run on its own sequence, and has the bytes of its sequence run
    alone through the single-sequence call."""
    lq = [37, 0, 130, 64, 5]
    lk = [90, 20, 130, 30, 200]
    cq, ck = _cu(lq), _cu(lk)
    q, k, v = _inputs(int(cq[-1]), int(ck[-1]), 4, 2, base=1020 + causal, extra=64)
    got, ws = mot.joint_attention_varlen(dev(q), dev(k), dev(v), dev(torch.from_numpy(cq)),
                                         dev(torch.from_numpy(ck)), max(lq), 4, 2, causal=causal)
    assert mot.read_device_error(ws) == 0
    gb = bits(got)
    ref, rne = oracle.attention_varlen(W.bits(q), W.bits(k), W.bits(v), cq, ck, 4, 2, causal)
    check_parity(gb[:, :4 * D], ref, rne, f"attn varlen causal={causal}", one_step=False)
    for b in range(len(lq)):
        if lq[b] == 0:
            continue
        alone = mot.joint_attention(dev(q[cq[b]:cq[b + 1]]), dev(k[ck[b]:ck[b + 1]]), dev(v[ck[b]:ck[b + 1]]), 4, 2,
                                    causal=causal)
        torch.cuda.synchronize()
        assert np.array_equal(gb[cq[b]:cq[b + 1]], bits(alone)), b


def test_attention_varlen_cfg_pack_sampled():
    """The three-branch CFG pack as three requests and a prompt-only tail
    (28 q / 4 kv heads): the branches' rows never see each other, sampled
    rows against the oracle."""
    lq = [1101, 1101, 1101, 77, 77, 77, 562]
    cq = _cu(lq)
    T = int(cq[-1])
    q, k, v = _inputs(T, T, W.N_Q_HEADS, W.N_K_HEADS, base=1030)
    got, ws = mot.joint_attention_varlen(dev(q), dev(k), dev(v), dev(torch.from_numpy(cq)),
                                         dev(torch.from_numpy(cq)), max(lq), W.N_Q_HEADS, W.N_K_HEADS, causal=True)
    assert mot.read_device_error(ws) == 0
    gb = bits(got)
    for b in (0, 2, 5, 6):
        rows = np.unique(np.r_[0, lq[b] - 1, np.random.default_rng(20 + b).integers(0, lq[b], 4)])
        ref, rne = oracle.attention(W.bits(q)[cq[b]:cq[b + 1]], W.bits(k)[cq[b]:cq[b + 1]],
                                    W.bits(v)[cq[b]:cq[b + 1]], W.N_Q_HEADS, W.N_K_HEADS, True, rows=rows)
        check_parity(gb[cq[b] + rows], ref, rne, f"attn varlen cfg branch {b}", one_step=False)


def test_attention_varlen_gen_step_sampled():
    """One denoising step of the three-branch pack: every row of a branch
    sees all 1101 keys of its branch (no causal mask: the latent queries
    attend to the prompt and to each other), sampled rows against the oracle,
    and a branch's bytes equal its own single-sequence call."""
    lq = [1101, 1101, 1101]
    cq = _cu(lq)
    T = int(cq[-1])
    q, k, v = _inputs(T, T, W.N_Q_HEADS, W.N_K_HEADS, base=1040)
    got, ws = mot.joint_attention_varlen(dev(q), dev(k), dev(v), dev(torch.from_numpy(cq)),
                                         dev(torch.from_numpy(cq)), max(lq), W.N_Q_HEADS, W.N_K_HEADS, causal=False)
    assert mot.read_device_error(ws) == 0
    gb = bits(got)
    for b in range(3):
        rows = np.unique(np.r_[0, 76, 77, lq[b] - 1, np.random.default_rng(30 + b).integers(77, lq[b], 4)])
        ref, rne = oracle.attention(W.bits(q)[cq[b]:cq[b + 1]], W.bits(k)[cq[b]:cq[b + 1]],
                                    W.bits(v)[cq[b]:cq[b + 1]], W.N_Q_HEADS, W.N_K_HEADS, False, rows=rows)
        check_parity(gb[cq[b] + rows], ref, rne, f"attn gen step branch {b}", one_step=False)
    b = 1
    alone = mot.joint_attention(dev(q[cq[b]:cq[b + 1]]), dev(k[cq[b]:cq[b + 1]]), dev(v[cq[b]:cq[b + 1]]),
                                W.N_Q_HEADS, W.N_K_HEADS, causal=False)
    torch.cuda.synchronize()
    assert np.array_equal(gb[cq[b]:cq[b + 1]], bits(alone))


@pytest.mark.parametrize("bad", ["decreasing", "wrong_total", "too_long"])
def test_attention_varlen_rejects_bad_lengths(bad):
    """Lengths that break the rules raise MOT_ERR_SEQLENS on the device and
    leave the output untouched."""
    lq, lk = [40, 30], [50, 20]
    cq, ck = _cu(lq), _cu(lk)
    q, k, v = _inputs(70, 70, 2, 1, base=1040)
    max_q = 40
    if bad == "decreasing":
        cq = np.array([0, 50, 40, 70], np.int32)[[0, 1, 3]]
        cq[1] = 80  # 0, 80, 70: the second sequence has a negative length
    elif bad == "wrong_total":
        ck = np.array([0, 50, 69], np.int32)
    else:
        max_q = 30
    out = torch.full((70, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    _, ws = mot.joint_attention_varlen(dev(q), dev(k), dev(v), dev(torch.from_numpy(cq)), dev(torch.from_numpy(ck)),
                                       max_q, 2, 1, causal=True, out=out)
    assert mot.read_device_error(ws) == 8  # MOT_ERR_SEQLENS
    assert bool((out == 7.0).all())
