"""GPU parity of the routed backward (RFC page "[RFC][BAGEL-7B-MoT] WS1/WS2
kernel roadmap", section 1: Phase A trains only the generation expert; the
frozen understanding operators still need dX) against the CPU oracle.

dX = dY W_{m(t)} runs the forward's routed GEMM on transposed weights; the
generation set's dW = sum over gen rows of dY[t]^T X[t] runs it over the
tokens on transposed, masked operands (rows folded in ascending 16-row
chunks).  The transpose itself is pure data movement and is checked bit for
bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_transformers_token_amd as mot
import oracle
import workloads as W
from helpers import _abs_bits, bits, check_parity, dev, raw_equal

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("rows,cols,pad,masked", [(1, 8, 1, False), (77, 200, 128, True),
                                                  (300, 64, 320, False), (4096, 4608, 4096, True)])
def test_transpose_is_exact(rows, cols, pad, masked):
    x = W.normal_bf16((rows, cols), 500 + rows)
    m = W.pattern(rows)
    out = mot.transpose(dev(x), modality=dev(torch.from_numpy(m)) if masked else None, keep=1,
                        rows_pad=pad if pad >= rows else rows)
    torch.cuda.synchronize()
    want = x.clone()
    if masked:
        want[torch.from_numpy(m != 1)] = 0
    full = torch.zeros((cols, out.shape[1]), dtype=torch.bfloat16)
    full[:, :rows] = want.T
    assert raw_equal(out.cpu(), full)


def _dx_parity(T, N, K, m, base, rows=None):
    dy = W.normal_bf16((T, N), W.seed_of(base, 1))
    wu = W.normal_bf16((N, K), W.seed_of(base, 2), 0.02)
    wg = W.normal_bf16((N, K), W.seed_of(base, 3), 0.02)
    dx = mot.routed_gemm_dx(dev(dy), dev(wu), dev(wg), dev(torch.from_numpy(m)))
    torch.cuda.synchronize()
    sel = np.arange(T) if rows is None else rows
    args = (W.bits(dy)[sel], W.bits(wu), W.bits(wg), m[sel])
    ref, rne = oracle.routed_gemm_dx(*args)
    # fp32 sum of N products per element: N 2^-23 sum_n |dy||w|
    mag, _ = oracle.routed_gemm_dx(*(_abs_bits(a) for a in args[:3]), m[sel])
    check_parity(bits(dx)[sel], ref, rne, f"dX T={T} N={N} K={K}", bound=N * (2.0 ** -23 + 2.0 ** -52) * mag)


@pytest.mark.parametrize("T,N,K", [(1, 64, 64), (77, 128, 192), (333, 320, 256), (1101, 448, 320)])
def test_dx_small(T, N, K):
    m = W.pattern(T)
    m[::5] = 1 - m[::5]
    _dx_parity(T, N, K, m, base=510 + T)


def test_dx_qkv_shape_sampled():
    """dY [4096, 4608] (the QKV output's gradient) -> dX [4096, 3584]."""
    m = W.pattern(4096)
    _dx_parity(4096, W.QKV_DIM, W.HIDDEN, m, base=520, rows=W.sample_rows(m, 48, seed=4))


def _grad_parity(T, N, K, m, base, cols=None):
    dy = W.normal_bf16((T, N), W.seed_of(base, 1))
    x = W.normal_bf16((T, K), W.seed_of(base, 4))
    dw = mot.grad_w(dev(dy), dev(x), dev(torch.from_numpy(m)), keep=1)
    torch.cuda.synchronize()
    sel = np.arange(N) if cols is None else cols
    # dW[n] depends on column n of dY only: the oracle on sampled columns is
    # the exact restriction
    dys = np.ascontiguousarray(W.bits(dy)[:, sel])
    ref, rne = oracle.grad_w(dys, W.bits(x), m, keep=1)
    # fp32 fold over the (padded) rows: at most 64 * ceil(T / 64) additions
    mag, _ = oracle.grad_w(_abs_bits(dys), _abs_bits(W.bits(x)), m, keep=1)
    nadd = 64 * ((T + 63) // 64)
    check_parity(bits(dw)[sel], ref, rne, f"dW_gen T={T} N={N} K={K}", bound=nadd * (2.0 ** -23 + 2.0 ** -52) * mag)


@pytest.mark.parametrize("T,N,K", [(1, 64, 64), (100, 128, 64), (333, 192, 256), (1101, 256, 128)])
def test_grad_w_small(T, N, K):
    m = W.pattern(T)
    m[::4] = 1 - m[::4]
    _grad_parity(T, N, K, m, base=530 + T)


def test_grad_w_qkv_shape_sampled():
    """The generation set's QKV weight gradient, dW [4608, 3584] over the
    3788 gen rows of the 4096-row BAGEL pack, on sampled output rows."""
    m = W.pattern(4096)
    cols = np.random.default_rng(6).choice(W.QKV_DIM, 24, replace=False)
    _grad_parity(4096, W.QKV_DIM, W.HIDDEN, m, base=540, cols=np.sort(cols))


@pytest.mark.parametrize("T,N,K", [(1, 64, 64), (77, 128, 192), (300, 320, 256), (1101, 448, 320),
                                   (4096, 4608, 3584), (9000, 256, 192)])
def test_dx_weights_as_they_lie_equal_the_transposed_product(T, N, K):
    """mot_routed_gemm_dx reads the forward's [N, K] weights where they lie
    (contraction-major weight stages, transposing LDS reads) and gives, bit
    for bit, the routed GEMM's bytes on the transposed weights, whatever
    tile shapes that call picks (256 x 256 big tiles here, small tiles or the
    small-pack kernel there): same MFMA chain, same k order.  T = 9000 takes
    the segment list from the plan kernel instead of building it in-kernel."""
    base = 600 + T
    dy = dev(W.normal_bf16((T, N), W.seed_of(base, 1)))
    wu = dev(W.normal_bf16((N, K), W.seed_of(base, 2), 0.02))
    wg = dev(W.normal_bf16((N, K), W.seed_of(base, 3), 0.02))
    m = W.pattern(T)
    m[::5] = 1 - m[::5]
    md = dev(torch.from_numpy(m))
    got = mot.routed_gemm_dx(dy, wu, wg, md)
    want = mot.routed_gemm_dx(dy, wu, wg, md, wt=(mot.transpose(wu), mot.transpose(wg)))
    torch.cuda.synchronize()
    assert raw_equal(got, want), f"T={T} N={N} K={K}"


def test_dx_weights_as_they_lie_plan_ready_and_bad_bytes():
    """The ready-plan form gives the same bytes; an invalid modality byte
    makes the call write nothing and raises the error word."""
    T, N, K = 500, 256, 192
    dy = dev(W.normal_bf16((T, N), 620))
    wu = dev(W.normal_bf16((N, K), 621, 0.02))
    wg = dev(W.normal_bf16((N, K), 622, 0.02))
    md = dev(torch.from_numpy(W.pattern(T)))
    ws = mot.new_workspace(T, dy.device)
    mot.routing_plan(md, workspace=ws)
    a = mot.routed_gemm_dx(dy, wu, wg, md, workspace=ws, plan_ready=True)
    b = mot.routed_gemm_dx(dy, wu, wg, md)
    torch.cuda.synchronize()
    assert raw_equal(a, b)
    bad = W.pattern(T)
    bad[123] = 7
    out = torch.full((T, K), 3.0, dtype=torch.bfloat16, device="cuda")
    ws2 = mot.new_workspace(T, dy.device)
    mot.routed_gemm_dx(dy, wu, wg, dev(torch.from_numpy(bad)), out=out, workspace=ws2)
    assert mot.read_device_error(ws2) == 6  # MOT_ERR_MODALITY
    assert bool((out == 3.0).all())


def _grad_w_transposed(dy, x, m, keep, f32):
    """The same weight gradient as a routed GEMM over the tokens, on
    transposed copies (x's other-set rows zeroed, both padded to 64 rows)."""
    T, N = dy.shape
    Tp = max(64, (T + 63) // 64 * 64)
    dyt = mot.transpose(dy, rows_pad=Tp)
    xt = mot.transpose(x, modality=m, keep=keep, rows_pad=Tp)
    sets = torch.zeros(N, dtype=torch.uint8, device=dy.device)
    return (mot.routed_gemm_f32 if f32 else mot.routed_gemm)(dyt, xt, xt, sets)


@pytest.mark.parametrize("T,N,K,keep,pitch", [(0, 64, 64, 1, 0), (1, 64, 64, 1, 0), (63, 200, 64, 1, 8),
                                              (100, 256, 320, 0, 0), (333, 300, 256, 1, 4),
                                              (1101, 520, 192, 1, 0), (4096, 4608, 3584, 1, 0)])
@pytest.mark.parametrize("f32", [False, True])
def test_grad_w_is_the_transposed_product(T, N, K, keep, pitch, f32):
    """mot_grad_w reads dY and X where they lie (token-major tiles, transposing
    LDS reads) and gives, bit for bit, the routed GEMM's bytes on their
    transposes: the same 16-row MFMA steps in the same order, the other
    set's rows zero.  Ragged row counts, padded row pitches, keep = 0 and
    invalid modality bytes (dropped like the other set's rows) included."""
    base = 560 + T + N
    dyb = W.normal_bf16((T, N + pitch), W.seed_of(base, 1))
    x = W.normal_bf16((T, K), W.seed_of(base, 4))
    m = W.pattern(T) if T else np.zeros(0, np.uint8)
    if T > 7:
        m[3::7] = 9  # neither set: dropped by both forms
    dy_d, x_d, m_d = dev(dyb)[:, :N], dev(x), dev(torch.from_numpy(m))
    got = mot.grad_w(dy_d, x_d, m_d, keep=keep, out_dtype=torch.float32 if f32 else torch.bfloat16)
    want = _grad_w_transposed(dy_d, x_d, m_d, keep, f32)
    torch.cuda.synchronize()
    assert tuple(got.shape) == (N, K)
    view = torch.int32 if f32 else torch.int16
    assert torch.equal(got.view(view), want.view(view)), f"T={T} N={N} K={K} keep={keep} f32={f32}"


def test_dx_rows_batch_invariant():
    """dX runs the forward's routed GEMM: a row's bytes do not depend on the
    pack around it (probe rows alone, inside a larger mixed pack, permuted)."""
    N, K = 512, 384
    wu = dev(W.normal_bf16((N, K), 550, 0.02))
    wg = dev(W.normal_bf16((N, K), 551, 0.02))
    wt = (mot.transpose(wu), mot.transpose(wg))
    probe = W.normal_bf16((200, N), 552)
    pm = W.pattern(200)
    ref = mot.routed_gemm_dx(dev(probe), wu, wg, dev(torch.from_numpy(pm)), wt=wt)
    fill = W.normal_bf16((900, N), 553)
    fm = np.random.default_rng(9).integers(0, 2, 900).astype(np.uint8)
    dy = torch.cat([fill[:450], probe, fill[450:]])
    m = np.concatenate([fm[:450], pm, fm[450:]])
    perm = W.permutation(dy.shape[0], 10).numpy()
    out = mot.routed_gemm_dx(dev(dy[perm]), wu, wg, dev(torch.from_numpy(m[perm])), wt=wt)
    pos = np.empty(perm.size, np.int64)
    pos[perm] = np.arange(perm.size)
    got = out[torch.from_numpy(pos[450:650]).cuda()]
    torch.cuda.synchronize()
    assert raw_equal(got, ref)
