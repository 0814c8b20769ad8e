"""The QKV projection with the per-head QK RMSNorm and rotary embedding fused
into its epilogue (mot_routed_gemm_qk_norm_rope), through the C ABI: its bytes
equal the two-kernel path (mot_routed_gemm, then mot_qk_norm_rope on its
rows) bit for bit in every launch shape, it meets the gate against the
oracle's own chain (GEMM, then QK norm + rotary on the oracle's bf16 GEMM
output), rows with a bad position keep the GEMM's bytes, and a row's bytes do
not depend on the pack (RL-Kernel RFC page, sections 3 and 5)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_transformers_token_amd as mot
import oracle
import workloads as W
from helpers import bits, check_parity, dev, raw_equal

pytestmark = pytest.mark.gpu

HQ, HK = W.N_Q_HEADS, W.N_K_HEADS


def _inputs(T, K, N, base, m=None):
    if m is None:
        m = W.pattern(T)
        m[::7] = 1 - m[::7]
    x = W.normal_bf16((T, K), W.seed_of(base, 1))
    wu = W.normal_bf16((N, K), W.seed_of(base, 2), 0.02)
    wg = W.normal_bf16((N, K), W.seed_of(base, 3), 0.02)
    qn, kn = W.qk_norm_weights(base=base)
    cos_t, sin_t, pos = W.rope_inputs(T, 4096, base=base)
    return m, x, wu, wg, qn, kn, cos_t, sin_t, pos


def _two_kernel(m, x, wu, wg, qn, kn, cos_t, sin_t, pos, hq, hk, tile=None):
    md = dev(torch.from_numpy(m))
    y = mot.routed_gemm(dev(x), dev(wu), dev(wg), md, tile=tile)
    ws = mot.new_workspace(0, "cuda")
    mot.qk_norm_rope(y, hq, hk, md, tuple(dev(t) for t in qn), tuple(dev(t) for t in kn), dev(pos), dev(cos_t),
                     dev(sin_t), workspace=ws)
    return y, mot.read_device_error(ws)


def _fused(m, x, wu, wg, qn, kn, cos_t, sin_t, pos, hq, hk, tile=None, out=None):
    ws = mot.new_workspace(x.shape[0], "cuda")
    y = mot.routed_gemm_qk_norm_rope(dev(x), dev(wu), dev(wg), dev(torch.from_numpy(m)), hq, hk,
                                     tuple(dev(t) for t in qn), tuple(dev(t) for t in kn), dev(pos), dev(cos_t),
                                     dev(sin_t), out=out, workspace=ws, tile=tile)
    return y, mot.read_device_error(ws)


@pytest.mark.parametrize("T", [1, 40, 64, 65, 128, 129, 200, 1101, 4096, 9001])
def test_fused_equals_two_kernel_path(T):
    """Packs of at most 128 rows (the small-pack GEMM, then the QK kernel),
    mid-size packs (128 x 128 tiles), 256 x 256 tiles with a partial round,
    and a pack above the in-kernel segment list's limit (plan kernel)."""
    args = _inputs(T, 512 if T != 4096 else W.HIDDEN, W.QKV_DIM, base=700 + T)
    ref, e_ref = _two_kernel(*args, HQ, HK)
    got, e_got = _fused(*args, HQ, HK)
    torch.cuda.synchronize()
    assert e_ref == 0 and e_got == 0
    assert raw_equal(got, ref), f"T={T}: {int((got.view(torch.int16) != ref.view(torch.int16)).sum())} elements differ"


@pytest.mark.parametrize("tile", ["256x256", "128x128"])
@pytest.mark.parametrize("T", [77, 1101])
def test_fused_forced_tiles(T, tile):
    args = _inputs(T, 320, W.QKV_DIM, base=720 + T)
    ref, _ = _two_kernel(*args, HQ, HK, tile=tile)
    got, _ = _fused(*args, HQ, HK, tile=tile)
    torch.cuda.synchronize()
    assert raw_equal(got, ref)


@pytest.mark.parametrize("hq,hk,N", [(3, 1, 640), (2, 1, 448), (1, 0, 128), (5, 2, 1024)])
def test_fused_other_head_layouts(hq, hk, N):
    """An odd head count (a 256-column tile holding a q/k head and a v head),
    a last head cut at a 64-column edge, q heads only, and a wider v part."""
    T = 333
    args = _inputs(T, 256, N, base=740 + N)
    ref, _ = _two_kernel(*args, hq, hk)
    got, _ = _fused(*args, hq, hk)
    torch.cuda.synchronize()
    assert raw_equal(got, ref)


def test_fused_qkv_full_size_against_oracle():
    """The BAGEL QKV shape (T=4096, K=3584, 28 q + 4 k heads + v) on sampled
    rows, against the oracle's GEMM followed by its QK norm + rotary on its
    own bf16 GEMM output (a two-step chain: held to the gate)."""
    T = 4096
    x, wu, wg, m = W.qkv(T)
    qn, kn = W.qk_norm_weights(base=760)
    cos_t, sin_t, pos = W.rope_inputs(T, 4096, base=760)
    got, err = _fused(m, x, wu, wg, qn, kn, cos_t, sin_t, pos, HQ, HK)
    assert err == 0
    rows = W.sample_rows(m, 32, seed=15)
    _, y_or = oracle.routed_gemm(W.bits(x)[rows], W.bits(wu), W.bits(wg), m[rows])
    ref, out, e_or = oracle.qk_norm_rope(y_or, HQ, HK, m[rows], tuple(W.bits(t) for t in qn),
                                         tuple(W.bits(t) for t in kn), pos.numpy()[rows], W.bits(cos_t), W.bits(sin_t))
    assert e_or == 0
    cols = 128 * (HQ + HK)
    g = bits(got)[rows]
    check_parity(g[:, :cols], ref[:, :cols], out[:, :cols], "fused QKV + QK norm/rotary", one_step=False)
    # the v columns are the GEMM's own output
    ref_v, rne_v = oracle.routed_gemm(W.bits(x)[rows], W.bits(wu)[cols:], W.bits(wg)[cols:], m[rows])
    from helpers import gemm_bound
    check_parity(g[:, cols:], ref_v, rne_v, "fused QKV: v columns",
                 bound=gemm_bound(W.bits(x)[rows], W.bits(wu)[cols:], W.bits(wg)[cols:], m[rows]))


def test_fused_bad_positions_and_bytes():
    """Rows whose position lies outside the table keep the GEMM's bytes (as
    the two-kernel path leaves them) and raise MOT_ERR_POSITION; an invalid
    modality byte writes nothing and raises MOT_ERR_MODALITY."""
    T = 1101
    m, x, wu, wg, qn, kn, cos_t, sin_t, pos = _inputs(T, 256, W.QKV_DIM, base=780)
    pos = pos.clone()
    pos[5] = 4096
    pos[700] = -3
    ref, e_ref = _two_kernel(m, x, wu, wg, qn, kn, cos_t, sin_t, pos, HQ, HK)
    got, e_got = _fused(m, x, wu, wg, qn, kn, cos_t, sin_t, pos, HQ, HK)
    torch.cuda.synchronize()
    assert e_ref == e_got == 7
    assert raw_equal(got, ref)
    m_bad = m.copy()
    m_bad[17] = 3
    out = torch.full((T, W.QKV_DIM), 5.0, dtype=torch.bfloat16, device="cuda")
    _, e = _fused(m_bad, x, wu, wg, qn, kn, cos_t, sin_t, W.rope_inputs(T, 4096, base=780)[2], HQ, HK, out=out)
    assert e == 6 and torch.all(out == 5.0)
    # a small pack takes the small-pack GEMM then the QK kernel: same rules
    ms = m[:40].copy()
    ms[3] = 9
    out = torch.full((40, W.QKV_DIM), 5.0, dtype=torch.bfloat16, device="cuda")
    _, e = _fused(ms, x[:40], wu, wg, qn, kn, cos_t, sin_t, W.rope_inputs(40, 4096, base=780)[2], HQ, HK, out=out)
    assert e == 6 and torch.all(out == 5.0)


def test_fused_rows_invariant_across_packs():
    """The probe rows' bytes are the same alone, inside a larger pack and
    permuted."""
    Tp, Tf = 1024, 2048
    m_all, x, wu, wg, qn, kn, cos_t, sin_t, pos = _inputs(Tp + Tf, 512, W.QKV_DIM, base=790)
    probe = _fused(m_all[:Tp].copy(), x[:Tp], wu, wg, qn, kn, cos_t, sin_t, pos[:Tp], HQ, HK)[0]
    perm = W.permutation(Tp + Tf, 7).numpy()
    full = _fused(m_all[perm].copy(), x[perm], wu, wg, qn, kn, cos_t, sin_t, pos[perm], HQ, HK)[0]
    where = np.empty(Tp + Tf, np.int64)
    where[perm] = np.arange(Tp + Tf)
    torch.cuda.synchronize()
    assert raw_equal(full[torch.from_numpy(where[:Tp]).cuda()], probe)
