"""Empty inputs through the C ABI: every entry point accepts a pack of zero
rows (or requests of zero rows) as a no-op that writes nothing and leaves
the error word clear, the degenerate case of each operation."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_transformers_token_amd as mot
import workloads as W
from helpers import dev

pytestmark = pytest.mark.gpu


def _e(shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype, device="cuda")


def test_routed_calls_on_an_empty_pack():
    K, N, F = 256, 384, 128
    x, md = _e((0, K)), _e((0,), torch.uint8)
    wu, wg = dev(W.normal_bf16((N, K), 1, 0.02)), dev(W.normal_bf16((N, K), 2, 0.02))
    ws = mot.new_workspace(0, "cuda")
    y = mot.routed_gemm(x, wu, wg, md, workspace=ws)
    assert tuple(y.shape) == (0, N) and mot.read_device_error(ws) == 0
    gu, gg = dev(W.normal_bf16((2 * F, K), 3, 0.02)), dev(W.normal_bf16((2 * F, K), 4, 0.02))
    a = mot.routed_gemm_swiglu(x, gu, gg, md, workspace=ws)
    assert tuple(a.shape) == (0, F) and mot.read_device_error(ws) == 0
    y0 = mot.routed_gemm_noalloc(x, wu, wg, md, _e((0, N)))
    assert tuple(y0.shape) == (0, N)
    nwu, nwg = (dev(t) for t in W.norm_weights(K))
    out, rstd = mot.fused_add_rmsnorm(x, _e((0, K)), nwu, nwg, md)
    assert tuple(out.shape) == (0, K) and tuple(rstd.shape) == (0,)
    torch.cuda.synchronize()


def test_qk_steps_on_an_empty_pack():
    hq, hk = 2, 1
    N = 128 * (hq + hk) + 128
    qn, kn = W.qk_norm_weights()
    qn, kn = tuple(dev(t) for t in qn), tuple(dev(t) for t in kn)
    cos_t, sin_t, _ = W.rope_inputs(1, 16)
    pos, md = _e((0,), torch.int32), _e((0,), torch.uint8)
    ws = mot.new_workspace(0, "cuda")
    mot.qk_norm_rope(_e((0, N)), hq, hk, md, qn, kn, pos, dev(cos_t), dev(sin_t), workspace=ws)
    assert mot.read_device_error(ws) == 0
    wu, wg = dev(W.normal_bf16((N, 256), 5, 0.02)), dev(W.normal_bf16((N, 256), 6, 0.02))
    y = mot.routed_gemm_qk_norm_rope(_e((0, 256)), wu, wg, md, hq, hk, qn, kn, pos, dev(cos_t), dev(sin_t),
                                     workspace=ws)
    assert tuple(y.shape) == (0, N) and mot.read_device_error(ws) == 0
    torch.cuda.synchronize()


def test_index_sets_of_an_empty_pack():
    m, ws = mot.modality_from_index_sets(_e((0,), torch.int32), _e((0,), torch.int32), 0)
    assert m.numel() == 0 and mot.read_device_error(ws) == 0


def test_latent_step_with_empty_requests():
    C = 64
    rows = 5
    cu = dev(torch.tensor([0, 0, rows, rows], dtype=torch.int32))  # requests 0 and 2 are empty
    g = torch.Generator().manual_seed(3)
    vc, vt, vi, x, z = (dev(torch.randn((rows, C), generator=g)) for _ in range(5))
    t = dev(torch.tensor([0.5, 0.5, 0.5], dtype=torch.float32))
    out, ws = mot.cfg_combine_renorm(vc, vt, vi, cu, rows, t, 4.0, 1.5, 0.0, 1.0, 0.2, "global")
    assert mot.read_device_error(ws) == 0 and torch.isfinite(out).all()
    tn = dev(torch.tensor([0.4, 0.4, 0.4], dtype=torch.float32))
    xn, lp, ws2 = mot.flow_sde_step_logp(x, vc, cu, rows, t, tn, 1.0, noise=z)
    assert mot.read_device_error(ws2) == 0
    lpc = lp.cpu().numpy()
    assert lpc[0] == 0.0 and lpc[2] == 0.0 and np.isfinite(lpc[1])
    # no rows at all: one empty request (max_rows >= 1 by contract)
    cu0 = dev(torch.tensor([0, 0], dtype=torch.int32))
    e = _e((0, C), torch.float32)
    out0, ws3 = mot.cfg_combine_renorm(e, e, None, cu0, 1, t[:1], 4.0, 1.5, 0.0, 1.0, 0.2, "global")
    assert out0.numel() == 0 and mot.read_device_error(ws3) == 0
    _, lp0, ws4 = mot.flow_sde_step_logp(e, e, cu0, 1, t[:1], tn[:1], 1.0, noise=e)
    assert mot.read_device_error(ws4) == 0 and float(lp0.cpu()[0]) == 0.0
