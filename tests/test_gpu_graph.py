"""The library's calls captured in a HIP graph (through torch.cuda.graph) and
replayed: every replay, with eager work and synchronisation between them,
gives the eager result bit for bit.  The calls allocate nothing and record
no memset, so their kernels are plain graph nodes."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_transformers_token_amd as mot
import workloads as W
from helpers import dev, raw_equal

pytestmark = pytest.mark.gpu


def _replays_match(run, out, ref, n=3):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()
    for i in range(n):
        out.fill_(float(i + 3))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert raw_equal(out, ref), f"replay {i} differs from the eager result"


@pytest.mark.parametrize("T", [8, 200, 4096])
def test_routed_gemm_graph(T):
    m = W.pattern(T)
    x, wu, wg, _ = W.gemm_case(T, W.HIDDEN, W.QKV_DIM, m, base=1200 + T)
    xd, wud, wgd, md = dev(x), dev(wu), dev(wg), dev(torch.from_numpy(m))
    ref = mot.routed_gemm(xd, wud, wgd, md)
    out = torch.empty_like(ref)
    ws = mot.new_workspace(T, xd.device)
    _replays_match(lambda: mot.routed_gemm(xd, wud, wgd, md, out=out, workspace=ws), out, ref)


def test_swiglu_graph():
    T, K, F = 300, 512, 1024
    m = W.pattern(T)
    x = dev(W.normal_bf16((T, K), 1301))
    wu = dev(W.normal_bf16((2 * F, K), 1302, 0.05))
    wg = dev(W.normal_bf16((2 * F, K), 1303, 0.05))
    md = dev(torch.from_numpy(m))
    ref = mot.routed_gemm_swiglu(x, wu, wg, md)
    out = torch.empty_like(ref)
    ws = mot.new_workspace(T, x.device)
    _replays_match(lambda: mot.routed_gemm_swiglu(x, wu, wg, md, out=out, workspace=ws), out, ref)


@pytest.mark.parametrize("f32", [False, True])
def test_backward_graph(f32):
    """dX with the weights as they lie and dW over token-major operands
    replay to the eager bytes."""
    T, N, K = 700, 512, 384
    m = W.pattern(T)
    dy = dev(W.normal_bf16((T, N), 1340))
    x = dev(W.normal_bf16((T, K), 1341))
    wu = dev(W.normal_bf16((N, K), 1342, 0.05))
    wg = dev(W.normal_bf16((N, K), 1343, 0.05))
    md = dev(torch.from_numpy(m))
    ref = mot.routed_gemm_dx(dy, wu, wg, md)
    out = torch.empty_like(ref)
    ws = mot.new_workspace(T, dy.device)
    _replays_match(lambda: mot.routed_gemm_dx(dy, wu, wg, md, out=out, workspace=ws), out, ref)
    dt = torch.float32 if f32 else torch.bfloat16
    ref_w = mot.grad_w(dy, x, md, keep=1, out_dtype=dt)
    out_w = torch.empty_like(ref_w)
    _replays_match(lambda: mot.grad_w(dy, x, md, keep=1, out_dtype=dt, out=out_w), out_w, ref_w)


def test_qk_norm_rope_graph():
    """The in-place op, captured with the copy that restores its input."""
    T = 512
    qkv0 = dev(W.normal_bf16((T, W.QKV_DIM), 1311, 1.2))
    m = dev(torch.from_numpy(W.pattern(T)))
    qn, kn = W.qk_norm_weights(base=1312)
    qn, kn = tuple(dev(t) for t in qn), tuple(dev(t) for t in kn)
    c, s, pos = (dev(t) for t in W.rope_inputs(T, 1024, base=1312))
    ws = mot.new_workspace(0, qkv0.device)
    ref = qkv0.clone()
    mot.qk_norm_rope(ref, W.N_Q_HEADS, W.N_K_HEADS, m, qn, kn, pos, c, s, workspace=ws)
    assert mot.read_device_error(ws) == 0
    buf = torch.empty_like(qkv0)

    def run():
        buf.copy_(qkv0)
        mot.qk_norm_rope(buf, W.N_Q_HEADS, W.N_K_HEADS, m, qn, kn, pos, c, s, workspace=ws)

    _replays_match(run, buf, ref)
    assert mot.read_device_error(ws) == 0


def test_joint_attention_graph():
    """Both attention calls (the packed form with its lengths check) replay
    to the eager bytes."""
    T = 700
    qkv = dev(W.normal_bf16((T, W.QKV_DIM), 1320))
    q, k, v = qkv[:, :W.Q_DIM], qkv[:, W.Q_DIM:W.Q_DIM + W.KV_DIM], qkv[:, W.Q_DIM + W.KV_DIM:]
    ref = mot.joint_attention(q, k, v, W.N_Q_HEADS, W.N_K_HEADS, causal=True)
    out = torch.empty_like(ref)
    _replays_match(lambda: mot.joint_attention(q, k, v, W.N_Q_HEADS, W.N_K_HEADS, causal=True, out=out), out, ref)
    cu = dev(torch.from_numpy(W.cu_lengths([300, 0, 77, 323])))
    ref2, _ = mot.joint_attention_varlen(q, k, v, cu, cu, 323, W.N_Q_HEADS, W.N_K_HEADS, causal=True)
    out2 = torch.empty_like(ref2)
    ws2 = torch.empty(mot.attention_varlen_workspace_bytes(T, 4, W.N_K_HEADS), dtype=torch.uint8, device="cuda")
    _replays_match(lambda: mot.joint_attention_varlen(q, k, v, cu, cu, 323, W.N_Q_HEADS, W.N_K_HEADS, causal=True,
                                                      out=out2, workspace=ws2), out2, ref2)
    assert mot.read_device_error(ws2) == 0


def test_fused_qk_and_wide_gemm_graph():
    """The QKV GEMM with the QK norm + rotary epilogue (its error-word clear
    is a kernel, not a memset), and a down-shaped GEMM that runs 256 x 224
    tiles on a pack of whole row blocks."""
    T = 1024
    m = np.concatenate([np.zeros(256, np.uint8), np.ones(768, np.uint8)])
    x = dev(W.normal_bf16((T, 512), 1401))
    wu, wg = dev(W.normal_bf16((W.QKV_DIM, 512), 1402, 0.02)), dev(W.normal_bf16((W.QKV_DIM, 512), 1403, 0.02))
    md = dev(torch.from_numpy(m))
    qn, kn = W.qk_norm_weights(base=1404)
    qn, kn = tuple(dev(t) for t in qn), tuple(dev(t) for t in kn)
    c, s, pos = (dev(t) for t in W.rope_inputs(T, 2048, base=1404))
    ref = mot.routed_gemm_qk_norm_rope(x, wu, wg, md, W.N_Q_HEADS, W.N_K_HEADS, qn, kn, pos, c, s)
    out = torch.empty_like(ref)
    ws = mot.new_workspace(T, x.device)
    _replays_match(lambda: mot.routed_gemm_qk_norm_rope(x, wu, wg, md, W.N_Q_HEADS, W.N_K_HEADS, qn, kn, pos, c,
                                                         s, out=out, workspace=ws), out, ref)
    assert mot.read_device_error(ws) == 0
    T2 = 4096
    m2 = np.concatenate([np.zeros(1024, np.uint8), np.ones(3072, np.uint8)])
    x2 = dev(W.normal_bf16((T2, 256), 1405))
    du, dg = dev(W.normal_bf16((3584, 256), 1406, 0.02)), dev(W.normal_bf16((3584, 256), 1407, 0.02))
    md2 = dev(torch.from_numpy(m2))
    ref2 = mot.routed_gemm(x2, du, dg, md2)
    out2 = torch.empty_like(ref2)
    ws2 = mot.new_workspace(T2, x2.device)
    _replays_match(lambda: mot.routed_gemm(x2, du, dg, md2, out=out2, workspace=ws2), out2, ref2)


def test_noalloc_and_index_sets_graph():
    """The allocation-free GEMM (its scratch is the library's) and the
    index-set conversion, captured together."""
    T = 300
    m = W.pattern(T)
    und = dev(torch.from_numpy(np.flatnonzero(m == 0).astype(np.int32)[::-1].copy()))
    gen = dev(torch.from_numpy(np.flatnonzero(m == 1).astype(np.int32)))
    x = dev(W.normal_bf16((T, 256), 1411))
    wu, wg = dev(W.normal_bf16((384, 256), 1412, 0.02)), dev(W.normal_bf16((384, 256), 1413, 0.02))
    md = torch.empty(T, dtype=torch.uint8, device="cuda")
    wsi = mot.new_workspace(T, x.device)
    mot.modality_from_index_sets(und, gen, T, out=md, workspace=wsi)
    ref = mot.routed_gemm(x, wu, wg, md)
    out = torch.empty_like(ref)

    def run():
        mot.modality_from_index_sets(und, gen, T, out=md, workspace=wsi)
        mot.routed_gemm_noalloc(x, wu, wg, md, out)

    _replays_match(run, out, ref)
    assert mot.read_device_error(wsi) == 0


def test_latent_step_graph():
    """The CFG combine and the SDE step (their check kernels clear the error
    word), captured and replayed."""
    C, lens = 64, [300, 0, 77]
    cu = dev(torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32))
    rows = int(sum(lens))
    g = torch.Generator().manual_seed(9)
    vc, vt, vi, xl, z = (dev(torch.randn((rows, C), generator=g)) for _ in range(5))
    t = dev(torch.tensor([0.7, 0.5, 1.0], dtype=torch.float32))
    tn = dev(torch.tensor([0.6, 0.4, 0.95], dtype=torch.float32))
    ref, _ = mot.cfg_combine_renorm(vc, vt, vi, cu, 300, t, 4.0, 1.5, 0.0, 1.0, 0.2, "global")
    xref, lref, _ = mot.flow_sde_step_logp(xl, ref, cu, 300, t, tn, 0.7, noise=z)
    out = torch.empty_like(ref)
    xo = torch.empty_like(xref)
    lp = torch.empty_like(lref)
    ws = torch.zeros(mot.latent_workspace_bytes(3, 300), dtype=torch.uint8, device="cuda")
    both = torch.empty((rows * C + rows * C + 3,), dtype=torch.float32, device="cuda")
    refs = torch.cat([ref.view(-1), xref.view(-1), lref.view(-1)])

    def run():
        mot.cfg_combine_renorm(vc, vt, vi, cu, 300, t, 4.0, 1.5, 0.0, 1.0, 0.2, "global", out=out, workspace=ws)
        mot.flow_sde_step_logp(xl, out, cu, 300, t, tn, 0.7, noise=z, out=xo, logp=lp, workspace=ws)
        torch.cat([out.view(-1), xo.view(-1), lp.view(-1)], out=both)

    _replays_match(run, both, refs)
    assert mot.read_device_error(ws) == 0
