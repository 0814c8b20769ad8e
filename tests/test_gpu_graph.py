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
    """Both attention calls (V transpose + attention; the packed form with
    its lengths check and packed V transpose) replay to the eager bytes."""
    T = 700
    qkv = dev(W.normal_bf16((T, W.QKV_DIM), 1320))
    q, k, v = qkv[:, :W.Q_DIM], qkv[:, W.Q_DIM:W.Q_DIM + W.KV_DIM], qkv[:, W.Q_DIM + W.KV_DIM:]
    ref = mot.joint_attention(q, k, v, W.N_Q_HEADS, W.N_K_HEADS, causal=True)
    out = torch.empty_like(ref)
    ws = torch.empty(mot.attention_workspace_bytes(T, W.N_K_HEADS), dtype=torch.uint8, device="cuda")
    _replays_match(lambda: mot.joint_attention(q, k, v, W.N_Q_HEADS, W.N_K_HEADS, causal=True, out=out,
                                               workspace=ws), out, ref)
    cu = dev(torch.from_numpy(W.cu_lengths([300, 0, 77, 323])))
    ref2, _ = mot.joint_attention_varlen(q, k, v, cu, cu, 323, W.N_Q_HEADS, W.N_K_HEADS, causal=True)
    out2 = torch.empty_like(ref2)
    ws2 = torch.empty(mot.attention_varlen_workspace_bytes(T, 4, W.N_K_HEADS), dtype=torch.uint8, device="cuda")
    _replays_match(lambda: mot.joint_attention_varlen(q, k, v, cu, cu, 323, W.N_Q_HEADS, W.N_K_HEADS, causal=True,
                                                      out=out2, workspace=ws2), out2, ref2)
    assert mot.read_device_error(ws2) == 0
