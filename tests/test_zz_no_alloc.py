"""The allocation-free routed GEMM (mot_routed_gemm_noalloc), through the C
ABI: for callers that cannot allocate, its scratch is the library's per-GPU
static array.  Its output must be mot_routed_gemm's, bit for bit, call after
call on the same GPU (the second call smaller than the first, so stale
scratch contents from the larger call would show)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import mixture_transformers_token_amd as mot
import workloads as W
from helpers import dev, raw_equal

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p


def _noalloc(x, wu, wg, md, y, err, flags=0):
    T, K = x.shape
    N = wu.shape[0]
    return mot.lib().mot_routed_gemm_noalloc(
        P(x.data_ptr()), x.stride(0), P(wu.data_ptr()), P(wg.data_ptr()), P(md.data_ptr()), P(y.data_ptr()),
        y.stride(0), T, K, N, None, None, None, P(err.data_ptr()) if err is not None else None, flags,
        P(torch.cuda.current_stream().cuda_stream))


def _case(T, K, N, base, bad_row=None):
    m = W.pattern(T)
    m[::5] = 1 - m[::5]
    if bad_row is not None:
        m[bad_row] = 7
    x, wu, wg, _ = W.gemm_case(T, K, N, np.where(m > 1, 0, m).astype(np.uint8), base=base)
    return dev(x), dev(wu), dev(wg), dev(torch.from_numpy(m))


@pytest.mark.parametrize("sizes", [(4096, 1101), (9000, 40), (64, 1), (65536, 300)])
def test_noalloc_matches_routed_gemm_twice(sizes):
    K, N = 256, 320
    err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    for i, T in enumerate(sizes):
        x, wu, wg, md = _case(T, K, N, base=2000 + T + i)
        want = mot.routed_gemm(x, wu, wg, md)
        y = torch.full((T, N), 3.0, dtype=torch.bfloat16, device="cuda")
        assert _noalloc(x, wu, wg, md, y, err) == 0
        torch.cuda.synchronize()
        assert raw_equal(y, want), (sizes, T)
        assert int(err.item()) == 0


def test_noalloc_qkv_shape_then_smaller():
    x, wu, wg, m = W.qkv(4096)
    md = dev(torch.from_numpy(m))
    xd, wud, wgd = dev(x), dev(wu), dev(wg)
    want = mot.routed_gemm(xd, wud, wgd, md)
    y = torch.empty_like(want)
    assert _noalloc(xd, wud, wgd, md, y, None) == 0
    torch.cuda.synchronize()
    assert raw_equal(y, want)
    rows = np.arange(0, 4096, 3)
    md2 = dev(torch.from_numpy(m[rows].copy()))
    y2 = torch.empty((rows.size, wu.shape[0]), dtype=torch.bfloat16, device="cuda")
    assert _noalloc(xd[torch.from_numpy(rows).cuda()].contiguous(), wud, wgd, md2, y2, None) == 0
    torch.cuda.synchronize()
    assert raw_equal(y2, want[torch.from_numpy(rows).cuda()])


def test_noalloc_reports_bad_bytes_and_limits():
    K, N = 128, 128
    x, wu, wg, md = _case(500, K, N, base=2100, bad_row=123)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = torch.full((500, N), 3.0, dtype=torch.bfloat16, device="cuda")
    assert _noalloc(x, wu, wg, md, y, err) == 0
    torch.cuda.synchronize()
    assert int(err.item()) == 6 and torch.all(y == 3.0)
    # the next good call reports no error
    x, wu, wg, md = _case(200, K, N, base=2101)
    y = torch.empty((200, N), dtype=torch.bfloat16, device="cuda")
    assert _noalloc(x, wu, wg, md, y, err) == 0
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and raw_equal(y, mot.routed_gemm(x, wu, wg, md))
    # host-checked limits: a pack above the scratch's size, a ready plan
    big = torch.empty((mot.NOALLOC_MAX_T + 1, K), dtype=torch.bfloat16, device="cuda")
    ybig = torch.empty((mot.NOALLOC_MAX_T + 1, N), dtype=torch.bfloat16, device="cuda")
    mbig = torch.zeros(mot.NOALLOC_MAX_T + 1, dtype=torch.uint8, device="cuda")
    assert _noalloc(big, wu, wg, mbig, ybig, err) == 2
    assert _noalloc(x, wu, wg, md, y, err, flags=1) == 1
