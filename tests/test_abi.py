"""The C-ABI library loads, exports every declared symbol, and fails closed on
host-checkable errors before touching the GPU (no compute here)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import mixture_transformers_token_amd as mot

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mot.h")

# error codes of include/mot.h
OK, INVALID, SHAPE, MISALIGNED, WORKSPACE, DEVICE, MODALITY = range(7)

A = 1 << 20  # fake, 256-byte aligned device addresses: never dereferenced


def _header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(mot_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = mot.lib()
    declared = _header_functions()
    assert set(declared) == set(mot.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    nm = os.popen(f"nm -D --defined-only {mot.LIB_PATH}").read()
    for name in declared:
        assert re.search(rf"\bT {name}\b", nm), name


def test_abi_version_matches_header():
    text = open(HEADER).read()
    v = int(re.search(r"#define MOT_ABI_VERSION (\d+)", text).group(1))
    assert mot.abi_version() == v == mot.ABI_VERSION


def test_status_strings():
    for code, name in mot.STATUS.items():
        assert mot.status_string(code).startswith(name)
    assert "unknown" in mot.status_string(99)


def test_workspace_bytes():
    assert mot.workspace_bytes(0) == 256
    assert mot.workspace_bytes(1) == 512
    assert mot.workspace_bytes(64) == 512
    assert mot.workspace_bytes(65) == 768
    assert mot.workspace_bytes(4096) == 256 + 4 * 4096


def _gemm(**kw):
    args = dict(x=A, ldx=256, wu=2 * A, wg=3 * A, m=4 * A, y=5 * A, ldy=384, T=64, K=256, N=384,
                rstd=None, nwu=None, nwg=None, ws=6 * A, wsb=1 << 20, flags=0)
    args.update(kw)
    return mot.lib().mot_routed_gemm(args["x"], args["ldx"], args["wu"], args["wg"], args["m"],
                                     args["y"], args["ldy"], args["T"], args["K"], args["N"],
                                     args["rstd"], args["nwu"], args["nwg"], args["ws"], args["wsb"],
                                     args["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID),
    (dict(T=0, x=None), OK),                  # T == 0 is a no-op
    (dict(x=None), INVALID),
    (dict(wg=None), INVALID),                 # both weight sets are required
    (dict(m=None), INVALID),
    (dict(y=None), INVALID),
    (dict(K=100), SHAPE),
    (dict(N=100, ldy=128), SHAPE),
    (dict(K=0), SHAPE),
    (dict(T=(1 << 24) + 1), SHAPE),
    (dict(ldx=128), INVALID),                 # ldx < K
    (dict(ldy=256), INVALID),                 # ldy < N
    (dict(ldx=260), MISALIGNED),
    (dict(x=A + 2), MISALIGNED),
    (dict(y=5 * A + 8), MISALIGNED),
    (dict(ws=None), WORKSPACE),
    (dict(wsb=300), WORKSPACE),
    (dict(ws=6 * A + 16), MISALIGNED),
    (dict(rstd=7 * A), INVALID),              # prologue pointers all or none
    (dict(rstd=7 * A, nwu=8 * A), INVALID),
    (dict(flags=4), INVALID),
    (dict(flags=0x30), INVALID),              # two tile shapes at once
    (dict(flags=0x40), INVALID),
    (dict(y=A + 1024), INVALID),              # y overlaps x
    (dict(y=2 * A), INVALID),                 # y overlaps a weight set
    (dict(K=(1 << 20) + 64, ldx=(1 << 20) + 64), SHAPE),
])
def test_gemm_fails_closed(kw, code):
    assert _gemm(**kw) == code


def _gemm_f32(**kw):
    args = dict(x=A, ldx=256, wu=2 * A, wg=3 * A, m=4 * A, y=5 * A, ldy=384, T=64, K=256, N=384,
                ws=6 * A, wsb=1 << 20, flags=0)
    args.update(kw)
    return mot.lib().mot_routed_gemm_f32(args["x"], args["ldx"], args["wu"], args["wg"], args["m"],
                                         args["y"], args["ldy"], args["T"], args["K"], args["N"],
                                         args["ws"], args["wsb"], args["flags"], None)


G = 1 << 36  # far-apart fake addresses for the large-extent case


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID),
    (dict(T=0, y=None), OK),
    (dict(y=None), INVALID),
    (dict(wu=None), INVALID),
    (dict(N=96, ldy=128), SHAPE),
    (dict(ldy=388), MISALIGNED),
    (dict(y=5 * A + 8), MISALIGNED),
    (dict(wsb=300), WORKSPACE),
    (dict(flags=0x10), INVALID),              # no tile override
    (dict(flags=0x20), INVALID),
    (dict(flags=2), INVALID),
    # the fp32 extent (64 rows x 384 x 4 bytes) reaches w_und; half of it would not
    (dict(y=2 * A - 64 * 384 * 4 + 256), INVALID),
    # 2^20 rows x 1024 fp32 columns = 4 GiB: past the 32-bit byte offsets
    (dict(x=G, wu=2 * G, wg=3 * G, m=4 * G, y=5 * G, ws=6 * G, T=1 << 20, N=1024, ldy=1024,
          wsb=1 << 23), SHAPE),
])
def test_gemm_f32_fails_closed(kw, code):
    assert _gemm_f32(**kw) == code


def test_swiglu_fails_closed():
    L = mot.lib()
    # F not a multiple of 64
    assert L.mot_routed_gemm_swiglu(A, 256, 2 * A, 3 * A, 4 * A, 5 * A, 96, 64, 256, 96,
                                    None, None, None, 6 * A, 1 << 20, 0, None) == SHAPE
    assert L.mot_routed_gemm_swiglu(A, 256, 2 * A, None, 4 * A, 5 * A, 128, 64, 256, 128,
                                    None, None, None, 6 * A, 1 << 20, 0, None) == INVALID


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID),
    (dict(eps=0.0), INVALID),
    (dict(eps=float("inf")), INVALID),
    (dict(eps=float("nan")), INVALID),
    (dict(x=None), INVALID),
    (dict(out=None, rstd=None), INVALID),
    (dict(H=100), SHAPE),
    (dict(H=16384 + 64), SHAPE),
    (dict(x=A + 4), MISALIGNED),
    (dict(out=A), INVALID),                   # out aliases x
    (dict(res=A + 64), INVALID),              # residual overlaps x
    (dict(T=0, x=None), OK),
])
def test_norm_fails_closed(kw, code):
    a = dict(x=A, res=2 * A, wu=3 * A, wg=4 * A, m=5 * A, eps=1e-6, out=6 * A, rstd=7 * A, T=64, H=3584,
             ws=None)
    a.update(kw)
    L = mot.lib()
    st = L.mot_fused_add_rmsnorm(a["x"], a["res"], a["wu"], a["wg"], a["m"], a["eps"], a["out"],
                                 a["rstd"], a["T"], a["H"], a["ws"], None)
    assert st == code


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(m=None), INVALID), (dict(ws=None), WORKSPACE),
    (dict(wsb=100), WORKSPACE), (dict(T=0, m=None), OK), (dict(ws=A + 8), MISALIGNED),
])
def test_plan_fails_closed(kw, code):
    a = dict(m=A, T=100, ws=2 * A, wsb=4096)
    a.update(kw)
    assert mot.lib().mot_routing_plan(a["m"], a["T"], a["ws"], a["wsb"], None) == code


def test_read_device_error_needs_workspace():
    assert mot.lib().mot_read_device_error(None, None) == INVALID


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), INVALID),
    (dict(rows_pad=50), INVALID),             # rows_pad < rows
    (dict(rows=0, rows_pad=0, inp=None), OK), # nothing to write
    (dict(cols=0), OK),
    (dict(inp=None), INVALID),
    (dict(out=None), INVALID),
    (dict(keep=2, m=3 * A), INVALID),       # keep is read only with a modality
    (dict(ld_in=100), INVALID),               # ld_in < cols
    (dict(ld_out=64), INVALID),               # ld_out < rows_pad
    (dict(ld_in=132), MISALIGNED),
    (dict(ld_out=132, rows_pad=130), MISALIGNED),
    (dict(inp=A + 2), MISALIGNED),
    (dict(out=2 * A + 8), MISALIGNED),
    (dict(out=A + 64), INVALID),              # out overlaps in
    (dict(rows_pad=(1 << 24) + 8, ld_out=(1 << 24) + 8), SHAPE),
])
def test_transpose_fails_closed(kw, code):
    a = dict(inp=A, ld_in=128, rows=100, cols=128, m=None, keep=1, out=2 * A, ld_out=128, rows_pad=128)
    a.update(kw)
    st = mot.lib().mot_transpose_bf16(a["inp"], a["ld_in"], a["rows"], a["cols"], a["m"], a["keep"],
                                      a["out"], a["ld_out"], a["rows_pad"], None)
    assert st == code


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID),
    (dict(T=0, qkv=None), OK),                # no-op
    (dict(eps=0.0), INVALID),
    (dict(eps=float("nan")), INVALID),
    (dict(qkv=None), INVALID),
    (dict(pos=None), INVALID),
    (dict(kwg=None), INVALID),
    (dict(hq=0, hk=0), INVALID),
    (dict(hq=-1), INVALID),
    (dict(n_pos=0), INVALID),
    (dict(ld=4096 - 8), INVALID),             # ld shorter than the heads
    (dict(ld=4612), MISALIGNED),
    (dict(qkv=A + 4), MISALIGNED),
    (dict(cos=9 * A + 2), MISALIGNED),
    (dict(ws=None), WORKSPACE),
    (dict(wsb=16), WORKSPACE),
    (dict(ws=12 * A + 8), MISALIGNED),
    (dict(pos=A + 4096), INVALID),            # positions inside the rows rewritten in place
    (dict(hq=8192), SHAPE),
    (dict(T=(1 << 24) + 1), SHAPE),
])
def test_qk_norm_rope_fails_closed(kw, code):
    a = dict(qkv=A, ld=4608, T=64, hq=28, hk=4, m=2 * A, qwu=3 * A, qwg=4 * A, kwu=5 * A, kwg=6 * A,
             pos=7 * A, cos=8 * A, sin=9 * A, n_pos=4096, eps=1e-6, ws=12 * A, wsb=256)
    a.update(kw)
    st = mot.lib().mot_qk_norm_rope(a["qkv"], a["ld"], a["T"], a["hq"], a["hk"], a["m"], a["qwu"], a["qwg"],
                                    a["kwu"], a["kwg"], a["pos"], a["cos"], a["sin"], a["n_pos"], a["eps"],
                                    a["ws"], a["wsb"], None)
    assert st == code


def _attn(**kw):
    args = dict(q=A, ldq=512, k=2 * A, ldk=256, v=3 * A, ldv=256, out=4 * A, ldo=512, Tq=64, Tk=100, hq=4,
                hkv=2, D=128, causal=1, ws=6 * A, wsb=1 << 20)
    args.update(kw)
    return mot.lib().mot_joint_attention(args["q"], args["ldq"], args["k"], args["ldk"], args["v"], args["ldv"],
                                         args["out"], args["ldo"], args["Tq"], args["Tk"], args["hq"],
                                         args["hkv"], args["D"], args["causal"], args["ws"], args["wsb"], None)


def test_attention_workspace_bytes():
    # V is read in place: the single-sequence call needs no workspace
    for tk, hkv in ((0, 4), (1, 4), (4096, 4), (4097, 1)):
        assert mot.attention_workspace_bytes(tk, hkv) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(Tq=-1), INVALID),
    (dict(Tk=-1), INVALID),
    (dict(Tq=0, q=None), OK),                 # Tq == 0 is a no-op
    (dict(hq=3), INVALID),                    # hq % hkv != 0
    (dict(hkv=0), INVALID),
    (dict(causal=2), INVALID),
    (dict(D=64), SHAPE),                      # head dimension 128 only
    (dict(hq=512, hkv=2, ldq=512 * 128, ldo=512 * 128), SHAPE),
    (dict(Tq=(1 << 24) + 1), SHAPE),
    (dict(q=None), INVALID),
    (dict(out=None), INVALID),
    (dict(k=None), INVALID),
    (dict(ldq=384), INVALID),                 # narrower than the q heads
    (dict(ldo=384), INVALID),
    (dict(ldk=128), INVALID),
    (dict(ldq=516), MISALIGNED),
    (dict(v=3 * A + 8), MISALIGNED),
    (dict(out=A + 1024), INVALID),            # out overlaps q
    (dict(out=2 * A), INVALID),               # out overlaps k
    (dict(out=3 * A + 512), INVALID),         # out overlaps v
    # 2^20 keys at a 4096-column pitch: K past the 32-bit byte offsets
    (dict(q=G, k=2 * G, v=3 * G, out=4 * G, Tk=1 << 20, ldk=4096, ldv=4096), SHAPE),
    # the same for V alone (K at a 256-column pitch fits)
    (dict(q=G, k=2 * G, v=3 * G, out=4 * G, Tk=1 << 20, ldk=256, ldv=4096), SHAPE),
])
def test_attention_fails_closed(kw, code):
    assert _attn(**kw) == code


def _dx(**kw):
    args = dict(dy=A, lddy=256, wu=2 * A, wg=3 * A, m=4 * A, dx=5 * A, lddx=128, T=100, N=256, K=128, ws=6 * A,
                wsb=1 << 20, flags=0)
    args.update(kw)
    return mot.lib().mot_routed_gemm_dx(args["dy"], args["lddy"], args["wu"], args["wg"], args["m"], args["dx"],
                                        args["lddx"], args["T"], args["N"], args["K"], args["ws"], args["wsb"],
                                        args["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID),
    (dict(T=0), OK),                                      # empty pack: a no-op
    (dict(flags=0x10), INVALID),                          # no tile override (256 x 256 tiles only)
    (dict(wg=None), INVALID),
    (dict(m=None), INVALID),
    (dict(N=100, lddy=104), SHAPE),                       # contraction % 64 != 0
    (dict(K=96, lddx=96), SHAPE),                         # output width % 64 != 0
    (dict(lddy=128), INVALID),                            # narrower than N
    (dict(lddx=64), INVALID),
    (dict(lddx=132), MISALIGNED),
    (dict(wu=2 * A + 8), MISALIGNED),
    (dict(ws=None), WORKSPACE),
    (dict(dx=2 * A + 1024), INVALID),                     # dx overlaps w_und
])
def test_dx_fails_closed(kw, code):
    assert _dx(**kw) == code


def _grad_w(**kw):
    args = dict(dy=A, lddy=256, x=2 * A, ldx=128, m=3 * A, keep=1, T=100, N=256, K=128, out=4 * A, ldo=128,
                f32=0)
    args.update(kw)
    return mot.lib().mot_grad_w(args["dy"], args["lddy"], args["x"], args["ldx"], args["m"], args["keep"],
                                args["T"], args["N"], args["K"], args["out"], args["ldo"], args["f32"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID),
    (dict(N=-1), INVALID),
    (dict(keep=2), INVALID),
    (dict(f32=2), INVALID),
    (dict(N=0, dy=None, x=None, m=None, out=None), OK),   # empty output: a no-op
    (dict(K=0), OK),
    (dict(out=None), INVALID),
    (dict(dy=None), INVALID),
    (dict(m=None), INVALID),
    (dict(K=96, ldx=96, ldo=96), SHAPE),                  # K % 64 != 0
    (dict(T=(1 << 24) + 1), SHAPE),
    (dict(lddy=128), INVALID),                            # narrower than N
    (dict(ldo=64), INVALID),
    (dict(lddy=260), MISALIGNED),
    (dict(x=2 * A + 8), MISALIGNED),
    (dict(out=2 * A + 1024), INVALID),                    # out overlaps x
    (dict(out=3 * A), INVALID),                           # out overlaps modality
    # 2^20 rows at a 4096-column pitch: dY past the 32-bit byte offsets
    (dict(dy=G, x=2 * G, m=3 * G, out=4 * G, T=1 << 20, lddy=4096), SHAPE),
])
def test_grad_w_fails_closed(kw, code):
    assert _grad_w(**kw) == code


def _attn_varlen(**kw):
    args = dict(q=A, ldq=512, k=2 * A, ldk=256, v=3 * A, ldv=256, out=4 * A, ldo=512, cq=5 * A, ck=5 * A + 64,
                n=3, Tq=64, Tk=100, maxq=64, hq=4, hkv=2, D=128, causal=1, ws=6 * A, wsb=1 << 20)
    args.update(kw)
    return mot.lib().mot_joint_attention_varlen(
        args["q"], args["ldq"], args["k"], args["ldk"], args["v"], args["ldv"], args["out"], args["ldo"],
        args["cq"], args["ck"], args["n"], args["Tq"], args["Tk"], args["maxq"], args["hq"], args["hkv"], args["D"],
        args["causal"], args["ws"], args["wsb"], None)


def test_attention_varlen_workspace_bytes():
    # the header with the lengths check's error word only (V is read in place)
    assert mot.attention_varlen_workspace_bytes(100, 0, 2) == 0
    assert mot.attention_varlen_workspace_bytes(100, 3, 2) == 256
    assert mot.attention_varlen_workspace_bytes(0, 1, 1) == 256


@pytest.mark.parametrize("kw,code", [
    (dict(Tq=0, q=None), OK),
    (dict(n=0), INVALID),
    (dict(maxq=0), INVALID),
    (dict(cq=None), INVALID),
    (dict(ck=5 * A + 2), MISALIGNED),
    (dict(hq=3), INVALID),
    (dict(D=64), SHAPE),
    (dict(n=65537), SHAPE),
    (dict(ws=None), WORKSPACE),
    (dict(wsb=255), WORKSPACE),
    (dict(ws=6 * A + 16), MISALIGNED),
    (dict(out=A + 1024), INVALID),
    (dict(ws=3 * A + 256), INVALID),          # workspace overlaps v
])
def test_attention_varlen_fails_closed(kw, code):
    assert _attn_varlen(**kw) == code


def _index_sets(**kw):
    args = dict(u=A, nu=24, g=2 * A, ng=40, m=3 * A, T=64, ws=4 * A, wsb=1 << 20)
    args.update(kw)
    return mot.lib().mot_modality_from_index_sets(args["u"], args["nu"], args["g"], args["ng"], args["m"],
                                                  args["T"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID),
    (dict(nu=-1, ng=65), INVALID),
    (dict(nu=24, ng=41), INVALID),            # n_und + n_gen != T: some row in neither or in both
    (dict(nu=0, ng=0, T=0, u=None, g=None, m=None), OK),  # empty pack
    (dict(m=None), INVALID),
    (dict(u=None), INVALID),
    (dict(g=None), INVALID),
    (dict(u=A + 2), MISALIGNED),
    (dict(ws=None), WORKSPACE),
    (dict(wsb=300), WORKSPACE),
    (dict(ws=4 * A + 16), MISALIGNED),
    (dict(m=A + 8), INVALID),                 # modality overlaps the und list
    (dict(ws=3 * A), INVALID),                # workspace overlaps modality
    (dict(T=(1 << 24) + 1, nu=(1 << 24) + 1, ng=0), SHAPE),
])
def test_index_sets_fail_closed(kw, code):
    assert _index_sets(**kw) == code


def _cfg(**kw):
    F = ctypes.c_float
    args = dict(vc=A, vt=2 * A, vi=3 * A, out=4 * A, cu=5 * A, n=2, rows=100, C=64, maxr=64, t=6 * A, s1=4.0, s2=1.5,
                lo=0.0, hi=1.0, rmin=0.0, kind=1, ws=7 * A, wsb=1 << 20)
    args.update(kw)
    return mot.lib().mot_cfg_combine_renorm(args["vc"], args["vt"], args["vi"], args["out"], args["cu"], args["n"],
                                            args["rows"], args["C"], args["maxr"], args["t"], args["s1"], args["s2"],
                                            args["lo"], args["hi"], args["rmin"], args["kind"], args["ws"], args["wsb"],
                                            None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0, rows=0), OK),
    (dict(n=-1), INVALID),
    (dict(C=0), INVALID),
    (dict(C=66), SHAPE),
    (dict(C=8192), SHAPE),
    (dict(maxr=0), INVALID),
    (dict(vc=None), INVALID),
    (dict(vt=None), INVALID),
    (dict(out=None), INVALID),
    (dict(t=None), INVALID),
    (dict(cu=None), INVALID),
    (dict(kind=3), INVALID),
    (dict(rmin=1.5), INVALID),
    (dict(s1=float("inf")), INVALID),
    (dict(vc=A + 4), MISALIGNED),
    (dict(cu=5 * A + 2), MISALIGNED),
    (dict(ws=None), WORKSPACE),
    (dict(wsb=200), WORKSPACE),
    (dict(ws=7 * A + 16), MISALIGNED),
    (dict(out=A + 1024), INVALID),            # out overlaps v_cond
    (dict(n=0), INVALID),                      # rows without requests
])
def test_cfg_fails_closed(kw, code):
    assert _cfg(**kw) == code


def _sde(**kw):
    args = dict(x=A, v=2 * A, z=3 * A, xin=None, xout=4 * A, lp=5 * A, cu=6 * A, n=2, rows=100, C=64, maxr=64,
                tc=7 * A, tn=8 * A, eta=0.7, ws=9 * A, wsb=1 << 20)
    args.update(kw)
    return mot.lib().mot_flow_sde_step_logp(args["x"], args["v"], args["z"], args["xin"], args["xout"], args["lp"],
                                            args["cu"], args["n"], args["rows"], args["C"], args["maxr"], args["tc"],
                                            args["tn"], args["eta"], args["ws"], args["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0, rows=0), OK),
    (dict(x=None), INVALID),
    (dict(lp=None), INVALID),
    (dict(tn=None), INVALID),
    (dict(xout=None), INVALID),                   # sampling needs x_next_out
    (dict(xin=10 * A), INVALID),                  # both modes at once
    (dict(z=None, xout=None), INVALID),           # neither mode
    (dict(eta=0.0), INVALID),
    (dict(eta=float("nan")), INVALID),
    (dict(C=30), SHAPE),
    (dict(xout=4 * A + 8), MISALIGNED),
    (dict(lp=5 * A + 2), MISALIGNED),
    (dict(wsb=100), WORKSPACE),
    (dict(xout=A + 512), INVALID),                # x_next_out overlaps x
    (dict(lp=2 * A + 64), INVALID),               # logp overlaps v
])
def test_sde_fails_closed(kw, code):
    assert _sde(**kw) == code


def test_latent_workspace_bytes():
    assert mot.latent_workspace_bytes(0, 64) == 0
    assert mot.latent_workspace_bytes(3, 1024) == 256 + 3 * 16 * 8
    assert mot.latent_workspace_bytes(1, 65) == 256 + 2 * 8
