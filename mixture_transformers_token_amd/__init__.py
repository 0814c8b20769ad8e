"""MI355X-native Mixture-of-Transformers token-routed projection.

Thin ctypes binding of libmot (include/mot.h): argument checking and
marshalling only.  Every step of the path runs in the HIP library; PyTorch
provides device memory and the current stream.  There is no fallback: if
libmot.so is missing or stale, every call raises.

Functions mirror the C ABI:
  modality_from_index_sets, routing_plan, routed_gemm, routed_gemm_f32, routed_gemm_swiglu,
  fused_add_rmsnorm, transpose, qk_norm_rope, joint_attention,
  joint_attention_varlen, read_device_error,
  workspace_bytes, abi_version, routed_gemm_dx, grad_w.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MotError", "ABI_VERSION", "lib", "abi_version", "workspace_bytes", "new_workspace",
    "routing_plan", "modality_from_index_sets", "routed_gemm_noalloc", "NOALLOC_MAX_T", "plan_view", "routed_gemm", "routed_gemm_f32", "routed_gemm_swiglu", "fused_add_rmsnorm",
    "transpose", "routed_gemm_dx", "grad_w", "qk_norm_rope", "joint_attention",
    "attention_workspace_bytes", "joint_attention_varlen", "attention_varlen_workspace_bytes",
    "read_device_error", "status_string", "LIB_PATH", "latent_workspace_bytes", "cfg_combine_renorm",
    "flow_sde_step_logp", "RENORM", "routed_gemm_qk_norm_rope",
]

ABI_VERSION = 14
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmot.so")
WS_HEADER_BYTES = 256
FLAG_PLAN_READY = 1
# tile-shape overrides (the library picks the shape by default; every shape
# gives the same bytes)
TILE_FLAGS = {None: 0x00, "auto": 0x00, "256x256": 0x10, "128x128": 0x20}

# exported symbols, as declared in include/mot.h
EXPORTS = (
    "mot_abi_version", "mot_status_string", "mot_workspace_bytes", "mot_routing_plan",
    "mot_routed_gemm", "mot_routed_gemm_swiglu", "mot_fused_add_rmsnorm", "mot_read_device_error",
    "mot_transpose_bf16", "mot_qk_norm_rope", "mot_routed_gemm_f32", "mot_attention_workspace_bytes",
    "mot_joint_attention", "mot_attention_varlen_workspace_bytes", "mot_joint_attention_varlen", "mot_grad_w",
    "mot_routed_gemm_dx",
    "mot_modality_from_index_sets", "mot_routed_gemm_noalloc", "mot_latent_workspace_bytes",
    "mot_cfg_combine_renorm", "mot_flow_sde_step_logp", "mot_routed_gemm_qk_norm_rope",
)

STATUS = {
    0: "MOT_OK", 1: "MOT_ERR_INVALID_ARG", 2: "MOT_ERR_UNSUPPORTED_SHAPE", 3: "MOT_ERR_MISALIGNED",
    4: "MOT_ERR_WORKSPACE", 5: "MOT_ERR_DEVICE", 6: "MOT_ERR_MODALITY", 7: "MOT_ERR_POSITION",
    8: "MOT_ERR_SEQLENS", 9: "MOT_ERR_PLAN", 10: "MOT_ERR_INDEX_SET", 11: "MOT_ERR_SCHEDULE",
}


class MotError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = int(status)
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def lib():
    """Load libmot.so (once) and check its ABI version; raise if unavailable."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libmot.so not built at {LIB_PATH}: "
                           "run python mixture_transformers_token_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, SZ, U = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint
    L.mot_abi_version.restype = ctypes.c_int
    L.mot_abi_version.argtypes = []
    L.mot_status_string.restype = ctypes.c_char_p
    L.mot_status_string.argtypes = [ctypes.c_int]
    L.mot_workspace_bytes.restype = SZ
    L.mot_workspace_bytes.argtypes = [I64]
    L.mot_routing_plan.restype = ctypes.c_int
    L.mot_routing_plan.argtypes = [P, I64, P, SZ, P]
    L.mot_routed_gemm.restype = ctypes.c_int
    L.mot_routed_gemm.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I64, P, P, P, P, SZ, U, P]
    L.mot_routed_gemm_f32.restype = ctypes.c_int
    L.mot_routed_gemm_f32.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I64, P, SZ, U, P]
    L.mot_routed_gemm_swiglu.restype = ctypes.c_int
    L.mot_routed_gemm_swiglu.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I64, P, P, P, P, SZ, U, P]
    L.mot_fused_add_rmsnorm.restype = ctypes.c_int
    L.mot_fused_add_rmsnorm.argtypes = [P, P, P, P, P, ctypes.c_float, P, P, I64, I64, P, P]
    L.mot_read_device_error.restype = ctypes.c_int
    L.mot_read_device_error.argtypes = [P, P]
    L.mot_transpose_bf16.restype = ctypes.c_int
    L.mot_transpose_bf16.argtypes = [P, I64, I64, I64, P, ctypes.c_int, P, I64, I64, P]
    L.mot_qk_norm_rope.restype = ctypes.c_int
    L.mot_qk_norm_rope.argtypes = [P, I64, I64, I64, I64, P, P, P, P, P, P, P, P, I64, ctypes.c_float, P, SZ, P]
    L.mot_attention_workspace_bytes.restype = SZ
    L.mot_attention_workspace_bytes.argtypes = [I64, I64]
    L.mot_joint_attention.restype = ctypes.c_int
    L.mot_joint_attention.argtypes = [P, I64, P, I64, P, I64, P, I64, I64, I64, I64, I64, I64, ctypes.c_int, P,
                                      SZ, P]
    L.mot_routed_gemm_dx.restype = ctypes.c_int
    L.mot_routed_gemm_dx.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I64, P, SZ, U, P]
    L.mot_grad_w.restype = ctypes.c_int
    L.mot_grad_w.argtypes = [P, I64, P, I64, P, ctypes.c_int, I64, I64, I64, P, I64, ctypes.c_int, P]
    L.mot_attention_varlen_workspace_bytes.restype = SZ
    L.mot_attention_varlen_workspace_bytes.argtypes = [I64, I64, I64]
    L.mot_joint_attention_varlen.restype = ctypes.c_int
    L.mot_joint_attention_varlen.argtypes = [P, I64, P, I64, P, I64, P, I64, P, P, I64, I64, I64, I64, I64, I64, I64,
                                             ctypes.c_int, P, SZ, P]
    F = ctypes.c_float
    L.mot_latent_workspace_bytes.restype = SZ
    L.mot_latent_workspace_bytes.argtypes = [I64, I64]
    L.mot_cfg_combine_renorm.restype = ctypes.c_int
    L.mot_cfg_combine_renorm.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, F, F, F, F, F, ctypes.c_int, P, SZ, P]
    L.mot_flow_sde_step_logp.restype = ctypes.c_int
    L.mot_flow_sde_step_logp.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, P, P, F, P, SZ, P]
    L.mot_routed_gemm_qk_norm_rope.restype = ctypes.c_int
    L.mot_routed_gemm_qk_norm_rope.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I64, I64, I64, P, P, P, P, P, P, P,
                                               I64, ctypes.c_float, P, SZ, U, P]
    L.mot_routed_gemm_noalloc.restype = ctypes.c_int
    L.mot_routed_gemm_noalloc.argtypes = [P, I64, P, P, P, P, I64, I64, I64, I64, P, P, P, P, U, P]
    L.mot_modality_from_index_sets.restype = ctypes.c_int
    L.mot_modality_from_index_sets.argtypes = [P, I64, P, I64, P, I64, P, SZ, P]
    v = L.mot_abi_version()
    if v != ABI_VERSION:
        raise RuntimeError(f"stale libmot.so: ABI {v}, binding expects {ABI_VERSION}; rebuild it")
    _lib = L
    return L


def abi_version() -> int:
    return int(lib().mot_abi_version())


def status_string(status: int) -> str:
    try:
        return lib().mot_status_string(int(status)).decode()
    except Exception:
        return STATUS.get(int(status), "unknown")


def workspace_bytes(T: int) -> int:
    return int(lib().mot_workspace_bytes(int(T)))


def _check(status: int, where: str):
    if status != 0:
        raise MotError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _req(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _rows(t, name):
    """Leading dimension of a row-major 2-D tensor (unit column stride)."""
    if t.shape[0] > 0 and t.shape[1] > 0 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def new_workspace(T: int, device) -> torch.Tensor:
    """A routed workspace for packs of up to T rows, zero-filled (so that its
    error word reads 0 until a call writes it: calls on an empty pack are
    no-ops that leave the workspace untouched)."""
    return torch.zeros(workspace_bytes(T), dtype=torch.uint8, device=device)


def routing_plan(modality: torch.Tensor, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Build the segment list of a pack in a workspace (returned)."""
    _req(modality, "modality", torch.uint8, 1)
    T = modality.shape[0]
    if workspace is None:
        workspace = new_workspace(T, modality.device)
    _check(lib().mot_routing_plan(_ptr(modality.contiguous()), T, _ptr(workspace),
                                  workspace.numel(), _stream(modality.device)), "mot_routing_plan")
    return workspace


def modality_from_index_sets(und_idx: torch.Tensor, gen_idx: torch.Tensor, T: int, out=None,
                             workspace: torch.Tensor | None = None):
    """Per-row modality bytes [T] uint8 from the understanding and generation
    row index lists (int32 GPU tensors, any order).  Every row must be in
    exactly one list once; otherwise the device raises MOT_ERR_INDEX_SET in
    the workspace's error word (read_device_error) and marks those rows with
    the invalid byte 0xFF.  Returns (modality, workspace)."""
    _req(und_idx, "und_idx", torch.int32, 1)
    _req(gen_idx, "gen_idx", torch.int32, 1)
    T = int(T)
    if out is None:
        out = torch.empty(T, dtype=torch.uint8, device=und_idx.device)
    _req(out, "out", torch.uint8, 1)
    if out.shape[0] != T or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{T}] uint8 tensor")
    if workspace is None:
        workspace = new_workspace(T, und_idx.device)
    u, g = und_idx.contiguous(), gen_idx.contiguous()
    st = lib().mot_modality_from_index_sets(_ptr(u), u.shape[0], _ptr(g), g.shape[0], _ptr(out), T,
                                            _ptr(workspace), workspace.numel(), _stream(und_idx.device))
    _check(st, "mot_modality_from_index_sets")
    return out, workspace


def plan_view(workspace: torch.Tensor, T: int):
    """(header int32[4], perm int32[T]) views of a workspace (documented layout)."""
    hdr = workspace[:16].view(torch.int32)
    perm = workspace[WS_HEADER_BYTES:WS_HEADER_BYTES + 4 * T].view(torch.int32)
    return hdr, perm


def _routed(fn, name, x, w_und, w_gen, modality, out, norm, workspace, plan_ready, swiglu, tile,
            out_dtype=torch.bfloat16):
    _req(x, "x", torch.bfloat16, 2)
    _req(w_und, "w_und", torch.bfloat16, 2)
    _req(w_gen, "w_gen", torch.bfloat16, 2)
    _req(modality, "modality", torch.uint8, 1)
    if w_und.shape != w_gen.shape:
        raise ValueError("w_und and w_gen must have the same shape (both weight sets are required)")
    if not (w_und.is_contiguous() and w_gen.is_contiguous()):
        raise ValueError("weights must be contiguous [rows, K]")
    T, K = x.shape
    rows = w_und.shape[0]
    if w_und.shape[1] != K:
        raise ValueError(f"weights have K={w_und.shape[1]}, x has K={K}")
    if modality.shape[0] != T:
        raise ValueError("modality must have one byte per row")
    if swiglu and rows % 2:
        raise ValueError("gate/up weights need an even number of rows")
    N = rows // 2 if swiglu else rows
    if out is None:
        out = torch.empty((T, N), dtype=out_dtype, device=x.device)
    _req(out, "out", out_dtype, 2)
    if tuple(out.shape) != (T, N):
        raise ValueError(f"out must be [{T}, {N}]")
    if workspace is None:
        if plan_ready:
            raise ValueError("plan_ready needs the workspace that holds the plan")
        workspace = new_workspace(T, x.device)
    rstd = nw_u = nw_g = None
    if norm is not None:
        rstd, nw_u, nw_g = norm
        _req(rstd, "rstd", torch.float32, 1)
        _req(nw_u, "norm w_und", torch.bfloat16, 1)
        _req(nw_g, "norm w_gen", torch.bfloat16, 1)
        if rstd.shape[0] != T or nw_u.shape[0] != K or nw_g.shape[0] != K:
            raise ValueError("prologue shapes: rstd [T], norm weights [K]")
    if tile not in TILE_FLAGS:
        raise ValueError(f"tile must be one of {sorted(k for k in TILE_FLAGS if k)}")
    mod = modality.contiguous()
    flags = (FLAG_PLAN_READY if plan_ready else 0) | TILE_FLAGS[tile]
    if out_dtype == torch.float32:
        if norm is not None or TILE_FLAGS[tile]:
            raise ValueError("fp32 output: no prologue and no tile override")
        st = fn(_ptr(x), _rows(x, "x"), _ptr(w_und), _ptr(w_gen), _ptr(mod), _ptr(out), _rows(out, "out"),
                T, K, N, _ptr(workspace), workspace.numel(), flags, _stream(x.device))
    else:
        st = fn(_ptr(x), _rows(x, "x"), _ptr(w_und), _ptr(w_gen), _ptr(mod), _ptr(out), _rows(out, "out"),
                T, K, N, _ptr(rstd), _ptr(nw_u), _ptr(nw_g), _ptr(workspace), workspace.numel(),
                flags, _stream(x.device))
    _check(st, name)
    return out


def routed_gemm(x, w_und, w_gen, modality, out=None, norm=None, workspace=None, plan_ready=False,
                tile=None):
    """y[t] = x[t] @ W_{modality[t]}^T in bf16 (fp32 accumulate).  W_* are [N, K].
    norm=(rstd [T] fp32, nw_und [K], nw_gen [K]) applies the routed-RMSNorm prologue.
    tile: None (library's choice) or "256x256" / "128x128" (force one tile shape)."""
    return _routed(lib().mot_routed_gemm, "mot_routed_gemm", x, w_und, w_gen, modality, out, norm,
                   workspace, plan_ready, swiglu=False, tile=tile)


NOALLOC_MAX_T = 65536


def routed_gemm_noalloc(x, w_und, w_gen, modality, out, norm=None, error_out=None, tile=None):
    """routed_gemm without a workspace: the library's own per-GPU scratch
    holds the segment list (packs of up to NOALLOC_MAX_T rows), so the call
    allocates nothing; `out` must be given.  error_out: None or an int32 GPU
    tensor of one element that receives the device error word.  Calls that
    overlap on one GPU share the scratch and must be ordered."""
    _req(x, "x", torch.bfloat16, 2)
    _req(w_und, "w_und", torch.bfloat16, 2)
    _req(w_gen, "w_gen", torch.bfloat16, 2)
    _req(modality, "modality", torch.uint8, 1)
    _req(out, "out", torch.bfloat16, 2)
    if w_und.shape != w_gen.shape or not (w_und.is_contiguous() and w_gen.is_contiguous()):
        raise ValueError("w_und and w_gen must be contiguous and of the same shape")
    T, K = x.shape
    N = w_und.shape[0]
    if w_und.shape[1] != K or modality.shape[0] != T or tuple(out.shape) != (T, N):
        raise ValueError("shapes: x [T, K], weights [N, K], modality [T], out [T, N]")
    if not modality.is_contiguous():
        raise ValueError("modality must be contiguous (no copy is made)")
    rstd = nw_u = nw_g = None
    if norm is not None:
        rstd, nw_u, nw_g = norm
    if error_out is not None:
        _req(error_out, "error_out", torch.int32, 1)
    if tile not in TILE_FLAGS:
        raise ValueError(f"tile must be one of {sorted(k for k in TILE_FLAGS if k)}")
    st = lib().mot_routed_gemm_noalloc(_ptr(x), _rows(x, "x"), _ptr(w_und), _ptr(w_gen), _ptr(modality),
                                       _ptr(out), _rows(out, "out"), T, K, N, _ptr(rstd), _ptr(nw_u), _ptr(nw_g),
                                       _ptr(error_out), TILE_FLAGS[tile], _stream(x.device))
    _check(st, "mot_routed_gemm_noalloc")
    return out


def routed_gemm_qk_norm_rope(x, w_und, w_gen, modality, n_q_heads, n_k_heads, q_norm, k_norm, positions,
                             cos_table, sin_table, eps=1e-6, out=None, workspace=None, tile=None):
    """The QKV projection with the per-head QK RMSNorm and rotary embedding in
    its epilogue: the bytes of routed_gemm followed by qk_norm_rope on its
    output, in one call.  q_norm, k_norm: (und, gen) pairs of [128] bf16;
    positions [T] int32; cos_table, sin_table [n_pos, 64] bf16.  Rows whose
    position is outside the table keep the GEMM's bytes and raise the
    workspace's error word (MOT_ERR_POSITION).  Returns out [T, N]."""
    _req(x, "x", torch.bfloat16, 2)
    _req(w_und, "w_und", torch.bfloat16, 2)
    _req(w_gen, "w_gen", torch.bfloat16, 2)
    _req(modality, "modality", torch.uint8, 1)
    _req(positions, "positions", torch.int32, 1)
    for t, name in ((cos_table, "cos_table"), (sin_table, "sin_table")):
        _req(t, name, torch.bfloat16, 2)
    if w_und.shape != w_gen.shape or not (w_und.is_contiguous() and w_gen.is_contiguous()):
        raise ValueError("w_und and w_gen must be contiguous and of the same shape")
    T, K = x.shape
    N = w_und.shape[0]
    if modality.shape[0] != T or positions.shape[0] != T or w_und.shape[1] != K:
        raise ValueError("shapes: x [T, K], weights [N, K], modality and positions [T]")
    if cos_table.shape != sin_table.shape or cos_table.shape[1] != 64:
        raise ValueError("cos_table and sin_table must both be [n_pos, 64]")
    if out is None:
        out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
    _req(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (T, N):
        raise ValueError(f"out must be [{T}, {N}]")
    if workspace is None:
        workspace = new_workspace(T, x.device)
    if tile not in TILE_FLAGS:
        raise ValueError(f"tile must be one of {sorted(k for k in TILE_FLAGS if k)}")
    tensors = [*(w.contiguous() for w in (*q_norm, *k_norm)), positions.contiguous(), cos_table.contiguous(),
               sin_table.contiguous()]
    st = lib().mot_routed_gemm_qk_norm_rope(_ptr(x), _rows(x, "x"), _ptr(w_und), _ptr(w_gen),
                                            _ptr(modality.contiguous()), _ptr(out), _rows(out, "out"), T, K, N,
                                            int(n_q_heads), int(n_k_heads), *(_ptr(t) for t in tensors),
                                            cos_table.shape[0], float(eps), _ptr(workspace), workspace.numel(),
                                            TILE_FLAGS[tile], _stream(x.device))
    _check(st, "mot_routed_gemm_qk_norm_rope")
    return out


def routed_gemm_f32(x, w_und, w_gen, modality, out=None, workspace=None, plan_ready=False):
    """The routed GEMM's fp32 sums, uncast: y[t] = x[t] @ W_{modality[t]}^T in
    fp32 (routed_gemm returns bf16_rne of exactly these values)."""
    return _routed(lib().mot_routed_gemm_f32, "mot_routed_gemm_f32", x, w_und, w_gen, modality, out, None,
                   workspace, plan_ready, False, None, out_dtype=torch.float32)


def routed_gemm_swiglu(x, wgu_und, wgu_gen, modality, out=None, norm=None, workspace=None,
                       plan_ready=False, tile=None):
    """act[t] = silu(g) * u with [g | u] = x[t] @ Wgu_{modality[t]}^T; Wgu_* are [2F, K]."""
    return _routed(lib().mot_routed_gemm_swiglu, "mot_routed_gemm_swiglu", x, wgu_und, wgu_gen,
                   modality, out, norm, workspace, plan_ready, swiglu=True, tile=tile)


def fused_add_rmsnorm(x, residual, w_und, w_gen, modality, eps=1e-6, out=True, rstd=True,
                      workspace=None):
    """Routed fused add-RMSNorm.  residual (or None) is updated in place with h.
    out / rstd: True to allocate, a tensor to fill, or None to skip.
    Returns (out, rstd)."""
    _req(x, "x", torch.bfloat16, 2)
    _req(modality, "modality", torch.uint8, 1)
    _req(w_und, "w_und", torch.bfloat16, 1)
    _req(w_gen, "w_gen", torch.bfloat16, 1)
    T, H = x.shape
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if residual is not None:
        _req(residual, "residual", torch.bfloat16, 2)
        if tuple(residual.shape) != (T, H) or not residual.is_contiguous():
            raise ValueError("residual must be contiguous [T, H]")
    if out is True:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if rstd is True:
        rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    if out is not None:
        _req(out, "out", torch.bfloat16, 2)
        if tuple(out.shape) != (T, H) or not out.is_contiguous():
            raise ValueError("out must be contiguous [T, H]")
    if rstd is not None:
        _req(rstd, "rstd", torch.float32, 1)
        if rstd.shape[0] != T:
            raise ValueError("rstd must be [T]")
    if modality.shape[0] != T or w_und.shape[0] != H or w_gen.shape[0] != H:
        raise ValueError("shapes: modality [T], weights [H]")
    st = lib().mot_fused_add_rmsnorm(_ptr(x), _ptr(residual), _ptr(w_und), _ptr(w_gen),
                                     _ptr(modality.contiguous()), float(eps), _ptr(out), _ptr(rstd),
                                     T, H, _ptr(workspace), _stream(x.device))
    _check(st, "mot_fused_add_rmsnorm")
    return out, rstd


def read_device_error(workspace: torch.Tensor) -> int:
    """Synchronises the current stream; returns the workspace's error status."""
    return int(lib().mot_read_device_error(_ptr(workspace), _stream(workspace.device)))


def _pad64(n: int) -> int:
    return (n + 63) // 64 * 64


def transpose(x, modality=None, keep=1, rows_pad=None):
    """out [cols, rows_pad] with out[c][r] = x[r][c]; rows whose modality byte
    differs from `keep` (if modality is given) and rows past x's are zero."""
    _req(x, "x", torch.bfloat16, 2)
    rows, cols = x.shape
    rows_pad = rows if rows_pad is None else int(rows_pad)
    ld_out = max(8, (rows_pad + 7) // 8 * 8)  # the library takes 16-byte row pitches
    out = torch.empty((cols, ld_out), dtype=torch.bfloat16, device=x.device)[:, :rows_pad]
    if modality is not None:
        _req(modality, "modality", torch.uint8, 1)
        if modality.shape[0] != rows:
            raise ValueError("modality must have one byte per row")
        modality = modality.contiguous()
    ld_in = _rows(x, "x") if rows > 0 else max(cols, 8)
    st = lib().mot_transpose_bf16(_ptr(x) if rows > 0 else None, ld_in, rows, cols, _ptr(modality),
                                  int(keep), _ptr(out), ld_out, rows_pad, _stream(x.device))
    _check(st, "mot_transpose_bf16")
    return out


def routed_gemm_dx(dy, w_und, w_gen, modality, wt=None, out=None, workspace=None, plan_ready=False):
    """dX[t] = dY[t] @ W_{modality[t]} (the routed backward for the inputs);
    W_* are the forward's [N, K] weights, read as they lie (mot_routed_gemm_dx,
    256 x 256 tiles).  wt = (W_und^T, W_gen^T) from transpose() runs the
    routed GEMM on them instead (its tile choice, small packs included); both
    forms give the same bytes."""
    if wt is not None:
        return routed_gemm(dy, wt[0], wt[1], modality, out=out, workspace=workspace, plan_ready=plan_ready)
    _req(dy, "dy", torch.bfloat16, 2)
    _req(w_und, "w_und", torch.bfloat16, 2)
    _req(w_gen, "w_gen", torch.bfloat16, 2)
    _req(modality, "modality", torch.uint8, 1)
    if w_und.shape != w_gen.shape or not (w_und.is_contiguous() and w_gen.is_contiguous()):
        raise ValueError("w_und and w_gen must be contiguous and of the same shape [N, K]")
    T, N = dy.shape
    if w_und.shape[0] != N or modality.shape[0] != T:
        raise ValueError("shapes: dy [T, N], weights [N, K], modality [T]")
    K = w_und.shape[1]
    if out is None:
        out = torch.empty((T, K), dtype=torch.bfloat16, device=dy.device)
    _req(out, "out", torch.bfloat16, 2)
    if tuple(out.shape) != (T, K):
        raise ValueError(f"out must be [{T}, {K}]")
    if workspace is None:
        if plan_ready:
            raise ValueError("plan_ready needs the workspace that holds the plan")
        workspace = new_workspace(T, dy.device)
    st = lib().mot_routed_gemm_dx(_ptr(dy), _rows(dy, "dy"), _ptr(w_und), _ptr(w_gen), _ptr(modality.contiguous()),
                                  _ptr(out), _rows(out, "out"), T, N, K, _ptr(workspace), workspace.numel(),
                                  FLAG_PLAN_READY if plan_ready else 0, _stream(dy.device))
    _check(st, "mot_routed_gemm_dx")
    return out


def grad_w(dy, x, modality, keep=1, out_dtype=torch.bfloat16, out=None):
    """dW[n][k] = sum over rows t with modality[t] == keep of dY[t][n] * X[t][k]
    (fp32, rows folded in ascending order in 16-row chunks), as [N, K] in
    out_dtype: bf16 (one cast) or fp32 (the sums themselves).  One kernel
    reads dy and x as they lie (mot_grad_w); the same bytes as routed_gemm on
    their transposes (transpose, with x's other-set rows zeroed)."""
    _req(dy, "dy", torch.bfloat16, 2)
    _req(x, "x", torch.bfloat16, 2)
    _req(modality, "modality", torch.uint8, 1)
    T, N = dy.shape
    K = x.shape[1]
    if x.shape[0] != T or modality.shape[0] != T:
        raise ValueError("dy, x and modality must have the same rows")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("grad_w: out_dtype must be torch.bfloat16 or torch.float32")
    f32 = out_dtype == torch.float32
    if out is None:
        out = torch.empty((N, K), dtype=out_dtype, device=dy.device)
    _req(out, "out", out_dtype, 2)
    if tuple(out.shape) != (N, K):
        raise ValueError(f"out must be [{N}, {K}]")
    st = lib().mot_grad_w(_ptr(dy), _rows(dy, "dy"), _ptr(x), _rows(x, "x"), _ptr(modality.contiguous()),
                          int(keep), T, N, K, _ptr(out), _rows(out, "out"), 1 if f32 else 0, _stream(dy.device))
    _check(st, "mot_grad_w")
    return out


def qk_norm_rope(qkv, n_q_heads, n_k_heads, modality, q_norm, k_norm, positions, cos_table, sin_table,
                 eps=1e-6, workspace=None):
    """In place on qkv [T, ld] bf16: per-head (128 columns) routed RMSNorm of
    the q heads (columns [0, 128*n_q_heads)) and k heads (the next
    128*n_k_heads), then the rotate-half rotary embedding in bf16.  q_norm,
    k_norm: (und, gen) pairs of [128] bf16; positions [T] int32; cos_table,
    sin_table [n_pos, 64] bf16.  Rows with an invalid modality byte or
    position keep their bytes and raise the workspace's error word
    (read_device_error).  Returns qkv."""
    _req(qkv, "qkv", torch.bfloat16, 2)
    if qkv.stride(1) != 1:
        raise ValueError("qkv must have unit column stride")
    T = qkv.shape[0]
    _req(modality, "modality", torch.uint8, 1)
    _req(positions, "positions", torch.int32, 1)
    for t, name in ((cos_table, "cos_table"), (sin_table, "sin_table")):
        _req(t, name, torch.bfloat16, 2)
    if modality.shape[0] != T or positions.shape[0] != T:
        raise ValueError("modality and positions need one entry per row")
    if cos_table.shape != sin_table.shape or cos_table.shape[1] != 64:
        raise ValueError("cos_table and sin_table must both be [n_pos, 64]")
    ws = workspace if workspace is not None else new_workspace(0, qkv.device)
    tensors = [modality.contiguous(), *(w.contiguous() for w in (*q_norm, *k_norm)), positions.contiguous(),
               cos_table.contiguous(), sin_table.contiguous()]
    st = lib().mot_qk_norm_rope(_ptr(qkv), qkv.stride(0), T, int(n_q_heads), int(n_k_heads),
                                *(_ptr(t) for t in tensors), cos_table.shape[0], float(eps), _ptr(ws),
                                ws.numel(), _stream(qkv.device))
    _check(st, "mot_qk_norm_rope")
    return qkv


def attention_workspace_bytes(Tk: int, n_kv_heads: int) -> int:
    return int(lib().mot_attention_workspace_bytes(int(Tk), int(n_kv_heads)))


def joint_attention(q, k, v, n_q_heads, n_kv_heads, causal=True, out=None, workspace=None):
    """Shared joint attention over the pack (both modalities, not routed):
    out[i] = softmax(q_i k^T / sqrt(128)) v per q head, kv heads shared by
    groups of n_q_heads / n_kv_heads; causal: row i sees keys
    j <= i + (Tk - Tq) (bottom-right aligned).  q [Tq, >= 128 hq], k and v
    [Tk, >= 128 hkv] bf16 row-major views (column ranges of one QKV buffer
    are fine).  Returns out [Tq, 128 hq] bf16."""
    _req(q, "q", torch.bfloat16, 2)
    _req(k, "k", torch.bfloat16, 2)
    _req(v, "v", torch.bfloat16, 2)
    Tq, Tk = q.shape[0], k.shape[0]
    if v.shape[0] != Tk:
        raise ValueError("k and v must have the same rows")
    width = 128 * int(n_q_heads)
    if q.shape[1] < width or k.shape[1] < 128 * int(n_kv_heads) or v.shape[1] < 128 * int(n_kv_heads):
        raise ValueError("q, k or v narrower than its heads")
    if out is None:
        out = torch.empty((Tq, width), dtype=torch.bfloat16, device=q.device)
    _req(out, "out", torch.bfloat16, 2)
    if out.shape[0] != Tq or out.shape[1] < width:
        raise ValueError(f"out must be [{Tq}, >= {width}]")
    # (the call reads V in place and needs no workspace; one passed in is unused)
    st = lib().mot_joint_attention(_ptr(q), _rows(q, "q"), _ptr(k), _rows(k, "k"), _ptr(v), _rows(v, "v"),
                                   _ptr(out), _rows(out, "out"), Tq, Tk, int(n_q_heads), int(n_kv_heads), 128,
                                   1 if causal else 0, _ptr(workspace),
                                   0 if workspace is None else workspace.numel(), _stream(q.device))
    _check(st, "mot_joint_attention")
    return out


def attention_varlen_workspace_bytes(Tk: int, n_seqs: int, n_kv_heads: int) -> int:
    return int(lib().mot_attention_varlen_workspace_bytes(int(Tk), int(n_seqs), int(n_kv_heads)))


def joint_attention_varlen(q, k, v, cu_q, cu_k, max_q, n_q_heads, n_kv_heads, causal=True, out=None,
                           workspace=None):
    """joint_attention over packed sequences: sequence b has the q rows
    [cu_q[b], cu_q[b+1]) and the keys [cu_k[b], cu_k[b+1]) (int32 GPU
    tensors of n_seqs + 1 entries, checked on the device; max_q bounds one
    sequence's rows).  Returns (out, workspace); mot_read_device_error on the
    workspace reports MOT_ERR_SEQLENS for invalid lengths."""
    _req(q, "q", torch.bfloat16, 2)
    _req(k, "k", torch.bfloat16, 2)
    _req(v, "v", torch.bfloat16, 2)
    _req(cu_q, "cu_q", torch.int32, 1)
    _req(cu_k, "cu_k", torch.int32, 1)
    if cu_q.shape != cu_k.shape or cu_q.shape[0] < 1:
        raise ValueError("cu_q and cu_k must both hold n_seqs + 1 entries")
    n_seqs = cu_q.shape[0] - 1
    Tq, Tk = q.shape[0], k.shape[0]
    if v.shape[0] != Tk:
        raise ValueError("k and v must have the same rows")
    width = 128 * int(n_q_heads)
    if out is None:
        out = torch.empty((Tq, width), dtype=torch.bfloat16, device=q.device)
    _req(out, "out", torch.bfloat16, 2)
    if out.shape[0] != Tq or out.shape[1] < width:
        raise ValueError(f"out must be [{Tq}, >= {width}]")
    if workspace is None:
        workspace = torch.empty(max(attention_varlen_workspace_bytes(Tk, max(n_seqs, 1), n_kv_heads), 256),
                                dtype=torch.uint8, device=q.device)
    cq, ck = cu_q.contiguous(), cu_k.contiguous()
    st = lib().mot_joint_attention_varlen(_ptr(q), _rows(q, "q"), _ptr(k), _rows(k, "k"), _ptr(v), _rows(v, "v"),
                                          _ptr(out), _rows(out, "out"), _ptr(cq), _ptr(ck), n_seqs, Tq, Tk,
                                          int(max_q), int(n_q_heads), int(n_kv_heads), 128, 1 if causal else 0,
                                          _ptr(workspace), workspace.numel(), _stream(q.device))
    _check(st, "mot_joint_attention_varlen")
    return out, workspace


# ---- latent step: renormalised CFG combine, flow SDE step ---------------------

RENORM = {"none": 0, "global": 1, "channel": 2}


def latent_workspace_bytes(n_req: int, max_rows: int) -> int:
    return int(lib().mot_latent_workspace_bytes(int(n_req), int(max_rows)))


def _latent_common(arrs, cu_rows, name):
    for a, nm in arrs:
        if a is not None:
            _req(a, nm, torch.float32, 2)
            if not a.is_contiguous():
                raise ValueError(f"{nm} must be contiguous [rows, C]")
    _req(cu_rows, "cu_rows", torch.int32, 1)
    if cu_rows.shape[0] < 1:
        raise ValueError("cu_rows must hold n_req + 1 entries")
    return cu_rows.contiguous()


def cfg_combine_renorm(v_cond, v_text_uncond, v_img_uncond, cu_rows, max_rows, t, s_text, s_img, t_lo, t_hi,
                       renorm_min=0.0, renorm="global", out=None, workspace=None):
    """Guided velocity per request (rows [cu_rows[b], cu_rows[b+1]) of the
    fp32 [rows, C] branches; v_img_uncond None for two branches), inside the
    window t_lo < t[b] <= t_hi, with the norm-ratio rescale clamped to
    [renorm_min, 1] per request ("global"), per row ("channel") or none.
    t: fp32 [n_req] GPU tensor.  Returns (out, workspace)."""
    cu = _latent_common(((v_cond, "v_cond"), (v_text_uncond, "v_text_uncond"), (v_img_uncond, "v_img_uncond")),
                        cu_rows, "cfg")
    rows, C = v_cond.shape
    for a in (v_text_uncond, v_img_uncond):
        if a is not None and a.shape != v_cond.shape:
            raise ValueError("the branches must have the same shape")
    _req(t, "t", torch.float32, 1)
    n = cu.shape[0] - 1
    if renorm not in RENORM:
        raise ValueError(f"renorm must be one of {sorted(RENORM)}")
    if out is None:
        out = torch.empty_like(v_cond)
    if workspace is None:
        workspace = torch.empty(max(latent_workspace_bytes(n, max_rows), 256), dtype=torch.uint8,
                                device=v_cond.device)
    st = lib().mot_cfg_combine_renorm(_ptr(v_cond), _ptr(v_text_uncond), _ptr(v_img_uncond), _ptr(out), _ptr(cu), n,
                                      rows, C, int(max_rows), _ptr(t.contiguous()), float(s_text), float(s_img),
                                      float(t_lo), float(t_hi), float(renorm_min), RENORM[renorm], _ptr(workspace),
                                      workspace.numel(), _stream(v_cond.device))
    _check(st, "mot_cfg_combine_renorm")
    return out, workspace


def flow_sde_step_logp(x, v, cu_rows, max_rows, t_cur, t_next, eta, noise=None, x_next=None, out=None, logp=None,
                       workspace=None):
    """One flow SDE step per request from t_cur[b] to t_next[b] (fp32 [n_req]
    GPU tensors): with noise, sample x_next (returned in `out`); with x_next,
    evaluate it.  Either way returns (x_next or None, logp [n_req] fp32,
    workspace)."""
    cu = _latent_common(((x, "x"), (v, "v"), (noise, "noise"), (x_next, "x_next")), cu_rows, "sde")
    rows, C = x.shape
    _req(t_cur, "t_cur", torch.float32, 1)
    _req(t_next, "t_next", torch.float32, 1)
    n = cu.shape[0] - 1
    if (noise is None) == (x_next is None):
        raise ValueError("give exactly one of noise (sampling) and x_next (evaluation)")
    if noise is not None and out is None:
        out = torch.empty_like(x)
    if logp is None:
        logp = torch.empty(n, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(latent_workspace_bytes(n, max_rows), 256), dtype=torch.uint8, device=x.device)
    st = lib().mot_flow_sde_step_logp(_ptr(x), _ptr(v), _ptr(noise), _ptr(x_next), _ptr(out if noise is not None
                                                                                         else None),
                                      _ptr(logp), _ptr(cu), n, rows, C, int(max_rows), _ptr(t_cur.contiguous()),
                                      _ptr(t_next.contiguous()), float(eta), _ptr(workspace), workspace.numel(),
                                      _stream(x.device))
    _check(st, "mot_flow_sde_step_logp")
    return (out if noise is not None else None), logp, workspace
