"""Seeded synthetic inputs for the MoT token-routed projection.

This module is shared by the CPU oracle side and the HIP side of every test
and of the benchmark.  It holds shapes, modality patterns and seeded random
draws only -- none of the method's arithmetic lives here.

Modality follows the BAGEL Mixture-of-Transformers description on the
RL-Kernel RFC page ("[RFC][BAGEL-7B-MoT] WS1/WS2 kernel roadmap", section 1):
text and ViT rows use the understanding weight set (modality 0), VAE-latent
rows use the generation set (modality 1).  Random draws use one seeded CPU
generator per tensor, with the device, dtype and order of the draws fixed, as
the same page's numerical rules ask of the sampling noise (section 3).
"""
from __future__ import annotations

import math

import numpy as np
import torch

UND = 0
GEN = 1

# Qwen2.5-7B-shaped decoder sizes used by BAGEL-7B-MoT.
HIDDEN = 3584
Q_DIM = 3584
KV_DIM = 512
QKV_DIM = Q_DIM + 2 * KV_DIM  # 4608: q rows, then k rows, then v rows
HEAD_DIM = 128
N_Q_HEADS = Q_DIM // HEAD_DIM   # 28
N_K_HEADS = KV_DIM // HEAD_DIM  # 4
FFN = 18944

# One BAGEL text-to-image packing unit: 77 prompt rows (und) then a 32x32
# latent grid of 1024 rows (gen).
BAGEL_UNIT = ((UND, 77), (GEN, 1024))


def seed_of(base: int, tensor_id: int) -> int:
    """Seed of one tensor: 1000*base + tensor_id."""
    return 1000 * base + tensor_id


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return g


def normal_bf16(shape, seed: int, std: float = 1.0, mean: float = 0.0) -> torch.Tensor:
    """CPU bf16 tensor drawn as mean + std*N(0,1) in fp32, then cast (RNE)."""
    t = torch.randn(tuple(shape), generator=_gen(seed), dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(torch.bfloat16)


def permutation(n: int, seed: int) -> torch.Tensor:
    return torch.randperm(n, generator=_gen(seed))


def pattern(T: int, unit=BAGEL_UNIT) -> np.ndarray:
    """Modality bytes: the packing unit cycled and truncated at T rows."""
    one = np.concatenate([np.full(n, m, dtype=np.uint8) for m, n in unit])
    reps = -(-T // len(one)) if T > 0 else 0
    return np.tile(one, reps)[:T].copy()


def tiny_modality() -> np.ndarray:
    """Tiny case: first 24 rows und, last 40 rows gen."""
    return np.concatenate([np.zeros(24, np.uint8), np.ones(40, np.uint8)])


def cfg_pack_modality() -> np.ndarray:
    """Three CFG branches of one prompt+latent unit, three extra prompt-only
    branches of 77 rows, then 562 und padding rows up to 4096."""
    body = np.concatenate([pattern(1101)] * 3 + [np.zeros(77, np.uint8)] * 3)
    assert body.size == 3534
    return np.concatenate([body, np.zeros(4096 - 3534, np.uint8)])


def cfg_pack_lengths() -> list:
    """Rows per request of the CFG pack: the three branches, the three
    prompt-only branches and the padding rows, each its own sequence."""
    return [1101, 1101, 1101, 77, 77, 77, 4096 - 3534]


def cu_lengths(lengths) -> np.ndarray:
    """Cumulative row counts [0, l0, l0 + l1, ...] as int32."""
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw uint16 view of a CPU bf16 tensor (for the oracle)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


# --- the workloads -------------------------------------------------------------

def gemm_case(T: int, K: int, N: int, modality: np.ndarray, base: int = 0,
              x_std: float = 1.0, w_std: float = 0.02):
    """X ~ N(0,1) bf16 [T,K]; W_und, W_gen ~ N(0,0.02) bf16 [N,K]."""
    assert modality.shape == (T,)
    x = normal_bf16((T, K), seed_of(base, 1), x_std)
    w_und = normal_bf16((N, K), seed_of(base, 2), w_std)
    w_gen = normal_bf16((N, K), seed_of(base, 3), w_std)
    return x, w_und, w_gen, modality


def tiny(base: int = 0):
    return gemm_case(64, 256, 384, tiny_modality(), base)


def qkv(T: int = 4096, base: int = 0, modality: np.ndarray | None = None):
    m = pattern(T) if modality is None else modality
    return gemm_case(T, HIDDEN, QKV_DIM, m, base)


def norm_weights(H: int, base: int = 0):
    """Per-set RMSNorm weights ~ 1 + N(0, 0.1), bf16."""
    return (normal_bf16((H,), seed_of(base, 4), 0.1, 1.0),
            normal_bf16((H,), seed_of(base, 5), 0.1, 1.0))


def qk_norm_weights(base: int = 0, head_dim: int = 128):
    """Per-set QK norm weights ~ 1 + N(0, 0.1), bf16: ((q_und, q_gen), (k_und, k_gen))."""
    return ((normal_bf16((head_dim,), seed_of(base, 11), 0.1, 1.0), normal_bf16((head_dim,), seed_of(base, 12), 0.1, 1.0)),
            (normal_bf16((head_dim,), seed_of(base, 13), 0.1, 1.0), normal_bf16((head_dim,), seed_of(base, 14), 0.1, 1.0)))


def rope_inputs(T: int, n_pos: int, base: int = 0, half: int = 64):
    """Rotary tables and positions as data: cos and sin [n_pos, half] bf16 of
    seeded phases uniform on [0, 2*pi) (rounded from fp64), and positions
    [T] int32 uniform on [0, n_pos)."""
    ph = torch.rand((n_pos, half), generator=_gen(seed_of(base, 15)), dtype=torch.float64) * (2 * math.pi)
    pos = torch.randint(0, n_pos, (T,), generator=_gen(seed_of(base, 16)), dtype=torch.int64).to(torch.int32)
    return ph.cos().to(torch.bfloat16), ph.sin().to(torch.bfloat16), pos


def residual_inputs(T: int, H: int, base: int = 0):
    """Hidden input x and residual r ~ N(0,1) bf16 [T,H]."""
    return normal_bf16((T, H), seed_of(base, 6)), normal_bf16((T, H), seed_of(base, 7))


def mlp_weights(K: int = HIDDEN, F: int = FFN, base: int = 0):
    """Gate/up [2F,K] (rows [0,F) gate, [F,2F) up) and down [K_out=K, F] per set."""
    return (normal_bf16((2 * F, K), seed_of(base, 8), 0.02),
            normal_bf16((2 * F, K), seed_of(base, 9), 0.02),
            normal_bf16((K, F), seed_of(base, 10), 0.02),
            normal_bf16((K, F), seed_of(base, 11), 0.02))


def o_weights(H: int = HIDDEN, base: int = 0):
    return (normal_bf16((H, Q_DIM), seed_of(base, 12), 0.02),
            normal_bf16((H, Q_DIM), seed_of(base, 13), 0.02))


def sample_rows(modality: np.ndarray, n: int, seed: int) -> np.ndarray:
    """Seeded row sample stratified by modality that always contains every
    segment boundary (first/last row of each maximal run) plus the pack ends."""
    T = modality.size
    if T == 0:
        return np.zeros(0, np.int64)
    edges = {0, T - 1}
    change = np.nonzero(modality[1:] != modality[:-1])[0]
    for c in change:
        edges.update((int(c), int(c) + 1))
    rng = np.random.default_rng(seed)
    picked = set(edges)
    for m in (UND, GEN):
        rows = np.nonzero(modality == m)[0]
        if rows.size:
            k = min(rows.size, max(1, n // 2))
            picked.update(int(r) for r in rng.choice(rows, size=k, replace=False))
    return np.array(sorted(picked), dtype=np.int64)
