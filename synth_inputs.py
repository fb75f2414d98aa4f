"""Seeded synthetic inputs for the W8A8 DiT block: shapes and random draws only.

This module holds none of the block's arithmetic. It draws the tensors that both the
HIP path and the CPU oracle consume, so that the two can be compared on identical
inputs. Every draw comes from a torch Generator seeded from (base seed, block index,
tensor id); the same call on the same device always returns the same tensor.

Workload shapes (d, heads, MLP width, token grid) follow the DiT denoiser the pages
describe ("h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section
"고성능 추론 프리셋": 50 transformer blocks), sized like a 512x512 short clip
(4x64x64 latent grid) and a long clip (16x64x64).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Tuple

import torch

BASE_SEED = 20260811

# tensor ids (stable; used to derive per-tensor seeds)
_TID = {"x": 1, "cond": 2, "w_ada": 3, "w_qkv": 4, "w_o": 5, "w_up": 6, "w_down": 7,
        "outlier_ch": 8}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    d: int
    n_heads: int
    head_dim: int
    d_ff: int
    d_cond: int
    grid: Tuple[int, int, int]          # (T, Hg, Wg); token l = (t*Hg + h)*Wg + w
    n_blocks: int = 1
    tr_range: Tuple[int, int] = (0, 0)  # token-reduced blocks [begin, end); begin == end: off
    outliers: int = 0                   # channels of x scaled by outlier_scale
    outlier_scale: float = 20.0
    seed: int = BASE_SEED

    @property
    def L(self) -> int:
        t, h, w = self.grid
        return t * h * w


def _dit(name, grid, **kw):
    return Workload(name=name, d=5120, n_heads=40, head_dim=128, d_ff=20480, d_cond=5120,
                    grid=grid, **kw)


WORKLOADS = {
    # tiny 2-block stack: d=256, 4 heads x 64, MLP 1024, 8x8x8 grid (512 tokens)
    "tiny": Workload(name="tiny", d=256, n_heads=4, head_dim=64, d_ff=1024, d_cond=256,
                     grid=(8, 8, 8), n_blocks=2, seed=BASE_SEED + 0),
    # one block, 4x32x32 grid (4096 tokens), 8 outlier channels at 20x
    "block_l4096": _dit("block_l4096", (4, 32, 32), outliers=8, seed=BASE_SEED + 1),
    # one block, 4x64x64 grid (16384 tokens): a 512x512 short-clip canvas
    "block_l16384": _dit("block_l16384", (4, 64, 64), seed=BASE_SEED + 2),
    # 50-block stack at 16384 tokens, horizontal token pairing in blocks [10, 40)
    "stack50_l16384": _dit("stack50_l16384", (4, 64, 64), n_blocks=50, tr_range=(10, 40),
                           seed=BASE_SEED + 3),
    # one block, 16x64x64 grid (65536 tokens): long clip, attention dominated
    "block_l65536": _dit("block_l65536", (16, 64, 64), seed=BASE_SEED + 4),
}


def derive_seed(base: int, block: int, tensor: str) -> int:
    """64-bit seed from (base, block, tensor) via SHA-256 (stable across runs and hosts)."""
    h = hashlib.sha256(f"{base}:{block}:{_TID[tensor]}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, std: float, seed: int, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """N(0, std^2) draws in fp32, rounded (RNE) to `dtype`."""
    t = torch.randn(*shape, generator=_gen(device, seed), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def activations(wl: Workload, device="cpu", L: Optional[int] = None,
                dtype=torch.bfloat16) -> torch.Tensor:
    """x ~ N(0,1) [L, d]; `wl.outliers` distinct channels are scaled by `outlier_scale`
    before rounding to `dtype`."""
    L = wl.L if L is None else L
    x = torch.randn(L, wl.d, generator=_gen(device, derive_seed(wl.seed, 0, "x")),
                    device=device, dtype=torch.float32)
    if wl.outliers:
        ch = outlier_channels(wl)
        x[:, ch.to(device)] *= wl.outlier_scale
    return x.to(dtype)


def outlier_channels(wl: Workload) -> torch.Tensor:
    g = _gen("cpu", derive_seed(wl.seed, 0, "outlier_ch"))
    return torch.randperm(wl.d, generator=g)[: wl.outliers].sort().values


def conditioning(wl: Workload, device="cpu") -> torch.Tensor:
    """Timestep conditioning vector c ~ N(0,1) [d_cond], fp32."""
    return torch.randn(wl.d_cond, generator=_gen(device, derive_seed(wl.seed, 0, "cond")),
                       device=device, dtype=torch.float32)


def block_weights_bf16(wl: Workload, block: int, device="cpu", std: float = 0.02) -> dict:
    """Dense bf16 weights of one block, each ~ N(0, std^2), row-major [out, in]:
    w_ada [6d, d_cond], w_qkv [3d, d], w_o [d, d], w_up [F, d], w_down [d, F]."""
    d, F, dc = wl.d, wl.d_ff, wl.d_cond
    shapes = {"w_ada": (6 * d, dc), "w_qkv": (3 * d, d), "w_o": (d, d),
              "w_up": (F, d), "w_down": (d, F)}
    return {k: normal(s, std, derive_seed(wl.seed, block, k), device)
            for k, s in shapes.items()}
