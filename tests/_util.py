"""Shared helpers for the parity tests: workload construction on the GPU and conversion of
the same tensors for the oracle. Holds none of the block's arithmetic."""
from __future__ import annotations

import numpy as np
import torch

import synth_inputs as S


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype != torch.float64 \
        else t.detach().cpu().numpy()


def gpu_available() -> bool:
    return torch.cuda.is_available()


def gpu_block(wl: S.Workload, block: int = 0, keep_bf16: bool = False, gen_device: str = "cpu"):
    """Dense bf16 weights of `block` (drawn on gen_device), moved to the GPU and quantised
    there by the library. Returns (BlockWeights, dense dict on GPU)."""
    from video_diffusion_transformer_03_amd import h3k
    wb = S.block_weights_bf16(wl, block, device=gen_device)
    wb = {k: v.to("cuda") for k, v in wb.items()}
    return h3k.quantize_block(wb, keep_bf16=keep_bf16), wb


def oracle_weights(bw, dense=None) -> dict:
    """Oracle weight dict from the GPU's quantised weights (and dense bf16 if given)."""
    w = {"w_ada": np64(bw.w_ada)}
    for k in ("qkv", "o", "up", "down"):
        w["q_" + k] = getattr(bw, "w_" + k).cpu().numpy()
        w["s_" + k] = getattr(bw, "s_" + k).cpu().numpy()
        if dense is not None:
            w["w_" + k] = np64(dense["w_" + k])
    return w


def code_match(a: np.ndarray, b: np.ndarray):
    """(fraction identical, max |difference|) of two int8 code arrays."""
    a = a.astype(np.int32)
    b = b.astype(np.int32)
    return float(np.mean(a == b)), int(np.max(np.abs(a - b))) if a.size else 0
