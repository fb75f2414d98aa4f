"""CPU twin of the block library's C ABI: the oracle behind the same entry points.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests, the smoke check
and the benchmark's CPU baseline use it, and it shares no code with the HIP library or
its binding.

Each h3k_ref_<name> takes the arguments of the C function h3k_<name>, in the same order
and with the same meaning, with these differences:
  - host arrays (numpy) stand where the C call takes device pointers; outputs are
    written into caller-provided arrays (any float dtype for activations, int8 and fp32
    for quantised weights), inputs are read as the values they hold;
  - the dims argument is any object with the fields of h3k_dims (d, n_heads, head_dim,
    d_ff, d_cond, grid_t, grid_h, grid_w, rope_theta, ln_eps), e.g. the binding's struct;
  - a block's weights are any object or mapping with the field names of
    h3k_block_weights (w_ada; w_qkv, s_qkv, w_o, s_o, w_up, s_up, w_down, s_down as int8
    codes and fp32 scales; wb_qkv, wb_o, wb_up, wb_down as the dense matrices for the
    bf16 projections, else None); the tiled copies of the codes (wt_*), a layout the GPU
    GEMM reads, are not read: the twin needs the row-major codes;
  - workspace and stream arguments are accepted and ignored.
The return codes are those of the C ABI. The twin checks the method's own consistency
conditions (H3K_EINVAL: sizes that do not fit together, a bad pairing range, a
non-positive scale), not the GPU library's support limits (head_dim, multiples of 256,
L % 8), which a plain implementation does not have. A precision flag combination outside
the oracle's precision series (W8A8; int8 MLP + QKV; int8 MLP; all bf16) returns
H3K_EUNSUPPORTED, and so does a stack that is not W8A8 or does not use the default
LayerNorm eps and RoPE base.

Precision: by default the oracle's plain definition (every float fp64, the quantisers'
decisions in fp32); outputs take the type of the caller's array when they are written.
With the fp32 debug flag the tensors that path stores (Q, K, V, O, x1, g and the block
output) are rounded to fp32 where they are produced, since fp32 storage is part of that
path's definition. The attention call rounds its output to its dtype argument.
"""
import math
from typing import Optional

import numpy as np

from . import h3k_oracle as O

# return codes and flags, with the values of the C header
OK, EINVAL, EUNSUPPORTED = 0, -1, -2
F_BF16_GEMM, F_FP32_DEBUG, F_SYNC = 1, 2, 4
F_BF16_QKV, F_BF16_OUT, F_BF16_MLP = 8, 16, 32
F_ATTN_BF16 = 64
F_Q_BASE2 = 128
DT_F32, DT_BF16, DT_F16 = 0, 1, 2
_KNOWN_FLAGS = F_BF16_GEMM | F_FP32_DEBUG | F_SYNC | F_BF16_QKV | F_BF16_OUT | F_BF16_MLP | F_ATTN_BF16

_DENSE = (F_BF16_QKV, F_BF16_OUT, F_BF16_MLP)
# (qkv, out, mlp) projections run dense -> the oracle's variant of the precision series
_VARIANTS = {(False, False, False): "w8a8", (False, True, False): "int8_mlp_qkv",
             (True, True, False): "int8_mlp", (True, True, True): "bf16gemm"}


def _field(obj, name):
    return obj[name] if isinstance(obj, dict) else getattr(obj, name)


def _host(a) -> np.ndarray:
    return np.asarray(a, np.float64)


def _variant(flags: int) -> Optional[str]:
    dense = tuple(bool(flags & (F_BF16_GEMM | f)) for f in _DENSE)
    return _VARIANTS.get(dense)


def _storage(flags: int) -> str:
    return "fp32" if flags & F_FP32_DEBUG else "fp64"


def _oracle_weights(w, variant: str) -> dict:
    out = {"w_ada": _host(_field(w, "w_ada"))}
    dense = set(("_qkv", "_o", "_up", "_down")) - set(O.INT8_PROJECTIONS[variant])
    for k in ("qkv", "o", "up", "down"):
        if "_" + k in dense:
            out["w_" + k] = _host(_field(w, "wb_" + k))
        else:
            out["q_" + k] = np.asarray(_field(w, "w_" + k), np.int8)
            out["s_" + k] = np.asarray(_field(w, "s_" + k), np.float32)
    return out


def _dims_ok(dm, L: int) -> bool:
    pos = all(int(getattr(dm, f)) > 0 for f in ("d", "n_heads", "head_dim", "d_ff", "d_cond",
                                                 "grid_t", "grid_h", "grid_w"))
    return (pos and dm.d == dm.n_heads * dm.head_dim and dm.head_dim % 2 == 0 and L > 0
            and dm.grid_t * dm.grid_h * dm.grid_w == L and dm.ln_eps > 0 and dm.rope_theta > 0)


def _write(out, values) -> None:
    np.copyto(out, np.asarray(values).reshape(out.shape), casting="unsafe")


def h3k_ref_quantize_weights(w, w_dtype, n_out, k_in, q_out, scale_out, stream=None) -> int:
    """Per-output-channel int8 quantisation of w [n_out, k_in] (oracle quantize_weights)."""
    if w_dtype not in (DT_F32, DT_BF16) or n_out <= 0 or k_in <= 0:
        return EINVAL
    wm = _host(w)
    if wm.size != n_out * k_in or q_out.size != n_out * k_in or scale_out.size != n_out:
        return EINVAL
    q, s = O.quantize_weights(wm.reshape(n_out, k_in))
    _write(q_out, q)
    _write(scale_out, s)
    return OK


def h3k_ref_block_forward_grid(x_in, x_out, cond, w, dm, T, Hg, Wg, w_pos_scale, w_pos_offset,
                               flags, ws=None, ws_bytes=0, stream=None) -> int:
    """One block on the token grid (T, Hg, Wg), w positions w * w_pos_scale + w_pos_offset
    (oracle block_forward with the storage of the flags)."""
    L = T * Hg * Wg
    if min(T, Hg, Wg) <= 0 or not _dims_ok(_Grid(dm, T, Hg, Wg), L):
        return EINVAL
    if flags & ~_KNOWN_FLAGS:
        return EINVAL
    variant = _variant(flags)
    if variant is None:
        return EUNSUPPORTED
    x = _host(x_in)
    if x.size != L * dm.d or x_out.size != L * dm.d or np.size(cond) != dm.d_cond:
        return EINVAL
    st = _storage(flags)
    y = O.block_forward(x.reshape(L, dm.d), _host(cond), _oracle_weights(w, variant),
                        n_heads=dm.n_heads, head_dim=dm.head_dim, grid=(T, Hg, Wg),
                        variant=variant, w_scale=w_pos_scale, w_offset=w_pos_offset,
                        eps=float(dm.ln_eps), theta=float(dm.rope_theta), attn_inputs=st,
                        act_store=st)
    _write(x_out, y)
    return OK


def h3k_ref_block_forward(x_in, x_out, cond, w, dm, L, flags, ws=None, ws_bytes=0,
                          stream=None) -> int:
    """One block on the grid of dm (w positions 0, 1, ...)."""
    if not _dims_ok(dm, L):
        return EINVAL
    return h3k_ref_block_forward_grid(x_in, x_out, cond, w, dm, dm.grid_t, dm.grid_h,
                                      dm.grid_w, 1.0, 0.0, flags)


def h3k_ref_attention(q, k, v, o, n_heads, L, head_dim, softmax_scale, dtype, flags,
                      stream=None) -> int:
    """o[l, e*Dh + j] = sum_k softmax_k(q[e,l,:] . k[e,k,:] * softmax_scale) v[e,j,k]
    with q, k [H, L, Dh], v transposed [H, Dh, L] and o [L, H*Dh], computed from the
    values q, k, v hold and rounded once to `dtype` (the type the call's o has). With
    F_Q_BASE2, q holds base-2 logits (q * softmax_scale * log2 e), so the scores are
    q . k * ln 2. The oracle's attention scales by 1/sqrt(Dh), so q enters multiplied by
    softmax_scale * sqrt(Dh)."""
    if n_heads <= 0 or L <= 0 or head_dim <= 0 or not softmax_scale > 0:
        return EINVAL
    if dtype not in (DT_F32, DT_BF16, DT_F16) or flags & ~(F_SYNC | F_Q_BASE2):
        return EINVAL
    if flags & F_Q_BASE2:
        if dtype == DT_F32:
            return EINVAL
        # q holds q * scale * log2(e): softmax_2(q . k) = softmax(q . k * ln 2)
        softmax_scale = math.log(2.0)
    n = n_heads * L * head_dim
    if np.size(q) != n or np.size(k) != n or np.size(v) != n or np.size(o) != n:
        return EINVAL
    qh = _host(q).reshape(n_heads, L, head_dim).transpose(1, 0, 2)
    kh = _host(k).reshape(n_heads, L, head_dim).transpose(1, 0, 2)
    vh = _host(v).reshape(n_heads, head_dim, L).transpose(2, 0, 1)
    res = O.attention(qh * (softmax_scale * math.sqrt(head_dim)), kh, vh)
    store = {DT_F32: O.round_f32, DT_BF16: O.round_bf16, DT_F16: O.round_f16}[dtype]
    _write(o, store(res.reshape(L, n_heads * head_dim)))
    return OK


def h3k_ref_stack_forward(x_in, x_out, cond, blocks, n_blocks, dm, L, tr_begin, tr_end, flags,
                          ws=None, ws_bytes=0, stream=None) -> int:
    """n_blocks blocks sharing cond; blocks [tr_begin, tr_end) on horizontally paired
    tokens (oracle stack_forward)."""
    if not _dims_ok(dm, L) or n_blocks <= 0 or len(blocks) < n_blocks:
        return EINVAL
    if not (0 <= tr_begin <= tr_end <= n_blocks) or (tr_begin < tr_end and dm.grid_w % 2):
        return EINVAL
    if flags & ~_KNOWN_FLAGS:
        return EINVAL
    variant = _variant(flags)
    # the oracle stack runs W8A8 blocks with the default LayerNorm eps and RoPE base
    if (variant != "w8a8" or np.float32(dm.ln_eps) != np.float32(O.LN_EPS)
            or np.float32(dm.rope_theta) != np.float32(O.ROPE_THETA)):
        return EUNSUPPORTED
    x = _host(x_in)
    if x.size != L * dm.d or x_out.size != L * dm.d or np.size(cond) != dm.d_cond:
        return EINVAL
    st = _storage(flags)
    y = O.stack_forward(x.reshape(L, dm.d), _host(cond),
                        [_oracle_weights(b, variant) for b in blocks[:n_blocks]],
                        n_heads=dm.n_heads, head_dim=dm.head_dim,
                        grid=(dm.grid_t, dm.grid_h, dm.grid_w), tr_begin=tr_begin,
                        tr_end=tr_end, variant=variant, attn_inputs=st, act_store=st)
    _write(x_out, y)
    return OK


class _Grid:
    """dm with its grid fields replaced (for the explicit-grid block call)."""

    def __init__(self, dm, T, Hg, Wg):
        self._dm, self.grid_t, self.grid_h, self.grid_w = dm, T, Hg, Wg

    def __getattr__(self, name):
        return getattr(self._dm, name)
