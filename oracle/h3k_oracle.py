"""CPU oracle for the W8A8 DiT block forward: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module. The product path (the HIP library and its Python
binding) never imports, calls or falls back to it, and it shares no code with that
path.

Precision: every float is fp64 and every int8 product is accumulated exactly. The one
exception is each quantiser's rounding decision, which is taken in fp32 because the
pages fix the scales as F32 values ("맥북에서 AI 영상 생성 모델 돌리기 - MiniMax H3 로컬
실행과 30초 애니메이션 만들기", section "int8 이 뭔가요": one F32 scale per weight output
channel, activations quantised on the fly with one F32 scale per row).

What the block computes. The pages name the parts but print no equation; where they are
silent the plainest reading consistent with them is taken (the readings are listed in the
design notes):
  m  = W_ada c                                   -> shift1 scale1 gate1 shift2 scale2 gate2
  h  = LN(x) * (1 + scale1) + shift1             (gated AdaLN, LayerNorm without affine)
  qa = quant(h)                                  (dynamic per-token int8)
  y  = (qa Wq_qkv^T) * s_a[l] * s_w[n]           (W8A8 QKV, per-output-channel scales)
  Q, K = RoPE(Q), RoPE(K)                        (3D axial RoPE over the (t, h, w) grid)
  O  = softmax(Q K^T / sqrt(Dh)) V   per head    (no mask)
  x1 = x + gate1 * dequant(quant(O) Wq_o^T)
  h2 = LN(x1) * (1 + scale2) + shift2
  g  = GELU(dequant(quant(h2) Wq_up^T))           (exact erf GELU)
  x2 = x1 + gate2 * dequant(quant(g) Wq_down^T)
Pages: "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", sections "Int8 양자화"
(int8 MLP with dynamic activation quantisation and per-output-channel weight scales,
int8 QKV, quantisers folded into the gated AdaLN kernel) and "Metal 4 및 TensorOps"
(QKV and attention-output projections feeding head-major attention inputs); the
comparison page "MiniMax-H3在Apple Silicon上的兩種推理實現工程取舍", section 性能上限
(AdaLN gating, RoPE and quantisation folded into the preceding kernel).

Parity pins: every function below is pinned by tests that do not re-run its own
formula (brute force on tiny inputs, library routines, closed forms, invariants). The
composed block and stack values are pinned only through their parts, the invariants and
a brute-force loop implementation on a tiny case: the pages print no tensor values.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

QMAX = 127
LN_EPS = 1e-6
ROPE_THETA = 10000.0


# --------------------------------------------------------------------------- quantiser
def quantize_rows(v) -> Tuple[np.ndarray, np.ndarray]:
    """Symmetric per-row absmax int8 quantiser (the pages' "one F32 scale per row";
    the same rule gives "one F32 scale per output channel" for weight rows).

    Decision taken in fp32: v is rounded to fp32; a = max|v|; s = a/127 (fp32);
    q = clamp(RNE(v * (127/a)), -127, 127) with the reciprocal and the product each
    rounded to fp32. A row with a = 0 gets s = 0 and all-zero codes.
    Returns (q int8 [..., K], s fp32 [...]).
    """
    v32 = np.asarray(v).astype(np.float32)
    a = np.max(np.abs(v32), axis=-1)
    s = (a / np.float32(QMAX)).astype(np.float32)
    safe = np.where(a > 0, a, np.float32(1))
    inv = np.where(a > 0, np.float32(QMAX) / safe, np.float32(0)).astype(np.float32)
    prod = (v32 * inv[..., None]).astype(np.float32)
    q = np.clip(np.rint(prod), -QMAX, QMAX).astype(np.int8)
    return q, s


def dequantize_rows(q, s) -> np.ndarray:
    return q.astype(np.float64) * np.asarray(s, np.float64)[..., None]


def quantize_weights(w) -> Tuple[np.ndarray, np.ndarray]:
    """Weight quantisation, one scale per output channel (row of w [N, K])."""
    return quantize_rows(w)


# --------------------------------------------------------------------------- 16-bit rounding
def round_bf16(v) -> np.ndarray:
    """Round to the nearest bfloat16 value (8 significant bits), ties to even, from the
    exact fp64 value (one rounding). Zero, inf and NaN pass through; values are assumed
    to lie in the normal bf16 range."""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)                   # v = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def round_f16(v) -> np.ndarray:
    """Round to the nearest IEEE binary16 value, ties to even, from the exact fp64 value
    (one rounding): 11 significant bits for |v| >= 2^-14; below that a fixed step of 2^-24
    (the subnormals). Magnitudes that round above 65504 become infinite. Written out from
    the format rather than through a library conversion."""
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)                   # v = m * 2**e, 0.5 <= |m| < 1
    # quantum of the binade: 2^(e - 11) for normal values, 2^-24 for subnormal ones
    q = np.ldexp(1.0, np.maximum(e - 11, -24))
    r = np.rint(v / q) * q               # exact: v / q and the product are powers-of-two scalings
    return np.where(np.abs(r) > 65504.0, np.copysign(np.inf, v), r)


# --------------------------------------------------------------------------- int8 GEMM
def int8_matmul(qa, qw) -> np.ndarray:
    """acc[m, n] = sum_k qa[m, k] * qw[n, k], exact, as int64.

    The fp64 product is exact: every term and partial sum is an integer of magnitude at
    most 127*127*K, below 2**53 for any K used here."""
    qa = np.asarray(qa)
    qw = np.asarray(qw)
    K = qa.shape[-1]
    assert qw.shape[-1] == K
    assert QMAX * QMAX * K < 2 ** 31, "int32 accumulator would overflow"
    return (qa.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)


def w8a8_linear(h, qw, sw) -> np.ndarray:
    """Dynamic per-token activation quantisation, int8 GEMM, dequant: acc * s_a * s_w."""
    qa, sa = quantize_rows(h)
    acc = int8_matmul(qa, qw)
    return acc.astype(np.float64) * sa.astype(np.float64)[:, None] * \
        np.asarray(sw, np.float64)[None, :]


# --------------------------------------------------------------------------- AdaLN
def adaln_modulation(w_ada, cond) -> np.ndarray:
    """m = W_ada c (a plain linear layer, no bias, no activation), fp64 [6d]."""
    return np.asarray(w_ada, np.float64) @ np.asarray(cond, np.float64)


def round_f32(v) -> np.ndarray:
    """Round to the nearest fp32 value (RNE), returned as fp64."""
    return np.asarray(v, np.float64).astype(np.float32).astype(np.float64)


def split_modulation(m, d: int) -> Dict[str, np.ndarray]:
    names = ("shift1", "scale1", "gate1", "shift2", "scale2", "gate2")
    return {k: m[i * d:(i + 1) * d] for i, k in enumerate(names)}


def layer_norm(x, eps: float = LN_EPS) -> np.ndarray:
    """Per-row LayerNorm without affine: (x - mean) / sqrt(var + eps), population var."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(n, shift, scale) -> np.ndarray:
    return n * (1.0 + scale) + shift


# --------------------------------------------------------------------------- RoPE
def rope_axis_pairs(head_dim: int) -> Tuple[int, int, int]:
    """Split of the head_dim/2 rotation pairs over the (t, h, w) axes: the h and w axes
    get floor(P/3) pairs each and t takes the rest (Dh=128 -> 22/21/21)."""
    P = head_dim // 2
    p3 = P // 3
    return P - 2 * p3, p3, p3


def token_positions(grid, w_scale: float = 1.0, w_offset: float = 0.0) -> np.ndarray:
    """Positions [L, 3] (t, h, w) for tokens l = (t*Hg + h)*Wg + w. With token pairing
    the reduced grid's w index j stands for position w_scale*j + w_offset (2j + 0.5)."""
    T, Hg, Wg = grid
    l = np.arange(T * Hg * Wg)
    t = l // (Hg * Wg)
    h = (l // Wg) % Hg
    w = l % Wg
    return np.stack([t, h, w * w_scale + w_offset], axis=1).astype(np.float64)


def rope_angles(pos, head_dim: int, theta: float = ROPE_THETA) -> np.ndarray:
    """Angle [L, Dh/2] of each rotation pair: pair j of axis a (P_a pairs on that axis)
    turns by pos_a * theta**(-j / P_a)."""
    counts = rope_axis_pairs(head_dim)
    cols = []
    for axis, P_a in enumerate(counts):
        j = np.arange(P_a, dtype=np.float64)
        cols.append(pos[:, axis:axis + 1] * theta ** (-j / P_a)[None, :])
    return np.concatenate(cols, axis=1)


def apply_rope(u, ang) -> np.ndarray:
    """Rotate interleaved pairs (u[2i], u[2i+1]) of u [L, H, Dh] by ang [L, Dh/2]."""
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = u[..., 0::2]
    b = u[..., 1::2]
    out = np.empty_like(u, dtype=np.float64)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


# --------------------------------------------------------------------------- attention
def attention(q, k, v, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Multi-head softmax attention, no mask. q, k, v [L, H, Dh] -> O [n, H, Dh] for the
    query rows `rows` (all rows if None). S = q k^T / sqrt(Dh); softmax over keys with
    the row maximum subtracted; O = P v."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if rows is not None:
        q = q[np.asarray(rows)]
    Dh = q.shape[-1]
    out = np.empty((q.shape[0], q.shape[1], Dh))
    for h in range(q.shape[1]):
        s = (q[:, h, :] @ k[:, h, :].T) / math.sqrt(Dh)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ v[:, h, :]
    return out


def gelu(z) -> np.ndarray:
    """Exact GELU: z * Phi(z) with the standard normal CDF Phi(z) = erfc(-z / sqrt(2)) / 2,
    the same function as z/2 * (1 + erf(z / sqrt(2))) written without the cancellation of
    1 + erf for negative z, so that the tail keeps its relative accuracy (Phi(-10) is
    7.6e-24; 1 + erf(-10 / sqrt 2) is 0 in fp64)."""
    from scipy.special import erfc
    z = np.asarray(z, np.float64)
    return 0.5 * z * erfc(-z / math.sqrt(2.0))


# --------------------------------------------------------------------------- block
def quantize_block_weights(wb: Dict[str, np.ndarray]) -> Dict[str, np.ndarray]:
    """Per-output-channel int8 quantisation of the four projection matrices."""
    out = {"w_ada": np.asarray(wb["w_ada"], np.float64)}
    for k in ("w_qkv", "w_o", "w_up", "w_down"):
        q, s = quantize_weights(wb[k])
        out["q" + k[1:]] = q
        out["s" + k[1:]] = s
        out[k] = np.asarray(wb[k], np.float64)
    return out


# Projections computed in W8A8 for each variant; the others use the dense weights with no
# activation quantisation. The two middle variants are the steps of the pages' precision
# series (page "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section
# "Int8 양자화": int8 MLP first, then int8 QKV on top of it).
INT8_PROJECTIONS = {
    "w8a8": ("_qkv", "_o", "_up", "_down"),
    "int8_mlp_qkv": ("_qkv", "_up", "_down"),
    "int8_mlp": ("_up", "_down"),
    "bf16gemm": (),
}


def _linear(h, w, name: str, variant: str, dense_inputs: str = "fp64") -> np.ndarray:
    """One projection. A dense (bf16) projection multiplies by the dense weights; with
    dense_inputs="bf16" its activation operand is first rounded to bfloat16, since a bf16
    GEMM takes bf16 operands (BF16 TensorOps projections: page "h3-metal: Apple Silicon을
    위한 네이티브 MiniMax-H3 추론", section "Metal 4 및 TensorOps")."""
    if variant not in INT8_PROJECTIONS:
        raise ValueError(variant)
    if name in INT8_PROJECTIONS[variant]:
        return w8a8_linear(h, w["q" + name], w["s" + name])
    if dense_inputs == "bf16":
        h = round_bf16(h)
    elif dense_inputs != "fp64":
        raise ValueError(dense_inputs)
    return h @ w["w" + name].T


def block_forward(x, cond, w, *, n_heads: int, head_dim: int, grid,
                  variant: str = "w8a8", rows: Optional[Sequence[int]] = None,
                  w_scale: float = 1.0, w_offset: float = 0.0,
                  eps: float = LN_EPS, theta: float = ROPE_THETA,
                  attn_inputs: str = "fp64", dense_inputs: str = "fp64",
                  act_store: str = "fp64", return_parts: bool = False):
    """One DiT block forward. x [L, d] (fp64 view of the input values), cond [d_cond];
    w holds w_ada and, per projection, int8 codes q_* with fp32 scales s_* and/or the
    dense matrices w_*. variant selects the projections computed in W8A8 (see
    INT8_PROJECTIONS): "w8a8" all, "int8_mlp_qkv" all but the output projection,
    "int8_mlp" the MLP only, "bf16gemm" none (dense, no activation quantisation).

    The plain definition is the default: every float exact (fp64), only the quantisers'
    decisions in fp32. The storage options below round the tensors a path hands from one
    kernel to the next, each as itself, where it is produced; they serve diagnosis and a
    path whose storage type is part of its definition (the fp32 debug path).
    attn_inputs: "fp64" keeps Q, K, V exact; "bf16", "fp16" or "fp32" rounds each of them
    (after RoPE) to that type before attention (page "h3-metal: Apple Silicon을 위한
    네이티브 MiniMax-H3 추론", section "Metal 4 및 TensorOps": the QKV projection routed into
    head-major attention inputs).
    dense_inputs: "fp64" multiplies dense projections by the exact activations; "bf16"
    rounds each dense projection's activation operand to bfloat16 first (see _linear).
    act_store: "fp64" keeps the attention output O, the residual stream x1, the GELU output
    g and the block output exact; "bf16" or "fp32" rounds each of them to that type where
    it is produced.

    rows: token rows whose output is wanted (all if None). Q, K and V are formed for
    every token (attention needs them); everything after attention is per token and is
    computed only for `rows`."""
    x = np.asarray(x, np.float64)
    L, d = x.shape
    assert d == n_heads * head_dim and L == grid[0] * grid[1] * grid[2]
    # the modulation is stored as an fp32 vector for the kernels that use it
    mod = split_modulation(round_f32(adaln_modulation(w["w_ada"], cond)), d)
    h = modulate(layer_norm(x, eps), mod["shift1"], mod["scale1"])
    y = _linear(h, w, "_qkv", variant, dense_inputs)
    q = y[:, 0:d].reshape(L, n_heads, head_dim)
    k = y[:, d:2 * d].reshape(L, n_heads, head_dim)
    v = y[:, 2 * d:3 * d].reshape(L, n_heads, head_dim)
    ang = rope_angles(token_positions(grid, w_scale, w_offset), head_dim, theta)
    q = apply_rope(q, ang)
    k = apply_rope(k, ang)
    rq = {"fp64": None, "bf16": round_bf16, "fp16": round_f16, "fp32": round_f32}
    if attn_inputs not in rq:
        raise ValueError(attn_inputs)
    if rq[attn_inputs] is not None:
        r = rq[attn_inputs]
        q, k, v = r(q), r(k), r(v)
    sel = np.arange(L) if rows is None else np.asarray(rows)
    if act_store == "bf16":
        store = round_bf16
    elif act_store == "fp32":
        store = round_f32
    elif act_store == "fp64":
        store = lambda t: t
    else:
        raise ValueError(act_store)
    o = store(attention(q, k, v, sel).reshape(len(sel), d))
    xs = x[sel]
    x1 = store(xs + mod["gate1"] * _linear(o, w, "_o", variant, dense_inputs))
    h2 = modulate(layer_norm(x1, eps), mod["shift2"], mod["scale2"])
    g = store(gelu(_linear(h2, w, "_up", variant, dense_inputs)))
    x2 = store(x1 + mod["gate2"] * _linear(g, w, "_down", variant, dense_inputs))
    if return_parts:
        return x2, {"m": np.concatenate([mod[k] for k in mod]), "h": h, "q": q, "k": k,
                    "v": v, "o": o, "x1": x1, "h2": h2, "g": g, "rows": sel}
    return x2


# --------------------------------------------------------------------------- token reduction
def token_pair(x, grid) -> np.ndarray:
    """Horizontal token pairing: xr[t, h, j] = (x[t, h, 2j] + x[t, h, 2j+1]) / 2.
    Page "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section
    "속도 및 품질 트레이드오프" (token reduction pairs horizontal video tokens in the
    middle blocks)."""
    T, Hg, Wg = grid
    assert Wg % 2 == 0
    x = np.asarray(x, np.float64).reshape(T, Hg, Wg // 2, 2, -1)
    return x.mean(axis=3).reshape(T * Hg * (Wg // 2), -1)


def token_unpair(x_pre, xr_out, xr_in, grid) -> np.ndarray:
    """x[t, h, 2j+s] = x_pre[t, h, 2j+s] + (xr_out[t, h, j] - xr_in[t, h, j]): both
    members of a pair receive the reduced blocks' update."""
    T, Hg, Wg = grid
    delta = (np.asarray(xr_out, np.float64) - np.asarray(xr_in, np.float64))
    delta = delta.reshape(T, Hg, Wg // 2, 1, -1)
    x = np.asarray(x_pre, np.float64).reshape(T, Hg, Wg // 2, 2, -1) + delta
    return x.reshape(T * Hg * Wg, -1)


def stack_forward(x, cond, blocks, *, n_heads: int, head_dim: int, grid,
                  tr_begin: int = 0, tr_end: int = 0, variant: str = "w8a8",
                  attn_inputs: str = "fp64", act_store: str = "fp64"):
    """Blocks 0..n-1 in order, sharing cond. Blocks [tr_begin, tr_end) run on the
    horizontally paired grid (T, Hg, Wg/2) with w positions 2j + 0.5. With act_store
    "bf16" the paired and unpaired token tensors are rounded to bfloat16 as well."""
    x = np.asarray(x, np.float64)
    T, Hg, Wg = grid
    tr_on = tr_end > tr_begin
    x_pre = xr_in = None
    for b, w in enumerate(blocks):
        if tr_on and b == tr_begin:
            x_pre = x
            x = token_pair(x, grid)
            if act_store == "bf16":
                x = round_bf16(x)
            xr_in = x
        if tr_on and tr_begin <= b < tr_end:
            x = block_forward(x, cond, w, n_heads=n_heads, head_dim=head_dim,
                              grid=(T, Hg, Wg // 2), variant=variant,
                              w_scale=2.0, w_offset=0.5, attn_inputs=attn_inputs,
                              act_store=act_store)
        else:
            x = block_forward(x, cond, w, n_heads=n_heads, head_dim=head_dim,
                              grid=grid, variant=variant, attn_inputs=attn_inputs,
                              act_store=act_store)
        if tr_on and b == tr_end - 1:
            x = token_unpair(x_pre, x, xr_in, grid)
            if act_store == "bf16":
                x = round_bf16(x)
    return x


# --------------------------------------------------------------------------- denoising loop
def fresh_steps(steps: int, reuse: int) -> list:
    """Steps k at which the whole denoiser is evaluated afresh: k % reuse == 0 and the last
    step (page "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section
    "속도 및 품질 트레이드오프": reuse cuts 20 passes to 11 or 8 fresh evaluations)."""
    return [k for k in range(steps) if k % reuse == 0 or k == steps - 1]


def denoise(x, core, *, steps: int, reuse: int = 1, core_reuse: int = 1,
            store_bf16: bool = False, store_f32: bool = False) -> np.ndarray:
    """Euler steps of a flow-matching sampler on t_k = 1 - k / steps (same page and section
    give the controls --steps, --reuse, --core-reuse; the formulas are the plainest reading):
    at fresh steps (fresh_steps) every core_reuse-th evaluation and the last one run the
    core, y = core(x), caching r = y - x and setting v = y; the other fresh steps set
    v = x + r; other steps keep v. Then x <- x + (t_{k+1} - t_k) v. core: callable on
    [L, d] arrays (the stack of the active blocks). store_bf16 rounds y and each new x to
    bfloat16, as the path that stores activations in bf16 does. store_f32 rounds y, r, a
    reused v and each new x to fp32, as a path that computes in fp64 and keeps the sampler
    state in fp32 does."""
    x = np.asarray(x, np.float64).copy()
    dt = -1.0 / steps
    fresh = set(fresh_steps(steps, reuse))
    v = r = None
    f = 0
    for k in range(steps):
        last = k == steps - 1
        if k in fresh:
            if f % core_reuse == 0 or last:
                y = core(x)
                if store_bf16:
                    y = round_bf16(y)
                if store_f32:
                    y = round_f32(y)
                r = y - x
                if store_f32:
                    r = round_f32(r)
                v = y
            else:
                v = x + r
                if store_f32:
                    v = round_f32(v)
            f += 1
        x = x + dt * v
        if store_bf16:
            x = round_bf16(x)
        if store_f32:
            x = round_f32(x)
    return x

