"""The oracle's CPU twin of the C ABI (h3k_ref_*): argument order and layouts, the flag ->
precision mapping, and the return codes. The twin only marshals; its arithmetic is the
oracle's, which the oracle tests pin."""
import math
from types import SimpleNamespace

import numpy as np
import pytest

import oracle as O
from oracle import ref_abi as R

H, DH, F, DC = 2, 8, 32, 8
D = H * DH
GRID = (2, 2, 4)
L = GRID[0] * GRID[1] * GRID[2]


def _dims(**kw):
    base = dict(d=D, n_heads=H, head_dim=DH, d_ff=F, d_cond=DC, grid_t=GRID[0], grid_h=GRID[1],
                grid_w=GRID[2], rope_theta=np.float32(O.ROPE_THETA), ln_eps=np.float32(O.LN_EPS))
    base.update(kw)
    return SimpleNamespace(**base)


def _weights(seed):
    """C-struct field names; int8 codes made by the twin's own quantiser entry point."""
    rng = np.random.default_rng(seed)
    w = {"w_ada": rng.standard_normal((6 * D, DC)) * 0.1}
    for k, (n, kk) in {"qkv": (3 * D, D), "o": (D, D), "up": (F, D), "down": (D, F)}.items():
        dense = rng.standard_normal((n, kk)) * 0.2
        q, s = np.zeros((n, kk), np.int8), np.zeros(n, np.float32)
        assert R.h3k_ref_quantize_weights(dense, R.DT_F32, n, kk, q, s) == R.OK
        w["w_" + k], w["s_" + k], w["wb_" + k] = q, s, dense
    return w


def _inputs(seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((L, D)), rng.standard_normal(DC)


def _oracle_w(w, dense):
    o = {"w_ada": w["w_ada"]}
    for k in ("qkv", "o", "up", "down"):
        o["q_" + k], o["s_" + k] = w["w_" + k], w["s_" + k]
        if dense:
            o["w_" + k] = w["wb_" + k]
    return o


def test_quantize_weights_twin():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((5, 7))
    q, s = np.zeros((5, 7), np.int8), np.zeros(5, np.float32)
    assert R.h3k_ref_quantize_weights(w, R.DT_BF16, 5, 7, q, s) == R.OK
    q_ref, s_ref = O.quantize_weights(w)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)
    assert R.h3k_ref_quantize_weights(w, R.DT_F32, 5, 6, q, s) == R.EINVAL
    assert R.h3k_ref_quantize_weights(w, 7, 5, 7, q, s) == R.EINVAL


@pytest.mark.parametrize("flags,variant,store", [
    (0, "w8a8", "fp64"), (R.F_ATTN_BF16, "w8a8", "fp64"), (R.F_FP32_DEBUG, "w8a8", "fp32"),
    (R.F_BF16_OUT, "int8_mlp_qkv", "fp64"), (R.F_BF16_QKV | R.F_BF16_OUT, "int8_mlp", "fp64"),
    (R.F_BF16_GEMM, "bf16gemm", "fp64"), (R.F_BF16_QKV | R.F_BF16_OUT | R.F_BF16_MLP, "bf16gemm", "fp64")])
def test_block_twin_maps_flags_to_the_precision_series(flags, variant, store):
    # the 16-bit paths' twin is the plain definition; the fp32 debug path's stores fp32
    w = _weights(1)
    x, c = _inputs()
    out = np.zeros((L, D), np.float64)
    assert R.h3k_ref_block_forward(x, out, c, w, _dims(), L, flags) == R.OK
    ref = O.block_forward(x, c, _oracle_w(w, variant != "w8a8"), n_heads=H, head_dim=DH, grid=GRID,
                          variant=variant, eps=float(np.float32(O.LN_EPS)), attn_inputs=store,
                          act_store=store)
    assert np.array_equal(out, ref)
    if store == "fp32":  # the output holds fp32 values
        assert np.array_equal(out, O.round_f32(out))
    # an fp32 output array receives the values rounded to fp32 once
    out32 = np.zeros((L, D), np.float32)
    assert R.h3k_ref_block_forward(x, out32, c, w, _dims(), L, flags) == R.OK
    assert np.array_equal(out32, ref.astype(np.float32))


def test_block_grid_twin_positions():
    # the explicit-grid call with scale 2 and offset 0.5 is the paired blocks' RoPE
    w = _weights(2)
    rng = np.random.default_rng(4)
    g2 = (GRID[0], GRID[1], GRID[2] // 2)
    n = g2[0] * g2[1] * g2[2]
    x, c = rng.standard_normal((n, D)), rng.standard_normal(DC)
    out = np.zeros((n, D))
    assert R.h3k_ref_block_forward_grid(x, out, c, w, _dims(), *g2, 2.0, 0.5, 0) == R.OK
    ref = O.block_forward(x, c, _oracle_w(w, False), n_heads=H, head_dim=DH, grid=g2, w_scale=2.0,
                          w_offset=0.5, eps=float(np.float32(O.LN_EPS)))
    assert np.array_equal(out, ref)


@pytest.mark.parametrize("dtype", [R.DT_BF16, R.DT_F16, R.DT_F32])
def test_attention_twin_layouts_bruteforce(dtype):
    # explicit loops over the C ABI's layouts: q, k [H, L, Dh], v [H, Dh, L], o [L, H*Dh];
    # a softmax scale other than 1/sqrt(Dh)
    rng = np.random.default_rng(5)
    h, n, dh, scale = 3, 6, 4, 0.37
    q, k, v = rng.standard_normal((h, n, dh)), rng.standard_normal((h, n, dh)), rng.standard_normal((h, dh, n))
    o = np.zeros((n, h * dh))
    assert R.h3k_ref_attention(q, k, v, o, h, n, dh, scale, dtype, 0) == R.OK
    ref = np.zeros((n, h * dh))
    for e in range(h):
        for i in range(n):
            s = [scale * sum(q[e, i, t] * k[e, j, t] for t in range(dh)) for j in range(n)]
            mx = max(s)
            p = [math.exp(a - mx) for a in s]
            z = sum(p)
            for t in range(dh):
                ref[i, e * dh + t] = sum(p[j] * v[e, t, j] for j in range(n)) / z
    # o holds values of the dtype, each within half a unit in the last place of the loop's
    # value (a value within rounding error of a boundary may go either way: one ulp)
    store, ulp = {R.DT_F32: (O.round_f32, 2.0 ** -23), R.DT_F16: (O.round_f16, 2.0 ** -10),
                  R.DT_BF16: (O.round_bf16, 2.0 ** -7)}[dtype]
    assert np.array_equal(o, store(o))
    assert np.max(np.abs(o - store(ref)) / np.abs(ref)) <= ulp
    assert np.allclose(o, ref, rtol=ulp / 2 * 1.0001, atol=0)
    # base-2 logits: q carrying scale * log2(e) gives the same attention (16-bit dtypes only)
    ob = np.zeros((n, h * dh))
    rc = R.h3k_ref_attention(q * (scale * math.log2(math.e)), k, v, ob, h, n, dh, scale, dtype, R.F_Q_BASE2)
    if dtype == R.DT_F32:
        assert rc == R.EINVAL
    else:
        assert rc == R.OK
        assert np.array_equal(ob, store(ob))
        assert np.max(np.abs(ob - store(ref)) / np.abs(ref)) <= ulp
    assert R.h3k_ref_attention(q, k, v, o, h, n, dh, 0.0, dtype, 0) == R.EINVAL
    assert R.h3k_ref_attention(q, k, v, o, h, n + 1, dh, scale, dtype, 0) == R.EINVAL
    assert R.h3k_ref_attention(q, k, v, o, h, n, dh, scale, 9, 0) == R.EINVAL


def test_stack_twin_matches_the_oracle_stack():
    blocks = [_weights(10 + b) for b in range(3)]
    x, c = _inputs(6)
    out = np.zeros((L, D))
    for tr in [(0, 0), (1, 2), (0, 3)]:
        assert R.h3k_ref_stack_forward(x, out, c, blocks, 3, _dims(), L, *tr, 0) == R.OK
        ref = O.stack_forward(x, c, [_oracle_w(b, False) for b in blocks], n_heads=H, head_dim=DH,
                              grid=GRID, tr_begin=tr[0], tr_end=tr[1])
        assert np.array_equal(out, ref), tr


def test_return_codes():
    w = _weights(7)
    x, c = _inputs()
    out = np.zeros((L, D))
    ok = R.h3k_ref_block_forward
    assert ok(x, out, c, w, _dims(), L, 0) == R.OK
    assert ok(x, out, c, w, _dims(n_heads=3), L, 0) == R.EINVAL          # d != H * Dh
    assert ok(x, out, c, w, _dims(), L - 1, 0) == R.EINVAL                # L != T * Hg * Wg
    assert ok(x, out, c, w, _dims(ln_eps=0.0), L, 0) == R.EINVAL
    assert ok(x[:-1], out, c, w, _dims(), L, 0) == R.EINVAL               # wrong buffer size
    assert ok(x, out, c, w, _dims(), L, R.F_BF16_MLP) == R.EUNSUPPORTED  # not in the series
    assert ok(x, out, c, w, _dims(), L, 1 << 12) == R.EINVAL              # unknown flag bit
    st = R.h3k_ref_stack_forward
    blocks = [w, w]
    assert st(x, out, c, blocks, 2, _dims(), L, 2, 1, 0) == R.EINVAL       # tr_begin > tr_end
    assert st(x, out, c, blocks, 2, _dims(), L, 0, 3, 0) == R.EINVAL       # beyond n_blocks
    assert st(x, out, c, blocks, 3, _dims(), L, 0, 0, 0) == R.EINVAL       # fewer blocks given
    odd = _dims(grid_w=3, grid_h=4, grid_t=4, d=D)
    x12 = np.zeros((48, D))
    assert st(x12, np.zeros((48, D)), c, blocks, 2, odd, 48, 0, 1, 0) == R.EINVAL  # odd grid_w
    assert st(x, out, c, blocks, 2, _dims(), L, 0, 0, R.F_BF16_GEMM) == R.EUNSUPPORTED
    assert st(x, out, c, blocks, 2, _dims(rope_theta=np.float32(500.0)), L, 0, 0, 0) == R.EUNSUPPORTED
