"""Teacher-forced stage-by-stage parity of one block run against the oracle: each oracle
stage is fed the GPU's own input to that stage, read from the block workspace."""
import numpy as np
import torch

import oracle as O
from tests._util import code_match, np64, oracle_weights, rel_l2
from video_diffusion_transformer_03_amd import h3k


def f32_stored(got, ref):
    """(fraction of elements identical to ref rounded to fp32, rel-L2 to it): a path that
    computes a stage in fp64 and stores it as fp32 matches the oracle's fp64 value rounded
    once, apart from the rare element whose two fp64 values straddle an fp32 rounding
    boundary (one ulp apart)."""
    r32 = O.round_f32(ref)
    return float(np.mean(got == r32)), rel_l2(got, r32)


def f32_stored_ok(got, ref):
    """f32_stored's bar: at most one element in 10^4 (and at least one element allowed)
    one rounding away, rel-L2 below 1e-8."""
    eq, rel = f32_stored(got, ref)
    return (1 - eq) * got.size <= max(1.0, 1e-4 * got.size) and rel < 1e-8, (eq, rel)


def check_stages(wl, r, rows, grid=None, w_scale=1.0, w_offset=0.0, label=None):
    """Teacher-forced per-stage parity on token rows `rows` (W8A8 path) of the block run
    recorded in `r` (inputs, weights, workspace); `grid` and the w-position mapping give
    the token grid the block ran on (default: the workload's)."""
    grid = wl.grid if grid is None else grid
    L = grid[0] * grid[1] * grid[2]
    d, F, H, Dh = wl.d, wl.d_ff, wl.n_heads, wl.head_dim
    f32 = bool(r["flags"] & h3k.F_FP32_DEBUG)
    T = torch.float32 if f32 else torch.bfloat16
    ws, lay = r["ws"], r["lay"]
    V = lambda n, dt, shape: h3k.ws_view(ws, lay, n, dt, shape)
    w = oracle_weights(r["bw"])
    rows = np.asarray(rows)
    tq = torch.as_tensor(rows, device="cuda")
    stats = {}

    m_gpu = np64(V("m", torch.float32, (6 * d,)))
    stats["m"] = rel_l2(m_gpu, O.adaln_modulation(w["w_ada"], np64(r["c"])))
    assert stats["m"] < 1e-6
    mod = O.split_modulation(m_gpu, d)

    x = np64(r["x"][tq])
    qa_ref, sa_ref = O.quantize_rows(O.modulate(O.layer_norm(x), mod["shift1"], mod["scale1"]))
    qa = V("qa", torch.int8, (L, d))[tq].cpu().numpy()
    sa = V("s_a", torch.float32, (L,))[tq].cpu().numpy()
    stats["qa_match"], mx = code_match(qa, qa_ref)
    assert stats["qa_match"] >= 0.9999 and mx <= 1
    assert np.allclose(sa, sa_ref, rtol=1e-6, atol=0)

    # QKV from the GPU's own codes and scales
    y = O.int8_matmul(qa, w["q_qkv"]) * sa.astype(np.float64)[:, None] * w["s_qkv"].astype(np.float64)
    ang = O.rope_angles(O.token_positions(grid, w_scale, w_offset)[rows], Dh)
    q_ref = O.apply_rope(y[:, :d].reshape(-1, H, Dh), ang)
    k_ref = O.apply_rope(y[:, d:2 * d].reshape(-1, H, Dh), ang)
    v_ref = y[:, 2 * d:].reshape(-1, H, Dh)
    q_all = V("q", T, (H, L, Dh))
    k_all = V("k", T, (H, L, Dh))
    vt_all = V("vt", T, (H, Dh, L))
    # on the bf16 path Q is stored with the base-2 softmax scale applied
    qs = 1.0 if f32 else O.q_handoff_scale(Dh)
    q_ref = q_ref * qs
    q_g = np64(q_all[:, tq, :]).transpose(1, 0, 2)
    k_g = np64(k_all[:, tq, :]).transpose(1, 0, 2)
    v_g = np64(vt_all[:, :, tq]).transpose(2, 0, 1)
    if f32:  # fp64 dequant and RoPE, one rounding to fp32
        for n, g_, ref in (("q", q_g, q_ref), ("k", k_g, k_ref), ("v", v_g, v_ref)):
            ok, (stats[n + "_eq"], stats[n]) = f32_stored_ok(g_, ref)
            assert ok, stats
    else:
        stats["q"], stats["k"], stats["v"] = rel_l2(q_g, q_ref), rel_l2(k_g, k_ref), rel_l2(v_g, v_ref)
        assert max(stats["q"], stats["k"], stats["v"]) < 4e-3, stats

    # attention rows from the GPU's full Q, K, V (O stored in the activation type)
    qf = np64(q_all).transpose(1, 0, 2) / qs
    kf = np64(k_all).transpose(1, 0, 2)
    vf = np64(vt_all).transpose(2, 0, 1)
    o_ref = O.attention(qf, kf, vf, rows).reshape(len(rows), d)
    o_g = np64(V("o", T, (L, d))[tq])
    if f32:  # fp64 attention, O rounded once to fp32
        ok, (stats["o_eq"], stats["o"]) = f32_stored_ok(o_g, o_ref)
        assert ok, stats
    else:
        stats["o"] = rel_l2(o_g, o_ref)
        assert stats["o"] < 1e-2, stats

    # quantiser of O on the GPU's own tensor: identical codes
    qo, so = O.quantize_rows(o_g)
    assert np.array_equal(V("qo", torch.int8, (L, d))[tq].cpu().numpy(), qo)
    assert np.array_equal(V("s_o", torch.float32, (L,))[tq].cpu().numpy(), so)

    # out-projection + gated residual from the GPU's O codes
    x1_ref = x + mod["gate1"] * (O.int8_matmul(qo, w["q_o"]) * so.astype(np.float64)[:, None] * w["s_o"])
    x1 = np64(V("x1", T, (L, d))[tq])
    if f32:
        ok, (stats["x1_eq"], stats["x1"]) = f32_stored_ok(x1, x1_ref)
        assert ok, stats
    else:
        stats["x1"] = rel_l2(x1, O.round_bf16(x1_ref))
        assert stats["x1"] < 1e-4, stats

    # second LN + quantiser from the GPU's x1
    qa2_ref, sa2_ref = O.quantize_rows(O.modulate(O.layer_norm(x1), mod["shift2"], mod["scale2"]))
    qa2 = V("qa2", torch.int8, (L, d))[tq].cpu().numpy()
    sa2 = V("s_a2", torch.float32, (L,))[tq].cpu().numpy()
    stats["qa2_match"], mx = code_match(qa2, qa2_ref)
    assert stats["qa2_match"] >= 0.9999 and mx <= 1
    assert np.allclose(sa2, sa2_ref, rtol=1e-6, atol=0)

    # MLP up + GELU from the GPU's codes
    u_ref = O.int8_matmul(qa2, w["q_up"]) * sa2.astype(np.float64)[:, None] * w["s_up"]
    g_ref = O.gelu(u_ref)
    g_g = np64(V("g", T, (L, F))[tq])
    if f32:
        ok, (stats["g_eq"], stats["g"]) = f32_stored_ok(g_g, g_ref)
        assert ok, stats
        # pointwise: fp64 GELU rounded to fp32, within one ulp (2^-23 relative) of the exact value
        bound = 2.0 ** -23 * np.abs(g_ref) + 1e-45
    else:
        stats["g"] = rel_l2(g_g, O.round_bf16(g_ref))
        assert stats["g"] < 1e-4, stats
        # pointwise: the fp32 dequant and the erf approximation stay within 1e-6 (1 + |u|);
        # storing g in bf16 (8 significant bits) adds at most 2^-8 of |g|
        bound = 1e-6 * (1 + np.abs(u_ref)) + 2.0 ** -8 * (np.abs(g_ref) + 1e-6 * (1 + np.abs(u_ref)))
    stats["g_pw"] = float(np.max(np.abs(g_g - g_ref) / bound))
    assert stats["g_pw"] <= 1.0, stats
    qg, sg = O.quantize_rows(g_g)
    stats["qg_match"], _ = code_match(V("qg", torch.int8, (L, F))[tq].cpu().numpy(), qg)
    assert stats["qg_match"] == 1.0
    assert np.array_equal(V("s_g", torch.float32, (L,))[tq].cpu().numpy(), sg)

    # MLP down + gated residual from the GPU's codes and x1
    x2_ref = x1 + mod["gate2"] * (O.int8_matmul(qg, w["q_down"]) * sg.astype(np.float64)[:, None] * w["s_down"])
    x2 = np64(r["out"][tq])
    if f32:
        ok, (stats["x2_eq"], stats["x2"]) = f32_stored_ok(x2, x2_ref)
    else:
        stats["x2"] = rel_l2(x2, x2_ref)
    print(label or wl.name, {k: (f"{v:.3e}" if isinstance(v, float) else v) for k, v in stats.items()})
    if f32:
        assert ok, stats
    else:
        assert stats["x2"] < 4e-3, stats
    return stats


def code_forced_output(wl, r, rows, grid=None, w_scale=1.0, w_offset=0.0):
    """The oracle's block output on `rows` with every quantiser's integer codes taken from
    the GPU run in `r` (qa for all tokens, qo, qa2 and qg for `rows`); everything else (scales,
    int8 products, RoPE, attention, LayerNorm, GELU, residuals) is the oracle's own. Codes may
    legitimately differ at near-ties between fp32 and fp64 inputs; forcing them isolates the
    float arithmetic of the path from the way a flipped code spreads (a flipped code changes a
    token's Q, K and V, and attention hands that to every query). The tensors the path stores
    are rounded as it stores them: the modulation to fp32, and Q, K, V, O, x1, g and the output
    to bf16 (Q times the base-2 softmax scale), or to fp32 on the debug path."""
    grid = wl.grid if grid is None else grid
    L = grid[0] * grid[1] * grid[2]
    d, F, H, Dh = wl.d, wl.d_ff, wl.n_heads, wl.head_dim
    f32 = bool(r["flags"] & h3k.F_FP32_DEBUG)
    rb = O.round_f32 if f32 else O.round_bf16
    ws, lay = r["ws"], r["lay"]
    V = lambda n, dt, shape: h3k.ws_view(ws, lay, n, dt, shape)
    w = oracle_weights(r["bw"])
    rows = np.asarray(rows)
    tq = torch.as_tensor(rows, device="cuda")
    codes = lambda n, cols: V(n, torch.int8, (L, cols))[tq].cpu().numpy()

    mod = O.split_modulation(O.round_f32(O.adaln_modulation(w["w_ada"], np64(r["c"]))), d)
    x = np64(r["x"])
    _, sa = O.quantize_rows(O.modulate(O.layer_norm(x), mod["shift1"], mod["scale1"]))
    qa = V("qa", torch.int8, (L, d)).cpu().numpy()
    y = O.int8_matmul(qa, w["q_qkv"]) * sa.astype(np.float64)[:, None] * w["s_qkv"]
    ang = O.rope_angles(O.token_positions(grid, w_scale, w_offset), Dh)
    q = O.apply_rope(y[:, :d].reshape(L, H, Dh), ang)
    k = O.apply_rope(y[:, d:2 * d].reshape(L, H, Dh), ang)
    v = y[:, 2 * d:].reshape(L, H, Dh)
    if f32:
        q, k, v = O.round_f32(q), O.round_f32(k), O.round_f32(v)
    else:
        c = O.q_handoff_scale(Dh)
        q, k, v = O.round_bf16(q * c) / c, O.round_bf16(k), O.round_bf16(v)
    o = rb(O.attention(q, k, v, rows).reshape(len(rows), d))
    _, so = O.quantize_rows(o)
    x1 = rb(x[rows] + mod["gate1"] * (O.int8_matmul(codes("qo", d), w["q_o"]) *
                                      so.astype(np.float64)[:, None] * w["s_o"]))
    _, sa2 = O.quantize_rows(O.modulate(O.layer_norm(x1), mod["shift2"], mod["scale2"]))
    g = rb(O.gelu(O.int8_matmul(codes("qa2", d), w["q_up"]) * sa2.astype(np.float64)[:, None] *
                  w["s_up"]))
    _, sg = O.quantize_rows(g)
    return rb(x1 + mod["gate2"] * (O.int8_matmul(codes("qg", F), w["q_down"]) *
                                   sg.astype(np.float64)[:, None] * w["s_down"]))
