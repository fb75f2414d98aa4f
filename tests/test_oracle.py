"""Pins for the CPU oracle: each check comes from something other than the oracle's own
formula (brute force on tiny inputs, library routines, closed forms, invariants,
textbook values). CPU only."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def _bf16(a):
    return torch.tensor(np.asarray(a), dtype=torch.float32).to(torch.bfloat16).float().numpy().astype(np.float64)


# ----------------------------------------------------------------------------- quantiser
def test_quant_golden_rows():
    for line in open(os.path.join(GOLD, "quant_ties.txt")):
        if line.startswith("#") or not line.strip():
            continue
        vals, codes, scale = [p.split() for p in line.split("|")]
        q, s = O.quantize_rows(np.array([float(v) for v in vals])[None, :])
        assert q[0].tolist() == [int(c) for c in codes]
        assert float(s[0]) == float(scale[0])


@pytest.mark.parametrize("K", [7, 64, 5120])
def test_quant_invariants(K):
    v = rng.standard_normal((33, K)) * rng.uniform(0.01, 50, size=(33, 1))
    v[3, 5 % K] *= 40.0  # outlier
    q, s = O.quantize_rows(v)
    v32 = v.astype(np.float32).astype(np.float64)
    # scale is the fp32 row absmax over 127
    assert np.array_equal(s, (np.abs(v.astype(np.float32)).max(1) / np.float32(127)).astype(np.float32))
    # reconstruction error within half a step (plus fp32 rounding of the reciprocal)
    err = np.abs(v32 - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 1e-4))
    # the absmax element maps to +-127
    j = np.abs(v32).argmax(1)
    assert np.all(np.abs(q[np.arange(33), j]) == 127)
    assert q.min() >= -127
    # odd symmetry
    qn, sn = O.quantize_rows(-v)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # re-quantising the dequantised row gives back the same codes
    q2, _ = O.quantize_rows(O.dequantize_rows(q, s))
    assert np.array_equal(q2, q)


def test_quant_zero_row():
    q, s = O.quantize_rows(np.zeros((2, 9)))
    assert np.all(q == 0) and np.all(s == 0)


# ----------------------------------------------------------------------------- bf16 rounding
def test_round_bf16_vs_torch_and_ties():
    v32 = (rng.standard_normal(20000) * rng.uniform(1e-3, 1e3, 20000)).astype(np.float32)
    want = torch.tensor(v32).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(O.round_bf16(v32.astype(np.float64)), want)
    one = 1.0
    ulp = 2.0 ** -7  # bf16 spacing just above 1
    assert O.round_bf16(one + ulp / 2) == one              # tie -> even (1.0)
    assert O.round_bf16(one + 3 * ulp / 2) == one + 2 * ulp  # tie -> even
    assert O.round_bf16(one + ulp / 2 + 1e-12) == one + ulp  # above the tie
    assert O.round_bf16(-(one + ulp / 2 + 1e-12)) == -(one + ulp)
    assert O.round_bf16(0.0) == 0.0


def test_round_f16_vs_library_and_ties():
    # normal, subnormal and overflowing magnitudes against numpy's binary16 conversion
    v = rng.standard_normal(40000) * np.exp(rng.uniform(-26 * math.log(2), 17 * math.log(2), 40000))
    with np.errstate(over="ignore"):
        want = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(O.round_f16(v), want)
    ulp = 2.0 ** -10  # fp16 spacing just above 1
    assert O.round_f16(1 + ulp / 2) == 1.0                  # tie -> even
    assert O.round_f16(1 + 3 * ulp / 2) == 1 + 2 * ulp      # tie -> even
    assert O.round_f16(-(1 + ulp / 2 + 1e-12)) == -(1 + ulp)
    sub = 2.0 ** -24  # smallest subnormal
    assert O.round_f16(sub / 2) == 0.0                      # tie -> even (0)
    assert O.round_f16(3 * sub / 2) == 2 * sub              # tie -> even
    assert O.round_f16(2.0 ** -14 + sub / 2) == 2.0 ** -14  # the normal range starts at 2^-14
    assert O.round_f16(65504.0) == 65504.0
    assert O.round_f16(65519.9) == 65504.0
    assert O.round_f16(65520.0) == np.inf                   # tie -> even: 2^16, out of range
    assert O.round_f16(-70000.0) == -np.inf and O.round_f16(0.0) == 0.0


# ----------------------------------------------------------------------------- int8 GEMM
def test_int8_matmul_bruteforce():
    a = rng.integers(-127, 128, size=(5, 11)).astype(np.int8)
    b = rng.integers(-127, 128, size=(6, 11)).astype(np.int8)
    acc = O.int8_matmul(a, b)
    for m in range(5):
        for n in range(6):
            assert acc[m, n] == sum(int(a[m, k]) * int(b[n, k]) for k in range(11))


def test_int8_matmul_extremes():
    K = 20480
    a = np.full((2, K), -127, np.int8)
    b = np.full((3, K), 127, np.int8)
    acc = O.int8_matmul(a, b)
    assert np.all(acc == -127 * 127 * K)
    b[1, ::2] = -127
    assert O.int8_matmul(a, b)[0, 1] == 0


# ----------------------------------------------------------------------------- AdaLN / LN
def test_adaln_bruteforce():
    w = rng.standard_normal((12, 5))
    c = rng.standard_normal(5)
    m = O.adaln_modulation(w, c)
    for i in range(12):
        assert math.isclose(m[i], math.fsum(w[i, j] * c[j] for j in range(5)), rel_tol=1e-12, abs_tol=1e-14)
    parts = O.split_modulation(m, 2)
    assert list(parts) == ["shift1", "scale1", "gate1", "shift2", "scale2", "gate2"]
    assert np.array_equal(parts["gate1"], m[4:6])


def test_layer_norm_vs_torch():
    x = rng.standard_normal((17, 320)) * 3 + 1.5
    ref = torch.nn.functional.layer_norm(torch.tensor(x), (320,), eps=1e-6).numpy()
    assert np.allclose(O.layer_norm(x), ref, rtol=1e-12, atol=1e-12)
    n = O.layer_norm(x)
    var = x.var(axis=1)
    assert np.allclose(n.mean(1), 0, atol=1e-12)
    assert np.allclose(n.var(1), var / (var + 1e-6), rtol=1e-12)


def test_modulate_special_cases():
    n = rng.standard_normal((3, 4))
    z = np.zeros(4)
    assert np.array_equal(O.modulate(n, z, z), n)
    sh = rng.standard_normal(4)
    assert np.allclose(O.modulate(n, sh, -np.ones(4)), np.broadcast_to(sh, n.shape))


# ----------------------------------------------------------------------------- RoPE
def test_rope_axis_split():
    assert O.rope_axis_pairs(128) == (22, 21, 21)
    assert O.rope_axis_pairs(64) == (12, 10, 10)
    assert O.rope_axis_pairs(6) == (1, 1, 1)


def test_rope_angles_closed_form():
    grid = (4, 5, 6)
    pos = O.token_positions(grid)
    ang = O.rope_angles(pos, 128)
    l = (2 * 5 + 3) * 6 + 4  # t=2, h=3, w=4
    assert tuple(pos[l]) == (2, 3, 4)
    assert ang[l, 0] == 2 and ang[l, 22] == 3 and ang[l, 43] == 4
    assert math.isclose(ang[l, 1], 2 * 10000 ** (-1 / 22), rel_tol=1e-14)
    assert math.isclose(ang[l, 22 + 20], 3 * 10000 ** (-20 / 21), rel_tol=1e-14)
    assert math.isclose(ang[l, 63], 4 * 10000 ** (-20 / 21), rel_tol=1e-14)
    pr = O.token_positions(grid, 2.0, 0.5)
    assert pr[l, 2] == 8.5


def test_rope_complex_and_invariants():
    grid = (3, 4, 4)
    L, H, Dh = 48, 2, 64
    u = rng.standard_normal((L, H, Dh))
    ang = O.rope_angles(O.token_positions(grid), Dh)
    r = O.apply_rope(u, ang)
    z = (u[..., 0::2] + 1j * u[..., 1::2]) * np.exp(1j * ang)[:, None, :]
    assert np.allclose(r[..., 0::2], z.real, atol=1e-13) and np.allclose(r[..., 1::2], z.imag, atol=1e-13)
    assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(u, axis=-1), rtol=1e-13)
    assert np.array_equal(r[0], u[0])  # position (0,0,0) is the identity
    # relative-position property: a common shift of every position along one axis
    # leaves all q.k scores unchanged
    q = rng.standard_normal((L, 1, Dh))
    k = rng.standard_normal((L, 1, Dh))
    pos = O.token_positions(grid)
    for axis in range(3):
        sh = pos.copy()
        sh[:, axis] += 7
        s0 = O.apply_rope(q, O.rope_angles(pos, Dh))[:, 0] @ O.apply_rope(k, O.rope_angles(pos, Dh))[:, 0].T
        s1 = O.apply_rope(q, O.rope_angles(sh, Dh))[:, 0] @ O.apply_rope(k, O.rope_angles(sh, Dh))[:, 0].T
        assert np.allclose(s0, s1, atol=1e-11)


# ----------------------------------------------------------------------------- attention
def test_attention_vs_sdpa():
    L, H, Dh = 40, 3, 16
    q, k, v = (rng.standard_normal((L, H, Dh)) * 2 for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(
        *(torch.tensor(t).permute(1, 0, 2) for t in (q, k, v))).permute(1, 0, 2).numpy()
    assert np.allclose(O.attention(q, k, v), ref, rtol=1e-11, atol=1e-12)
    assert np.allclose(O.attention(q, k, v, rows=[3, 17]), ref[[3, 17]], rtol=1e-11, atol=1e-12)


def test_attention_bruteforce_and_invariants():
    L, H, Dh = 6, 1, 4
    q, k, v = (rng.standard_normal((L, H, Dh)) for _ in range(3))
    o = O.attention(q, k, v)
    for i in range(L):
        s = [sum(q[i, 0, e] * k[j, 0, e] for e in range(Dh)) / 2.0 for j in range(L)]
        w = [math.exp(t) for t in s]
        z = math.fsum(w)
        for e in range(Dh):
            assert math.isclose(o[i, 0, e], math.fsum(w[j] / z * v[j, 0, e] for j in range(L)),
                                rel_tol=1e-10, abs_tol=1e-12)
    # constant V -> that row; L = 1 -> v; q = 0 -> mean of V
    vc = np.broadcast_to(rng.standard_normal((1, H, Dh)), (L, H, Dh))
    assert np.allclose(O.attention(q, k, vc), vc, atol=1e-13)
    assert np.allclose(O.attention(q[:1], k[:1], v[:1]), v[:1], atol=1e-15)
    assert np.allclose(O.attention(np.zeros_like(q), k, v), np.broadcast_to(v.mean(0), v.shape), atol=1e-13)


# ----------------------------------------------------------------------------- GELU
def test_gelu_textbook():
    for line in open(os.path.join(GOLD, "normal_cdf.txt")):
        if line.startswith("#") or not line.strip():
            continue
        z, phi = map(float, line.split())
        # relative accuracy everywhere, the deep negative tail included
        assert math.isclose(float(O.gelu(z)), z * phi, rel_tol=1e-12, abs_tol=0.0), z
    z = rng.standard_normal(100) * 4
    assert np.allclose(O.gelu(z) - O.gelu(-z), z, atol=1e-13)
    assert O.gelu(0.0) == 0.0


def test_normal_tail_fixture_matches_asymptotic_series():
    # the tail rows of the CDF fixture against A&S 26.2.12, summed to its 20th term
    for line in open(os.path.join(GOLD, "normal_cdf.txt")):
        if line.startswith("#") or not line.strip():
            continue
        z, phi = map(float, line.split())
        if z > -8:
            continue
        x = -z
        term, acc = 1.0, 0.0
        for n in range(20):
            acc += term
            term *= -(2 * n + 1) / (x * x)
        series = math.exp(-x * x / 2) / math.sqrt(2 * math.pi) / x * acc
        assert math.isclose(phi, series, rel_tol=1e-11), (z, phi, series)


# ----------------------------------------------------------------------------- block (brute force)
def _bf_block(x, c, w, H, Dh, grid, variant, w_scale=1.0, w_offset=0.0, round_dense=False,
              qkv_type=None, store_type=None):
    """Independent scalar-loop implementation of the block on tiny shapes. round_dense:
    dense projections take bf16-rounded activations; qkv_type ("bf16", "fp16", "fp32"):
    Q, K (after RoPE) and V are each rounded to that type before attention; store_type
    ("bf16", "fp32"): the attention output, the residual after the attention half, the GELU
    output and the block output are rounded to that type where they are produced. The
    roundings are library conversions (torch's to bf16, numpy's to fp16 and fp32)."""

    def rnd(vals, t):
        if t == "fp32":
            return [float(np.float32(v)) for v in vals]
        if t == "fp16":
            return np.asarray(vals, np.float64).astype(np.float16).astype(np.float64).tolist()
        return torch.tensor(vals, dtype=torch.float64).to(torch.bfloat16).double().tolist()

    def rq(vals):
        return rnd(vals, qkv_type) if qkv_type else vals

    def rs(vals):
        return rnd(vals, store_type) if store_type else vals
    L, d = len(x), len(x[0])
    F = len(w["w_up"])
    # the modulation is stored as fp32 (nearest, ties to even)
    m = [float(np.float32(math.fsum(w["w_ada"][i][j] * c[j] for j in range(len(c))))) for i in range(6 * d)]
    sh1, sc1, g1, sh2, sc2, g2 = (m[i * d:(i + 1) * d] for i in range(6))

    def ln_mod(row, sh, sc):
        mu = math.fsum(row) / d
        var = math.fsum((t - mu) ** 2 for t in row) / d
        r = 1.0 / math.sqrt(var + 1e-6)
        return [((row[i] - mu) * r) * (1 + sc[i]) + sh[i] for i in range(d)]

    def quant(row):
        a = float(np.float32(max(abs(float(np.float32(t))) for t in row)))
        if a == 0:
            return [0] * len(row), 0.0
        inv = np.float32(127) / np.float32(a)
        codes = []
        for t in row:
            p = float(np.float32(np.float32(t) * inv))
            fl = math.floor(p)
            rem = p - fl
            r = fl + 1 if rem > 0.5 or (rem == 0.5 and fl % 2 == 1) else fl
            codes.append(max(-127, min(127, int(r))))
        return codes, float(np.float32(a) / np.float32(127))

    int8 = {"w8a8": {"_qkv", "_o", "_up", "_down"}, "int8_mlp_qkv": {"_qkv", "_up", "_down"},
            "int8_mlp": {"_up", "_down"}, "bf16gemm": set()}[variant]

    def lin(row, name):
        if name in int8:
            codes, s = quant(row)
            Wq, Ws = w["q" + name], w["s" + name]
            return [sum(codes[k] * int(Wq[n][k]) for k in range(len(row))) * s * float(Ws[n])
                    for n in range(len(Wq))]
        Wd = w["w" + name]
        if round_dense:
            row = torch.tensor(row, dtype=torch.float64).to(torch.bfloat16).double().tolist()
        return [math.fsum(row[k] * Wd[n][k] for k in range(len(row))) for n in range(len(Wd))]

    T, Hg, Wg = grid
    P = Dh // 2
    counts = [P - 2 * (P // 3), P // 3, P // 3]

    def rope(vec, l):
        pos = [l // (Hg * Wg), (l // Wg) % Hg, (l % Wg) * w_scale + w_offset]
        out = list(vec)
        i = 0
        for ax in range(3):
            for j in range(counts[ax]):
                phi = pos[ax] * 10000.0 ** (-j / counts[ax])
                a, b = vec[2 * i], vec[2 * i + 1]
                out[2 * i] = a * math.cos(phi) - b * math.sin(phi)
                out[2 * i + 1] = a * math.sin(phi) + b * math.cos(phi)
                i += 1
        return out

    qkv = [lin(ln_mod(x[l], sh1, sc1), "_qkv") for l in range(L)]
    Q = [[rq(rope(qkv[l][e * Dh:(e + 1) * Dh], l)) for e in range(H)] for l in range(L)]
    K = [[rq(rope(qkv[l][d + e * Dh:d + (e + 1) * Dh], l)) for e in range(H)] for l in range(L)]
    V = [[rq(qkv[l][2 * d + e * Dh:2 * d + (e + 1) * Dh]) for e in range(H)] for l in range(L)]
    out = []
    for l in range(L):
        o = []
        for e in range(H):
            s = [sum(Q[l][e][i] * K[j][e][i] for i in range(Dh)) / math.sqrt(Dh) for j in range(L)]
            mx = max(s)
            p = [math.exp(t - mx) for t in s]
            z = math.fsum(p)
            o += [math.fsum(p[j] * V[j][e][i] for j in range(L)) / z for i in range(Dh)]
        y = lin(rs(o), "_o")
        x1 = rs([x[l][i] + g1[i] * y[i] for i in range(d)])
        u = lin(ln_mod(x1, sh2, sc2), "_up")
        g = rs([0.5 * t * (1 + math.erf(t / math.sqrt(2))) for t in u])
        y2 = lin(g, "_down")
        out.append(rs([x1[i] + g2[i] * y2[i] for i in range(d)]))
    return np.array(out)


def _tiny_weights(d, F, dc, seed):
    r = np.random.default_rng(seed)
    wb = {"w_ada": _bf16(r.standard_normal((6 * d, dc)) * 0.3),
          "w_qkv": _bf16(r.standard_normal((3 * d, d)) * 0.3),
          "w_o": _bf16(r.standard_normal((d, d)) * 0.3),
          "w_up": _bf16(r.standard_normal((F, d)) * 0.3),
          "w_down": _bf16(r.standard_normal((d, F)) * 0.3)}
    return O.quantize_block_weights(wb)


@pytest.mark.parametrize("variant", ["w8a8", "int8_mlp_qkv", "int8_mlp", "bf16gemm"])
def test_block_bruteforce_tiny(variant):
    d, H, Dh, F, dc, grid = 12, 2, 6, 24, 5, (2, 2, 2)
    w = _tiny_weights(d, F, dc, 7)
    r = np.random.default_rng(8)
    x = _bf16(r.standard_normal((8, d)))
    c = r.standard_normal(dc)
    got = O.block_forward(x, c, w, n_heads=H, head_dim=Dh, grid=grid, variant=variant)
    ref = _bf_block(x.tolist(), c.tolist(), {k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in w.items()},
                    H, Dh, grid, variant)
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-9)
    # reduced-grid positions (2j + 0.5) go through the same path
    got_r = O.block_forward(x, c, w, n_heads=H, head_dim=Dh, grid=grid, variant=variant,
                            w_scale=2.0, w_offset=0.5)
    ref_r = _bf_block(x.tolist(), c.tolist(), {k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in w.items()},
                      H, Dh, grid, variant, 2.0, 0.5)
    assert np.allclose(got_r, ref_r, rtol=1e-9, atol=1e-9)
    # row subsets are the same rows of the full output
    sub = O.block_forward(x, c, w, n_heads=H, head_dim=Dh, grid=grid, variant=variant, rows=[5, 1])
    assert np.array_equal(sub, got[[5, 1]])


@pytest.mark.parametrize("variant", ["int8_mlp", "bf16gemm"])
def test_block_bruteforce_dense_bf16_inputs(variant):
    d, H, Dh, F, dc, grid = 12, 2, 6, 24, 5, (2, 2, 2)
    w = _tiny_weights(d, F, dc, 11)
    r = np.random.default_rng(12)
    x = _bf16(r.standard_normal((8, d)))
    c = r.standard_normal(dc)
    got = O.block_forward(x, c, w, n_heads=H, head_dim=Dh, grid=grid, variant=variant,
                          dense_inputs="bf16")
    ref = _bf_block(x.tolist(), c.tolist(), {k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in w.items()},
                    H, Dh, grid, variant, round_dense=True)
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-9)
    # rounding the operands changes the result (the option is not a no-op)
    plain = O.block_forward(x, c, w, n_heads=H, head_dim=Dh, grid=grid, variant=variant)
    assert not np.allclose(got, plain, rtol=1e-9, atol=1e-9)


@pytest.mark.parametrize("variant", ["w8a8", "bf16gemm"])
@pytest.mark.parametrize("attn_inputs,act_store", [("bf16", "fp64"), ("fp64", "bf16"), ("bf16", "bf16"),
                                                   ("fp16", "fp64"), ("fp32", "fp32")])
def test_block_bruteforce_storage_options(variant, attn_inputs, act_store):
    d, H, Dh, F, dc, grid = 12, 2, 6, 24, 5, (2, 2, 2)
    w = _tiny_weights(d, F, dc, 13)
    r = np.random.default_rng(14)
    x = _bf16(r.standard_normal((8, d)))
    c = r.standard_normal(dc)
    got = O.block_forward(x, c, w, n_heads=H, head_dim=Dh, grid=grid, variant=variant,
                          attn_inputs=attn_inputs, act_store=act_store)
    ref = _bf_block(x.tolist(), c.tolist(), {k: (v.tolist() if hasattr(v, "tolist") else v) for k, v in w.items()},
                    H, Dh, grid, variant, qkv_type=None if attn_inputs == "fp64" else attn_inputs,
                    store_type=None if act_store == "fp64" else act_store)
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-9)
    plain = O.block_forward(x, c, w, n_heads=H, head_dim=Dh, grid=grid, variant=variant)
    assert not np.allclose(got, plain, rtol=1e-9, atol=1e-9)
    rnd = O.round_f32 if act_store == "fp32" else O.round_bf16
    if act_store != "fp64":
        assert np.array_equal(got, rnd(got))
    # the stored intermediates are values of the storage type and x2 is built from them
    x2, parts = O.block_forward(x, c, w, n_heads=H, head_dim=Dh, grid=grid, variant=variant,
                                attn_inputs=attn_inputs, act_store=act_store, return_parts=True)
    assert np.array_equal(x2, got)
    if act_store != "fp64":
        for name in ("o", "x1", "g"):
            assert np.array_equal(parts[name], rnd(parts[name])), name


def test_block_zero_gates_identity():
    d, H, Dh, F, dc, grid = 24, 2, 12, 48, 8, (2, 2, 4)
    w = _tiny_weights(d, F, dc, 9)
    for gate in (2, 5):  # zero the rows of W_ada that produce gate1 and gate2
        w["w_ada"][gate * d:(gate + 1) * d] = 0.0
    x = _bf16(np.random.default_rng(3).standard_normal((16, d)))
    out = O.block_forward(x, np.ones(dc), w, n_heads=H, head_dim=Dh, grid=grid)
    assert np.array_equal(out, x)


# ----------------------------------------------------------------------------- token reduction / stack
def test_token_pair_closed_form():
    grid = (2, 3, 4)
    x = rng.standard_normal((24, 5))
    xr = O.token_pair(x, grid)
    assert xr.shape == (12, 5)
    # token (t=1, h=2, j=1) pairs w = 2 and 3
    assert np.allclose(xr[(1 * 3 + 2) * 2 + 1], (x[(1 * 3 + 2) * 4 + 2] + x[(1 * 3 + 2) * 4 + 3]) / 2)
    dup = np.repeat(rng.standard_normal((12, 5)), 2, axis=0)
    assert np.array_equal(O.token_pair(dup, grid), dup[::2])
    # unpair with an unchanged reduced state gives back x exactly
    assert np.array_equal(O.token_unpair(x, xr, xr, grid), x)
    delta = rng.standard_normal((12, 5))
    up = O.token_unpair(x, xr + delta, xr, grid)
    assert np.allclose(up[(1 * 3 + 2) * 4 + 3] - x[(1 * 3 + 2) * 4 + 3], delta[(1 * 3 + 2) * 2 + 1])


def test_stack_composition_and_identity():
    d, H, Dh, F, dc, grid = 24, 2, 12, 48, 8, (2, 2, 4)
    blocks = [_tiny_weights(d, F, dc, 20 + b) for b in range(3)]
    x = _bf16(np.random.default_rng(4).standard_normal((16, d)))
    c = np.random.default_rng(5).standard_normal(dc)
    kw = dict(n_heads=H, head_dim=Dh, grid=grid)
    seq = x
    for w in blocks:
        seq = O.block_forward(seq, c, w, **kw)
    assert np.array_equal(O.stack_forward(x, c, blocks, **kw), seq)
    # with reduction on block 1: pair, run block 1 on the half-width grid, unpair
    y0 = O.block_forward(x, c, blocks[0], **kw)
    xr = O.token_pair(y0, grid)
    xr1 = O.block_forward(xr, c, blocks[1], n_heads=H, head_dim=Dh, grid=(2, 2, 2), w_scale=2.0, w_offset=0.5)
    y1 = O.token_unpair(y0, xr1, xr, grid)
    y2 = O.block_forward(y1, c, blocks[2], **kw)
    assert np.array_equal(O.stack_forward(x, c, blocks, tr_begin=1, tr_end=2, **kw), y2)
    # zero gates everywhere: the stack (with reduction) is the identity
    for w in blocks:
        w["w_ada"][2 * d:3 * d] = 0.0
        w["w_ada"][5 * d:6 * d] = 0.0
    assert np.array_equal(O.stack_forward(x, c, blocks, tr_begin=1, tr_end=3, **kw), x)


# ----------------------------------------------------------------------------- denoising loop
def test_fresh_steps_match_pages():
    # page "h3-metal: Apple Silicon을 위한 네이티브 MiniMax-H3 추론", section "속도 및 품질
    # 트레이드오프": reuse 2 and 3 cut 20 denoising passes to 11 and 8 fresh DiT evaluations
    assert len(O.fresh_steps(20, 1)) == 20
    assert len(O.fresh_steps(20, 2)) == 11
    assert len(O.fresh_steps(20, 3)) == 8
    assert O.fresh_steps(4, 2) == [0, 2, 3]


def test_denoise_linear_core_closed_forms():
    """With a linear core y = a x the Euler sampler has products of (1 + c dt a) factors."""
    a = 0.7
    x0 = np.array([[1.0, -2.0, 0.5]])
    core = lambda x: a * x  # noqa: E731
    # no reuse: x_N = x_0 (1 + dt a)^N
    N = 6
    got = O.denoise(x0, core, steps=N)
    assert np.allclose(got, x0 * (1 - a / N) ** N, rtol=1e-14, atol=0)
    # whole reuse 2, 4 steps: fresh at k = 0, 2, 3 -> x_4 = x_0 (1 + 2 dt a)(1 + dt a)^2
    dt = -1 / 4
    got = O.denoise(x0, core, steps=4, reuse=2)
    assert np.allclose(got, x0 * (1 + 2 * dt * a) * (1 + dt * a) ** 2, rtol=1e-14, atol=0)
    # core reuse 2, 3 steps: k=0 runs the core (r = (a-1) x_0), k=1 uses v = x_1 + r,
    # k=2 (last) runs the core again
    dt = -1 / 3
    x1 = x0 * (1 + dt * a)
    x2 = x1 + dt * (x1 + (a - 1) * x0)
    x3 = x2 * (1 + dt * a)
    got = O.denoise(x0, core, steps=3, core_reuse=2)
    assert np.allclose(got, x3, rtol=1e-14, atol=0)
    # store_bf16 rounds every state: the result is exactly representable in bf16
    got = O.denoise(x0, core, steps=3, store_bf16=True)
    assert np.array_equal(got, O.round_bf16(got))
    # store_f32 likewise in fp32, and within fp32 rounding of the exact closed form
    core32 = lambda x: O.round_f32(a * x)  # noqa: E731
    got = O.denoise(x0, core32, steps=3, core_reuse=2, store_f32=True)
    assert np.array_equal(got, O.round_f32(got))
    assert np.allclose(got, x3, rtol=1e-6, atol=0) and not np.array_equal(got, x3)
