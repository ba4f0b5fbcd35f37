"""Pins of the oracle's float64 arithmetic against closed forms, library routines,
invariants and brute force on tiny inputs.

Each test is chosen so that a plausible slip in ``oracle/dit.py`` (a transposed weight, a
dropped term, a wrong sign or index, the wrong axis) fails it.  Library routines used as
independent references: torch.nn.functional (layer_norm, rms_norm, linear,
scaled_dot_product_attention, gelu) in float64 on the CPU, math.erf, complex arithmetic.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as tF

from oracle import dit, host

RNG = np.random.default_rng(1234)


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


# ----------------------------------------------------------------- timestep / modulation
def test_timestep_embedding_closed_forms():
    e0 = dit.timestep_embedding(0.0)
    np.testing.assert_array_equal(e0[:128], 1.0)   # cos half first
    np.testing.assert_array_equal(e0[128:], 0.0)   # sin half second
    # frequency j=64 is 10000^(-1/2) = 1/100; at t = 50 pi its angle is pi/2
    e = dit.timestep_embedding(50 * math.pi / 1000.0)
    assert abs(e[64]) < 1e-12 and abs(e[128 + 64] - 1.0) < 1e-12
    # frequency j=0 is 1: angle = t = 1000 sigma
    e = dit.timestep_embedding(0.25)
    assert e[0] == pytest.approx(math.cos(250.0), abs=1e-12)
    assert e[128] == pytest.approx(math.sin(250.0), abs=1e-12)
    # every (cos, sin) pair lies on the unit circle
    np.testing.assert_allclose(e[:128] ** 2 + e[128:] ** 2, 1.0, atol=1e-12)
    # highest frequency index 127 has w = 10000^(-127/128)
    w127 = 10000.0 ** (-127 / 128)
    assert e[127] == pytest.approx(math.cos(250.0 * w127), abs=1e-12)


def _loops_linear(x, w, b):
    return [sum(x[k] * w[o][k] for k in range(len(x))) + b[o] for o in range(len(w))]


def test_modulation_brute_force_tiny():
    d, nb = 4, 3
    g = {"t1_w": RNG.normal(size=(d, 256)), "t1_b": RNG.normal(size=d),
         "t2_w": RNG.normal(size=(d, d)), "t2_b": RNG.normal(size=d),
         "mod_w": RNG.normal(size=(6 * d, d)), "mod_b": RNG.normal(size=6 * d),
         "fin_w": RNG.normal(size=(2 * d, d)), "fin_b": RNG.normal(size=2 * d),
         "fin_t": RNG.normal(size=(2, d)), "mod_table": RNG.normal(size=(nb, 6, d))}
    sigma = 0.37
    mod, fin = dit.modulation(g, sigma)
    e = list(dit.timestep_embedding(sigma))
    silu = lambda v: v / (1 + math.exp(-v))
    h = [silu(v) for v in _loops_linear(e, g["t1_w"].tolist(), g["t1_b"].tolist())]
    temb = _loops_linear(h, g["t2_w"].tolist(), g["t2_b"].tolist())
    u = [silu(v) for v in temb]
    m = _loops_linear(u, g["mod_w"].tolist(), g["mod_b"].tolist())
    f = _loops_linear(u, g["fin_w"].tolist(), g["fin_b"].tolist())
    for b in range(nb):
        for r in range(6):
            for c in range(d):
                assert mod[b, r, c] == pytest.approx(m[r * d + c] + g["mod_table"][b, r, c], rel=1e-12)
    for r in range(2):
        for c in range(d):
            assert fin[r, c] == pytest.approx(f[r * d + c] + g["fin_t"][r, c], rel=1e-12)


def test_modulation_zero_weights_gives_bias_plus_table():
    d, nb = 8, 2
    z = lambda *s: np.zeros(s)
    g = {"t1_w": z(d, 256), "t1_b": z(d), "t2_w": z(d, d), "t2_b": z(d),
         "mod_w": z(6 * d, d), "mod_b": RNG.normal(size=6 * d), "fin_w": z(2 * d, d),
         "fin_b": RNG.normal(size=2 * d), "fin_t": RNG.normal(size=(2, d)),
         "mod_table": RNG.normal(size=(nb, 6, d))}
    mod, fin = dit.modulation(g, 0.8)
    np.testing.assert_array_equal(mod, g["mod_b"].reshape(6, d)[None] + g["mod_table"])
    np.testing.assert_array_equal(fin, g["fin_b"].reshape(2, d) + g["fin_t"])


# ----------------------------------------------------------------- norms
def test_layer_norm_matches_torch():
    x = RNG.normal(size=(7, 48)) * 3 + 1
    want = tF.layer_norm(t64(x), (48,), eps=1e-6).numpy()
    np.testing.assert_allclose(dit.layer_norm(x), want, rtol=1e-12, atol=1e-12)


def test_adaln_reduces_and_modulates():
    x = RNG.normal(size=(5, 16))
    z = np.zeros(16)
    np.testing.assert_array_equal(dit.adaln(x, z, z), dit.layer_norm(x))
    sh, sc = RNG.normal(size=16), RNG.normal(size=16)
    want = tF.layer_norm(t64(x), (16,), weight=t64(1 + sc), bias=t64(sh), eps=1e-6).numpy()
    np.testing.assert_allclose(dit.adaln(x, sh, sc), want, rtol=1e-12, atol=1e-12)
    # scale = -1 leaves only the shift
    np.testing.assert_allclose(dit.adaln(x, sh, -np.ones(16)), np.broadcast_to(sh, x.shape), atol=0)


def test_gated_residual_zero_gate_exact():
    x, y = RNG.normal(size=(4, 8)), RNG.normal(size=(4, 8))
    np.testing.assert_array_equal(dit.gated_residual(x, np.zeros(8), y), x)
    g = RNG.normal(size=8)
    np.testing.assert_allclose(dit.gated_residual(x, g, y) - x, g * y, rtol=1e-14)


def test_rms_norm_matches_torch_and_unit_rms():
    t = RNG.normal(size=(6, 3, 12)) * 5
    gamma = RNG.normal(size=12)
    want = tF.rms_norm(t64(t), (12,), weight=t64(gamma), eps=1e-6).numpy()
    np.testing.assert_allclose(dit.rms_norm_heads(t, gamma), want, rtol=1e-12, atol=1e-12)
    out = dit.rms_norm_heads(t, np.ones(12))
    np.testing.assert_allclose(np.sqrt((out ** 2).mean(-1)), 1.0, rtol=1e-6)


# ----------------------------------------------------------------- RoPE
def test_rope_split_sizes():
    assert dit.rope_split(128) == (44, 42, 42)
    assert dit.rope_split(64) == (24, 20, 20)
    for dh in (12, 24, 64, 96, 128):
        a, b, c = dit.rope_split(dh)
        assert a + b + c == dh and a % 2 == 0 and b % 2 == 0 and b == c


def _rope_complex(t, coords):
    # independent statement: each pair is a complex number multiplied by exp(i * angle)
    n, nh, dh = t.shape
    out = np.empty_like(t)
    off = 0
    for axis, da in enumerate(dit.rope_split(dh)):
        z = t[:, :, off:off + da:2] + 1j * t[:, :, off + 1:off + da:2]
        freqs = 1.0 / (10000.0 ** (np.arange(0, da, 2) / da))
        rot = np.exp(1j * coords[:, axis:axis + 1] * freqs[None, :])
        z = z * rot[:, None, :]
        out[:, :, off:off + da:2] = z.real
        out[:, :, off + 1:off + da:2] = z.imag
        off += da
    return out


def test_rope_matches_complex_form():
    coords = dit.rope_coords(2, 3, 4, 1.0)
    t = RNG.normal(size=(24, 2, 64))
    np.testing.assert_allclose(dit.rope_apply(t, coords), _rope_complex(t, coords), atol=1e-12)


def test_rope_coords_order_and_halving():
    c = dit.rope_coords(2, 3, 4, 1.0)
    # token n = (f*3 + h)*4 + w
    n = (1 * 3 + 2) * 4 + 3
    np.testing.assert_array_equal(c[n], [1, 2, 3])
    ch = dit.rope_coords(2, 8, 8, 0.5)
    n = (1 * 8 + 6) * 8 + 5
    np.testing.assert_array_equal(ch[n], [1, 3.0, 2.5])


def test_rope_identity_at_origin_and_norm_preserved():
    t = RNG.normal(size=(5, 2, 24))
    z = np.zeros((5, 3))
    np.testing.assert_array_equal(dit.rope_apply(t, z), t)
    coords = RNG.normal(size=(5, 3)) * 10
    r = dit.rope_apply(t, coords)
    np.testing.assert_allclose((r[..., 0::2] ** 2 + r[..., 1::2] ** 2), (t[..., 0::2] ** 2 + t[..., 1::2] ** 2),
                               rtol=1e-12)


def test_rope_relative_position():
    dh = 64
    q, k = RNG.normal(size=(1, 1, dh)), RNG.normal(size=(1, 1, dh))
    a, b = np.array([[3.0, 1.5, 2.0]]), np.array([[1.0, 4.0, 0.5]])
    shift = np.array([[7.0, -2.5, 11.0]])
    d1 = (dit.rope_apply(q, a) * dit.rope_apply(k, b)).sum()
    d2 = (dit.rope_apply(q, a + shift) * dit.rope_apply(k, b + shift)).sum()
    assert d1 == pytest.approx(d2, rel=1e-10, abs=1e-10)


def test_rope_halved_coords_equal_halved_frequencies():
    # rotating by coordinate c/2 equals rotating with every frequency halved at coordinate c
    t = RNG.normal(size=(64, 1, 24))
    full = dit.rope_coords(1, 8, 8, 1.0)
    half = dit.rope_coords(1, 8, 8, 0.5)
    got = dit.rope_apply(t, half)
    want = np.empty_like(t)
    off = 0
    for axis, da in enumerate(dit.rope_split(24)):
        for j in range(da // 2):
            f = 10000.0 ** (-2.0 * j / da) * (0.5 if axis > 0 else 1.0)
            ang = full[:, axis] * f
            a, b = t[:, 0, off + 2 * j], t[:, 0, off + 2 * j + 1]
            want[:, 0, off + 2 * j] = a * np.cos(ang) - b * np.sin(ang)
            want[:, 0, off + 2 * j + 1] = a * np.sin(ang) + b * np.cos(ang)
        off += da
    np.testing.assert_allclose(got, want, atol=1e-12)


def test_rope_merged_coords_are_pair_means():
    plan = host.token_plan(1, 2, 5, 0, 10)
    c = dit.rope_coords(1, 2, 5, 1.0, plan["pairs"])
    np.testing.assert_array_equal(c[:, 2], [0.5, 2.5, 4.0, 0.5, 2.5, 4.0])
    np.testing.assert_array_equal(c[:, 1], [0, 0, 0, 1, 1, 1])


# ----------------------------------------------------------------- attention
def test_attention_matches_torch_sdpa():
    q, k, v = RNG.normal(size=(9, 3, 16)), RNG.normal(size=(13, 3, 16)), RNG.normal(size=(13, 3, 16))
    want = tF.scaled_dot_product_attention(t64(q).transpose(0, 1), t64(k).transpose(0, 1),
                                           t64(v).transpose(0, 1)).transpose(0, 1).numpy()
    np.testing.assert_allclose(dit.attention(q, k, v), want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dit.attention(q, k, v, chunk=4), want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dit.attention(q, k, v, rows=[2, 7]), want[[2, 7]], rtol=1e-12)


def test_attention_brute_force_and_closed_forms():
    q, k, v = RNG.normal(size=(3, 1, 4)), RNG.normal(size=(5, 1, 4)), RNG.normal(size=(5, 1, 4))
    got = dit.attention(q, k, v)
    for i in range(3):
        s = [sum(q[i, 0, c] * k[j, 0, c] for c in range(4)) / 2.0 for j in range(5)]
        e = [math.exp(x) for x in s]
        for c in range(4):
            assert got[i, 0, c] == pytest.approx(sum(e[j] * v[j, 0, c] for j in range(5)) / sum(e), rel=1e-12)
    # zero query: uniform weights -> mean of values
    np.testing.assert_allclose(dit.attention(np.zeros((2, 1, 4)), k, v)[0], v.mean(0), rtol=1e-12)
    # one key: output is that value
    np.testing.assert_allclose(dit.attention(q, k[:1], v[:1]), np.broadcast_to(v[:1], (3, 1, 4)), rtol=1e-12)


def test_gelu_matches_erf():
    x = np.linspace(-6, 6, 97)
    want = [0.5 * a * (1 + math.erf(a / math.sqrt(2))) for a in x]
    np.testing.assert_allclose(dit.gelu(x), want, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(dit.gelu(x), tF.gelu(t64(x)).numpy(), rtol=1e-14, atol=1e-15)


def test_linear_orientation():
    x, w, b = RNG.normal(size=(3, 5)), RNG.normal(size=(4, 5)), RNG.normal(size=4)
    got = dit.linear(x, w, b)
    for r in range(3):
        np.testing.assert_allclose(got[r], _loops_linear(x[r], w, b), rtol=1e-13)


# ----------------------------------------------------------------- int8
def test_bf16_rounding_matches_torch():
    x = (RNG.normal(size=4096) * 10.0 ** RNG.integers(-8, 8, size=4096)).astype(np.float32)
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # ties to even
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(dit.f32_to_bf16(x), want)


def test_quantize_rows_scalar_brute_force():
    h = (RNG.normal(size=(4, 2048)) * 3).astype(np.float32)
    h[1] = 0.0
    h[2, 5] = 1e-30
    for group in (None, 1024):
        q, s = dit.quantize_rows(h, group)
        g = 2048 if group is None else group
        assert s.shape == (4, 2048 // g)
        for r in range(4):
            for gi in range(2048 // g):
                seg = h[r, gi * g:(gi + 1) * g]
                amax = np.float32(max(abs(float(v)) for v in seg))
                sc = np.float32(amax / np.float32(127))
                assert s[r, gi] == sc
                for kk in range(0, g, 97):
                    v = seg[kk]
                    want = 0 if sc == 0 else int(np.clip(np.rint(np.float32(v / sc)), -127, 127))
                    assert q[r, gi * g + kk] == want
    q, s = dit.quantize_rows(h, None)
    assert (q[1] == 0).all() and s[1, 0] == 0
    assert np.abs(q).max() == 127 and q.dtype == np.int8


def test_quantize_error_bound():
    h = RNG.normal(size=(8, 1024)).astype(np.float32)
    q, s = dit.quantize_rows(h)
    err = np.abs(h.astype(np.float64) - q.astype(np.float64) * s.astype(np.float64))
    assert (err <= s.astype(np.float64) * 0.5 * (1 + 1e-5) + 1e-30).all()
    # the absmax element lands on +-127
    r = np.arange(8)
    assert (np.abs(q[r, np.abs(h).argmax(1)]) == 127).all()


def test_round_half_even_decision():
    # values exactly half-way between codes round to the even code
    h = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5]], dtype=np.float32)  # s = 1
    q, s = dit.quantize_rows(h)
    assert s[0, 0] == 1.0
    np.testing.assert_array_equal(q[0], [127, 0, 2, 2, 0, -2])


def test_int8_accumulate_exact():
    qa = RNG.integers(-127, 128, size=(3, 64)).astype(np.int8)
    qw = RNG.integers(-127, 128, size=(5, 64)).astype(np.int8)
    acc = dit.int8_accumulate(qa, qw, 32)
    for g in range(2):
        for r in range(3):
            for n in range(5):
                assert acc[g, r, n] == sum(int(qa[r, k]) * int(qw[n, k]) for k in range(32 * g, 32 * g + 32))
    full = dit.int8_accumulate(qa, qw)
    np.testing.assert_array_equal(full[0], acc.sum(0))


def test_int8_accumulate_exact_at_the_extremes():
    # the largest sums an FC2 row can reach (every code +-127 over 20480 channels) and sums
    # that cancel to small values: integer brute force with Python ints
    k = 20480
    qa = np.full((2, k), 127, dtype=np.int8)
    qa[1, ::2] = -127
    qw = np.full((3, k), -127, dtype=np.int8)
    qw[1] = 127
    qw[2, 1::3] = 1
    acc = dit.int8_accumulate(qa, qw, 1024)
    for r in range(2):
        for n in range(3):
            for g in range(k // 1024):
                ref = sum(int(qa[r, c]) * int(qw[n, c]) for c in range(1024 * g, 1024 * g + 1024))
                assert acc[g, r, n] == ref
    full = dit.int8_accumulate(qa, qw)
    assert full[0, 0, 0] == -127 * 127 * k and full[0, 0, 1] == 127 * 127 * k
    assert full.dtype == np.int64


def test_dequant_fixed_order_float32():
    acc = RNG.integers(-10 ** 7, 10 ** 7, size=(3, 2, 4))
    sa = RNG.random(size=(2, 3)).astype(np.float32)
    sw = RNG.random(size=4).astype(np.float32)
    b = RNG.normal(size=4).astype(np.float32)
    got = dit.dequant(acc, sa, sw, b)
    for r in range(2):
        for n in range(4):
            t = np.float32(0)
            for g in range(3):
                t = np.float32(t + np.float32(np.float32(acc[g, r, n]) * sa[r, g]))
            want = np.float32(np.float32(t * sw[n]) + b[n])
            assert got[r, n] == want


def test_int8_fc2_close_to_bf16_product():
    h = RNG.normal(size=(6, 2048)) * 0.5
    blk = {"fc2_w": RNG.normal(size=(16, 2048)) * 0.02, "fc2_b": RNG.normal(size=16) * 0.02}
    ref = dit.fc2(h, blk, "bf16")
    for mode in ("row", "grouped"):
        got = dit.fc2(h, blk, mode)
        # error bound: sum_k |w| s_a/2 + |h| s_w/2 (plus float32 rounding)
        qa, sa = dit.quantize_rows(h, None if mode == "row" else 1024)
        qw, sw = dit.quantize_weight(blk["fc2_w"])
        sa_full = np.repeat(sa, 2048 // sa.shape[1], axis=1)
        bound = (np.abs(blk["fc2_w"])[None] * sa_full[:, None, :] / 2).sum(-1) + \
                (np.abs(h)[:, None, :] * sw[None, :, 0:1] / 2).sum(-1) + \
                (sa_full[:, None, :] * sw[None, :, 0:1] / 4).sum(-1)
        assert (np.abs(got - ref) <= bound * 1.01 + 1e-6).all()


def test_linear_int8_exact_when_quantisation_is_lossless():
    # activations on the grid s_a * k (|k| <= 127, 127 reached, s_a a power of two so the bf16
    # rounding and the division are exact) and weights on s_w * j: the int8 product is then
    # the exact product, up to the float32 rounding of the dequantisation
    qa = RNG.integers(-127, 128, size=(4, 96))
    qa[:, 0] = 127
    qw = RNG.integers(-127, 128, size=(6, 96))
    qw[:, 5] = -127
    sa = 2.0 ** -RNG.integers(3, 9, size=(4, 1))
    sw = 2.0 ** -RNG.integers(6, 12, size=(6, 1))
    a, w = qa * sa, qw * sw
    b = RNG.normal(size=6) * 0.01
    b = b.astype(np.float32).astype(np.float64)
    got = dit.linear_int8(a, w, b)
    want = tF.linear(t64(a), t64(w), t64(b)).numpy()
    np.testing.assert_allclose(got, want, rtol=2e-7, atol=1e-9)


def test_linear_int8_rounds_the_activation_to_bf16_first():
    a = RNG.normal(size=(3, 64))
    w = RNG.normal(size=(5, 64)) * 0.02
    b = np.zeros(5)
    ab = torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(dit.linear_int8(a, w, b), dit.linear_int8(ab, w, b))


def test_linear_int8_within_quantisation_bound_of_the_float64_product():
    a = RNG.normal(size=(5, 512))
    w = RNG.normal(size=(12, 512)) * 0.02
    b = RNG.normal(size=12) * 0.02
    ab = torch.from_numpy(a).to(torch.bfloat16).double().numpy()
    ref = tF.linear(t64(ab), t64(w), t64(b)).numpy()
    got = dit.linear_int8(a, w, b)
    _, sa = dit.quantize_rows(ab.astype(np.float32))
    _, sw = dit.quantize_weight(w.astype(np.float32))
    bound = (np.abs(w)[None] * sa[:, None, :] / 2).sum(-1) + \
            (np.abs(ab)[:, None, :] * sw[None, :, 0:1] / 2).sum(-1) + \
            (sa[:, None, :] * sw[None, :, 0:1] / 4).sum(-1)
    assert (np.abs(got - ref) <= bound * 1.01 + 1e-6).all()
    assert np.abs(got - ref).max() > 0   # it is a different product


# ----------------------------------------------------------------- token pairing
def test_merge_restore_identity_and_delta():
    plan = host.token_plan(2, 3, 5, 0, 10)
    s = RNG.normal(size=(30, 6))
    xr = dit.token_merge(s, plan["pairs"])
    assert xr.shape == (18, 6)
    np.testing.assert_array_equal(dit.token_restore(s, xr, plan["pairs"]), s)
    # a change of the pair mean is added to both members; the odd column is a singleton
    delta = RNG.normal(size=(18, 6))
    x = dit.token_restore(s, xr + delta, plan["pairs"])
    np.testing.assert_allclose(x[0], s[0] + delta[0], rtol=1e-14)
    np.testing.assert_allclose(x[1], s[1] + delta[0], rtol=1e-14)
    np.testing.assert_allclose(x[4], s[4] + delta[2], rtol=1e-14)   # column 4 alone
    # constant pairs merge to the row itself
    c = np.repeat(RNG.normal(size=(15, 6)), 2, axis=0)
    pc = host.token_plan(1, 3, 10, 0, 10)["pairs"]
    np.testing.assert_array_equal(dit.token_merge(c, pc), c[0::2])


def test_euler_constant_velocity():
    x0, v = RNG.normal(size=(4, 3)), RNG.normal(size=(4, 3))
    for steps in (1, 4, 20):
        sig, _ = host.schedule(steps)
        x = x0
        for i in range(steps):
            x = dit.euler_step(x, v, sig[i], sig[i + 1])
        np.testing.assert_allclose(x, x0 - v, rtol=1e-12, atol=1e-12)
