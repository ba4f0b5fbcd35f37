"""Pins of the oracle's block, forward and loop composition.

The block is restated with torch.nn.functional library routines in float64 (layer_norm
with weight/bias, linear, rms_norm, scaled_dot_product_attention, gelu) and a complex
RoPE, and must agree with ``oracle.dit.block_forward``.  Structural cases (zero gates,
merge/restore plumbing, reuse counts, constant velocity) pin the forward and the loop.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as tF

from oracle import dit, host
from tests.test_oracle_dit import _rope_complex

RNG = np.random.default_rng(99)


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def tiny_model(d=24, heads=2, ffn=48, ctx_len=5, nb=3, c=6, std=0.2):
    dh = d // heads
    n = lambda *s: RNG.normal(size=s) * std
    g = {"t1_w": n(d, 256), "t1_b": n(d), "t2_w": n(d, d), "t2_b": n(d), "mod_w": n(6 * d, d),
         "mod_b": n(6 * d), "fin_w": n(2 * d, d), "fin_b": n(2 * d), "fin_t": n(2, d),
         "mod_table": n(nb, 6, d), "patch_w": n(d, c), "patch_b": n(d), "head_w": n(c, d),
         "head_b": n(c)}
    blocks = []
    for _ in range(nb):
        blocks.append({"qkv_w": n(3 * d, d), "qkv_b": n(3 * d), "qc_w": n(d, d), "qc_b": n(d),
                       "kc_w": n(d, d), "kc_b": n(d), "vc_w": n(d, d), "vc_b": n(d),
                       "o_w": n(d, d), "o_b": n(d), "oc_w": n(d, d), "oc_b": n(d),
                       "q_gamma": 1 + n(dh), "k_gamma": 1 + n(dh), "fc1_w": n(ffn, d),
                       "fc1_b": n(ffn), "fc2_w": n(d, ffn), "fc2_b": n(d)})
    return {"global": g, "blocks": blocks, "ctx": RNG.normal(size=(ctx_len, d))}


def torch_block(x, blk, mod, ctx, coords, heads):
    n, d = x.shape
    dh = d // heads
    X = t64(x)
    sh1, sc1, g1, sh2, sc2, g2 = [t64(m) for m in mod]
    n1 = tF.layer_norm(X, (d,), weight=1 + sc1, bias=sh1, eps=1e-6)
    qkv = tF.linear(n1, t64(blk["qkv_w"]), t64(blk["qkv_b"]))
    q, k, v = qkv.split(d, dim=1)
    q = tF.rms_norm(q.reshape(n, heads, dh), (dh,), weight=t64(blk["q_gamma"]), eps=1e-6)
    k = tF.rms_norm(k.reshape(n, heads, dh), (dh,), weight=t64(blk["k_gamma"]), eps=1e-6)
    q = t64(_rope_complex(q.numpy(), coords))
    k = t64(_rope_complex(k.numpy(), coords))
    v = v.reshape(n, heads, dh)
    o = tF.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1))
    o = o.transpose(0, 1).reshape(n, d)
    C = t64(ctx)
    kc = tF.linear(C, t64(blk["kc_w"]), t64(blk["kc_b"])).reshape(-1, heads, dh).transpose(0, 1)
    vc = tF.linear(C, t64(blk["vc_w"]), t64(blk["vc_b"])).reshape(-1, heads, dh).transpose(0, 1)
    qc = tF.linear(n1, t64(blk["qc_w"]), t64(blk["qc_b"])).reshape(n, heads, dh).transpose(0, 1)
    oc = tF.scaled_dot_product_attention(qc, kc, vc).transpose(0, 1).reshape(n, d)
    y = tF.linear(o, t64(blk["o_w"]), t64(blk["o_b"])) + tF.linear(oc, t64(blk["oc_w"]), t64(blk["oc_b"]))
    x1 = X + g1 * y
    n2 = tF.layer_norm(x1, (d,), weight=1 + sc2, bias=sh2, eps=1e-6)
    h = tF.gelu(tF.linear(n2, t64(blk["fc1_w"]), t64(blk["fc1_b"])))
    m = tF.linear(h, t64(blk["fc2_w"]), t64(blk["fc2_b"]))
    return (x1 + g2 * m).numpy()


def test_block_matches_torch_composition():
    mdl = tiny_model()
    mod, _ = dit.modulation(mdl["global"], 0.6)
    coords = dit.rope_coords(2, 2, 3, 1.0)
    x = RNG.normal(size=(12, 24))
    for b in range(3):
        got = dit.block_forward(x, mdl["blocks"][b], mod[b], mdl["ctx"], coords, 2)
        want = torch_block(x, mdl["blocks"][b], mod[b], mdl["ctx"], coords, 2)
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-11)


def test_block_trace_consistent():
    mdl = tiny_model()
    mod, _ = dit.modulation(mdl["global"], 0.3)
    coords = dit.rope_coords(1, 3, 4, 1.0)
    x = RNG.normal(size=(12, 24))
    tr = {}
    out = dit.block_forward(x, mdl["blocks"][0], mod[0], mdl["ctx"], coords, 2, trace=tr)
    np.testing.assert_allclose(tr["x1"], x + mod[0][2] * tr["y"], rtol=1e-14)
    np.testing.assert_allclose(out, tr["x1"] + mod[0][5] * tr["m"], rtol=1e-14)


def test_zero_gates_leave_stream_unchanged():
    mdl = tiny_model()
    mod, _ = dit.modulation(mdl["global"], 0.5)
    mod = mod.copy()
    mod[:, 2] = 0
    mod[:, 5] = 0
    x = RNG.normal(size=(12, 24))
    coords = dit.rope_coords(1, 3, 4, 1.0)
    for b in range(3):
        np.testing.assert_array_equal(dit.block_forward(x, mdl["blocks"][b], mod[b], mdl["ctx"], coords, 2), x)


def test_qk_norm_switch():
    mdl = tiny_model()
    blk = dict(mdl["blocks"][0])
    mod, _ = dit.modulation(mdl["global"], 0.5)
    x = RNG.normal(size=(6, 24))
    coords = dit.rope_coords(1, 2, 3, 1.0)
    tr_on, tr_off = {}, {}
    dit.block_forward(x, blk, mod[0], mdl["ctx"], coords, 2, qk_norm=True, trace=tr_on)
    dit.block_forward(x, blk, mod[0], mdl["ctx"], coords, 2, qk_norm=False, trace=tr_off)
    # without the norm, q is only rotated: its per-pair norms equal those of the projection
    q_proj = tr_off["qkv"][:, :24].reshape(6, 2, 12)
    np.testing.assert_allclose((tr_off["q"] ** 2).sum(-1), (q_proj ** 2).sum(-1), rtol=1e-12)
    assert not np.allclose(tr_on["q"], tr_off["q"])


def _zero_gate_model(mdl):
    g = dict(mdl["global"])
    t = g["mod_table"].copy()
    # cancel the shared gate rows: gates = 0 for every block
    mod0, _ = dit.modulation(g, 0.7)
    t[:, 2] -= mod0[:, 2]
    t[:, 5] -= mod0[:, 5]
    g["mod_table"] = t
    return {"global": g, "blocks": mdl["blocks"], "ctx": mdl["ctx"]}


def test_forward_with_zero_gates_is_patch_then_head():
    mdl = _zero_gate_model(tiny_model(nb=5))
    geom = dict(f_lat=1, grid_h=2, grid_w=3, scale=1.0)
    lat = RNG.normal(size=(6, 6))
    _, fin = dit.modulation(mdl["global"], 0.7)
    want = dit.final_head(dit.patch_embed(lat, mdl["global"]), mdl["global"], fin)
    for tr in (False, True):
        v = dit.dit_forward(lat, mdl, 0.7, [0, 1, 2, 3, 4], geom, 2, token_reduction=tr)
        np.testing.assert_allclose(v, want, rtol=1e-12, atol=1e-12)


def test_forward_token_reduction_runs_reduced_blocks():
    mdl = tiny_model(nb=5)
    geom = dict(f_lat=1, grid_h=2, grid_w=3, scale=1.0)
    lat = RNG.normal(size=(6, 6))
    active = [0, 1, 2, 3, 4]
    v_tr = dit.dit_forward(lat, mdl, 0.7, active, geom, 2, token_reduction=True)
    # hand-composed: 3 full blocks, merge, 2 reduced blocks, restore before the head
    g = mdl["global"]
    mod, fin = dit.modulation(g, 0.7)
    x = dit.patch_embed(lat, g)
    full = dit.rope_coords(1, 2, 3, 1.0)
    for b in range(3):
        x = dit.block_forward(x, mdl["blocks"][b], mod[b], mdl["ctx"], full, 2)
    plan = host.token_plan(1, 2, 3, 0, 5)
    s = x
    x = dit.token_merge(s, plan["pairs"])
    red = dit.rope_coords(1, 2, 3, 1.0, plan["pairs"])
    assert x.shape[0] == 4
    for b in range(3, 5):
        x = dit.block_forward(x, mdl["blocks"][b], mod[b], mdl["ctx"], red, 2)
    x = dit.token_restore(s, x, plan["pairs"])
    np.testing.assert_allclose(v_tr, dit.final_head(x, g, fin), rtol=1e-12, atol=1e-12)
    v_full = dit.dit_forward(lat, mdl, 0.7, active, geom, 2)
    assert not np.allclose(v_tr, v_full)


def test_denoise_counts_and_reuse_hold():
    mdl = tiny_model(nb=2)
    geom = dict(f_lat=1, grid_h=2, grid_w=2, scale=1.0)
    lat = RNG.normal(size=(4, 6))
    for steps, reuse, want in [(4, 1, 4), (5, 2, 3), (7, 3, 3), (8, 3, 4), (1, 1, 1)]:
        _, ev = dit.denoise(lat, mdl, steps, reuse, [0, 1], geom, 2)
        assert ev == want
    # one step from sigma=1 to 0 is x0 - v(x0, 1)
    x1, _ = dit.denoise(lat, mdl, 1, 1, [0, 1], geom, 2)
    v = dit.dit_forward(lat, mdl, 1.0, [0, 1], geom, 2)
    np.testing.assert_allclose(x1, lat - v, rtol=1e-13, atol=1e-13)
    # reuse 2 over 2 steps: the second step reuses the first velocity and the last step is fresh
    x2, ev = dit.denoise(lat, mdl, 3, 2, [0, 1], geom, 2)
    sig, _ = host.schedule(3, 2)
    v0 = dit.dit_forward(lat, mdl, float(sig[0]), [0, 1], geom, 2, 0)
    xa = dit.euler_step(lat, v0, sig[0], sig[1])
    xb = dit.euler_step(xa, v0, sig[1], sig[2])
    v2 = dit.dit_forward(xb, mdl, float(sig[2]), [0, 1], geom, 2, 1)
    np.testing.assert_allclose(x2, dit.euler_step(xb, v2, sig[2], sig[3]), rtol=1e-13, atol=1e-13)
    assert ev == 2


def test_core_reuse_cached_evaluation_at_the_fresh_point_is_the_fresh_velocity():
    # x_0 + (x_L - x_0) = x_L: a reused evaluation at the same latent and sigma reproduces
    # the fresh velocity; with token pairing the delta is taken after the bypass restore
    mdl = tiny_model(nb=5)
    geom = dict(f_lat=1, grid_h=2, grid_w=3, scale=1.0)
    lat = RNG.normal(size=(6, 6))
    for tr in (False, True):
        v, delta = dit.dit_forward_cached(lat, mdl, 0.6, [0, 1, 2, 3, 4], geom, 2,
                                          token_reduction=tr)
        np.testing.assert_allclose(v, dit.dit_forward(lat, mdl, 0.6, [0, 1, 2, 3, 4], geom, 2,
                                                      token_reduction=tr), rtol=1e-13, atol=1e-13)
        v2, d2 = dit.dit_forward_cached(lat, mdl, 0.6, [0, 1, 2, 3, 4], geom, 2, core_delta=delta)
        assert d2 is delta
        np.testing.assert_allclose(v2, v, rtol=1e-12, atol=1e-12)
        assert np.abs(delta).max() > 1e-3


def test_core_reuse_with_zero_gates_has_zero_delta():
    mdl = _zero_gate_model(tiny_model(nb=3))
    geom = dict(f_lat=1, grid_h=2, grid_w=2, scale=1.0)
    lat = RNG.normal(size=(4, 6))
    _, delta = dit.dit_forward_cached(lat, mdl, 0.7, [0, 1, 2], geom, 2)
    np.testing.assert_allclose(delta, 0.0, atol=1e-13)


def test_core_reuse_loop_refreshes_patch_and_head_only():
    # --core-reuse 2 over 3 steps: steps 0 and 2 run the core; step 1 reuses step 0's delta
    # with its own latent and its own sigma in the head
    mdl = tiny_model(nb=2)
    geom = dict(f_lat=1, grid_h=2, grid_w=2, scale=1.0)
    lat = RNG.normal(size=(4, 6))
    g = mdl["global"]
    x3, ev = dit.denoise(lat, mdl, 3, 1, [0, 1], geom, 2, core_reuse=2)
    assert ev == 2
    sig, fresh = host.schedule(3, 1, 2)
    assert list(fresh) == [1, 0, 1]
    tr = {}
    v0 = dit.dit_forward(lat, mdl, float(sig[0]), [0, 1], geom, 2, trace=tr)
    delta = tr["x_core_out"] - dit.patch_embed(lat, g)
    xa = dit.euler_step(lat, v0, sig[0], sig[1])
    _, fin1 = dit.modulation(g, float(sig[1]))
    v1 = dit.final_head(dit.patch_embed(xa, g) + delta, g, fin1)
    xb = dit.euler_step(xa, v1, sig[1], sig[2])
    v2 = dit.dit_forward(xb, mdl, float(sig[2]), [0, 1], geom, 2, 1)
    np.testing.assert_allclose(x3, dit.euler_step(xb, v2, sig[2], sig[3]), rtol=1e-12, atol=1e-12)
    # and it differs from whole-velocity reuse, which would keep v0 on step 1
    x3r, _ = dit.denoise(lat, mdl, 3, 2, [0, 1], geom, 2)
    assert not np.allclose(x3, x3r)
