"""GPU parity of the whole fresh evaluation (h3_dit_forward) and of the Euler loop against
the oracle.

Bars: velocity per evaluation within rel-L2 2e-2; latent after the full step loop within
rel-L2 5e-2, and so is x_N - x_0 (the part the loop changed).
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import dit, host
from tests.gpu_util import DEV, assert_close, bits, f64, rel_l2, zero_gates
from tests.oracle_model import oracle_active, oracle_geom, oracle_latent, oracle_model
from video_diffusion_transformer_fwd_amd import binding as B
from video_diffusion_transformer_fwd_amd import synthetic as S
from video_diffusion_transformer_fwd_amd.runtime import DiTModel

pytestmark = pytest.mark.gpu

# A small model with token pairing: 160x128 output -> 4x5 grid (odd width), 2 latent frames,
# 32 blocks so that the bypass restore lands inside the active list (before position 30 for
# evaluations past the tenth) as well as before the head.
TR_SMALL = S.Workload("tr_160x128_5f", 160, 128, 5, 512, 8, 2048, 32, 32, steps=12, reuse=1,
                      layers=31, token_reduction=True)


def loop_parity(w, model, om, opts_kw, steps, reuse, active):
    geo = oracle_geom(w)
    lat0 = model.initial_latent()
    x = lat0.clone()
    opts = model.opts(**opts_kw)
    ev = model.denoise(x, steps, reuse, active, opts)
    torch.cuda.synchronize()
    ref, ev_ref = dit.denoise(f64(lat0), om, steps, reuse, active, geo, w.n_heads,
                              fc2_mode=opts_kw.get("fc2_mode", "bf16"),
                              token_reduction=opts_kw.get("token_reduction", False),
                              int8_linear=opts_kw.get("int8_linear", False))
    assert ev == ev_ref
    got = f64(x)
    assert np.isfinite(got).all()
    r1 = rel_l2(got, ref)
    r2 = rel_l2(got - f64(lat0), ref - f64(lat0))
    assert r1 < 5e-2 and r2 < 5e-2, (r1, r2)
    return r1, r2


# Bar on the blocks' own contribution at the small workload.  There the two blocks move the
# velocity by only ~5% of its norm (the latent by ~2%), so the whole-output bars alone would
# pass a forward that skipped them.  The contribution c = v - v(zero gates) is gated instead,
# relative to the oracle's c: a skipped block gives 1, a sign error 2.  Its floor is the bf16
# storage of the stream and of the head's input: each store rounds to 2^-9 of |x| (|n|), not of
# the ~20x smaller |g y|, so three roundings (two block outputs, the final AdaLN) leave about
# 2^-9 * sqrt(3) * 20 ~ 7e-2 of |c| (measured 8.4e-2 on the velocity): the bar sits ~2x above
# that and ~7x below a skipped block.  The per-block branch outputs carry 2e-2 bars at this size.
CONTRIB_REL = 0.15


def test_tiny_forward_and_loop():
    w = S.WORKLOADS["tiny_256sq_5f"]
    model = DiTModel(w)
    om = oracle_model(w)
    geo = oracle_geom(w)
    assert (geo["f_lat"], geo["grid_h"], geo["grid_w"], geo["scale"], geo["n"]) == (2, 8, 8, 0.5, 128)
    g = model.geo
    assert (g.f_lat, g.grid_h, g.grid_w, g.scale, g.n_tokens) == (2, 8, 8, 0.5, 128)
    assert oracle_active(w, om) == [0, 1]
    lat = model.initial_latent()
    for sigma, ev in [(1.0, 0), (0.5, 3)]:
        v = model.forward(lat, sigma, eval_index=ev).clone()
        with zero_gates(model):
            v0 = model.forward(lat, sigma, eval_index=ev).clone()
        torch.cuda.synchronize()
        ref = dit.dit_forward(f64(lat), om, sigma, [0, 1], geo, w.n_heads)
        ref0 = dit.dit_forward(f64(lat), om, sigma, [], geo, w.n_heads)
        assert_close(f64(v), ref, rel=2e-2, elem=8e-2, what=f"velocity sigma={sigma}")
        rc = rel_l2(f64(v) - f64(v0), ref - ref0)
        print(f"sigma={sigma}: velocity rel-L2 {rel_l2(f64(v), ref):.2e}, blocks' contribution "
              f"rel-L2 {rc:.2e} (contribution / velocity {rel_l2(ref0, ref):.2e})")
        assert rc <= CONTRIB_REL, rc
    # the Euler loop, whole and as the blocks' contribution
    lat0 = model.initial_latent()
    x = lat0.clone()
    model.denoise(x, w.steps, w.reuse, [0, 1])
    x0 = lat0.clone()
    with zero_gates(model):
        model.denoise(x0, w.steps, w.reuse, [0, 1])
    ref, _ = dit.denoise(f64(lat0), om, w.steps, w.reuse, [0, 1], geo, w.n_heads)
    ref0, _ = dit.denoise(f64(lat0), om, w.steps, w.reuse, [], geo, w.n_heads)
    r1 = rel_l2(f64(x), ref)
    r2 = rel_l2(f64(x) - f64(lat0), ref - f64(lat0))
    rc = rel_l2(f64(x) - f64(x0), ref - ref0)
    print(f"loop: latent {r1:.2e}, x_N - x_0 {r2:.2e}, blocks' contribution {rc:.2e}")
    assert r1 < 5e-2 and r2 < 5e-2 and rc <= CONTRIB_REL, (r1, r2, rc)
    # int8 FC2 modes through the whole evaluation, also as the blocks' contribution
    model8 = DiTModel(w, with_int8=True)
    with zero_gates(model8):
        v0 = model8.forward(lat, 1.0).clone()
    ref0 = dit.dit_forward(f64(lat), om, 1.0, [], geo, w.n_heads)
    for mode in ("row", "grouped"):
        v = model8.forward(lat, 1.0, opts=model8.opts(fc2_mode=mode))
        torch.cuda.synchronize()
        ref = dit.dit_forward(f64(lat), om, 1.0, [0, 1], geo, w.n_heads, fc2_mode=mode)
        assert rel_l2(f64(v), ref) < 2e-2
        rc = rel_l2(f64(v) - f64(v0), ref - ref0)
        assert rc <= CONTRIB_REL, (mode, rc)


def test_token_reduction_forward_and_loop():
    w = TR_SMALL
    model = DiTModel(w)
    om = oracle_model(w)
    active = oracle_active(w, om)
    assert model.active() == active
    lat = model.initial_latent()
    for ev in (0, 10):   # restore before the head / before active position 30
        v = model.forward(lat, 0.6, active, eval_index=ev)
        torch.cuda.synchronize()
        ref = dit.dit_forward(f64(lat), om, 0.6, active, oracle_geom(w), w.n_heads,
                              eval_index=ev, token_reduction=True)
        assert_close(f64(v), ref, rel=2e-2, elem=8e-2, what=f"token-reduced velocity eval {ev}")
        ref_full = dit.dit_forward(f64(lat), om, 0.6, active, oracle_geom(w), w.n_heads)
        assert rel_l2(ref, ref_full) > 2 * rel_l2(f64(v), ref), "pairing must change the result"
    loop_parity(w, model, om, {"token_reduction": True}, w.steps, 1, active)
    loop_parity(w, model, om, {"token_reduction": True}, 5, 2, active)


@pytest.mark.parametrize("int8_linear", [False, True])
def test_unfused_forward_bit_identical_to_fused(int8_linear):
    # every fusion (gate + AdaLN-2, MLP gate + next AdaLN-1, Q/K RMSNorm + RoPE in the QKV
    # epilogue, final AdaLN inside the head product) on and off, with and without token pairing,
    # bf16 and int8 QKV / FC1
    w = dataclasses.replace(TR_SMALL, int8_linear=int8_linear)
    model = DiTModel(w)
    lat = model.initial_latent()
    outs = []
    for fused in (1, 0):
        for tr in (False, True):
            v = model.forward(lat, 0.8, eval_index=0,
                              opts=model.opts(fused_gate_adaln=fused, fused_cross_block=fused,
                                              fused_qk_rope=fused, fused_head_adaln=fused,
                                              token_reduction=tr))
            torch.cuda.synchronize()
            outs.append(bits(v))
    assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[1], outs[3])
    # the head fusion alone, where the final AdaLN would otherwise come from the last block's
    # MLP gate (no pairing; pairing restored before active position 30, evaluation 10) or from
    # its own kernel after the bypass restore (pairing restored before the head, evaluation 0)
    for tr, ev in ((False, 0), (True, 10), (True, 0)):
        v = [bits(model.forward(lat, 0.8, eval_index=ev,
                                opts=model.opts(fused_head_adaln=fh, token_reduction=tr)).clone())
             for fh in (1, 0)]
        assert np.array_equal(v[0], v[1]), (tr, ev)


def test_512sq_loop_reduced_depth():
    # the 512x512x22 shape with 2 blocks, --steps 4 --reuse 1
    w = dataclasses.replace(S.WORKLOADS["512sq_22f"], n_blocks=2)
    model = DiTModel(w)
    om = oracle_model(w)
    loop_parity(w, model, om, {}, 4, 1, [0, 1])


def test_512sq_full_depth_zero_gates_and_determinism():
    # all 50 blocks at the full shape, in the launch configuration the benchmark times.
    # With every gate forced to zero the blocks must leave the residual untouched, so the
    # velocity is the head of the patch embedding (computed by the oracle at full size).
    w = S.WORKLOADS["512sq_22f"]
    model = DiTModel(w)
    lat = model.initial_latent()
    v1 = model.forward(lat, 1.0).clone()
    v2 = model.forward(lat, 1.0).clone()
    torch.cuda.synchronize()
    assert np.array_equal(bits(v1), bits(v2)), "forward not deterministic"
    assert np.isfinite(f64(v1)).all()
    d = w.d_model
    for r in (2, 5):  # gate rows of the shared projection and of every block's table
        model.gw["mod_w"][r * d:(r + 1) * d].zero_()
        model.gw["mod_b"][r * d:(r + 1) * d].zero_()
        model.gw["mod_table"][:, r].zero_()
    v0 = model.forward(lat, 1.0)
    torch.cuda.synchronize()
    # the oracle's weights from the seeded generator (the zeroed gate rows do not enter the head)
    g = oracle_model(w, blocks=[])["global"]
    _, fin = dit.modulation(g, 1.0)
    ref = dit.final_head(dit.patch_embed(oracle_latent(w), g), g, fin)
    assert_close(f64(v0), ref, rel=2e-2, elem=8e-2, what="zero-gate velocity")


def test_512sq_token_reduction_loop_reduced_depth():
    # the 512x512x22 shape with 5 blocks and token pairing (1536 -> 768 tokens after the third
    # block, restored before the head), --steps 2 --reuse 1
    w = dataclasses.replace(S.WORKLOADS["512sq_22f_tr"], n_blocks=5, layers=0, steps=2, reuse=1)
    model = DiTModel(w)
    om = oracle_model(w)
    loop_parity(w, model, om, {"token_reduction": True}, 2, 1, [0, 1, 2, 3, 4])


def test_864x480_loop_reduced_depth():
    # the 864x480x22 shape (2430 tokens: ragged tiles in every product and attention) with 2
    # blocks, --steps 4 --reuse 1
    w = dataclasses.replace(S.WORKLOADS["864x480_22f"], n_blocks=2)
    model = DiTModel(w)
    assert model.geo.n_tokens == 2430
    om = oracle_model(w)
    loop_parity(w, model, om, {}, 4, 1, [0, 1])


def test_864x480_token_reduction_loop_reduced_depth():
    # odd grid width 27: token pairing leaves the last column of every row alone (2430 -> 1260)
    w = dataclasses.replace(S.WORKLOADS["864x480_22f_tr"], n_blocks=5, layers=0, steps=2, reuse=1)
    model = DiTModel(w)
    om = oracle_model(w)
    loop_parity(w, model, om, {"token_reduction": True}, 2, 1, [0, 1, 2, 3, 4])


def test_int8_path_forward_and_loop():
    # the whole int8 path: int8 QKV and FC1 with the fused row quantisation, grouped int8 FC2,
    # through the forward with token pairing and the Euler loop
    w = dataclasses.replace(TR_SMALL, fc2_mode="grouped", int8_linear=True, steps=6)
    model = DiTModel(w)
    om = oracle_model(w)
    active = oracle_active(w, om)
    assert model.active() == active
    lat = model.initial_latent()
    for tr in (False, True):
        v = model.forward(lat, 0.6, active, eval_index=3, opts=model.opts(token_reduction=tr))
        torch.cuda.synchronize()
        ref = dit.dit_forward(f64(lat), om, 0.6, active, oracle_geom(w), w.n_heads, eval_index=3,
                              fc2_mode="grouped", token_reduction=tr, int8_linear=True)
        assert_close(f64(v), ref, rel=2e-2, elem=8e-2, what=f"int8 velocity token_reduction={tr}")
    loop_parity(w, model, om, {"fc2_mode": "grouped", "int8_linear": True, "token_reduction": True},
                6, 2, active)


@pytest.mark.parametrize("tr", [False, True])
def test_core_reuse_cached_forward(tr):
    w = TR_SMALL
    model = DiTModel(w)
    om = oracle_model(w)
    active = oracle_active(w, om)
    assert model.active() == active
    lat = model.initial_latent()
    n, d = model.geo.n_tokens, w.d_model
    opts = model.opts(token_reduction=tr)
    v_plain = model.forward(lat, 0.6, active, 2, opts).clone()
    delta = torch.empty((n, d), dtype=torch.float32, device=DEV)
    v_fresh = model.forward_cached(lat, 0.6, True, delta, active, 2, opts).clone()
    torch.cuda.synchronize()
    # the fresh cached evaluation is the forward, bit for bit
    assert np.array_equal(bits(v_fresh), bits(v_plain))
    tr_ref = {}
    v_ref = dit.dit_forward(f64(lat), om, 0.6, active, oracle_geom(w), w.n_heads,
                            eval_index=2, token_reduction=tr, trace=tr_ref)
    _, d_ref = dit.dit_forward_cached(f64(lat), om, 0.6, active, oracle_geom(w), w.n_heads,
                                      eval_index=2, token_reduction=tr)
    # the delta is a small difference of two bf16 streams: besides 2e-2 of its own norm it
    # carries the bf16 rounding of every residual update of the stream, about sqrt(blocks)
    # units of 2^-9 relative to the stream (a wrong sign or a missed restore is far above)
    err = np.linalg.norm(f64(delta) - d_ref)
    floor = 2.0 ** -8 * np.sqrt(len(active)) * np.linalg.norm(tr_ref["x_core_out"])
    assert err <= 2e-2 * np.linalg.norm(d_ref) + floor, (err, np.linalg.norm(d_ref), floor)
    assert np.linalg.norm(d_ref) > 4 * floor   # the bar still resolves the delta itself
    # reused at the same latent and sigma: x_0 + delta is the core output again
    v_reuse = model.forward_cached(lat, 0.6, False, delta, active, 2, opts).clone()
    torch.cuda.synchronize()
    assert rel_l2(f64(v_reuse), f64(v_fresh)) < 1e-3
    # the final AdaLN inside the head product or as its own kernel: the same bits
    opts_u = model.opts(token_reduction=tr, fused_head_adaln=True)
    v_reuse_u = model.forward_cached(lat, 0.6, False, delta, active, 2, opts_u)
    v_plain_u = model.forward(lat, 0.6, active, 2, opts_u)
    torch.cuda.synchronize()
    assert np.array_equal(bits(v_reuse_u), bits(v_reuse))
    assert np.array_equal(bits(v_plain_u), bits(v_plain))
    # reused at another point: the oracle's patch + cached delta + head of that sigma
    lat2 = lat * 0.8
    v2 = model.forward_cached(lat2, 0.35, False, delta, active, 2, opts)
    torch.cuda.synchronize()
    ref2, _ = dit.dit_forward_cached(f64(lat2), om, 0.35, active, oracle_geom(w), w.n_heads,
                                     core_delta=f64(delta))
    assert_close(f64(v2), ref2, rel=2e-2, elem=8e-2, what="reused velocity")


def test_core_reuse_loop():
    w = dataclasses.replace(S.WORKLOADS["tiny_256sq_5f"], steps=7, core_reuse=3)
    model = DiTModel(w)
    om = oracle_model(w)
    lat0 = model.initial_latent()
    x = lat0.clone()
    ev = model.denoise(x, 7, 1, [0, 1], model.opts(), core_reuse=3)
    torch.cuda.synchronize()
    ref, ev_ref = dit.denoise(f64(lat0), om, 7, 1, [0, 1], oracle_geom(w), w.n_heads,
                              core_reuse=3)
    assert ev == ev_ref == 3
    r1 = rel_l2(f64(x), ref)
    r2 = rel_l2(f64(x) - f64(lat0), ref - f64(lat0))
    assert r1 < 5e-2 and r2 < 5e-2, (r1, r2)
