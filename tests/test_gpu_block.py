"""GPU parity of one DiT block (h3_dit_block_fwd) against the oracle, at the small workload's
shape and at the 512x512x22 shape, for every FC2 mode; fused and unfused gate/AdaLN
variants bit-identical.

The oracle receives the same seeded inputs (weights, residual x, text context) and the
modulation it computes itself; the GPU receives that modulation as float32.  Bars: the
block output within rel-L2 2e-2 of the oracle; the block delta (out - in) within 2e-2 of
its norm plus the bf16 rounding floor of the stored output; and, because the residual would
otherwise hide branch errors, the two branch outputs y (attention) and m (MLP), q after
RMSNorm + RoPE and both attention outputs, read back from the workspace, each within
rel-L2 2e-2.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import dit
from tests.gpu_util import DEV, assert_close, bits, f64, rel_l2
from tests.oracle_model import oracle_geom, oracle_model
from video_diffusion_transformer_fwd_amd import binding as B
from video_diffusion_transformer_fwd_amd import synthetic as S
from video_diffusion_transformer_fwd_amd.runtime import DiTModel

pytestmark = pytest.mark.gpu

_MODELS = {}


def gpu_model(name, n_blocks=2, fc2_mode="bf16", frames=None):
    key = (name, n_blocks, frames)
    if key not in _MODELS:
        w = dataclasses.replace(S.WORKLOADS[name], n_blocks=n_blocks, layers=0, fc2_mode=fc2_mode)
        if frames is not None:
            w = dataclasses.replace(w, frames=frames)
        _MODELS[key] = (w, DiTModel(w, with_int8=True, with_int8_linear=True), oracle_model(w))
    return _MODELS[key]


def ws_view(ws, off, shape, dtype=torch.bfloat16):
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + n].view(dtype).view(*shape)


def run_block(model, w, b, x, mod_dev, opts, n1_next=None, mod_next=None):
    ws = model.workspace(model.geo.n_tokens, opts)
    B.h3_dit_block_fwd(model.handle, b, model.geo.geom, opts, x, None, n1_next, mod_dev[b],
                       mod_next, model.ctx_kv[b], ws)
    torch.cuda.synchronize()
    return ws


@pytest.mark.parametrize("name", ["tiny_256sq_5f", "512sq_22f"])
@pytest.mark.parametrize("fc2_mode,int8_linear", [("bf16", False), ("row", False), ("grouped", False),
                                                  ("bf16", True), ("grouped", True)])
def test_block_parity(name, fc2_mode, int8_linear):
    w, model, om = gpu_model(name)
    n, d = model.geo.n_tokens, w.d_model
    sigma = 0.75
    mod, fin = dit.modulation(om["global"], sigma)
    mod_dev = torch.tensor(mod, dtype=torch.float32, device=DEV)
    geo = oracle_geom(w)
    assert geo["n"] == n
    coords = dit.rope_coords(geo["f_lat"], geo["grid_h"], geo["grid_w"], geo["scale"])
    x0 = S.normal("test.block.x", (n, d), 1.0)
    opts = B.make_opts(fc2_mode=fc2_mode, int8_linear=int8_linear, store_branches=True)
    for b in range(w.n_blocks):
        x = x0.to(DEV)
        ws = run_block(model, w, b, x, mod_dev, opts)
        lay = B.h3_workspace_layout(model.handle, n, opts)
        tr = {}
        ref = dit.block_forward(f64(x0), om["blocks"][b], mod[b], om["ctx"], coords, w.n_heads,
                                fc2_mode=fc2_mode, trace=tr, int8_linear=int8_linear)
        got = f64(x)
        tag = f"{name} {fc2_mode} int8_linear={int8_linear} block {b}"
        assert_close(got, ref, rel=2e-2, elem=6e-2, what=f"{tag} out")
        # block delta: the stored output is bf16, whose rounding (at most 2^-8 relative per
        # element) is a floor under any comparison of a delta that is small next to x
        dx, dref = got - f64(x0), ref - f64(x0)
        err = np.linalg.norm(dx - dref)
        assert err <= 2e-2 * np.linalg.norm(dref) + 2.0 ** -8 * np.linalg.norm(ref), f"{tag} delta"
        y = f64(ws_view(ws, lay.y, (n, d)))
        m = f64(ws_view(ws, lay.m, (n, d)))
        assert rel_l2(y, tr["y"]) < 2e-2, f"{tag} attention branch {rel_l2(y, tr['y'])}"
        assert rel_l2(m, tr["m"]) < 2e-2, f"{tag} MLP branch {rel_l2(m, tr['m'])}"
        # q after RMSNorm + RoPE, and the attention outputs, at the same bar
        qkvq = f64(ws_view(ws, lay.qkvq, (n, 4 * d)))
        assert rel_l2(qkvq[:, :d], tr["q"].reshape(n, d)) < 2e-2, f"{tag} q"
        attn = f64(ws_view(ws, lay.attn, (n, 2 * d)))
        assert rel_l2(attn[:, :d], tr["o"]) < 2e-2, f"{tag} self-attention"
        assert rel_l2(attn[:, d:], tr["oc"]) < 2e-2, f"{tag} cross-attention"


def valid_bytes(t, n, d, int8_linear):
    """The defined part of an AdaLN output buffer: bf16 [n, d], or int8 [n, d] + float [n]."""
    b = t.detach().contiguous().view(torch.uint8).reshape(-1)
    return (b[:n * d + 4 * n] if int8_linear else b).cpu().numpy()


@pytest.mark.parametrize("name", ["tiny_256sq_5f", "512sq_22f"])
@pytest.mark.parametrize("int8_linear", [False, True])
def test_fused_and_unfused_bit_identical(name, int8_linear):
    w, model, om = gpu_model(name)
    n, d = model.geo.n_tokens, w.d_model
    mod, fin = dit.modulation(om["global"], 0.5)
    mod_dev = torch.tensor(mod, dtype=torch.float32, device=DEV)
    x0 = S.normal("test.block.x2", (n, d), 1.0).to(DEV)
    outs = {}
    # (gate + AdaLN-2, MLP gate + next AdaLN-1, Q/K RMSNorm + RoPE in the QKV epilogue)
    for fg, fc, fq in [(1, 1, 1), (0, 0, 0), (1, 0, 0), (0, 1, 1)]:
        opts = B.make_opts(fused_gate_adaln=fg, fused_cross_block=fc, int8_linear=int8_linear,
                           fused_qk_rope=fq)
        x = x0.clone()
        n1n = torch.empty_like(x)
        ws = run_block(model, w, 0, x, mod_dev, opts, n1n, mod_dev[1])
        lay = B.h3_workspace_layout(model.handle, n, opts)
        outs[(fg, fc, fq)] = (bits(x), valid_bytes(n1n, n, d, int8_linear),
                              valid_bytes(ws_view(ws, lay.n2, (n, d)), n, d, int8_linear),
                              bits(ws_view(ws, lay.qkvq, (n, 4 * d))), x.clone(), n1n.clone())
    ref = outs[(1, 1, 1)]
    for k, v in outs.items():
        for a, b_, what in zip(v[:4], ref[:4], ("x", "n1_next", "n2", "qkvq")):
            assert np.array_equal(a, b_), f"{name} {what} differs for fused={k}"
    # n1_next is the next block's AdaLN-1 of the output stream (dequantised in int8 mode)
    want = dit.adaln(f64(ref[4]), mod[1][0], mod[1][1])
    if int8_linear:
        raw = ref[5].view(torch.uint8).reshape(-1)
        q = raw[:n * d].view(torch.int8).reshape(n, d).cpu().numpy().astype(np.float64)
        sc = raw[n * d:n * d + 4 * n].view(torch.float32).cpu().numpy().astype(np.float64)
        assert rel_l2(q * sc[:, None], want) < 2e-2
    else:
        assert_close(f64(ref[5]), want, rel=1e-2, elem=3e-2, what="n1_next")


def test_block_deterministic_run_to_run():
    w, model, om = gpu_model("512sq_22f")
    n, d = model.geo.n_tokens, w.d_model
    mod, _ = dit.modulation(om["global"], 1.0)
    mod_dev = torch.tensor(mod, dtype=torch.float32, device=DEV)
    x0 = S.normal("test.block.x3", (n, d), 1.0).to(DEV)
    res = []
    for _ in range(2):
        x = x0.clone()
        run_block(model, w, 1, x, mod_dev, B.make_opts())
        res.append(bits(x))
    assert np.array_equal(res[0], res[1])


def test_block_rejects_bad_arguments():
    w, model, om = gpu_model("tiny_256sq_5f")
    n, d = model.geo.n_tokens, w.d_model
    x = torch.zeros((n, d), dtype=torch.bfloat16, device=DEV)
    mod = torch.zeros((6, d), dtype=torch.float32, device=DEV)
    opts = B.make_opts()
    small = torch.empty(1024, dtype=torch.uint8, device=DEV)
    with pytest.raises(B.H3Error) as e:
        B.h3_dit_block_fwd(model.handle, 0, model.geo.geom, opts, x, None, None, mod, None,
                           model.ctx_kv[0], small)
    assert e.value.code == B.H3_EWORKSPACE
    ws = model.workspace(n, opts)
    with pytest.raises(B.H3Error) as e:
        B.h3_dit_block_fwd(model.handle, 5, model.geo.geom, opts, x, None, None, mod, None,
                           model.ctx_kv[0], ws)
    assert e.value.code == B.H3_EINVAL
    with pytest.raises(B.H3Error):
        B.h3_dit_block_fwd(model.handle, 0, model.geo.geom, opts, x, None, x, mod, None,
                           model.ctx_kv[0], ws)


@pytest.mark.parametrize("frames", [22, 5])
def test_int8_row_split_k_bit_identical_to_unsplit(frames):
    # inside the block the int8 FC2 at 1536 rows (22 frames: 384x192 tiles) or 512 rows (5
    # frames: 192x192 tiles) splits K over four workgroups per tile and adds the int32 partials
    # in a second launch; the standalone product runs unsplit.  Integer partial sums are exact,
    # so both must give the same bf16 bits from the same quantised input.
    w, model, om = gpu_model("512sq_22f", frames=frames)
    n, d, F = model.geo.n_tokens, w.d_model, w.ffn_dim
    mod, _ = dit.modulation(om["global"], 0.75)
    mod_dev = torch.tensor(mod, dtype=torch.float32, device=DEV)
    x = S.normal("test.block.x3", (n, d), 1.0).to(DEV)
    opts = B.make_opts(fc2_mode="row", store_branches=True)
    ws = run_block(model, w, 1, x, mod_dev, opts)
    lay = B.h3_workspace_layout(model.handle, n, opts)
    hq = ws_view(ws, lay.hq, (n, F), torch.int8).clone()
    hs = ws_view(ws, lay.hs, (n, 1), torch.float32).clone()
    m_blk = ws_view(ws, lay.m, (n, d)).clone()
    blk = model.blocks[1]
    out = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    B.h3_gemm_i8(hq, hs, blk["fc2_q"], blk["fc2_s"], blk["fc2_b"], out, F)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(m_blk))
    # and both equal the exact integer product dequantised by the oracle's rule, on sampled rows
    rows = np.array([0, 1, 317, n // 2 + 5, n - 1])
    qa = hq[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    sa = hs[torch.as_tensor(rows, device=DEV)].cpu().numpy()
    acc = dit.int8_accumulate(qa, blk["fc2_q"].cpu().numpy(), None)
    ref = dit.f32_to_bf16(dit.dequant(acc, sa, blk["fc2_s"].cpu().numpy().reshape(-1),
                                      f64(blk["fc2_b"]).astype(np.float32)))
    got = out[torch.as_tensor(rows, device=DEV)].cpu().to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
