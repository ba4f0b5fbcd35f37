"""Parity at the 768x1344x243-frame shapes (61,488 tokens, d = 5120, 40 heads x 128,
MLP 20480, 512 text tokens) in the launch configurations the forward uses.

The oracle cannot redo whole products at this size, so each kernel is checked on sampled
outputs it can compute one by one (dot products, single attention rows, single AdaLN rows)
from the same seeded inputs, and the whole forward through properties that hold at any
size (zero gates leave the residual untouched; fused and unfused variants are bit-identical).
"""
import numpy as np
import pytest
import torch

from oracle import dit
from tests.gpu_util import DEV, assert_close, f64
from tests.oracle_model import oracle_geom, oracle_latent, oracle_model
from video_diffusion_transformer_fwd_amd import binding as B
from video_diffusion_transformer_fwd_amd import synthetic as S

pytestmark = pytest.mark.gpu

N, D_MODEL, HEADS, HD, FFN, LCTX = 61488, 5120, 40, 128, 20480, 512


def randn_bf16(seed, shape, std=1.0):
    """Seeded N(0, std^2) bf16 tensor drawn on the device (the inputs are too large to draw on
    the host in reasonable time; only sampled rows travel back to the oracle)."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    return (torch.randn(shape, generator=g, device=DEV, dtype=torch.float32) * std).to(torch.bfloat16)


def sample_rows(n, k, seed):
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(n - 2, size=k - 2, replace=False))
    return np.concatenate([[0], rows + 1, [n - 1]])  # first, random, last (ragged tail)


@pytest.mark.parametrize("M,Nn,K,epi", [(N, FFN, D_MODEL, 1), (N, D_MODEL, FFN, 0), (N, 4 * D_MODEL, D_MODEL, 0)])
def test_gemm_sampled(M, Nn, K, epi):
    A = randn_bf16(M + K, (M, K))
    W = randn_bf16(Nn + K, (Nn, K), 0.02)
    b = randn_bf16(Nn, (Nn,), 0.02)
    C = torch.empty((M, Nn), dtype=torch.bfloat16, device=DEV)
    B.h3_gemm_bf16(A, W, C, bias=b, epilogue=epi)
    torch.cuda.synchronize()
    rows = sample_rows(M, 48, 1)
    cols = sample_rows(Nn, 64, 2)
    a = f64(A[torch.as_tensor(rows, device=DEV)])
    w = f64(W[torch.as_tensor(cols, device=DEV)])
    ref = dit.linear(a, w, f64(b)[cols])
    if epi:
        ref = dit.gelu(ref)
    got = f64(C[torch.as_tensor(rows, device=DEV)][:, torch.as_tensor(cols, device=DEV)])
    assert_close(got, ref, rel=6e-3, elem=1.5e-2, what="gemm sampled")


def test_self_attention_sampled_rows():
    d = HEADS * HD
    qkvq = randn_bf16(7, (N, 4 * d))
    O = torch.zeros((N, 2 * d), dtype=torch.bfloat16, device=DEV)
    B.h3_attention(qkvq[:, :d], qkvq[:, d:2 * d], qkvq[:, 2 * d:3 * d], O[:, :d], N, N, HEADS, HD)
    torch.cuda.synchronize()
    rows = sample_rows(N, 12, 3)
    heads = [0, 13, 39]
    k = f64(qkvq[:, d:2 * d]).reshape(N, HEADS, HD)[:, heads]
    v = f64(qkvq[:, 2 * d:3 * d]).reshape(N, HEADS, HD)[:, heads]
    q = f64(qkvq[torch.as_tensor(rows, device=DEV), :d]).reshape(len(rows), HEADS, HD)[:, heads]
    ref = dit.attention(q, k, v)
    got = f64(O[torch.as_tensor(rows, device=DEV), :d]).reshape(len(rows), HEADS, HD)[:, heads]
    assert_close(got, ref, rel=1e-2, elem=3e-2, what="self-attention rows")


def test_cross_attention_sampled_rows():
    d = HEADS * HD
    q = randn_bf16(8, (N, d))
    kv = randn_bf16(18, (2 * LCTX, d))
    O = torch.empty((N, d), dtype=torch.bfloat16, device=DEV)
    B.h3_attention(q, kv[:LCTX], kv[LCTX:], O, N, LCTX, HEADS, HD)
    torch.cuda.synchronize()
    rows = sample_rows(N, 64, 4)
    ref = dit.attention(f64(q[torch.as_tensor(rows, device=DEV)]).reshape(-1, HEADS, HD),
                        f64(kv[:LCTX]).reshape(LCTX, HEADS, HD), f64(kv[LCTX:]).reshape(LCTX, HEADS, HD))
    got = f64(O[torch.as_tensor(rows, device=DEV)]).reshape(-1, HEADS, HD)
    assert_close(got, ref, rel=1e-2, elem=3e-2, what="cross-attention rows")


def test_gate_adaln_full_size():
    rng = np.random.default_rng(9)
    x = randn_bf16(9, (N, D_MODEL))
    y = randn_bf16(19, (N, D_MODEL))
    vec = lambda: torch.tensor(rng.standard_normal(D_MODEL) * 0.2, dtype=torch.float32, device=DEV)
    g, sh, sc = vec(), vec(), vec()
    xf, nf = x.clone(), torch.empty_like(x)
    B.h3_gate_adaln(xf, y, g, xf, sh, sc, nf)
    xu, nu = x.clone(), torch.empty_like(x)
    B.h3_gate_adaln(xu, y, g, xu, None, None, None)
    B.h3_gate_adaln(xu, None, None, None, sh, sc, nu)
    torch.cuda.synchronize()
    assert torch.equal(xf.view(torch.int16), xu.view(torch.int16))
    assert torch.equal(nf.view(torch.int16), nu.view(torch.int16))
    rows = torch.as_tensor(sample_rows(N, 64, 5), device=DEV)
    gx = dit.gated_residual(f64(x[rows]), f64(g), f64(y[rows]))
    assert_close(f64(nf[rows]), dit.adaln(gx, f64(sh), f64(sc)), rel=1e-2, elem=3e-2, what="adaln rows")


def test_qk_norm_rope_full_geometry():
    geom = B.make_geom(61, 24, 42, 1.0, 0)
    assert B.h3_geom_tokens(geom) == N
    d = D_MODEL
    buf = randn_bf16(10, (N, 4 * d))
    before_rows = torch.as_tensor(sample_rows(N, 32, 6), device=DEV)
    before = f64(buf[before_rows])
    qg = torch.ones(HD, dtype=torch.bfloat16, device=DEV)
    table = torch.empty((N, HD // 2, 2), dtype=torch.float32, device=DEV)
    B.h3_rope_table(geom, HD, table)
    B.h3_qk_norm_rope(buf, N, d, HD, qg, qg, 1, table)
    torch.cuda.synchronize()
    coords = dit.rope_coords(61, 24, 42, 1.0)[before_rows.cpu().numpy()]
    q = dit.rms_norm_heads(before[:, :d].reshape(-1, HEADS, HD), np.ones(HD))
    ref = dit.rope_apply(q, coords).reshape(-1, d)
    assert_close(f64(buf[before_rows])[:, :d], ref, rel=6e-3, elem=2e-2, what="q rows")


def test_forward_full_size_zero_gates_and_fused_identity():
    w = S.WORKLOADS["768x1344_243f"]
    from video_diffusion_transformer_fwd_amd.runtime import DiTModel
    model = DiTModel(w)
    assert model.geo.n_tokens == N
    lat = model.initial_latent()
    v1 = model.forward(lat, 1.0).clone()
    v2 = model.forward(lat, 1.0, opts=model.opts(fused_gate_adaln=False, fused_cross_block=False,
                                                 fused_qk_rope=False, fused_head_adaln=False)).clone()
    torch.cuda.synchronize()
    assert torch.equal(v1.view(torch.int32), v2.view(torch.int32)), "fused and unfused forwards differ"
    assert torch.isfinite(v1).all()
    d = w.d_model
    for r in (2, 5):
        model.gw["mod_w"][r * d:(r + 1) * d].zero_()
        model.gw["mod_b"][r * d:(r + 1) * d].zero_()
        model.gw["mod_table"][:, r].zero_()
    v0 = model.forward(lat, 1.0)
    torch.cuda.synchronize()
    # the oracle's weights from the seeded generator (the zeroed gate rows do not enter the head)
    g = oracle_model(w, blocks=[])["global"]
    _, fin = dit.modulation(g, 1.0)
    rows_np = sample_rows(N, 256, 11)
    rows = torch.as_tensor(rows_np, device=DEV)
    ref = dit.final_head(dit.patch_embed(oracle_latent(w)[rows_np], g), g, fin)
    assert_close(f64(v0[rows]), ref, rel=2e-2, elem=8e-2, what="zero-gate velocity rows")
    model.close()


def test_block_local_chain_sampled_rows():
    """Blocks 0, 24 and 49 of the 768x1344 model, each on its own seeded bf16 input, in the
    forward's launch configuration (fused gates, Q/K RMSNorm + RoPE in the QKV epilogue).
    Every stage is checked on sampled token rows against the oracle applied to the GPU's own
    input to that stage, read back from the workspace: AdaLN-1 from x; QKV, q/k and qc from
    n1; both attentions from q or qc and all of the GPU's keys and values; the output
    projection from [O | Oc]; AdaLN-2 of x + g1 y from y; FC1 + GELU from n2; FC2 from h; and
    the block output x + g1 y + g2 m from m."""
    from video_diffusion_transformer_fwd_amd.runtime import DiTModel
    w = S.WORKLOADS["768x1344_243f"]
    model = DiTModel(w)
    d, H, F = w.d_model, w.n_heads, w.ffn_dim
    Dh = d // H
    geo = model.geo
    og = oracle_geom(w)
    assert og["n"] == N == geo.n_tokens
    g = oracle_model(w, blocks=[])["global"]
    mod, _ = dit.modulation(g, 0.75)
    mod_dev = torch.tensor(mod, dtype=torch.float32, device=DEV)
    coords = dit.rope_coords(og["f_lat"], og["grid_h"], og["grid_w"], og["scale"])
    opts = B.make_opts(store_branches=True)
    lay = B.h3_workspace_layout(model.handle, N, opts)
    rows = sample_rows(N, 10, 21)
    rt = torch.as_tensor(rows, device=DEV)

    def ws_view(ws, off, width, dtype=torch.bfloat16):
        n = N * width * torch.tensor([], dtype=dtype).element_size()
        return ws[off:off + n].view(dtype).view(N, width)

    for b in (0, 24, 49):
        print(f"block {b}", flush=True)
        x0 = randn_bf16(100 + b, (N, d))
        x = x0.clone()
        ws = model.workspace(N, opts)
        B.h3_dit_block_fwd(model.handle, b, geo.geom, opts, x, None, None, mod_dev[b], None,
                           model.ctx_kv[b], ws)
        torch.cuda.synchronize()
        sh1, sc1, g1, sh2, sc2, g2 = mod[b]
        blk = model.blocks[b]
        tag = f"block {b}"
        xr = f64(x0[rt])
        n1 = f64(ws_view(ws, lay.n1, d)[rt])
        assert_close(n1, dit.adaln(xr, sh1, sc1), what=f"{tag} n1")
        pre = dit.linear(n1, f64(blk["qkvq_w"]), f64(blk["qkvq_b"]))
        full = ws_view(ws, lay.qkvq, 4 * d)
        qkvq = f64(full[rt])
        q = dit.rope_apply(dit.rms_norm_heads(pre[:, :d].reshape(-1, H, Dh), f64(blk["q_gamma"])), coords[rows])
        k = dit.rope_apply(dit.rms_norm_heads(pre[:, d:2 * d].reshape(-1, H, Dh), f64(blk["k_gamma"])), coords[rows])
        assert_close(qkvq[:, :d], q.reshape(-1, d), what=f"{tag} q")
        assert_close(qkvq[:, d:2 * d], k.reshape(-1, d), what=f"{tag} k")
        assert_close(qkvq[:, 2 * d:], pre[:, 2 * d:], what=f"{tag} v, qc")
        kk = f64(full[:, d:2 * d]).reshape(N, H, Dh)
        vv = f64(full[:, 2 * d:3 * d]).reshape(N, H, Dh)
        o_ref = dit.attention(qkvq[:, :d].reshape(-1, H, Dh), kk, vv).reshape(-1, d)
        del kk, vv
        kc = f64(model.ctx_kv[b, 0]).reshape(-1, H, Dh)
        vc = f64(model.ctx_kv[b, 1]).reshape(-1, H, Dh)
        oc_ref = dit.attention(qkvq[:, 3 * d:].reshape(-1, H, Dh), kc, vc).reshape(-1, d)
        attn = f64(ws_view(ws, lay.attn, 2 * d)[rt])
        assert_close(attn[:, :d], o_ref, what=f"{tag} self-attention")
        assert_close(attn[:, d:], oc_ref, what=f"{tag} cross-attention")
        y_ref = dit.linear(attn, f64(blk["out_w"]), f64(blk["out_b"]) + f64(blk["outc_b"]))
        y = f64(ws_view(ws, lay.y, d)[rt])
        assert_close(y, y_ref, what=f"{tag} y")
        x1 = dit.gated_residual(xr, g1, y)
        n2 = f64(ws_view(ws, lay.n2, d)[rt])
        assert_close(n2, dit.adaln(x1, sh2, sc2), what=f"{tag} n2")
        h = f64(ws_view(ws, lay.h, F)[rt])
        assert_close(h, dit.gelu(dit.linear(n2, f64(blk["fc1_w"]), f64(blk["fc1_b"]))), what=f"{tag} h")
        m = f64(ws_view(ws, lay.m, d)[rt])
        assert_close(m, dit.linear(h, f64(blk["fc2_w"]), f64(blk["fc2_b"])), what=f"{tag} m")
        assert_close(f64(x[rt]), dit.gated_residual(x1, g2, m), what=f"{tag} output")
        del ws
    model.close()
