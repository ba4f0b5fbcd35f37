"""Oracle: float64 arithmetic of the MiniMax-H3 DiT denoiser (TEST INFRASTRUCTURE ONLY).

One fresh evaluation is: timestep embedding -> modulation -> patch embedding -> active
blocks (AdaLN, QKV, Q/K RMSNorm, 3D RoPE, self-attention, cross-attention, gated
residual, AdaLN, GELU MLP, gated residual) -> final AdaLN -> head.  The Euler loop
consumes the velocity under the --steps / --reuse / --layers schedule (``oracle.host``).

Everything is float64 NumPy; a matrix product (``@``) is the only library primitive.
Inputs are float64 arrays (exact images of the bf16 weights the GPU uses).  Nothing is
rounded to bf16 here except in the int8 FC2 helpers, whose quantisation decisions are
defined in float32 (see ``quantize_rows``).

Weights follow the ``[out, in]`` convention: ``linear(x, W, b) = x @ W.T + b``.
Model dict keys (d = width, F = MLP width, C = latent channels, D = head dim):
  global: t1_w [d,256] t1_b, t2_w [d,d] t2_b, mod_w [6d,d] mod_b [6d],
          fin_w [2d,d] fin_b [2d], fin_t [2,d], mod_table [n_blocks,6,d],
          patch_w [d,C] patch_b, head_w [C,d] head_b [C]
  block : qkv_w [3d,d] qkv_b, qc_w kc_w vc_w o_w oc_w [d,d] (+ _b), q_gamma k_gamma [D],
          fc1_w [F,d] fc1_b [F], fc2_w [d,F] fc2_b [d]
"""
from __future__ import annotations

import math

import numpy as np

from . import host

LN_EPS = 1e-6
RMS_EPS = 1e-6
ROPE_THETA = 10000.0
TIME_FREQ_DIM = 256


# --------------------------------------------------------------------------- timestep
def timestep_embedding(sigma: float) -> np.ndarray:
    """Sinusoidal embedding of the timestep, [256].

    The pages only say shift/scale/gate come from the timestep (P3 "DiT fusions").
    Reading: t = 1000 sigma; e = [cos(t w_j) for j<128] ++ [sin(t w_j) for j<128] with
    w_j = 10000^(-j/128).
    """
    t = 1000.0 * float(sigma)
    half = TIME_FREQ_DIM // 2
    j = np.arange(half, dtype=np.float64)
    w = np.power(10000.0, -j / half)
    return np.concatenate([np.cos(t * w), np.sin(t * w)])


def silu(x):
    return x / (1.0 + np.exp(-x))


def linear(x, w, b=None):
    y = x @ w.T
    if b is not None:
        y = y + b
    return y


def modulation(g: dict, sigma: float):
    """Per-block AdaLN parameters for one timestep.

    P3 "DiT fusions" / "aggressive levers": every block has AdaLN shift/scale and residual
    gates, and the gates differ per block (thinning ranks them).
    Reading: temb = t2(SiLU(t1(e))); M = mod(SiLU(temb)) in R^{6d}; block b uses
    M + T_b with T_b = mod_table[b] (rows sh1, sc1, g1, sh2, sc2, g2); the final AdaLN uses
    fin(SiLU(temb)) + fin_t (rows shift, scale).
    Returns (mod [n_blocks, 6, d], mod_final [2, d]).
    """
    e = timestep_embedding(sigma)
    temb = linear(silu(linear(e, g["t1_w"], g["t1_b"])), g["t2_w"], g["t2_b"])
    u = silu(temb)
    d = g["t2_w"].shape[0]
    m = linear(u, g["mod_w"], g["mod_b"]).reshape(6, d)
    mod = m[None, :, :] + g["mod_table"]
    fin = linear(u, g["fin_w"], g["fin_b"]).reshape(2, d) + g["fin_t"]
    return mod, fin


# --------------------------------------------------------------------------- norms
def layer_norm(z):
    """LayerNorm over the last axis without affine: (z - mean) / sqrt(var + 1e-6), biased var.

    Reading: the usual no-affine adaLN LayerNorm (pages: "AdaLN", P3 "DiT fusions").
    """
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    return (z - mu) / np.sqrt(var + LN_EPS)


def adaln(x, shift, scale):
    """AdaLN: LN(x) * (1 + scale) + shift (reading: standard adaLN modulation)."""
    return layer_norm(x) * (1.0 + scale) + shift


def gated_residual(x, gate, branch):
    """x + gate * branch (P3 "DiT fusions": residual gates; reading: ungated-by-tanh, plain product)."""
    return x + gate * branch


def rms_norm_heads(t, gamma):
    """Per-head RMSNorm over the head dim: t / sqrt(mean(t^2) + 1e-6) * gamma.

    P3 "the int8 path" names an RMS norm of Q and K before RoPE.  Reading: per head, over D,
    with one gain vector of length D shared by all heads.  t is [N, H, D].
    """
    ms = (t * t).mean(axis=-1, keepdims=True)
    return t / np.sqrt(ms + RMS_EPS) * gamma


# --------------------------------------------------------------------------- RoPE
def rope_split(head_dim: int):
    """Channel split (t, h, w) of one head for 3D RoPE.

    Reading (pages silent on the layout): the two spatial axes get 2*floor(D/6) channels
    each and time gets the rest (D=128 -> 44/42/42, D=64 -> 24/20/20).
    """
    hw = 2 * (head_dim // 6)
    return head_dim - 2 * hw, hw, hw


def rope_coords(f_lat, grid_h, grid_w, spatial_scale, pairs=None):
    """Per-token (f, h, w) RoPE coordinates, [N, 3] float64.

    P2 §5 / P3 "memory and resolution limits": at the 8x8 grid the spatial coordinates are
    halved (``spatial_scale`` = 0.5); time is unchanged.  For a paired (reduced) token the
    coordinates are the mean of its two source tokens (reading).
    """
    f, h, w = np.meshgrid(np.arange(f_lat), np.arange(grid_h), np.arange(grid_w), indexing="ij")
    c = np.stack([f.ravel(), h.ravel() * spatial_scale, w.ravel() * spatial_scale], axis=1)
    c = c.astype(np.float64)
    if pairs is not None:
        c = 0.5 * (c[pairs[:, 0]] + c[pairs[:, 1]])
    return c


def rope_apply(t, coords):
    """Rotate interleaved channel pairs of every head by coordinate-dependent angles.

    Reading: inside each axis slice of width Da, pair j = channels (2j, 2j+1) rotates by
    angle = coord_axis * 10000^(-2j/Da): (a, b) -> (a cos - b sin, a sin + b cos).
    t is [N, H, D]; coords [N, 3].
    """
    n, nh, d = t.shape
    out = t.copy()
    off = 0
    for axis, da in enumerate(rope_split(d)):
        for j in range(da // 2):
            ang = coords[:, axis] * ROPE_THETA ** (-2.0 * j / da)
            c, s = np.cos(ang)[:, None], np.sin(ang)[:, None]
            a = t[:, :, off + 2 * j]
            b = t[:, :, off + 2 * j + 1]
            out[:, :, off + 2 * j] = a * c - b * s
            out[:, :, off + 2 * j + 1] = a * s + b * c
        off += da
    return out


# --------------------------------------------------------------------------- attention
def attention(q, k, v, rows=None, chunk=1024):
    """softmax(q k^T / sqrt(D)) v per head, no mask.  q [Nq,H,D], k/v [Nk,H,D] -> [Nq,H,D].

    Reading: scale 1/sqrt(D), unmasked, softmax over all keys.  ``rows`` restricts the
    query rows computed (each row is independent); queries are processed in chunks only to
    bound memory.
    """
    if rows is not None:
        q = q[rows]
    nq, nh, dh = q.shape
    out = np.empty((nq, nh, v.shape[2]), dtype=np.float64)
    scale = 1.0 / math.sqrt(dh)
    for hh in range(nh):
        kh, vh = k[:, hh, :], v[:, hh, :]
        for s in range(0, nq, chunk):
            sc = (q[s:s + chunk, hh, :] @ kh.T) * scale
            sc = sc - sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            p /= p.sum(axis=1, keepdims=True)
            out[s:s + chunk, hh, :] = p @ vh
    return out


def gelu(x):
    """Exact (erf) GELU: x/2 (1 + erf(x / sqrt 2)).  Reading: the erf form of "GELU"."""
    from scipy.special import erf
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


# --------------------------------------------------------------------------- int8 FC2
def f32_to_bf16(x):
    """Round float32 values to the nearest bf16 (ties to even); returns float32 values.

    Used only by the int8 FC2 helpers, whose output the HIP path stores as bf16.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def quantize_rows(h, group=None):
    """Dynamic symmetric int8 quantisation of FC2 input rows, decided in float32.

    P2 §4 / P4 §4: ``--use-int8-row-fc2`` has one activation scale per FC2 row; P3 "the
    int8 path": the grouped engine has one scale per 1024 FC2-input channels and quantises
    activations dynamically.
    Reading: s = absmax / 127 (float32 division); q = clamp(rint(x / s), -127, 127) with
    round-half-even and float32 division; s = 0 gives q = 0.  ``group`` = channels per
    scale (None = whole row).  h [R, K] -> (q int8 [R,K], s float32 [R, K/group]).
    """
    h32 = np.asarray(h, dtype=np.float32)
    r, k = h32.shape
    g = k if group is None else group
    if k % g:
        raise ValueError("K must be a multiple of the group size")
    hv = h32.reshape(r, k // g, g)
    amax = np.abs(hv).max(axis=2)
    s = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    q = np.rint((hv / safe[:, :, None]).astype(np.float32))
    q = np.clip(q, -127, 127)
    q = np.where(s[:, :, None] > 0, q, 0).astype(np.int8)
    return q.reshape(r, k), s


def quantize_weight(w):
    """Per-output-channel int8 weights (P3 "the int8 path": per-output-channel weight scales).

    Same float32 rule as ``quantize_rows`` with one scale per output row of W [N, K].
    """
    return quantize_rows(w, None)


def int8_accumulate(qa, qw, group=None):
    """Exact integer products per K group: acc[g, r, n] = sum_{k in g} qa[r,k] qw[n,k] (int64).

    Each group's sum is one float64 matrix product.  It is exact: every product of two codes
    in [-127, 127] and every partial sum of at most 2^39 of them is an integer below 2^53 in
    magnitude, so no addition rounds, whatever order the product sums in.
    """
    r, k = qa.shape
    g = k if group is None else group
    if k > (1 << 39):
        raise ValueError("K too large for an exact float64 sum")
    a = qa.astype(np.float64)
    w = qw.astype(np.float64)
    out = np.empty((k // g, r, qw.shape[0]), dtype=np.int64)
    for gi in range(k // g):
        sl = slice(gi * g, (gi + 1) * g)
        out[gi] = (a[:, sl] @ w[:, sl].T).astype(np.int64)
    return out


def dequant(acc, sa, sw, bias):
    """FC2 output from int8 partial sums, float32 arithmetic in a fixed order.

    Reading: m = (sum over groups g ascending of float(acc_g) * s_a[r,g]) * s_w[n] + b[n],
    each operation rounded to float32 (no fused multiply-add).  Returns float32 [R, N].
    """
    ng = acc.shape[0]
    tot = np.zeros(acc.shape[1:], dtype=np.float32)
    for gi in range(ng):
        term = (acc[gi].astype(np.float32) * sa[:, gi:gi + 1].astype(np.float32)).astype(np.float32)
        tot = (tot + term).astype(np.float32)
    out = (tot * np.asarray(sw, np.float32)[None, :]).astype(np.float32)
    return (out + np.asarray(bias, np.float32)[None, :]).astype(np.float32)


def linear_int8(a, w, b):
    """int8 product of a row-quantised activation and per-output-channel int8 weights.

    P3 "the int8 path": the QKV projections and the MLP run as int8 products, activations
    quantised dynamically with per-output-channel weight scales, the quantisation fused into
    the gated-AdaLN kernel, which reads the rows as bf16 and writes int8.
    Reading: the activation is the bf16-rounded value the bf16 path would store; one scale
    per token row; quantisation, integer sums and dequantisation as in ``quantize_rows``,
    ``int8_accumulate`` and ``dequant`` (one group).  Returns the float32 result as float64.
    """
    ab = f32_to_bf16(np.asarray(a, dtype=np.float32))
    qa, sa = quantize_rows(ab, None)
    qw, sw = quantize_weight(np.asarray(w, dtype=np.float32))
    acc = int8_accumulate(qa, qw, None)
    return dequant(acc, sa, sw[:, 0], np.asarray(b, np.float32)).astype(np.float64)


def fc2(h, blk, mode="bf16", group=1024):
    """FC2 of the MLP in one of three modes: 'bf16' (float64 product), 'row', 'grouped'.

    The int8 modes quantise float32(h) and the bf16 weight with the rules above and return
    the float32 dequantised product as float64.
    """
    if mode == "bf16":
        return linear(h, blk["fc2_w"], blk["fc2_b"])
    qw, sw = quantize_weight(blk["fc2_w"])
    g = None if mode == "row" else group
    qa, sa = quantize_rows(h, g)
    acc = int8_accumulate(qa, qw, g)
    return dequant(acc, sa, sw[:, 0], blk["fc2_b"]).astype(np.float64)


# --------------------------------------------------------------------------- token pairing
def token_merge(s, pairs):
    """Average each horizontal pair: x_r[j] = (S[p0] + S[p1]) / 2 (P3 "aggressive levers")."""
    return 0.5 * (s[pairs[:, 0]] + s[pairs[:, 1]])


def token_restore(s, xr, pairs):
    """Bypass restore: x[p] = S[p] + (x_r[j] - merge(S)[j]) for both members of pair j.

    P3 "aggressive levers": a bypass brings back full resolution.  Reading: the saved
    full-resolution stream S keeps the intra-pair detail and receives the change the
    reduced blocks made to the pair mean; merge then restore with no block between is the
    identity.
    """
    delta = xr - token_merge(s, pairs)
    x = s.copy()
    x[pairs[:, 0]] = s[pairs[:, 0]] + delta
    x[pairs[:, 1]] = s[pairs[:, 1]] + delta
    return x


# --------------------------------------------------------------------------- block
def context_kv(ctx, blk):
    """Cross-attention keys/values of the text context for one block ([L, d] each)."""
    return linear(ctx, blk["kc_w"], blk["kc_b"]), linear(ctx, blk["vc_w"], blk["vc_b"])


def block_forward(x, blk, mod_b, ctx, coords, n_heads, qk_norm=True, fc2_mode="bf16",
                  trace=None, int8_linear=False):
    """One DiT block on the residual stream x [N, d].

    P3 "DiT fusions": each active block has an attention residual gate followed by the MLP
    AdaLN, and an MLP residual gate feeding the next block's attention AdaLN.  The block
    order (AdaLN, QKV, 3D-RoPE self-attention, cross-attention to text, gated residual,
    AdaLN, GELU MLP, gated residual) is the one the workload names.
    Reading: both attentions read the same AdaLN output n1 and their projections are summed
    inside the gated attention branch:
      n1 = AdaLN(x; sh1, sc1);  [q|k|v] = n1 Wqkv^T + b;  q,k <- RoPE(RMS(q)), RoPE(RMS(k))
      O  = SelfAttn(q, k, v);   Oc = CrossAttn(n1 Wqc^T + b, ctx Wkc^T + b, ctx Wvc^T + b)
      y  = O Wo^T + bo + Oc Woc^T + boc;  x <- x + g1 y
      n2 = AdaLN(x; sh2, sc2);  h = GELU(n2 W1^T + b1);  m = FC2(h);  x <- x + g2 m
    ``mod_b`` is [6, d] (sh1, sc1, g1, sh2, sc2, g2).  ``trace`` (a dict) receives the
    intermediates when given.  ``int8_linear``: the QKV, cross-attention Q and FC1 products
    run as ``linear_int8`` (P3 "the int8 path").
    """
    lin = linear_int8 if int8_linear else linear
    n, d = x.shape
    dh = d // n_heads
    sh1, sc1, g1, sh2, sc2, g2 = mod_b
    n1 = adaln(x, sh1, sc1)
    qkv = lin(n1, blk["qkv_w"], blk["qkv_b"])
    q = qkv[:, :d].reshape(n, n_heads, dh)
    k = qkv[:, d:2 * d].reshape(n, n_heads, dh)
    v = qkv[:, 2 * d:].reshape(n, n_heads, dh)
    if qk_norm:
        q = rms_norm_heads(q, blk["q_gamma"])
        k = rms_norm_heads(k, blk["k_gamma"])
    q = rope_apply(q, coords)
    k = rope_apply(k, coords)
    o = attention(q, k, v).reshape(n, d)
    kc, vc = context_kv(ctx, blk)
    qc = lin(n1, blk["qc_w"], blk["qc_b"])
    lc = ctx.shape[0]
    oc = attention(qc.reshape(n, n_heads, dh), kc.reshape(lc, n_heads, dh),
                   vc.reshape(lc, n_heads, dh)).reshape(n, d)
    y = linear(o, blk["o_w"], blk["o_b"]) + linear(oc, blk["oc_w"], blk["oc_b"])
    x1 = gated_residual(x, g1, y)
    n2 = adaln(x1, sh2, sc2)
    h = gelu(lin(n2, blk["fc1_w"], blk["fc1_b"]))
    m = fc2(h, blk, fc2_mode)
    x2 = gated_residual(x1, g2, m)
    if trace is not None:
        trace.update(n1=n1, qkv=qkv, q=q, k=k, v=v, o=o, qc=qc, oc=oc, y=y, x1=x1, n2=n2,
                     h=h, m=m, x2=x2)
    return x2


def final_head(x, g, mod_final):
    """Velocity head: (LN(x)(1 + sc_f) + sh_f) Whead^T + bhead (P3 "DiT fusions": final AdaLN + heads)."""
    return linear(adaln(x, mod_final[0], mod_final[1]), g["head_w"], g["head_b"])


def patch_embed(latent, g):
    """Latent tokens [N, C] -> residual stream [N, d] (reading: one Linear, token layout)."""
    return linear(latent, g["patch_w"], g["patch_b"])


# --------------------------------------------------------------------------- forward / loop
def dit_forward(latent, model, sigma, active, geom, n_heads, eval_index=0, qk_norm=True,
                fc2_mode="bf16", token_reduction=False, trace=None, int8_linear=False):
    """One fresh denoiser evaluation: latent [N, C] -> velocity [N, C].

    ``geom`` = dict(f_lat, grid_h, grid_w, scale).  ``active`` = ascending block indices.
    Token reduction follows ``host.token_plan`` for ``eval_index``.
    """
    g, blocks, ctx = model["global"], model["blocks"], model["ctx"]
    mod, fin = modulation(g, sigma)
    x = patch_embed(latent, g)
    f_lat, gh, gw, sc = geom["f_lat"], geom["grid_h"], geom["grid_w"], geom["scale"]
    full = rope_coords(f_lat, gh, gw, sc)
    coords = full
    plan = host.token_plan(f_lat, gh, gw, eval_index, len(active)) if token_reduction else None
    saved = None
    for pos, b in enumerate(active):
        if plan is not None and pos == plan["merge_after"]:
            saved = x
            x = token_merge(saved, plan["pairs"])
            coords = rope_coords(f_lat, gh, gw, sc, plan["pairs"])
        if plan is not None and saved is not None and pos == plan["restore_before"] - 1:
            x = token_restore(saved, x, plan["pairs"])
            saved, coords = None, full
        x = block_forward(x, blocks[b], mod[b], ctx, coords, n_heads, qk_norm, fc2_mode,
                          int8_linear=int8_linear)
        if trace is not None:
            trace.setdefault("x_after", []).append(x)
    if saved is not None:
        x = token_restore(saved, x, plan["pairs"])
    if trace is not None:
        trace["x_core_out"] = x
    return final_head(x, g, fin)


def dit_forward_cached(latent, model, sigma, active, geom, n_heads, core_delta=None,
                       eval_index=0, qk_norm=True, fc2_mode="bf16", token_reduction=False,
                       int8_linear=False):
    """One evaluation under core-residual reuse: returns (velocity, core delta).

    P2 §4 / P3 "aggressive levers": ``--core-reuse`` runs the expensive core less often while
    the patch and the timestep-dependent head stay fresh on every step.
    Reading: the core is the stack of active blocks; its residual delta is
    x_L - x_0, x_0 = patch(latent) and x_L the full-resolution stream after the last active
    block (after any bypass restore).  ``core_delta`` None: a fresh evaluation, which
    returns its velocity and its delta; otherwise the blocks are skipped and the stream
    patch(latent) + core_delta goes through the final AdaLN of this sigma and the head.
    """
    g = model["global"]
    if core_delta is None:
        tr = {}
        v = dit_forward(latent, model, sigma, active, geom, n_heads, eval_index, qk_norm,
                        fc2_mode, token_reduction, trace=tr, int8_linear=int8_linear)
        return v, tr["x_core_out"] - patch_embed(latent, g)
    _, fin = modulation(g, sigma)
    return final_head(patch_embed(latent, g) + core_delta, g, fin), core_delta


def euler_step(x, v, sigma_cur, sigma_next):
    """Euler transition of the flow: x + (sigma_next - sigma_cur) v (P4 §2: "Euler transition")."""
    return x + (float(sigma_next) - float(sigma_cur)) * v


def denoise(latent0, model, steps, reuse, active, geom, n_heads, qk_norm=True,
            fc2_mode="bf16", token_reduction=False, int8_linear=False, core_reuse=1,
            velocities=None):
    """The Euler loop: ``steps`` transitions, fresh evaluations per ``host.schedule``.

    Skipped steps reuse the last fresh velocity (P3 "aggressive levers": reuse extrapolates
    the skipped transitions).  With ``core_reuse`` > 1 every step evaluates the patch and the
    head and only the marked steps run the core (``dit_forward_cached``).  Returns (x_N,
    number of fresh (core) evaluations).  ``velocities`` (a list), when given, receives the
    velocity of every fresh evaluation in order.
    """
    sig, fresh = host.schedule(steps, reuse, core_reuse)
    x = np.asarray(latent0, dtype=np.float64)
    v, ev, delta = None, 0, None
    for i in range(steps):
        if core_reuse > 1:
            v, delta = dit_forward_cached(x, model, float(sig[i]), active, geom, n_heads,
                                          None if fresh[i] else delta, ev, qk_norm, fc2_mode,
                                          token_reduction, int8_linear)
            ev += int(fresh[i])
        elif fresh[i]:
            v = dit_forward(x, model, float(sig[i]), active, geom, n_heads, ev, qk_norm,
                            fc2_mode, token_reduction, int8_linear=int8_linear)
            ev += 1
            if velocities is not None:
                velocities.append(v)
        x = euler_step(x, v, sig[i], sig[i + 1])
    return x, ev
