"""GPU parity of every kernel of the path against the oracle, one operation at a time,
through the C ABI, on seeded inputs.

Tolerances (bf16 outputs): a bf16 store rounds to 2^-9 relative; float32 accumulation
adds far less.  rel-L2 <= 1e-2 and per-element |err| <= 3e-2 (|ref| + rms(ref)) leave
room for that rounding while catching any dropped term, wrong index or transposed operand
(each of which moves rel-L2 to O(1)).  Integer work (int8 codes, int32 sums, the
dequantised bf16 of identical inputs, token-pair indices) is compared bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import dit, host
from tests.gpu_util import DEV, assert_close, bf16_dev, bits, f64, randn_bf16, rel_l2
from video_diffusion_transformer_fwd_amd import binding as B
from video_diffusion_transformer_fwd_amd import synthetic as S

pytestmark = pytest.mark.gpu


def sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ GEMM
@pytest.mark.parametrize("M,N,K,epi,f32,two_bias", [
    (128, 512, 512, 0, 0, 0),
    (300, 384, 192, 1, 0, 1),       # ragged M, GELU, two biases
    (1536, 3072, 3072, 0, 0, 0),    # out-projection-sized tile grid
    (77, 200, 64, 0, 1, 0),         # ragged N, one K slice, float32 out
    (1, 128, 128, 0, 1, 0),         # single row
    (129, 12288, 512, 1, 0, 0),     # wide N (FC1 / QKV widths)
    (1000, 700, 256, 1, 0, 1),      # 192x192 tiles with ragged M and N
    (4100, 2304, 256, 0, 0, 0),     # 256x256 tiles, ragged M
    (4100, 2100, 128, 1, 0, 0),     # 256x256 tiles, ragged M and N, GELU
    (1500, 12200, 256, 1, 0, 1),    # 384x192 tiles, ragged M and N, GELU, two biases
    (1536, 12288, 64, 1, 0, 0),     # 384x192 tiles, one K slice (its held last step only)
    (1536, 12288, 192, 0, 1, 0),    # 384x192 tiles, odd slice count, float32 out
    (1260, 12288, 512, 1, 0, 0),    # wide product on 256x256 tiles (one wave of them)
    (1601, 8300, 256, 1, 0, 1),     # wide product on 256x256 tiles, ragged M and N
    (4100, 2048, 64, 0, 0, 0),      # 256x256 tiles, one K slice
    (900, 640, 320, 1, 0, 0),       # 192x192 tiles (three stages), five slices
    (300, 640, 64, 1, 0, 1),        # 192x192 tiles, two K-step groups over a single slice
    (768, 12288, 3072, 1, 0, 0),    # FC1 at 768 rows: 192x192 tiles, two K-step groups
])
def test_gemm_bf16(M, N, K, epi, f32, two_bias):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A = randn_bf16(rng, (M, K))
    W = randn_bf16(rng, (N, K), 0.02)
    b = randn_bf16(rng, (N,), 0.02)
    b2 = randn_bf16(rng, (N,), 0.02) if two_bias else None
    C = torch.empty((M, N), dtype=torch.float32 if f32 else torch.bfloat16, device=DEV)
    B.h3_gemm_bf16(A, W, C, bias=b, bias2=b2, epilogue=epi)
    sync()
    bias = f64(b) + (f64(b2) if two_bias else 0.0)
    ref = dit.linear(f64(A), f64(W), bias)
    if epi:
        ref = dit.gelu(ref)
    if f32:
        assert_close(f64(C), ref, rel=2e-5, elem=2e-4, what="gemm f32")
    else:
        assert_close(f64(C), ref, rel=6e-3, elem=1.5e-2, what="gemm bf16")


def test_gemm_tile_shape_keeps_the_bits():
    # the tile shape follows M (1536 rows: 384x192, 1260: 256x256, 129: 128x128); every shape
    # with one K-step group adds each output's K steps in the same order with the same MFMA and
    # applies the same epilogue, so the rows they share have the same bits
    rng = np.random.default_rng(77)
    N, K = 12288, 512
    A = randn_bf16(rng, (1536, K))
    W = randn_bf16(rng, (N, K), 0.02)
    b = randn_bf16(rng, (N,), 0.02)
    outs = {}
    for M in (1536, 1260, 129):
        C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        B.h3_gemm_bf16(A[:M], W, C, bias=b, epilogue=1)
        outs[M] = C
    sync()
    i16 = lambda t: t.contiguous().view(torch.int16)
    assert torch.equal(i16(outs[1536][:1260]), i16(outs[1260]))
    assert torch.equal(i16(outs[1536][:129]), i16(outs[129]))


def test_gemm_strided_operands():
    # operands that are column slices of wider rows (as the block's [O | Oc] and qkvq are)
    rng = np.random.default_rng(5)
    M, K, N = 200, 256, 320
    big = randn_bf16(rng, (M, 3 * K))
    A = big[:, K:2 * K]
    W = randn_bf16(rng, (N, K), 0.05)
    out = torch.zeros((M, 2 * N), dtype=torch.bfloat16, device=DEV)
    B.h3_gemm_bf16(A, W, out[:, N:], M=M, N=N, K=K, lda=3 * K, ldb=K, ldc=2 * N)
    sync()
    assert_close(f64(out[:, N:]), dit.linear(f64(A), f64(W)), rel=6e-3, elem=1.5e-2)
    assert (f64(out[:, :N]) == 0).all()


# ------------------------------------------------------------------ attention
@pytest.mark.parametrize("nq,nk,H,D", [
    (128, 128, 8, 64),     # the small workload's self-attention
    (128, 32, 8, 64),      # its cross-attention (32 text tokens)
    (300, 77, 3, 128),     # ragged queries and keys
    (1536, 1536, 2, 128),  # 512x512x22 self-attention length, two heads
    (1536, 256, 2, 128),   # cross-attention length
    (5, 1, 1, 64),         # one key: output is that value
    (64, 600, 2, 64),      # keys span several tiles with a ragged tail
    # more than 256 (128-query tile, head) pairs: eight-wave workgroups of 256 queries while
    # their grid takes at most 192 CUs, else four-wave workgroups; the cases above (fewer
    # pairs) take the eight-wave workgroups that split the key tiles between two wave groups
    (1040, 300, 32, 128),
    (1040, 300, 48, 128),
    (700, 100, 48, 64),
])
def test_attention(nq, nk, H, D):
    rng = np.random.default_rng(nq + 13 * nk + H * D)
    Q, K, V = (randn_bf16(rng, (n, H * D)) for n in (nq, nk, nk))
    O = torch.empty((nq, H * D), dtype=torch.bfloat16, device=DEV)
    B.h3_attention(Q, K, V, O, nq, nk, H, D)
    sync()
    ref = dit.attention(f64(Q).reshape(nq, H, D), f64(K).reshape(nk, H, D), f64(V).reshape(nk, H, D))
    assert_close(f64(O), ref.reshape(nq, H * D), rel=1e-2, elem=3e-2, what="attention")


def test_attention_long_sequence_sampled_rows():
    # 8192+ queries take the 8-wave workgroups, whose interior key tiles load without bounds
    # checks; ragged query and key counts exercise the last tiles.  The oracle computes a
    # sample of query rows (every key).
    rng = np.random.default_rng(23)
    nq, nk, H, D = 8200, 8263, 2, 128
    Q, K, V = (randn_bf16(rng, (n, H * D)) for n in (nq, nk, nk))
    O = torch.empty((nq, H * D), dtype=torch.bfloat16, device=DEV)
    B.h3_attention(Q, K, V, O, nq, nk, H, D)
    sync()
    rows = np.concatenate([np.arange(0, 40), rng.integers(40, nq - 40, 48), np.arange(nq - 40, nq)])
    ref = dit.attention(f64(Q)[rows].reshape(-1, H, D), f64(K).reshape(nk, H, D), f64(V).reshape(nk, H, D))
    assert_close(f64(O)[rows], ref.reshape(-1, H * D), rel=1e-2, elem=3e-2, what="long attention")


@pytest.mark.parametrize("nk", [1, 64, 65])
def test_attention_long_queries_short_keys(nk):
    # 8192 queries take the 8-wave workgroups; one key (every staged row repeats it), exactly
    # one tile, and one tile plus a one-key tail.  Sampled query rows against the oracle.
    rng = np.random.default_rng(31 + nk)
    nq, H, D = 8192, 2, 128
    Q, K, V = (randn_bf16(rng, (n, H * D)) for n in (nq, nk, nk))
    O = torch.empty((nq, H * D), dtype=torch.bfloat16, device=DEV)
    B.h3_attention(Q, K, V, O, nq, nk, H, D)
    sync()
    rows = np.concatenate([np.arange(0, 64), rng.integers(64, nq - 64, 64), np.arange(nq - 64, nq)])
    ref = dit.attention(f64(Q)[rows].reshape(-1, H, D), f64(K).reshape(nk, H, D), f64(V).reshape(nk, H, D))
    assert_close(f64(O)[rows], ref.reshape(-1, H * D), rel=1e-2, elem=3e-2, what=f"attention nk={nk}")


def planted_scores(nq, nk, H, D, tiles, seed):
    """Attention inputs whose scores jump far above the running maximum in later key tiles.

    Early keys are small (scores ~0).  For the even queries, which carry the planted
    direction, the key planted in the first tile of ``tiles`` scores 11 log2 units above them
    (2^11 times the softmax weight) and one in a second tile 9 more; odd queries see no jump,
    so within one wave some lanes move their softmax reference and others keep it.  Both jumps
    exceed the kernel's lazy threshold (8 log2 units), so each rescales the running sum and
    output, and what was accumulated before a jump keeps a weight that matters (the ~600
    small keys against 2^11 after one jump, the first planted key against 2^9 after the
    second): a wrong, missing or inverted rescale moves the output by O(1), about 10^-2 of
    which the test tolerates.  Returns Q, K, V as [n, H*D] bf16 on the device.
    """
    rng = np.random.default_rng(seed)
    c = np.log2(np.e) / np.sqrt(D)
    u = rng.choice([-1.0, 1.0], size=(H, D))
    a = np.where(np.arange(nq) % 2 == 0, 2.0, 0.0)
    q = a[:, None, None] * u[None] + 0.3 * rng.standard_normal((nq, H, D))
    k = 0.05 * rng.standard_normal((nk, H, D))
    for j, t in enumerate(tiles):
        k[64 * t + 7 + 3 * j] = u * ((11.0 + 9.0 * j) / c) / (2.0 * D)
    v = rng.standard_normal((nk, H, D))
    return tuple(bf16_dev(x.reshape(x.shape[0], H * D)) for x in (q, k, v))


@pytest.mark.parametrize("nq,nk,H,D,tiles", [
    (600, 700, 2, 128, (5,)),      # two key groups; the jump in the second group's tile
    (600, 700, 2, 128, (4,)),      # ... in the first group's tile
    (600, 700, 2, 128, (2, 6)),    # two jumps, one in each group
    (600, 256, 2, 128, (3,)),      # cross-attention length, two key groups
    (1040, 700, 48, 128, (5,)),    # four-wave workgroups
    (1040, 256, 48, 128, (1, 3)),  # four-wave, cross-attention length, two jumps
    (1040, 700, 32, 128, (2, 6)),  # eight-wave workgroups of 256 queries below 8192 queries
    (600, 600, 2, 64, (5,)),       # head dim 64, two key groups
    (600, 600, 2, 64, (4,)),
    (700, 600, 48, 64, (2, 5)),    # head dim 64, four-wave workgroups
    (8192, 700, 2, 128, (5,)),     # eight-wave workgroups (sampled rows)
    (8200, 512, 2, 128, (2, 7)),   # eight-wave, ragged queries, two jumps
])
def test_attention_softmax_rescale(nq, nk, H, D, tiles):
    Q, K, V = planted_scores(nq, nk, H, D, tiles, seed=nq + nk + sum(tiles))
    O = torch.empty((nq, H * D), dtype=torch.bfloat16, device=DEV)
    B.h3_attention(Q, K, V, O, nq, nk, H, D)
    sync()
    rows = np.arange(nq) if nq <= 2048 else np.concatenate([np.arange(0, 64), np.arange(4096, 4160),
                                                             np.arange(nq - 64, nq)])
    q, k, v = (f64(t).reshape(-1, H, D) for t in (Q, K, V))
    ref = dit.attention(q[rows], k, v)
    # the planted keys hold most but not all of the weight of the even queries
    sc = (k[:, 0] @ q[0, 0]) * np.log2(np.e) / np.sqrt(D)
    assert sc.max() - sc[:64].max() > 10.0
    assert_close(f64(O)[rows], ref.reshape(-1, H * D), rel=1e-2, elem=3e-2, what="rescaled attention")


@pytest.mark.parametrize("nq,nk,D,h_a,h_b", [
    (1040, 300, 128, 32, 48),   # 8-wave workgroups of 256 queries (32 heads) / 4-wave (48 heads)
    (1536, 256, 128, 24, 48),   # the 512x512x22f cross-attention shape: 8-wave / 4-wave
])
def test_attention_workgroup_form_keeps_the_bits(nq, nk, D, h_a, h_b):
    # which workgroup form runs (and the XCD order of its (tile, head) pairs) depends on the
    # head count; a query's arithmetic does not (the forms with two key groups excepted: each
    # group rounds its P to bf16 against its own softmax reference, so they are only checked
    # against the oracle).  The first h_a heads are computed by both launches.
    rng = np.random.default_rng(nq + nk + D)
    Q, K, V = (randn_bf16(rng, (n, h_b * D)) for n in (nq, nk, nk))
    Oa = torch.empty((nq, h_a * D), dtype=torch.bfloat16, device=DEV)
    Ob = torch.empty((nq, h_b * D), dtype=torch.bfloat16, device=DEV)
    B.h3_attention(Q[:, :h_a * D], K[:, :h_a * D], V[:, :h_a * D], Oa, nq, nk, h_a, D)
    B.h3_attention(Q, K, V, Ob, nq, nk, h_b, D)
    sync()
    assert torch.equal(Oa.view(torch.int16), Ob[:, :h_a * D].contiguous().view(torch.int16))


def test_attention_strided_views_of_qkvq():
    # the block's layout: q, k, v, qc as column slices of one [N, 4d] buffer, output into [N, 2d]
    rng = np.random.default_rng(11)
    n, H, D = 257, 4, 128
    d = H * D
    qkvq = randn_bf16(rng, (n, 4 * d))
    out = torch.zeros((n, 2 * d), dtype=torch.bfloat16, device=DEV)
    B.h3_attention(qkvq[:, :d], qkvq[:, d:2 * d], qkvq[:, 2 * d:3 * d], out[:, :d], n, n, H, D)
    sync()
    a = f64(qkvq)
    ref = dit.attention(a[:, :d].reshape(n, H, D), a[:, d:2 * d].reshape(n, H, D), a[:, 2 * d:3 * d].reshape(n, H, D))
    assert_close(f64(out[:, :d]), ref.reshape(n, d), rel=1e-2, elem=3e-2)
    assert (f64(out[:, d:]) == 0).all()


# ------------------------------------------------------------------ gate + AdaLN
@pytest.mark.parametrize("rows,d", [(5, 512), (1536, 3072), (130, 5120), (64, 1024)])
def test_gate_adaln_fused_bit_identical_and_oracle(rows, d):
    rng = np.random.default_rng(rows + d)
    x = randn_bf16(rng, (rows, d))
    y = randn_bf16(rng, (rows, d))
    gate = torch.tensor(rng.standard_normal(d) * 0.2, dtype=torch.float32, device=DEV)
    sh = torch.tensor(rng.standard_normal(d) * 0.2, dtype=torch.float32, device=DEV)
    sc = torch.tensor(rng.standard_normal(d) * 0.2, dtype=torch.float32, device=DEV)
    # fused
    xf = x.clone()
    nf = torch.empty_like(x)
    B.h3_gate_adaln(xf, y, gate, xf, sh, sc, nf)
    # unfused: gate, then AdaLN of the stored residual
    xu = x.clone()
    nu = torch.empty_like(x)
    B.h3_gate_adaln(xu, y, gate, xu, None, None, None)
    B.h3_gate_adaln(xu, None, None, None, sh, sc, nu)
    sync()
    assert np.array_equal(bits(xf), bits(xu)), "gated residual differs fused vs unfused"
    assert np.array_equal(bits(nf), bits(nu)), "AdaLN output differs fused vs unfused"
    gx = dit.gated_residual(f64(x), f64(gate), f64(y))
    assert_close(f64(xf), gx, rel=4e-3, elem=1e-2, what="gated residual")
    assert_close(f64(nf), dit.adaln(gx, f64(sh), f64(sc)), rel=1e-2, elem=3e-2, what="adaln(fused)")
    # AdaLN alone on the stored input is the oracle's AdaLN of that input
    n_only = torch.empty_like(x)
    B.h3_gate_adaln(x, None, None, None, sh, sc, n_only)
    sync()
    assert_close(f64(n_only), dit.adaln(f64(x), f64(sh), f64(sc)), rel=6e-3, elem=2e-2, what="adaln")


@pytest.mark.parametrize("rows,d,n_out", [
    (1536, 3072, 128),   # the 512x512x22 head: two waves per AdaLN row (even d/512, few rows)
    (300, 512, 128),     # one wave per row (odd d/512), ragged last tile
    (1000, 1536, 64),    # one wave per row, narrower head
    (2430, 3072, 8),     # the 864x480 token count, a head of one 8-wide tile column
    (17000, 1024, 128),  # one wave per row because of the row count (even d/512)
    (61488, 5120, 128),  # the 768x1344 head
])
def test_head_adaln_gemm_bit_identical_to_adaln_then_product(rows, d, n_out):
    # the final AdaLN applied while the head product stages its tiles equals the AdaLN kernel
    # followed by the product, bit for bit; and the oracle's AdaLN + head
    rng = np.random.default_rng(rows + d + n_out)
    x = randn_bf16(rng, (rows, d), 1.5)
    vec = lambda: torch.tensor(rng.standard_normal(d) * 0.2, dtype=torch.float32, device=DEV)
    sh, sc = vec(), vec()
    W = randn_bf16(rng, (n_out, d), 0.02)
    b = randn_bf16(rng, (n_out,), 0.02)
    fused = torch.empty((rows, n_out), dtype=torch.float32, device=DEV)
    B.h3_head_adaln_gemm(x, sh, sc, W, b, fused)
    n = torch.empty_like(x)
    B.h3_gate_adaln(x, None, None, None, sh, sc, n)
    plain = torch.empty_like(fused)
    B.h3_gemm_bf16(n, W, plain, bias=b)
    sync()
    assert np.array_equal(bits(fused), bits(plain)), "fused head differs from AdaLN + product"
    rows_s = np.arange(rows) if rows <= 4096 else np.concatenate([np.arange(64), rng.integers(64, rows, 128),
                                                                  np.arange(rows - 64, rows)])
    ref = dit.linear(dit.adaln(f64(x)[rows_s], f64(sh), f64(sc)), f64(W), f64(b))
    assert_close(f64(fused)[rows_s], ref, rel=1e-2, elem=3e-2, what="head")


def test_head_adaln_gemm_refuses_wide_heads():
    x = torch.zeros((64, 512), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros(512, dtype=torch.float32, device=DEV)
    W = torch.zeros((192, 512), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((64, 192), dtype=torch.float32, device=DEV)
    with pytest.raises(B.H3Error) as e:
        B.h3_head_adaln_gemm(x, v, v, W, None, out)
    assert e.value.code == B.H3_EUNSUPPORTED


def test_zero_gate_leaves_residual_bit_exact():
    rng = np.random.default_rng(2)
    x = randn_bf16(rng, (40, 3072))
    y = randn_bf16(rng, (40, 3072))
    z = torch.zeros(3072, dtype=torch.float32, device=DEV)
    out = torch.empty_like(x)
    B.h3_gate_adaln(x, y, z, out, None, None, None)
    sync()
    assert np.array_equal(bits(out), bits(x))


# ------------------------------------------------------------------ Q/K RMSNorm + RoPE
@pytest.mark.parametrize("geom_args,H,D,qk_norm", [
    ((2, 8, 8, 0.5, 0), 8, 64, 1),     # small workload: halved RoPE at the 8x8 grid
    ((6, 16, 16, 1.0, 0), 24, 128, 1), # 512x512x22
    ((6, 16, 16, 1.0, 1), 4, 128, 1),  # paired tokens
    ((1, 3, 5, 1.0, 1), 4, 128, 0),    # odd width pairing, no norm
    ((2, 8, 8, 1.0, 0), 8, 64, 1),     # reference RoPE coordinates
])
def test_qk_norm_rope(geom_args, H, D, qk_norm):
    f, gh, gw, sc, paired = geom_args
    geom = B.make_geom(f, gh, gw, sc, paired)
    n = B.h3_geom_tokens(geom)
    d = H * D
    rng = np.random.default_rng(n + d)
    buf = randn_bf16(rng, (n, 4 * d), 2.0)
    qg = bf16_dev(1 + rng.standard_normal(D) * 0.1)
    kg = bf16_dev(1 + rng.standard_normal(D) * 0.1)
    table = torch.empty((n, D // 2, 2), dtype=torch.float32, device=DEV)
    before = f64(buf)
    B.h3_rope_table(geom, D, table)
    B.h3_qk_norm_rope(buf, n, d, D, qg, kg, qk_norm, table)
    sync()
    after = f64(buf)
    pairs = host.token_plan(f, gh, gw, 0, 10)["pairs"] if paired else None
    coords = dit.rope_coords(f, gh, gw, sc, pairs)
    q = before[:, :d].reshape(n, H, D)
    k = before[:, d:2 * d].reshape(n, H, D)
    if qk_norm:
        q, k = dit.rms_norm_heads(q, f64(qg)), dit.rms_norm_heads(k, f64(kg))
    assert_close(after[:, :d], dit.rope_apply(q, coords).reshape(n, d), rel=6e-3, elem=2e-2, what="q")
    assert_close(after[:, d:2 * d], dit.rope_apply(k, coords).reshape(n, d), rel=6e-3, elem=2e-2, what="k")
    assert np.array_equal(after[:, 2 * d:], before[:, 2 * d:]), "v / qc must be untouched"


# ------------------------------------------------------------------ QKV product + Q/K epilogue
def _rand_table(rng, M, D):
    ang = rng.uniform(-np.pi, np.pi, size=(M, D // 2))
    return torch.tensor(np.stack([np.cos(ang), np.sin(ang)], -1), dtype=torch.float32, device=DEV)


# (M, d, head_dim, int8, fused form expected): 128x128 natural, 192x192 and 384x192 with the
# regrouped q/k-head columns (ragged rows, a partial last qc tile at d = 2048), 256x256 natural
# with ragged rows, head_dim 64 on 192-wide tiles (natural order), and an int8 plan that
# splits K (no fused form; a bf16 QKV product never splits: K = d gives pieces under 1024)
QKV_CASES = [
    (128, 512, 64, False, True), (300, 512, 64, False, True), (100, 3072, 128, False, True),
    (768, 3072, 128, False, True), (1000, 3072, 128, False, True), (1536, 3072, 128, False, True),
    (1536, 2048, 128, False, True), (1536, 3072, 64, False, True), (4100, 1024, 128, False, True),
    (128, 512, 64, True, True), (768, 3072, 128, True, True), (1536, 3072, 128, True, True),
    (1000, 2048, 128, True, True), (4100, 1024, 128, True, True), (300, 1024, 128, True, False),
]


# every shape with the RMSNorm, and RoPE alone on the small and the 1536-token shapes
QKV_PARAMS = [c + (1,) for c in QKV_CASES] + [c + (0,) for c in QKV_CASES if c[:2] in ((128, 512), (1536, 3072))]


@pytest.mark.parametrize("M,d,D,q8,expect_fused,qk_norm", QKV_PARAMS)
def test_qkv_gemm_fused_epilogue_bit_identical(M, d, D, q8, expect_fused, qk_norm):
    rng = np.random.default_rng(M * 7 + d + D + q8)
    N, K = 4 * d, d
    if q8:
        A = torch.from_numpy(rng.integers(-127, 128, size=(M, K)).astype(np.int8)).to(DEV)
        W = torch.from_numpy(rng.integers(-127, 128, size=(N, K)).astype(np.int8)).to(DEV)
        SA = torch.tensor(1e-3 + rng.random(M) * 4e-3, dtype=torch.float32, device=DEV)
        SW = torch.tensor(1e-3 + rng.random(N) * 4e-3, dtype=torch.float32, device=DEV)
    else:
        A, W, SA, SW = randn_bf16(rng, (M, K)), randn_bf16(rng, (N, K), 0.03), None, None
    bias = bf16_dev(rng.standard_normal(N) * 0.3)
    qg = bf16_dev(1 + rng.standard_normal(D) * 0.1)
    kg = bf16_dev(1 + rng.standard_normal(D) * 0.1)
    table = _rand_table(rng, M, D)
    ldc = N + (8 if M == 1000 else 0)  # one padded row stride
    # different fills, so an element one path leaves unwritten shows up
    Cf = torch.full((M, ldc), float("nan"), dtype=torch.bfloat16, device=DEV)
    Cu = torch.zeros((M, ldc), dtype=torch.bfloat16, device=DEV)
    used = B.h3_qkv_gemm(A, W, bias, Cf[:, :N], D, qg, kg, qk_norm, table, SA, SW, fused=True)
    used_u = B.h3_qkv_gemm(A, W, bias, Cu[:, :N], D, qg, kg, qk_norm, table, SA, SW, fused=False)
    sync()
    assert used == expect_fused and not used_u
    assert torch.equal(Cf[:, :N].view(torch.int16), Cu[:, :N].view(torch.int16))
    assert not torch.isnan(Cf[:, :N].float()).any()


def test_qkv_gemm_fused_matches_oracle():
    # 2 x 8 x 8 tokens (RoPE halved), d = 512, 8 heads of 64: product, per-head RMSNorm, RoPE
    f, gh, gw, sc = 2, 8, 8, 0.5
    geom = B.make_geom(f, gh, gw, sc, 0)
    M, d, D, H = 128, 512, 64, 8
    rng = np.random.default_rng(5)
    A, W = randn_bf16(rng, (M, d)), randn_bf16(rng, (4 * d, d), 0.03)
    bias = bf16_dev(rng.standard_normal(4 * d) * 0.3)
    qg = bf16_dev(1 + rng.standard_normal(D) * 0.1)
    kg = bf16_dev(1 + rng.standard_normal(D) * 0.1)
    table = torch.empty((M, D // 2, 2), dtype=torch.float32, device=DEV)
    B.h3_rope_table(geom, D, table)
    C_out = torch.empty((M, 4 * d), dtype=torch.bfloat16, device=DEV)
    assert B.h3_qkv_gemm(A, W, bias, C_out, D, qg, kg, 1, table)
    sync()
    lin = dit.linear(f64(A), f64(W), f64(bias))
    coords = dit.rope_coords(f, gh, gw, sc)
    q = dit.rope_apply(dit.rms_norm_heads(lin[:, :d].reshape(M, H, D), f64(qg)), coords).reshape(M, d)
    k = dit.rope_apply(dit.rms_norm_heads(lin[:, d:2 * d].reshape(M, H, D), f64(kg)), coords).reshape(M, d)
    got = f64(C_out)
    assert_close(got[:, :d], q, rel=8e-3, elem=3e-2, what="q")
    assert_close(got[:, d:2 * d], k, rel=8e-3, elem=3e-2, what="k")
    assert_close(got[:, 2 * d:], lin[:, 2 * d:], rel=8e-3, elem=3e-2, what="v | qc")


# ------------------------------------------------------------------ token pairing
@pytest.mark.parametrize("f,gh,gw,d", [(6, 16, 16, 3072), (1, 15, 27, 512), (2, 3, 5, 1024)])
def test_token_merge_restore_exact(f, gh, gw, d):
    geom = B.make_geom(f, gh, gw, 1.0, 0)
    n = f * gh * gw
    plan = host.token_plan(f, gh, gw, 0, 10)
    rng = np.random.default_rng(n)
    # values k/64 with |k| < 128: every pair mean is exactly representable in bf16, so the merge
    # must equal the oracle bit for bit and a wrong pair index shows as a mismatch
    S_np = rng.integers(-127, 128, size=(n, d)) / 64.0
    Sx = bf16_dev(S_np)
    xr = torch.empty((plan["n_reduced"], d), dtype=torch.bfloat16, device=DEV)
    B.h3_token_reduce(0, geom, d, Sx, None, xr)
    sync()
    assert np.array_equal(f64(xr), dit.token_merge(S_np, plan["pairs"]))
    # merge then restore with nothing between returns S bit for bit
    out = torch.empty_like(Sx)
    B.h3_token_reduce(1, geom, d, xr, Sx, out)
    sync()
    assert np.array_equal(bits(out), bits(Sx))
    # a changed reduced stream moves both pair members by the change (in place on the bypass)
    delta = rng.integers(-8, 9, size=xr.shape) / 64.0
    xr2 = bf16_dev(f64(xr) + delta)
    S2 = Sx.clone()
    B.h3_token_reduce(1, geom, d, xr2, S2, S2)
    sync()
    want = dit.f32_to_bf16(dit.token_restore(S_np, f64(xr2), plan["pairs"]).astype(np.float32))
    assert np.array_equal(f64(S2), want.astype(np.float64))


# ------------------------------------------------------------------ int8 FC2
@pytest.mark.parametrize("rows,K,group", [(300, 2048, 2048), (300, 2048, 1024), (1536, 12288, 12288),
                                          (64, 20480, 1024), (33, 20480, 20480),
                                          (70, 7168, 7168)])   # K / 1024 = 7: the generic row kernel
def test_quant_rows_bit_exact(rows, K, group):
    rng = np.random.default_rng(rows + K + group)
    X = randn_bf16(rng, (rows, K), 0.7)
    X[3] = 0            # zero row -> s = 0, q = 0
    X[4, :7] = 50.0     # an outlier row
    Q = torch.empty((rows, K), dtype=torch.int8, device=DEV)
    Sc = torch.empty((rows, K // group), dtype=torch.float32, device=DEV)
    B.h3_quant_rows(X, Q, Sc, group)
    sync()
    q_ref, s_ref = dit.quantize_rows(f64(X).astype(np.float32), None if group == K else group)
    assert np.array_equal(Q.cpu().numpy(), q_ref)
    assert np.array_equal(Sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("group", [2048, 1024])
def test_quant_rows_exact_half_way_quotients(group):
    # every group holds its absmax 127 c (c a power of two, so s = c exactly) and values
    # (k + 1/2) c: their quotients sit exactly half-way between codes and must round to even,
    # which the quantiser decides with the exact division
    K, rows = 2048, 4
    X = np.zeros((rows, K))
    k = (np.arange(K) % 253) - 126                      # -126 .. 126
    for r, c in enumerate([2.0 ** -3, 2.0 ** 5, 2.0 ** -20, 1.0]):
        X[r] = (k + 0.5) * c
        X[r, ::group] = 127 * c
        X[r, 1::7] = ((k[1::7] % 63) - 31 + 0.25) * c   # and some values off the half-way points
    Xd = torch.tensor(X, dtype=torch.float32).to(torch.bfloat16)
    assert np.array_equal(Xd.double().numpy(), X)      # the values are bf16-exact
    Q = torch.empty((rows, K), dtype=torch.int8, device=DEV)
    Sc = torch.empty((rows, K // group), dtype=torch.float32, device=DEV)
    B.h3_quant_rows(Xd.to(DEV), Q, Sc, group)
    sync()
    q_ref, s_ref = dit.quantize_rows(X.astype(np.float32), None if group == K else group)
    assert np.array_equal(Q.cpu().numpy(), q_ref)
    assert np.array_equal(Sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    half = np.zeros(K, bool)
    half[2::7] = True
    half[::group] = False                               # (not the absmax positions)
    assert (np.abs(q_ref[:, half]) % 2 == 0).all()      # the half-way values went to even codes


@pytest.mark.parametrize("M,N,K,group", [(300, 256, 2048, 2048), (300, 256, 2048, 1024),
                                         (1536, 3072, 12288, 12288), (130, 640, 4096, 1024),
                                         (4100, 700, 2048, 2048),    # 256x256 row tiles, ragged
                                         (4100, 400, 2048, 1024),    # 192x192 grouped tiles, ragged
                                         (700, 520, 4096, 4096)])    # 192x192 row tiles (unsplit)
def test_gemm_i8_bit_exact(M, N, K, group):
    rng = np.random.default_rng(M + N + K + group)
    qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sa = (rng.random((M, K // group)) * 0.01).astype(np.float32)
    sw = (rng.random(N) * 0.001).astype(np.float32)
    bias = bf16_dev(rng.standard_normal(N) * 0.02)
    Cm = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    B.h3_gemm_i8(torch.from_numpy(qa).to(DEV), torch.from_numpy(sa).to(DEV), torch.from_numpy(qw).to(DEV),
                 torch.from_numpy(sw).to(DEV), bias, Cm, group)
    sync()
    acc = dit.int8_accumulate(qa, qw, None if group == K else group)
    ref = dit.f32_to_bf16(dit.dequant(acc, sa, sw, f64(bias).astype(np.float32)))
    got = Cm.cpu().to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_int8_fc2_pipeline_bit_exact_on_seeded_input():
    # the same bf16 FC2 input through both quantisers and both int8 products
    w = S.WORKLOADS["tiny_256sq_5f"]
    blk = S.block_weights(w, 0)
    rng = np.random.default_rng(9)
    h = randn_bf16(rng, (128, w.ffn_dim), 0.5)
    W2 = blk["fc2_w"].to(DEV)
    b2 = blk["fc2_b"].to(DEV)
    for mode, group in (("row", w.ffn_dim), ("grouped", 1024)):
        qw = torch.empty((w.d_model, w.ffn_dim), dtype=torch.int8, device=DEV)
        sw = torch.empty((w.d_model, 1), dtype=torch.float32, device=DEV)
        B.h3_quant_rows(W2, qw, sw, w.ffn_dim)
        qa = torch.empty((128, w.ffn_dim), dtype=torch.int8, device=DEV)
        sa = torch.empty((128, w.ffn_dim // group), dtype=torch.float32, device=DEV)
        B.h3_quant_rows(h, qa, sa, group)
        out = torch.empty((128, w.d_model), dtype=torch.bfloat16, device=DEV)
        B.h3_gemm_i8(qa, sa, qw, sw, b2, out, group)
        sync()
        qw_ref, sw_ref = dit.quantize_weight(f64(W2).astype(np.float32))
        assert np.array_equal(qw.cpu().numpy(), qw_ref)
        g = None if mode == "row" else 1024
        qa_ref, sa_ref = dit.quantize_rows(f64(h).astype(np.float32), g)
        assert np.array_equal(qa.cpu().numpy(), qa_ref)
        acc = dit.int8_accumulate(qa_ref, qw_ref, g)
        ref = dit.f32_to_bf16(dit.dequant(acc, sa_ref, sw_ref[:, 0], f64(b2).astype(np.float32)))
        assert np.array_equal(out.cpu().to(torch.float32).numpy().view(np.uint32), ref.view(np.uint32))
        # and the int8 product stays close to the float64 bf16 product
        ref_f = dit.linear(f64(h), f64(W2), f64(b2))
        assert rel_l2(f64(out), ref_f) < 2e-2


@pytest.mark.parametrize("rows,d,gated", [(5, 512, True), (1536, 3072, True), (130, 5120, False),
                                          (64, 1024, True)])
def test_gate_adaln_quant_bit_identical_to_adaln_then_quant_rows(rows, d, gated):
    rng = np.random.default_rng(rows * 3 + d)
    x = randn_bf16(rng, (rows, d))
    y = randn_bf16(rng, (rows, d)) if gated else None
    vec = lambda: torch.tensor(rng.standard_normal(d) * 0.2, dtype=torch.float32, device=DEV)
    g, sh, sc = vec(), vec(), vec()
    # fused: gate, AdaLN and int8 row quantisation in one kernel
    xf = x.clone()
    qf = torch.empty((rows, d), dtype=torch.int8, device=DEV)
    sf = torch.empty((rows,), dtype=torch.float32, device=DEV)
    B.h3_gate_adaln_quant(xf, y, g if gated else None, xf if gated else None, sh, sc, qf, sf)
    # reference sequence: gate + AdaLN into bf16, then the row quantiser
    xu, nu = x.clone(), torch.empty_like(x)
    B.h3_gate_adaln(xu, y, g if gated else None, xu if gated else None, sh, sc, nu)
    qu = torch.empty_like(qf)
    su = torch.empty((rows, 1), dtype=torch.float32, device=DEV)
    B.h3_quant_rows(nu, qu, su, d)
    sync()
    assert torch.equal(xf.view(torch.int16), xu.view(torch.int16))
    assert torch.equal(qf, qu)
    assert torch.equal(sf.view(torch.int32), su.view(-1).view(torch.int32))
    # and the quantiser's output is the oracle's on the same bf16 rows
    q_ref, s_ref = dit.quantize_rows(f64(nu).astype(np.float32), None)
    assert np.array_equal(qf.cpu().numpy(), q_ref)


@pytest.mark.parametrize("M,N,K,sample", [(300, 640, 2048, False), (1536, 12288, 3072, True)])
def test_gemm_i8_gelu_epilogue(M, N, K, sample):
    # int8 FC1: dequantisation bit-exact, then GELU before the bf16 rounding; the exact-erf
    # GELU of the oracle and the kernel's may land on the two sides of a bf16 rounding
    # boundary, so the bar is one bf16 unit
    rng = np.random.default_rng(M + N)
    qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    # |acc| ~ sqrt(K) 127^2 / 3: scales of a few 1e-3 give dequantised values of order 1-10
    sa = (1e-3 + rng.random((M, 1)) * 4e-3).astype(np.float32)
    sw = (1e-3 + rng.random(N) * 4e-3).astype(np.float32)
    bias = bf16_dev(rng.standard_normal(N) * 0.5)
    Cm = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    B.h3_gemm_i8(torch.from_numpy(qa).to(DEV), torch.from_numpy(sa).to(DEV), torch.from_numpy(qw).to(DEV),
                 torch.from_numpy(sw).to(DEV), bias, Cm, K, epilogue=1)
    sync()
    rows = np.sort(rng.choice(M, 12, replace=False)) if sample else np.arange(M)
    cols = np.sort(rng.choice(N, 96, replace=False)) if sample else np.arange(N)
    acc = dit.int8_accumulate(qa[rows], qw[cols], None)
    v = dit.dequant(acc, sa[rows], sw[cols], f64(bias).astype(np.float32)[cols])
    ref = dit.gelu(v.astype(np.float64))
    got = Cm.cpu().to(torch.float32).numpy()[np.ix_(rows, cols)].astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 2e-6)
    assert np.abs(v).max() > 3 and (v < -1).any()   # both GELU regimes are exercised


# ------------------------------------------------------------------ Euler
def test_euler_step():
    rng = np.random.default_rng(4)
    n = 1536 * 128 + 3  # ragged tail after the 4-wide vectors
    x = torch.tensor(rng.standard_normal(n), dtype=torch.float32, device=DEV)
    v = torch.tensor(rng.standard_normal(n), dtype=torch.float32, device=DEV)
    x0 = f64(x)
    sig, _ = host.schedule(4)
    B.h3_euler_step(x, v, float(sig[1]), float(sig[2]))
    sync()
    ref = dit.euler_step(x0, f64(v), sig[1], sig[2])
    assert np.max(np.abs(f64(x) - ref)) <= 1e-6 * (1 + np.max(np.abs(ref)))


# ------------------------------------------------------------------ modulation
def test_modulation_matches_oracle():
    w = S.WORKLOADS["tiny_256sq_5f"]
    g = S.global_weights(w)
    gd = {k: v.to(DEV) for k, v in g.items()}
    dims = B.h3_dims(w.d_model, w.n_heads, w.ffn_dim, w.ctx_len, w.latent_ch, w.n_blocks)
    gs = B.h3_global_weights(*[gd[n].data_ptr() for n in B.GLOBAL_FIELDS])
    dummy = torch.zeros(w.ffn_dim * w.d_model, dtype=torch.bfloat16, device=DEV)
    blk = B.h3_block_weights(*([dummy.data_ptr()] * 15 + [None, None]))
    m = B.h3_model_create(dims, gs, [blk] * w.n_blocks)
    try:
        ws = torch.empty(B.h3_workspace_size(m, 1, B.make_opts()), dtype=torch.uint8, device=DEV)
        mod = torch.empty((w.n_blocks, 6, w.d_model), dtype=torch.float32, device=DEV)
        fin = torch.empty((2, w.d_model), dtype=torch.float32, device=DEV)
        g64 = {k: f64(v) for k, v in g.items()}
        for sigma in (1.0, 0.75, 0.25, 0.0):
            B.h3_modulation(m, sigma, mod, fin, ws)
            sync()
            mod_ref, fin_ref = dit.modulation(g64, sigma)
            assert_close(f64(mod), mod_ref, rel=1e-4, elem=1e-3, what=f"mod sigma={sigma}")
            assert_close(f64(fin), fin_ref, rel=1e-4, elem=1e-3, what=f"fin sigma={sigma}")
    finally:
        B.h3_model_destroy(m)
