"""h3_modulation_noalloc: the modulation with its intermediates in the library's static device
buffer (no workspace, no allocation) gives h3_modulation's results bit for bit, on two calls in
a row, the second with a smaller model width, and the oracle's within float32 rounding."""
import numpy as np
import pytest
import torch

from oracle import dit
from tests.gpu_util import DEV, assert_close, f64
from video_diffusion_transformer_fwd_amd import binding as B
from video_diffusion_transformer_fwd_amd import synthetic as S

pytestmark = pytest.mark.gpu


def globals_only_model(w):
    """A model handle with the workload's global weights; the blocks point at one zero buffer
    (the modulation reads only the global weights)."""
    g = S.global_weights(w)
    gd = {k: v.to(DEV) for k, v in g.items()}
    dims = B.h3_dims(w.d_model, w.n_heads, w.ffn_dim, w.ctx_len, w.latent_ch, w.n_blocks)
    gs = B.h3_global_weights(*[gd[n].data_ptr() for n in B.GLOBAL_FIELDS])
    dummy = torch.zeros(w.ffn_dim * w.d_model, dtype=torch.bfloat16, device=DEV)
    blk = B.h3_block_weights(*([dummy.data_ptr()] * 15 + [None] * 6))
    m = B.h3_model_create(dims, gs, [blk] * w.n_blocks)
    return m, g, (gd, dummy)


@pytest.mark.parametrize("sigmas", [(1.0, 0.25), (0.75, 0.0)])
def test_modulation_noalloc_matches_workspace_entry_point(sigmas):
    # first the 512x512x22 width (d = 3072, 50 blocks), then the small one (d = 512, 2 blocks)
    for w, sigma in zip((S.WORKLOADS["512sq_22f"], S.WORKLOADS["tiny_256sq_5f"]), sigmas):
        m, g, keep = globals_only_model(w)
        try:
            nb, d = w.n_blocks, w.d_model
            mod_a = torch.empty((nb, 6, d), dtype=torch.float32, device=DEV)
            fin_a = torch.empty((2, d), dtype=torch.float32, device=DEV)
            B.h3_modulation_noalloc(m, sigma, mod_a, fin_a)
            ws = torch.empty(B.h3_workspace_size(m, 1, B.make_opts()), dtype=torch.uint8, device=DEV)
            mod_b, fin_b = torch.empty_like(mod_a), torch.empty_like(fin_a)
            B.h3_modulation(m, sigma, mod_b, fin_b, ws)
            torch.cuda.synchronize()
            assert torch.equal(mod_a.view(torch.int32), mod_b.view(torch.int32)), (w.name, sigma)
            assert torch.equal(fin_a.view(torch.int32), fin_b.view(torch.int32)), (w.name, sigma)
            mod_ref, fin_ref = dit.modulation({k: f64(v) for k, v in g.items()}, sigma)
            assert_close(f64(mod_a), mod_ref, rel=1e-4, elem=1e-3, what=f"{w.name} mod")
            assert_close(f64(fin_a), fin_ref, rel=1e-4, elem=1e-3, what=f"{w.name} final")
        finally:
            B.h3_model_destroy(m)


def test_modulation_noalloc_at_the_widest_supported_width():
    # the widest model width the library accepts (8192) fills the static buffer: 256 + 8 * 8192
    # floats of its 264 KiB
    w = S.Workload("wide", 256, 256, 5, 8192, 64, 1024, 1, 2)
    m, g, keep = globals_only_model(w)
    try:
        mod = torch.empty((2, 6, 8192), dtype=torch.float32, device=DEV)
        fin = torch.empty((2, 8192), dtype=torch.float32, device=DEV)
        B.h3_modulation_noalloc(m, 0.5, mod, fin)
        torch.cuda.synchronize()
        mod_ref, fin_ref = dit.modulation({k: f64(v) for k, v in g.items()}, 0.5)
        assert_close(f64(fin), fin_ref, rel=1e-4, elem=1e-3, what="d 8192 final")
    finally:
        B.h3_model_destroy(m)
