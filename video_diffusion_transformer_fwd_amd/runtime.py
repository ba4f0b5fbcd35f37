"""Device-side setup around the C ABI: uploads a synthetic model, builds the pointer tables,
owns the workspace, and drives the Euler loop through the library's entry points.

PyTorch is used for device memory and streams only; every step of the path runs in the
library's kernels.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import torch

from . import binding as B
from . import synthetic as S


class Geometry:
    """Token geometry of a workload, from the library's host logic."""

    def __init__(self, w: S.Workload, reference_rope: bool = False):
        self.frames = B.h3_align_frames(w.frames)
        self.f_lat = B.h3_latent_frames(self.frames)
        self.grid_h, self.grid_w, self.scale = B.h3_token_grid(w.width, w.height, reference_rope)
        self.geom = B.make_geom(self.f_lat, self.grid_h, self.grid_w, self.scale, 0)
        self.n_tokens = B.h3_geom_tokens(self.geom)

    def as_dict(self):
        return dict(f_lat=self.f_lat, grid_h=self.grid_h, grid_w=self.grid_w, scale=self.scale)


def _upload_block(w: S.Workload, b: int, seed: int, device, with_int8: bool,
                  with_int8_linear: bool = False) -> dict:
    t = S.block_weights(w, b, seed)
    d, F = w.d_model, w.ffn_dim
    dev = {
        "qkvq_w": torch.cat([t["qkv_w"], t["qc_w"]], 0),
        "qkvq_b": torch.cat([t["qkv_b"], t["qc_b"]], 0),
        "kc_w": t["kc_w"], "kc_b": t["kc_b"], "vc_w": t["vc_w"], "vc_b": t["vc_b"],
        "out_w": torch.cat([t["o_w"], t["oc_w"]], 1),
        "out_b": t["o_b"], "outc_b": t["oc_b"],
        "q_gamma": t["q_gamma"], "k_gamma": t["k_gamma"],
        "fc1_w": t["fc1_w"], "fc1_b": t["fc1_b"], "fc2_w": t["fc2_w"], "fc2_b": t["fc2_b"],
    }
    out = {k: v.contiguous().to(device) for k, v in dev.items()}
    if with_int8:
        out["fc2_q"] = torch.empty((d, F), dtype=torch.int8, device=device)
        out["fc2_s"] = torch.empty((d,), dtype=torch.float32, device=device)
    if with_int8_linear:
        out["qkvq_q"] = torch.empty((4 * d, d), dtype=torch.int8, device=device)
        out["qkvq_s"] = torch.empty((4 * d,), dtype=torch.float32, device=device)
        out["fc1_q"] = torch.empty((F, d), dtype=torch.int8, device=device)
        out["fc1_s"] = torch.empty((F,), dtype=torch.float32, device=device)
    return out


class DiTModel:
    """A synthetic MiniMax-H3-shaped DiT resident in HBM, bound to the C ABI."""

    def __init__(self, w: S.Workload, seed: int = 0, device="cuda:0", with_int8=None,
                 workers=None, blocks=None, with_int8_linear=None):
        self.w, self.seed, self.device = w, seed, torch.device(device)
        self.with_int8 = (w.fc2_mode != "bf16") if with_int8 is None else with_int8
        self.with_int8_linear = w.int8_linear if with_int8_linear is None else with_int8_linear
        self.geo = Geometry(w)
        g = S.global_weights(w, seed)
        self.gw = {k: v.contiguous().to(self.device) for k, v in g.items()}
        self.mod_table_bits = g["mod_table"].view(torch.int16).numpy().view(np.uint16)
        nb = w.n_blocks
        self.blocks = [None] * nb
        workers = workers or min(16, max(1, len(os.sched_getaffinity(0))))
        prev = torch.get_num_threads()
        torch.set_num_threads(1)
        try:
            with cf.ThreadPoolExecutor(workers) as ex:
                futs = {ex.submit(_upload_block, w, b, seed, self.device, self.with_int8,
                                  self.with_int8_linear): b for b in range(nb)}
                for f in cf.as_completed(futs):
                    self.blocks[futs[f]] = f.result()
        finally:
            torch.set_num_threads(prev)
        torch.cuda.synchronize(self.device)
        self.dims = B.h3_dims(w.d_model, w.n_heads, w.ffn_dim, w.ctx_len, w.latent_ch, nb)
        self.g_struct = B.h3_global_weights(*[self.gw[n].data_ptr() for n in B.GLOBAL_FIELDS])
        self.b_structs = []
        for blk in self.blocks:
            vals = [blk[n].data_ptr() if n in blk else None for n in B.BLOCK_FIELDS]
            self.b_structs.append(B.h3_block_weights(*vals))
        self.handle = B.h3_model_create(self.dims, self.g_struct, self.b_structs)
        if self.with_int8:
            B.h3_quantize_fc2_weights(self.handle)
        if self.with_int8_linear:
            B.h3_quantize_linear_weights(self.handle)
        self.ctx = S.context(w, seed).to(self.device)
        self.ctx_kv = torch.empty((nb, 2, w.ctx_len, w.d_model), dtype=torch.bfloat16, device=self.device)
        B.h3_prepare_context(self.handle, self.ctx, self.ctx_kv)
        self._ws = {}

    # -------------------------------------------------------------- helpers
    def workspace(self, n_tokens: int, opts) -> torch.Tensor:
        size = B.h3_workspace_size(self.handle, n_tokens, opts)
        ws = self._ws.get("buf")
        if ws is None or ws.numel() < size:
            self._ws["buf"] = ws = torch.empty(size, dtype=torch.uint8, device=self.device)
        return ws

    def active(self, n_active=None):
        n_active = n_active or self.w.n_active
        if n_active == self.w.n_blocks:
            return list(range(self.w.n_blocks))
        return B.h3_select_layers(self.mod_table_bits, n_active)

    def opts(self, **kw):
        base = dict(fc2_mode=self.w.fc2_mode, token_reduction=self.w.token_reduction,
                    int8_linear=self.w.int8_linear)
        base.update(kw)
        return B.make_opts(**base)

    def initial_latent(self) -> torch.Tensor:
        return S.latent(self.w, self.geo.n_tokens, self.seed).to(self.device)

    # -------------------------------------------------------------- entry points
    def forward(self, latent, sigma, active=None, eval_index=0, opts=None, velocity=None):
        opts = opts or self.opts()
        active = self.active() if active is None else active
        n = self.geo.n_tokens
        if velocity is None:
            velocity = torch.empty((n, self.w.latent_ch), dtype=torch.float32, device=self.device)
        ws = self.workspace(n, opts)
        B.h3_dit_forward(self.handle, self.geo.geom, opts, latent, float(sigma), active, eval_index,
                         self.ctx_kv, velocity, ws)
        return velocity

    def forward_cached(self, latent, sigma, refresh_core, core_delta, active=None, eval_index=0,
                       opts=None, velocity=None):
        """One evaluation under core-residual reuse (``core_delta``: float32 [N, d])."""
        opts = opts or self.opts()
        active = self.active() if active is None else active
        n = self.geo.n_tokens
        if velocity is None:
            velocity = torch.empty((n, self.w.latent_ch), dtype=torch.float32, device=self.device)
        ws = self.workspace(n, opts)
        B.h3_dit_forward_cached(self.handle, self.geo.geom, opts, latent, float(sigma), active,
                                eval_index, self.ctx_kv, refresh_core, core_delta, velocity, ws)
        return velocity

    def denoise(self, latent, steps=None, reuse=None, active=None, opts=None, core_reuse=None):
        """Euler loop in place on ``latent``; returns the number of fresh (core) evaluations."""
        steps = steps or self.w.steps
        reuse = reuse or self.w.reuse
        core_reuse = core_reuse or self.w.core_reuse
        sig, fresh, _ = B.h3_schedule(steps, reuse, core_reuse)
        active = self.active() if active is None else active
        v = torch.empty((self.geo.n_tokens, self.w.latent_ch), dtype=torch.float32, device=self.device)
        delta = None
        if core_reuse > 1:
            delta = torch.empty((self.geo.n_tokens, self.w.d_model), dtype=torch.float32,
                                device=self.device)
        ev = 0
        for i in range(steps):
            if delta is not None:
                self.forward_cached(latent, float(sig[i]), bool(fresh[i]), delta, active, ev, opts, v)
                ev += int(fresh[i])
            elif fresh[i]:
                self.forward(latent, float(sig[i]), active, ev, opts, v)
                ev += 1
            B.h3_euler_step(latent, v, float(sig[i]), float(sig[i + 1]))
        return ev

    def close(self):
        if getattr(self, "handle", None):
            B.h3_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
