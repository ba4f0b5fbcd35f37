"""Float64 oracle view of a synthetic model (inputs drawn by the shared seeded generator).

Geometry, the active block list and the token-pair plan come from ``oracle.host`` only:
the oracle never takes a value the library under test computed.
"""
import numpy as np
import torch

from oracle import host
from video_diffusion_transformer_fwd_amd import synthetic as S


def to64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


class LazyBlocks:
    """``blocks[b]`` of a deep model, converted to float64 on access.

    The bf16 tensors of every block are drawn once and kept (2 bytes per weight); the
    float64 copy of one block exists only while the oracle runs it.
    """

    def __init__(self, w: S.Workload, seed: int = 0):
        self.w, self.seed = w, seed
        self._bf16 = {}

    def __len__(self):
        return self.w.n_blocks

    def __getitem__(self, b: int) -> dict:
        if not 0 <= b < self.w.n_blocks:
            raise IndexError(b)
        if b not in self._bf16:
            self._bf16[b] = S.block_weights(self.w, b, self.seed)
        return {k: to64(v) for k, v in self._bf16[b].items()}


def oracle_model(w: S.Workload, blocks=None, seed: int = 0, lazy: bool = False) -> dict:
    """Global weights, the requested blocks (all by default) and the text context, float64."""
    g = {k: to64(v) for k, v in S.global_weights(w, seed).items()}
    if lazy:
        bl = LazyBlocks(w, seed)
    else:
        idx = range(w.n_blocks) if blocks is None else blocks
        bl = {b: {k: to64(v) for k, v in S.block_weights(w, b, seed).items()} for b in idx}
        if blocks is None:
            bl = [bl[b] for b in range(w.n_blocks)]
    return {"global": g, "blocks": bl, "ctx": to64(S.context(w, seed))}


def oracle_geom(w: S.Workload, reference_rope: bool = False) -> dict:
    """Token geometry of a workload from the oracle's host logic: dict(f_lat, grid_h, grid_w,
    scale) as ``oracle.dit`` takes it, plus the token count under ``n``."""
    f_lat = host.latent_frames(host.align_frames(w.frames))
    gh, gw, scale = host.token_grid(w.width, w.height, reference_rope)
    return dict(f_lat=f_lat, grid_h=gh, grid_w=gw, scale=scale, n=host.n_tokens(f_lat, gh, gw))


def oracle_active(w: S.Workload, om: dict, n_active=None) -> list:
    """Active block list from the oracle's layer thinning over the model's gate table."""
    n_active = n_active or w.n_active
    return host.select_layers(om["global"]["mod_table"], n_active)


def oracle_latent(w: S.Workload, seed: int = 0) -> np.ndarray:
    """The workload's initial latent [N, C] at the oracle's token count, float64."""
    return to64(S.latent(w, oracle_geom(w)["n"], seed))
