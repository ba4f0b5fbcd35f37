"""Float64 oracle view of a synthetic model (inputs drawn by the shared seeded generator)."""
import numpy as np
import torch

from video_diffusion_transformer_fwd_amd import synthetic as S


def to64(t: torch.Tensor) -> np.ndarray:
    return t.to(torch.float64).numpy()


def oracle_model(w: S.Workload, blocks=None, seed: int = 0) -> dict:
    """Global weights, the requested blocks (all by default) and the text context, float64."""
    g = {k: to64(v) for k, v in S.global_weights(w, seed).items()}
    idx = range(w.n_blocks) if blocks is None else blocks
    bl = {b: {k: to64(v) for k, v in S.block_weights(w, b, seed).items()} for b in idx}
    if blocks is None:
        bl = [bl[b] for b in range(w.n_blocks)]
    return {"global": g, "blocks": bl, "ctx": to64(S.context(w, seed))}
