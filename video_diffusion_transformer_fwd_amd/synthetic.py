"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module holds no arithmetic of the denoiser: it only draws tensors.  Every tensor is
drawn from its own CPU stream, seeded by ``splitmix64(seed ^ fnv1a64(name))``, with torch's
CPU generator (``randn``) and rounded to bf16, so any single block can be regenerated on
the host without drawing the others.

Distributions (the workloads' description: weights N(0, 0.02) in bf16, latent N(0, 1)):
  * weights and biases of every Linear, the per-block modulation tables and the final
    modulation table: N(0, 0.02), bf16;
  * Q/K RMSNorm gains: 1 + N(0, 0.02), bf16 (not all ones, so a dropped gain is visible);
  * latent: N(0, 1), float32, [N, C] in token order (f, h, w);
  * text context: N(0, 1), bf16, [L_ctx, d].
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

MASK64 = (1 << 64) - 1


def fnv1a64(name: str) -> int:
    h = 0xCBF29CE484222325
    for byte in name.encode():
        h ^= byte
        h = (h * 0x100000001B3) & MASK64
    return h


def splitmix64(x: int) -> int:
    x = (x + 0x9E3779B97F4A7C15) & MASK64
    z = x
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def tensor_seed(seed: int, name: str) -> int:
    return splitmix64((seed ^ fnv1a64(name)) & MASK64) & 0x7FFF_FFFF_FFFF_FFFF


def normal(name: str, shape, std: float = 1.0, mean: float = 0.0, seed: int = 0,
           dtype=torch.bfloat16) -> torch.Tensor:
    """N(mean, std^2) drawn from the stream of ``name``, float32 then cast to ``dtype``."""
    g = torch.Generator().manual_seed(tensor_seed(seed, name))
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(dtype)


@dataclass(frozen=True)
class Workload:
    """Shape of one synthetic workload (the pages' output size and model width)."""
    name: str
    width: int
    height: int
    frames: int
    d_model: int
    n_heads: int
    ffn_dim: int
    ctx_len: int
    n_blocks: int
    latent_ch: int = 128
    steps: int = 1
    reuse: int = 1
    layers: int = 0            # 0 = all blocks
    token_reduction: bool = False
    fc2_mode: str = "bf16"
    int8_linear: bool = False  # int8 QKV and FC1 with row-quantised AdaLN outputs
    core_reuse: int = 1        # --core-reuse k (exclusive with reuse > 1)
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def head_dim(self) -> int:
        return self.d_model // self.n_heads

    @property
    def n_active(self) -> int:
        return self.layers or self.n_blocks


WORKLOADS = {
    # 256x256, 5 frames, 2 blocks, one Euler step (the small parity case)
    "tiny_256sq_5f": Workload("tiny_256sq_5f", 256, 256, 5, 512, 8, 2048, 32, 2, steps=1),
    # 512x512x22 frames, 50 blocks, --steps 4 --reuse 1
    "512sq_22f": Workload("512sq_22f", 512, 512, 22, 3072, 24, 12288, 256, 50, steps=4),
    # same shape, --steps 20 --layers 45 --reuse 2 --token-reduction
    "512sq_22f_tr": Workload("512sq_22f_tr", 512, 512, 22, 3072, 24, 12288, 256, 50,
                             steps=20, reuse=2, layers=45, token_reduction=True),
    # same shape, 50 blocks, per-row int8 FC2
    "512sq_22f_int8": Workload("512sq_22f_int8", 512, 512, 22, 3072, 24, 12288, 256, 50,
                               steps=4, fc2_mode="row"),
    # same shape, 50 blocks, int8 FC2 with one activation scale per 1024-channel group
    "512sq_22f_int8g": Workload("512sq_22f_int8g", 512, 512, 22, 3072, 24, 12288, 256, 50,
                                steps=4, fc2_mode="grouped"),
    # same shape with the whole int8 path: int8 QKV and FC1 (quantisation fused into the gated
    # AdaLN) and the per-row int8 FC2
    "512sq_22f_int8_all": Workload("512sq_22f_int8_all", 512, 512, 22, 3072, 24, 12288, 256, 50,
                                   steps=4, fc2_mode="row", int8_linear=True),
    # same shape, --steps 20 --layers 45 --core-reuse 4: the core runs on 6 of the 20 steps,
    # patch and head on every step
    "512sq_22f_core4": Workload("512sq_22f_core4", 512, 512, 22, 3072, 24, 12288, 256, 50,
                                steps=20, layers=45, core_reuse=4),
    # 768x1344, 243 frames, one forward
    "768x1344_243f": Workload("768x1344_243f", 1344, 768, 243, 5120, 40, 20480, 512, 50,
                              steps=1),
    # 864x480 (15 x 27 token grid: odd width), 22 frames, --steps 4 --reuse 1
    "864x480_22f": Workload("864x480_22f", 864, 480, 22, 3072, 24, 12288, 256, 50, steps=4),
    # same shape with --steps 20 --layers 45 --reuse 2 --token-reduction (singleton last column)
    "864x480_22f_tr": Workload("864x480_22f_tr", 864, 480, 22, 3072, 24, 12288, 256, 50,
                               steps=20, reuse=2, layers=45, token_reduction=True),
}

STD = 0.02

# name -> shape builder (d, F, C, D) for the global tensors
_GLOBAL = {
    "t1_w": lambda d, f, c, dh, nb: (d, 256), "t1_b": lambda d, f, c, dh, nb: (d,),
    "t2_w": lambda d, f, c, dh, nb: (d, d), "t2_b": lambda d, f, c, dh, nb: (d,),
    "mod_w": lambda d, f, c, dh, nb: (6 * d, d), "mod_b": lambda d, f, c, dh, nb: (6 * d,),
    "fin_w": lambda d, f, c, dh, nb: (2 * d, d), "fin_b": lambda d, f, c, dh, nb: (2 * d,),
    "fin_t": lambda d, f, c, dh, nb: (2, d),
    "mod_table": lambda d, f, c, dh, nb: (nb, 6, d),
    "patch_w": lambda d, f, c, dh, nb: (d, c), "patch_b": lambda d, f, c, dh, nb: (d,),
    "head_w": lambda d, f, c, dh, nb: (c, d), "head_b": lambda d, f, c, dh, nb: (c,),
}

_BLOCK = {
    "qkv_w": lambda d, f, dh: (3 * d, d), "qkv_b": lambda d, f, dh: (3 * d,),
    "qc_w": lambda d, f, dh: (d, d), "qc_b": lambda d, f, dh: (d,),
    "kc_w": lambda d, f, dh: (d, d), "kc_b": lambda d, f, dh: (d,),
    "vc_w": lambda d, f, dh: (d, d), "vc_b": lambda d, f, dh: (d,),
    "o_w": lambda d, f, dh: (d, d), "o_b": lambda d, f, dh: (d,),
    "oc_w": lambda d, f, dh: (d, d), "oc_b": lambda d, f, dh: (d,),
    "q_gamma": lambda d, f, dh: (dh,), "k_gamma": lambda d, f, dh: (dh,),
    "fc1_w": lambda d, f, dh: (f, d), "fc1_b": lambda d, f, dh: (f,),
    "fc2_w": lambda d, f, dh: (d, f), "fc2_b": lambda d, f, dh: (d,),
}
BLOCK_TENSORS = tuple(_BLOCK)
GLOBAL_TENSORS = tuple(_GLOBAL)


def global_weights(w: Workload, seed: int = 0) -> dict:
    """Global (non-block) bf16 tensors of the model, CPU."""
    out = {}
    for name, shp in _GLOBAL.items():
        out[name] = normal(f"global.{name}", shp(w.d_model, w.ffn_dim, w.latent_ch, w.head_dim,
                                                 w.n_blocks), STD, seed=seed)
    return out


def block_tensor(w: Workload, b: int, name: str, seed: int = 0) -> torch.Tensor:
    shp = _BLOCK[name](w.d_model, w.ffn_dim, w.head_dim)
    if name.endswith("_gamma"):
        return normal(f"block{b}.{name}", shp, STD, mean=1.0, seed=seed)
    return normal(f"block{b}.{name}", shp, STD, seed=seed)


def block_weights(w: Workload, b: int, seed: int = 0) -> dict:
    """bf16 tensors of block ``b``, CPU."""
    return {name: block_tensor(w, b, name, seed) for name in _BLOCK}


def latent(w: Workload, n_tokens: int, seed: int = 0) -> torch.Tensor:
    """Initial latent [N, C] float32, N(0, 1)."""
    return normal("latent", (n_tokens, w.latent_ch), 1.0, seed=seed, dtype=torch.float32)


def context(w: Workload, seed: int = 0) -> torch.Tensor:
    """Text context [L_ctx, d] bf16, N(0, 1)."""
    return normal("context", (w.ctx_len, w.d_model), 1.0, seed=seed)
