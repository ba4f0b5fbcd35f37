"""Oracle: integer host logic of the denoiser (TEST INFRASTRUCTURE ONLY).

Everything here is exact integer (or exactly-rounded float32) arithmetic, so the HIP
library's host layer must match it bit for bit.  Written in plain Python.
"""
from __future__ import annotations

import math

import numpy as np

FPS = 24
MAX_PIXELS = 768 * 1344
LATENT_TOKEN_PIXELS = 32


def align_frames(requested: int) -> int:
    """Smallest frame count of the form 5 + 17 n (n >= 0) not below ``requested``.

    P2 §5 and P3 "temporal shapes": requests are rounded up to 5 + 17 n (23 -> 39).
    Reading: n >= 0, so requests of 1..5 frames give 5.
    """
    if requested < 1:
        raise ValueError("frame request must be >= 1")
    n = 0
    while 5 + 17 * n < requested:
        n += 1
    return 5 + 17 * n


def frames_for_seconds(seconds: float) -> int:
    """``--seconds s``: ceil(24 s) frames at 24 fps, then aligned (P5 key facts: 10 s -> 243)."""
    if not (seconds > 0):
        raise ValueError("seconds must be > 0")
    return align_frames(int(math.ceil(FPS * seconds)))


def latent_frames(frames: int) -> int:
    """Latent frame count for an aligned frame count.

    Reading (pages silent): F_lat = 1 + floor((F - 1) / 4), which gives 5 -> 2, 22 -> 6 and
    243 -> 61, the three latent counts the workloads use.
    """
    if frames < 1:
        raise ValueError("frames must be >= 1")
    return 1 + (frames - 1) // 4


def token_grid(width: int, height: int, reference_rope: bool = False):
    """(grid_h, grid_w, rope_spatial_scale) for an output size.

    P2 §5 / P3 "memory and resolution limits": width and height are multiples of 32, at
    least 32, and width*height <= 768*1344.  One spatial token per 32x32 pixels (P2 §5:
    256x256 -> 8x8 grid).  At the 8x8 grid the spatial RoPE coordinates are halved unless
    ``--use-reference-rope`` asks for the released coordinates (P2 §5).
    Reading: only the mechanical limits are enforced (128x128 is accepted); the halving
    applies to the 8x8 grid only.
    """
    for v in (width, height):
        if v < LATENT_TOKEN_PIXELS or v % LATENT_TOKEN_PIXELS != 0:
            raise ValueError("width/height must be multiples of 32 and >= 32")
    if width * height > MAX_PIXELS:
        raise ValueError("width*height exceeds 768*1344")
    gh, gw = height // LATENT_TOKEN_PIXELS, width // LATENT_TOKEN_PIXELS
    scale = 0.5 if (gh == 8 and gw == 8 and not reference_rope) else 1.0
    return gh, gw, scale


def n_tokens(f_lat: int, grid_h: int, grid_w: int) -> int:
    """Video tokens in one latent: frames x rows x columns, order (f, h, w)."""
    return f_lat * grid_h * grid_w


def schedule(steps: int, reuse: int = 1, core_reuse: int = 1):
    """Sigma grid and fresh-evaluation mask of the Euler loop.

    P2 §2 / P4 §2: ``--steps N`` is exactly N denoising passes on the released linear base
    grid with one endpoint; P4 table / P3 "aggressive levers": at 20 steps ``--reuse``
    1/2/3 gives 20/11/8 fresh DiT evaluations and skipped transitions are extrapolated;
    P2 §4: ``--reuse`` and ``--core-reuse`` are mutually exclusive.
    Reading: sigma_i = (N - i) / N in float32, i = 0..N (so sigma_N = 0); step i is fresh
    iff i mod r == 0 or i == N - 1; a skipped step reuses the last fresh velocity.
    P2 §4 / P3 "aggressive levers": ``--core-reuse k`` runs the heavy core less often while
    the patch and the timestep-dependent head stay fresh every step; values above 6 are not
    offered.  Reading: the same rule with r = k marks the steps whose core runs fresh
    (``fresh`` then means "core fresh"); 1 <= k <= 6.
    Returns (sigmas float32[N+1], fresh uint8[N]).
    """
    if steps < 1 or reuse < 1 or core_reuse < 1:
        raise ValueError("steps, reuse, core_reuse must be >= 1")
    if reuse > 1 and core_reuse > 1:
        raise ValueError("--reuse and --core-reuse are mutually exclusive")
    if core_reuse > 6:
        raise ValueError("core_reuse must be at most 6")
    r = reuse if reuse > 1 else core_reuse
    n = np.float32(steps)
    sig = np.array([np.float32(steps - i) / n for i in range(steps + 1)], dtype=np.float32)
    fresh = np.array([1 if (i % r == 0 or i == steps - 1) else 0 for i in range(steps)],
                     dtype=np.uint8)
    return sig, fresh


def gate_scores(mod_table: np.ndarray) -> list:
    """Per-block gate magnitude: sum over channels of |T_b[g1]| + |T_b[g2]| in float64.

    ``mod_table`` is [n_blocks, 6, d] with rows (shift1, scale1, gate1, shift2, scale2,
    gate2).  The sum runs over channels in ascending order, g1 term then g2 term, in
    plain Python floats (IEEE double).
    """
    nb = mod_table.shape[0]
    out = []
    for b in range(nb):
        g1 = mod_table[b, 2]
        g2 = mod_table[b, 5]
        s = 0.0
        for c in range(mod_table.shape[2]):
            s += abs(float(g1[c]))
            s += abs(float(g2[c]))
        out.append(s)
    return out


def select_layers(mod_table: np.ndarray, n_active: int) -> list:
    """Active-block list for ``--layers L`` (ascending block indices).

    P3 "aggressive levers": thinning ranks the blocks by their AdaLN gates and protects
    the critical first and last blocks.
    Reading: the per-block learned gate table is the ranking key (gate_scores); blocks 0
    and n-1 are always kept; the n - L blocks with the smallest key are dropped, ties
    dropping the higher index first.  2 <= L <= n.
    """
    nb = mod_table.shape[0]
    if not (2 <= n_active <= nb):
        raise ValueError("n_active must be in [2, n_blocks]")
    scores = gate_scores(mod_table)
    candidates = list(range(1, nb - 1))
    # lowest score first; equal scores: higher index first
    candidates.sort(key=lambda b: (scores[b], -b))
    dropped = set(candidates[: nb - n_active])
    return [b for b in range(nb) if b not in dropped]


def token_plan(f_lat: int, grid_h: int, grid_w: int, eval_index: int, n_active: int):
    """Horizontal token pairing plan for one fresh evaluation.

    P3 "aggressive levers" / P1: adjacent horizontal video tokens are paired after block 3;
    a bypass restores full resolution before block 40 for the first 10 evaluations and
    before block 30 for later ones; the head sees full resolution.
    Reading: block numbers are 1-based positions in the active list; merging happens after
    position 3, restoring before position 40 (eval_index 0..9) or 30 (later), or before
    the head when the list is shorter.  Reduced token j of row (f, h) pairs columns 2j and
    2j+1; an odd last column pairs with itself.
    Returns dict(merge_after=3, restore_before=r (1-based position, n_active+1 = head),
    pairs=int32[N_r, 2] full-token indices, n_reduced=N_r).
    """
    if n_active <= 3:
        raise ValueError("token reduction needs more than 3 active blocks")
    restore = 40 if eval_index < 10 else 30
    restore = min(restore, n_active + 1)
    wr = (grid_w + 1) // 2
    pairs = []
    for f in range(f_lat):
        for h in range(grid_h):
            row = (f * grid_h + h) * grid_w
            for j in range(wr):
                a = 2 * j
                b = 2 * j + 1 if 2 * j + 1 < grid_w else 2 * j
                pairs.append((row + a, row + b))
    return dict(merge_after=3, restore_before=restore,
                pairs=np.array(pairs, dtype=np.int32).reshape(-1, 2), n_reduced=len(pairs))
