"""Writes the oracle's full-depth denoise loops at the 512x512x22-frame shape.

    python -m tests.golden.make_full_depth [512sq_22f 512sq_22f_tr 512sq_22f_int8 ...]

For each workload the float64 oracle (``oracle/``) runs the whole Euler loop on the seeded
synthetic model and latent (``synthetic.py``), every block of every fresh evaluation, and
the result is stored as ``tests/golden/full_depth_<workload>.npz``:

  velocities  float32 [n_fresh, N, C]  velocity of each fresh evaluation, in order
  latent      float32 [N, C]           the latent after the last Euler step
  meta        JSON string              workload, schedule, active list, sha256 of the oracle

Geometry, schedule, active list and token-pair plan come from ``oracle.host``.  Nothing here
calls the HIP library.  The loops take minutes each (about 4 s per 1536-token block on 8
cores); rerun this script after any change to the oracle's arithmetic.
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import dit, host  # noqa: E402
from tests.oracle_model import oracle_active, oracle_geom, oracle_latent, oracle_model  # noqa: E402
from video_diffusion_transformer_fwd_amd import synthetic as S  # noqa: E402

DEFAULT = ("512sq_22f", "512sq_22f_int8", "512sq_22f_tr")


def oracle_sha() -> str:
    h = hashlib.sha256()
    for f in ("dit.py", "host.py"):
        with open(os.path.join(ROOT, "oracle", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def path_for(name: str) -> str:
    return os.path.join(HERE, f"full_depth_{name}.npz")


class _Timed(list):
    """Velocity list that reports each fresh evaluation as it lands."""

    def __init__(self, name, t0):
        super().__init__()
        self.name, self.t0 = name, t0

    def append(self, v):
        super().append(v)
        print(f"  {self.name}: evaluation {len(self)} done at {time.time() - self.t0:.0f} s",
              flush=True)


def make(name: str) -> str:
    w = S.WORKLOADS[name]
    t0 = time.time()
    om = oracle_model(w, lazy=True)
    geo = oracle_geom(w)
    active = oracle_active(w, om)
    lat0 = oracle_latent(w)
    vel = _Timed(name, t0)
    x, n_fresh = dit.denoise(lat0, om, w.steps, w.reuse, active, geo, w.n_heads,
                             fc2_mode=w.fc2_mode, token_reduction=w.token_reduction,
                             int8_linear=w.int8_linear, velocities=vel)
    sig, fresh = host.schedule(w.steps, w.reuse)
    meta = dict(workload=name, seed=0, steps=w.steps, reuse=w.reuse, layers=w.n_active,
                fc2_mode=w.fc2_mode, token_reduction=w.token_reduction,
                int8_linear=w.int8_linear, n_fresh=n_fresh, active=list(map(int, active)),
                geometry={k: geo[k] for k in ("f_lat", "grid_h", "grid_w", "scale", "n")},
                sigmas=[float(s) for s in sig], oracle_sha256=oracle_sha(),
                seconds=round(time.time() - t0, 1))
    out = path_for(name)
    np.savez_compressed(out, velocities=np.stack(list(vel)).astype(np.float32),
                        latent=np.asarray(x, dtype=np.float32),
                        meta=np.array(json.dumps(meta)))
    print(f"{name}: {n_fresh} fresh evaluations, {meta['seconds']} s -> {out}", flush=True)
    return out


def load(name: str):
    """(velocities, latent, meta) of a stored loop, or None when the file is absent."""
    p = path_for(name)
    if not os.path.exists(p):
        return None
    with np.load(p, allow_pickle=False) as z:
        return z["velocities"], z["latent"], json.loads(str(z["meta"]))


if __name__ == "__main__":
    for nm in (sys.argv[1:] or DEFAULT):
        make(nm)
