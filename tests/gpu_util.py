"""Helpers shared by the GPU parity tests (inputs, conversions, comparisons)."""
import numpy as np
import torch

DEV = "cuda:0"


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 image of a device or host tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def bf16_dev(a, device=DEV) -> torch.Tensor:
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).to(device)


def randn_bf16(rng: np.random.Generator, shape, std=1.0, device=DEV) -> torch.Tensor:
    return bf16_dev(rng.standard_normal(shape) * std, device)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def assert_close(got, ref, rel=1e-2, elem=3e-2, what=""):
    """rel-L2 <= rel, and every element within elem * (|ref| + rms(ref))."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    assert r <= rel, f"{what}: rel-L2 {r:.3e} > {rel:.1e}"
    rms = np.sqrt(np.mean(ref * ref)) if ref.size else 0.0
    bound = elem * (np.abs(ref) + rms)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements outside bound, worst "
                           f"{float(np.max(np.abs(got - ref) - bound)):.3e}")
    return r


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bytes of a tensor for bit-identity checks."""
    return t.detach().to("cpu").contiguous().view(torch.uint8).numpy()


class zero_gates:
    """Context manager: the model's residual gates (rows g1 and g2 of the shared modulation
    projection, of its bias and of every block's table) are zero on the device inside, so
    every block leaves the residual stream as it is; the weights are restored on exit."""

    def __init__(self, model):
        self.m = model

    def __enter__(self):
        d, gw = self.m.w.d_model, self.m.gw
        self.saved = {k: gw[k].clone() for k in ("mod_w", "mod_b", "mod_table")}
        for r in (2, 5):
            gw["mod_w"][r * d:(r + 1) * d].zero_()
            gw["mod_b"][r * d:(r + 1) * d].zero_()
            gw["mod_table"][:, r].zero_()
        return self.m

    def __exit__(self, *exc):
        for k, v in self.saved.items():
            self.m.gw[k].copy_(v)
        torch.cuda.synchronize()
        return False
