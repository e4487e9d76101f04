"""Shared helpers for the GPU parity tests: device upload of synthetic layers, oracle
references on row subsets, and the tolerance rules.

The oracle never sees anything the HIP path produced: for a row subset it packs the
subset itself (from the seeded indices) and runs on that.
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = 2e-3  # max |y - y64| <= TOL * ||y64||_inf, fp32 accumulation


def f16_tensor(bits, device="cuda"):
    import torch

    if bits is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.float16).copy()).to(device)


def x_tensor(bits, dtype, device="cuda"):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(device)


class DeviceLayer:
    """A synthetic layer packed by the library's own packer and uploaded."""

    def __init__(self, vq, lay: dict, device="cuda"):
        import torch

        self.lay = lay
        self.desc = vq.make_desc(lay["n"], lay["in_features"], lay["v"], lay["bits1"], lay["bits2"])
        packed = vq.pack(self.desc, lay["idx1"], lay["idx2"])
        self.packed = torch.from_numpy(packed if packed.size else np.zeros(16, np.uint8)).to(device)
        self.cb1 = f16_tensor(lay["cb1"], device)
        self.cb2 = f16_tensor(lay["cb2"], device)
        self.scale = f16_tensor(lay["scale"], device)
        self.bias = f16_tensor(lay["bias"], device)

    def args(self):
        return (self.desc, self.packed, self.cb1, self.cb2, self.scale, self.bias)


def sub_layer(lay: dict, rows) -> dict:
    rows = np.asarray(rows)
    sub = dict(lay)
    sub["n"] = int(rows.size)
    sub["idx1"] = lay["idx1"][rows]
    sub["idx2"] = lay["idx2"][rows] if lay["bits2"] else None
    sub["scale"] = lay["scale"][rows] if lay["scale"] is not None else None
    sub["bias"] = lay["bias"][rows] if lay["bias"] is not None else None
    return sub


def oracle_packed(lay: dict) -> np.ndarray:
    return oracle.pack(lay["n"], lay["in_features"], lay["v"], lay["bits1"], lay["bits2"], lay["idx1"], lay["idx2"])


def oracle_w(lay: dict, rows=None) -> np.ndarray:
    """fp32 W^ rows from the oracle (packing the row subset itself)."""
    sub = lay if rows is None else sub_layer(lay, rows)
    p = oracle_packed(sub)
    return oracle.dequant(sub["n"], sub["in_features"], sub["v"], sub["bits1"], sub["bits2"], p, sub["cb1"],
                          sub["cb2"], sub["scale"])


def oracle_y(lay: dict, x_bits: np.ndarray, x_dtype: str, rows=None) -> np.ndarray:
    """y64 [M, rows] from the oracle."""
    sub = lay if rows is None else sub_layer(lay, rows)
    p = oracle_packed(sub)
    m = x_bits.shape[0]
    return oracle.forward(sub["n"], sub["in_features"], sub["v"], sub["bits1"], sub["bits2"], p, sub["cb1"],
                          sub["cb2"], sub["scale"], sub["bias"], x_bits, x_dtype == "bf16", m)


def half_ulp(ref: np.ndarray, out: str) -> np.ndarray:
    """Half a unit in the last place of the output format at |ref|."""
    mant, emin = (10, -14) if out == "f16" else (7, -126)
    a = np.maximum(np.abs(ref), 2.0 ** emin)
    e = np.floor(np.log2(a))
    return 0.5 * np.exp2(e - mant)


def check_y(y, y64: np.ndarray, out: str, tol: float = TOL, norm: float | None = None) -> float:
    """Asserts the tolerance rule; returns the error as a fraction of ||y64||_inf."""
    yd = y.float().cpu().numpy().astype(np.float64) if hasattr(y, "cpu") else np.asarray(y, np.float64)
    assert yd.shape == y64.shape, (yd.shape, y64.shape)
    assert np.isfinite(yd).all()
    norm = float(np.abs(y64).max()) if norm is None else norm
    err = np.abs(yd - y64)
    if out != "f32":
        err = err - half_ulp(y64, out)
    worst = float(err.max()) if err.size else 0.0
    frac = worst / norm if norm > 0 else worst
    assert worst <= tol * norm, "max error %.3e = %.3e of ||y||_inf (limit %.1e)" % (worst, frac, tol)
    return frac


def sample_rows(n: int, k: int, seed: int = 0) -> np.ndarray:
    g = np.random.default_rng(seed)
    base = [0, n - 1, n // 2]
    return np.unique(np.concatenate([base, g.integers(0, n, k)]))
