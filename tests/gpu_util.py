"""Helpers for GPU tests: move stored inputs to the device, run the library through its
C ABI binding, compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import exact_tiled_attention_03_amd as fa

# Elementwise bound |O_gpu - O_ref| <= TOL * max(1, |O_ref|); |lse_gpu - lse_ref| <= LSE_TOL.
TOL = {"f16": 2e-3, "bf16": 1e-2, "e4m3": 6e-2}
LSE_TOL = 1e-3
TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}


def to_dev(bits: np.ndarray, dtype: str, device="cuda:0") -> torch.Tensor:
    if dtype == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(bits)).to(device)
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(TORCH_DT[dtype])


def run(inp: dict, dtype: str, causal: bool, scale: float):
    """Run the library on stored inputs; returns (o, lse) device tensors."""
    q, k, v = (to_dev(inp[x], dtype) for x in "qkv")
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale, descale=inp.get("descale"),
                    dtype=dtype if dtype == "e4m3" else None)
    torch.cuda.synchronize()
    return o, lse


def host(o: torch.Tensor, lse: torch.Tensor):
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(o, o_ref, lse, lse_ref, dtype: str, what: str = ""):
    """Assert the parity bound; return (max scaled dO, max |dO|, max |dlse|)."""
    assert np.all(np.isfinite(o)), f"{what}: non-finite output"
    assert np.all(np.isfinite(lse)), f"{what}: non-finite lse"
    scaled = np.abs(o - o_ref) / np.maximum(1.0, np.abs(o_ref))
    e_o = float(scaled.max()) if scaled.size else 0.0
    e_abs = float(np.abs(o - o_ref).max()) if o.size else 0.0
    e_l = float(np.abs(lse - lse_ref).max()) if lse.size else 0.0
    assert e_o <= TOL[dtype], f"{what}: max scaled |dO| {e_o:.3e} > {TOL[dtype]} (abs {e_abs:.3e})"
    assert e_l <= LSE_TOL, f"{what}: max |dlse| {e_l:.3e} > {LSE_TOL}"
    return e_o, e_abs, e_l


def sample_rows(B: int, H: int, N: int, n_random: int, seed: int, br: int = 128) -> np.ndarray:
    """Rows (b, h, i) to spot-check: first and last positions, both sides of query-tile and
    key-tile boundaries, and random rows."""
    rng = np.random.default_rng(seed)
    fixed_i = sorted({0, 1, N - 1, N - 2, min(63, N - 1), min(64, N - 1), min(br - 1, N - 1), min(br, N - 1),
                      N // 2, (N // br) * br - 1 if N > br else 0})
    rows = []
    for i in fixed_i:
        rows.append((int(rng.integers(B)), int(rng.integers(H)), max(0, i)))
    rows.append((B - 1, H - 1, N - 1))
    rows.append((0, 0, 0))
    for _ in range(n_random):
        rows.append((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(N))))
    return np.array(rows, dtype=np.int64)
