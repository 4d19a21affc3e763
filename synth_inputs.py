"""Seeded synthetic inputs for the attention forward workloads.

This module draws random tensors and rounds them to the storage format handed to
the GPU library. It holds none of the attention arithmetic and is the only code
shared by the oracle side and the HIP side (both receive the same bit patterns).

Recipe (per tensor, in the order Q, K, V):
  * ``numpy.random.Generator(PCG64(seed))`` draws float32 standard normals in
    memory order [B, N, heads, d];
  * for the e4m3 workload, the same generator then draws U(0,1) per element and
    multiplies the entries with U < outlier_frac (0.1%) by outlier_mult (20);
  * f16 / bf16: round to nearest even (torch CPU casts);
  * e4m3: per-tensor scale = amax(|x|) / 448 (float32), x / scale clamped to
    [-448, 448], rounded to nearest even in OCP E4M3 (torch ``float8_e4m3fn``);
    the descale handed to the library is that scale.
Arrays are returned as bit patterns: uint16 for f16 / bf16, uint8 for e4m3.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    N: int
    d: int
    causal: bool
    dtype: str          # "f16", "bf16" or "e4m3"
    seed: int
    scale: float
    outlier_frac: float = 0.0
    outlier_mult: float = 20.0
    window: tuple | None = None     # (left, right) key window; negative side = unbounded
    fp8_block: bool = False         # e4m3 block-quantised on the GPU (drawn as bf16, rotated Q/K)
    backward: bool = False          # the gradient pass (upstream dO drawn with seed + 100)
    decode_nq: int = 0              # split-KV decode: Nq queries against N keys (0: square)
    sparse_density: float = 0.0     # block-sparse: share of random key blocks kept (0: dense)

    @property
    def flops(self) -> float:
        """4*B*H*N^2*d, halved under the causal mask (query heads H). With a key window:
        4*B*H*d times the number of (query, key) pairs inside the window. The gradient
        pass counts 2.5 times its forward (five N x N x d products instead of two)."""
        if self.backward:
            return 2.5 * replace(self, backward=False).flops
        if self.decode_nq:
            nq, nk = self.decode_nq, self.N
            pairs = nq * nk - (nq * (nq - 1) // 2 if self.causal else 0)
            return 4.0 * self.B * self.H * self.d * pairs
        if self.sparse_density:
            return 4.0 * self.B * self.d * float(block_mask_pairs(workload_block_mask(self), self.N, self.causal,
                                                                   self.H))
        if self.window is None:
            f = 4.0 * self.B * self.H * self.N * self.N * self.d
            return f / 2 if self.causal else f
        i = np.arange(self.N, dtype=np.int64)
        left, right = self.window
        lo = np.maximum(0, i - left) if left >= 0 else np.zeros_like(i)
        hi = i if self.causal else np.full_like(i, self.N - 1)
        if right >= 0:
            hi = np.minimum(hi, i + right)
        return 4.0 * self.B * self.H * self.d * float(np.sum(hi - lo + 1))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


def _w(name, B, H, Hkv, N, d, causal, dtype, seed, **kw):
    return Workload(name, B, H, Hkv, N, d, causal, dtype, seed, 1.0 / math.sqrt(d), **kw)


# The five workloads: a tiny fp16 case, bf16 multi-head, bf16 causal long sequence,
# bf16 causal grouped-query, and e4m3 with outliers; then a causal sliding-window case
# (each query sees itself and the 4095 keys before it), the e4m3 shape again drawn in
# bf16 for block quantisation with the Hadamard rotation (signs from the same seed), and
# the gradient pass on the multi-head and the causal grouped-query shapes (same inputs),
# and single-query decode against a 16384-key grouped-query cache (split-KV).
WORKLOADS = {
    w.name: w for w in [
        _w("tiny_f16_b1_h2_n128_d64", 1, 2, 2, 128, 64, False, "f16", 1001),
        _w("mha_bf16_b16_h16_n2048_d128", 16, 16, 16, 2048, 128, False, "bf16", 1002),
        _w("causal_bf16_b1_h16_n16384_d128", 1, 16, 16, 16384, 128, True, "bf16", 1003),
        _w("gqa_causal_bf16_b4_h32_kv8_n8192_d128", 4, 32, 8, 8192, 128, True, "bf16", 1004),
        _w("fp8_e4m3_b8_h16_n4096_d128", 8, 16, 16, 4096, 128, False, "e4m3", 1005,
           outlier_frac=1e-3, outlier_mult=20.0),
        _w("swa_causal_bf16_b1_h32_kv8_n32768_d128_w4096", 1, 32, 8, 32768, 128, True, "bf16", 1006,
           window=(4095, -1)),
        _w("fp8_block_hadamard_b8_h16_n4096_d128", 8, 16, 16, 4096, 128, False, "bf16", 1005,
           outlier_frac=1e-3, outlier_mult=20.0, fp8_block=True),
        _w("bwd_bf16_b16_h16_n2048_d128", 16, 16, 16, 2048, 128, False, "bf16", 1002, backward=True),
        _w("bwd_causal_gqa_bf16_b4_h32_kv8_n8192_d128", 4, 32, 8, 8192, 128, True, "bf16", 1004, backward=True),
        _w("decode_bf16_b8_h32_kv8_nq1_nk16384_d128", 8, 32, 8, 16384, 128, False, "bf16", 1007, decode_nq=1),
        _w("block_sparse_bf16_b1_h16_n16384_d128", 1, 16, 16, 16384, 128, False, "bf16", 1008,
           sparse_density=0.1),
    ]
}

SPARSE_BLOCK = 64      # queries and keys per block of a block-sparse mask


def random_block_mask(heads: int, N: int, density: float, seed: int, block: int = SPARSE_BLOCK) -> np.ndarray:
    """uint8 [heads, nb, nb] mask with each block kept with probability `density`
    (nb = ceil(N / block)), from numpy PCG64(seed)."""
    nb = (N + block - 1) // block
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.random((heads, nb, nb)) < density).astype(np.uint8)


def bigbird_block_mask(heads: int, N: int, density: float, seed: int, group: int = 4,
                       block: int = SPARSE_BLOCK) -> np.ndarray:
    """uint8 [heads, nb, nb] block mask in the local + global + random pattern of
    long-context sparse attention: for every group of `group` query blocks (the rows of a
    256-query tile at 64-row blocks), the key blocks of the three neighbouring groups, the
    first group of key blocks, and each other key block with probability `density`; rows
    of one group share their key blocks. From numpy PCG64(seed)."""
    nb = (N + block - 1) // block
    ng = (nb + group - 1) // group
    rng = np.random.Generator(np.random.PCG64(seed))
    keep_g = rng.random((heads, ng, nb)) < density
    kb_group = np.arange(nb) // group
    for g in range(ng):
        keep_g[:, g, (np.abs(kb_group - g) <= 1) | (kb_group == 0)] = True
    return np.repeat(keep_g, group, axis=1)[:, :nb].astype(np.uint8)


def block_mask_pairs(mask: np.ndarray, N: int, causal: bool, H: int, block: int = SPARSE_BLOCK) -> int:
    """Visible (query, key) pairs summed over the H query heads (a mask of one head
    applies to all): rows x keys of every kept block, ragged last block included, and under
    the causal mask only the pairs with key <= query."""
    nb = mask.shape[1]
    sizes = np.minimum(block, N - np.arange(nb) * block).astype(np.int64)
    per = mask.astype(np.int64) * np.outer(sizes, sizes)[None]
    if causal:
        qi = np.arange(N)
        below = np.zeros((nb, nb), dtype=np.int64)            # pairs with key <= query per block pair
        for qb in range(nb):
            rows = qi[qb * block:(qb + 1) * block]
            for kb in range(qb + 1):
                lo, hi = kb * block, min(N, (kb + 1) * block) - 1
                below[qb, kb] = int(np.sum(np.clip(np.minimum(rows, hi) - lo + 1, 0, None)))
        per = mask.astype(np.int64) * below[None]
    total = int(per.sum())
    return total * (H // mask.shape[0])


def workload_block_mask(w: Workload) -> np.ndarray:
    """The block mask of a block-sparse workload (one per query head)."""
    return bigbird_block_mask(w.H, w.N, w.sparse_density, w.seed + 200)

E4M3_MAX = 448.0


def _round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if dtype == "f16":
        return t.to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def quantize_e4m3(x: np.ndarray):
    """Per-tensor e4m3 quantisation. Returns (uint8 bit patterns, descale float)."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    scale = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    y = np.clip(x.astype(np.float32) / scale, -E4M3_MAX, E4M3_MAX)
    bits = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return bits, float(scale)


def draw(shape, rng: np.random.Generator, outlier_frac: float = 0.0, outlier_mult: float = 20.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if outlier_frac > 0:
        u = rng.random(size=shape, dtype=np.float32)
        x = np.where(u < outlier_frac, x * np.float32(outlier_mult), x).astype(np.float32)
    return x


def make_inputs(B: int, H: int, Hkv: int, N: int, d: int, dtype: str, seed: int,
                outlier_frac: float = 0.0, outlier_mult: float = 20.0, keep_f32: bool = False):
    """Draw Q [B,N,H,d], K and V [B,N,Hkv,d] and round them to `dtype`.

    Returns a dict with "q", "k", "v" (bit patterns), "descale" ((dq, dk, dv) for
    e4m3, else None) and, with keep_f32, the unrounded float32 draws "q32", "k32",
    "v32"."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    raw = {}
    for name, heads in (("q", H), ("k", Hkv), ("v", Hkv)):
        raw[name] = draw((B, N, heads, d), rng, outlier_frac, outlier_mult)
    if dtype == "e4m3":
        ds = []
        for name in ("q", "k", "v"):
            bits, s = quantize_e4m3(raw[name])
            out[name] = bits
            ds.append(s)
        out["descale"] = tuple(ds)
    else:
        for name in ("q", "k", "v"):
            out[name] = _round_bits(raw[name], dtype)
        out["descale"] = None
    if keep_f32:
        for name in ("q", "k", "v"):
            out[name + "32"] = raw[name]
    return out


def make_decode_inputs(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int, dtype: str, seed: int):
    """Q [B,Nq,H,d], then K and V [B,Nk,Hkv,d]: float32 N(0,1) from ``PCG64(seed)`` in that
    order, rounded to `dtype` (bit patterns)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {}
    for name, n, heads in (("q", Nq, H), ("k", Nk, Hkv), ("v", Nk, Hkv)):
        out[name] = _round_bits(rng.standard_normal(size=(B, n, heads, d), dtype=np.float32), dtype)
    out["descale"] = None
    return out


def make_dout(B: int, N: int, H: int, d: int, dtype: str, seed: int) -> np.ndarray:
    """An upstream gradient dO [B,N,H,d]: float32 N(0,1) from ``PCG64(seed)`` rounded to
    `dtype` (bit patterns)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _round_bits(rng.standard_normal(size=(B, N, H, d), dtype=np.float32), dtype)


def random_signs(d: int, seed: int) -> np.ndarray:
    """d random signs (+1.0 / -1.0, float32) for the incoherent-processing rotation: bit 0
    of ``PCG64(seed)`` 32-bit draws, 1 -> -1."""
    rng = np.random.Generator(np.random.PCG64(seed))
    bits = rng.integers(0, 2**32, size=d, dtype=np.uint64) & 1
    return np.where(bits == 1, -1.0, 1.0).astype(np.float32)


def workload_inputs(w: Workload, keep_f32: bool = False, **overrides):
    """Inputs of a named workload (optionally with some sizes overridden)."""
    if overrides:
        w = w.with_(**overrides)
    if w.decode_nq:
        return make_decode_inputs(w.B, w.H, w.Hkv, w.decode_nq, w.N, w.d, w.dtype, w.seed)
    return make_inputs(w.B, w.H, w.Hkv, w.N, w.d, w.dtype, w.seed, w.outlier_frac,
                       w.outlier_mult, keep_f32=keep_f32)
