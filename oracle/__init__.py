"""fp64 CPU oracle for the exact attention forward pass.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The product path (the
HIP library and its Python binding) never imports, links or falls back to it, and
the two share no code.

The arithmetic lives in ``attn_oracle.c`` (plain C, OpenMP over query rows, IEEE
double, no fast-math); this module compiles it with gcc when the shared object is
missing or older than the source, and marshals numpy arrays through ctypes.

What it computes is standard attention written out as a definition -- scores
S = scale * Q K^T, O = softmax(S) V -- following the section "The quadratic
bottleneck in standard attention" of the page "FlashAttention: The Algorithm That
Made Long-Context AI Possible". The tiled method reaches the same result exactly in
real arithmetic (abstract of "FlashAttention: Fast and Memory-Efficient Exact
Attention with IO-Awareness"), so no tiling or online softmax appears here.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_SOURCES = [_SRC, os.path.join(_HERE, "fp8_quant_oracle.c"), os.path.join(_HERE, "attn_bwd_oracle.c")]
_SO = os.path.join(_HERE, "liboracle.so")
_LOCK = threading.Lock()
_LIB = None

DTYPE_CODES = {"f16": 0, "bf16": 1, "e4m3": 2}


def build(force: bool = False) -> str:
    """Compile the oracle's C sources into liboracle.so with gcc (-O2, OpenMP, no
    fast-math, no contraction of a*b+c into fused multiply-adds)."""
    if force or not os.path.exists(_SO) or any(os.path.getmtime(_SO) < os.path.getmtime(s) for s in _SOURCES):
        tmp = _SO + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-Wall",
                        "-ffp-contract=off", "-o", tmp, *_SOURCES, "-lm"], check=True)
        os.replace(tmp, _SO)
    return _SO


def load(path: str):
    """Load a compiled oracle shared object and declare its C signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_decode.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, dp]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_attn_fwd_f64.argtypes = [dp, dp, dp, dp, dp] + [ctypes.c_int] * 6 + [ctypes.c_double]
    lib.oracle_attn_fwd_f64.restype = ctypes.c_int
    lib.oracle_attn_rows_f64.argtypes = ([dp, ctypes.c_int, dp, dp] + [ctypes.c_int] * 6 +
                                         [ctypes.c_double, ctypes.c_int64, i64p, dp, dp])
    lib.oracle_attn_rows_f64.restype = ctypes.c_int
    lib.oracle_attn_probs_f64.argtypes = ([dp, dp] + [ctypes.c_int] * 6 + [ctypes.c_double] +
                                          [ctypes.c_int, ctypes.c_int, dp])
    lib.oracle_attn_probs_f64.restype = ctypes.c_int
    lib.oracle_attn_fwd_local_f64.argtypes = ([dp, dp, dp, dp, dp] + [ctypes.c_int] * 8 +
                                              [ctypes.c_double])
    lib.oracle_attn_fwd_local_f64.restype = ctypes.c_int
    lib.oracle_attn_rows_local_f64.argtypes = ([dp, ctypes.c_int, dp, dp] + [ctypes.c_int] * 8 +
                                               [ctypes.c_double, ctypes.c_int64, i64p, dp, dp])
    lib.oracle_attn_rows_local_f64.restype = ctypes.c_int
    lib.oracle_attn_probs_local_f64.argtypes = ([dp, dp] + [ctypes.c_int] * 8 + [ctypes.c_double] +
                                                [ctypes.c_int, ctypes.c_int, dp])
    lib.oracle_attn_probs_local_f64.restype = ctypes.c_int
    u8p = ctypes.POINTER(ctypes.c_uint8)
    fp = ctypes.POINTER(ctypes.c_float)
    lib.oracle_e4m3_encode_array.argtypes = [fp, ctypes.c_int64, u8p]
    lib.oracle_e4m3_encode_array.restype = ctypes.c_int
    lib.oracle_fwht_rows_f32.argtypes = [fp, ctypes.c_int64, ctypes.c_int]
    lib.oracle_fwht_rows_f32.restype = ctypes.c_int
    lib.oracle_block_exponent.argtypes = [ctypes.c_float]
    lib.oracle_block_exponent.restype = ctypes.c_int
    lib.oracle_block_quantize_e4m3.argtypes = [dp] + [ctypes.c_int] * 5 + [fp, u8p, u8p]
    lib.oracle_block_quantize_e4m3.restype = ctypes.c_int
    lib.oracle_attn_bwd_f64.argtypes = [dp] * 7 + [ctypes.c_int] * 8 + [ctypes.c_double]
    lib.oracle_attn_bwd_f64.restype = ctypes.c_int
    lib.oracle_attn_bwd_dq_rows_f64.argtypes = [dp] * 4 + [ctypes.c_int] * 6 + [ctypes.c_double, ctypes.c_int64,
                                                                                i64p, dp, dp]
    lib.oracle_attn_bwd_dq_rows_f64.restype = ctypes.c_int
    lib.oracle_attn_bwd_dkdv_rows_f64.argtypes = [dp] * 6 + [ctypes.c_int] * 6 + [ctypes.c_double, ctypes.c_int64,
                                                                                  i64p, dp, dp, dp]
    lib.oracle_attn_bwd_dkdv_rows_f64.restype = ctypes.c_int
    lib.oracle_attn_fwd_kv_f64.argtypes = [dp] * 5 + [ctypes.c_int] * 7 + [ctypes.c_double]
    lib.oracle_attn_fwd_kv_f64.restype = ctypes.c_int
    lib.oracle_attn_fwd_block_f64.argtypes = ([dp, dp, dp, dp, dp] + [ctypes.c_int] * 6 +
                                              [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_double])
    lib.oracle_attn_fwd_block_f64.restype = ctypes.c_int
    lib.oracle_attn_rows_block_f64.argtypes = ([dp, ctypes.c_int, dp, dp] + [ctypes.c_int] * 6 +
                                               [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                                ctypes.c_int64, i64p, dp, dp])
    lib.oracle_attn_rows_block_f64.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    return lib


def _lib():
    global _LIB
    with _LOCK:
        if _LIB is None:
            _LIB = load(build())
    return _LIB


def _dptr(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all available)."""
    return int(_lib().oracle_num_threads())


def decode(raw: np.ndarray, dtype: str, mult: float = 1.0) -> np.ndarray:
    """Exact fp64 value of every stored element (bit patterns: uint16 for f16/bf16,
    uint8 for e4m3), multiplied by `mult` (the tensor's descale for e4m3)."""
    want = np.uint8 if dtype == "e4m3" else np.uint16
    raw = np.ascontiguousarray(raw)
    if raw.dtype != want:
        raise TypeError(f"{dtype} expects {want} bit patterns, got {raw.dtype}")
    out = np.empty(raw.shape, dtype=np.float64)
    rc = _lib().oracle_decode(DTYPE_CODES[dtype], raw.ctypes.data, raw.size, float(mult), _dptr(out))
    if rc:
        raise ValueError("oracle_decode rejected its arguments")
    return out


def _shape(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    if q.ndim != 4 or k.ndim != 4 or k.shape != v.shape:
        raise ValueError("q is [B,N,H,d]; k and v are [B,N,Hkv,d]")
    B, N, H, d = q.shape
    if k.shape[0] != B or k.shape[1] != N or k.shape[3] != d:
        raise ValueError("k/v shape does not match q")
    return B, N, H, k.shape[2], d


def _window(window):
    left, right = (-1, -1) if window is None else (int(window[0]), int(window[1]))
    return max(left, -1), max(right, -1)


def attn_fwd_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
                 window=None):
    """Attention forward on fp64 inputs. q [B,N,H,d], k/v [B,N,Hkv,d]. `window` =
    (left, right) keeps keys i-left <= j <= i+right for query i (negative: unbounded).
    Returns (o [B,N,H,d] float64, lse [B,H,N] float64)."""
    q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
    B, N, H, Hkv, d = _shape(q, k, v)
    left, right = _window(window)
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    rc = _lib().oracle_attn_fwd_local_f64(_dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(lse),
                                          B, H, Hkv, N, d, int(bool(causal)), left, right,
                                          float(scale))
    if rc:
        raise ValueError(f"oracle_attn_fwd_f64 failed ({rc})")
    return o, lse


def attn_rows_f64(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, H: int, rows: np.ndarray,
                  causal: bool, scale: float, window=None):
    """Selected query rows only. q_rows [R,d] are the fp64 query vectors of the rows
    rows[r] = (b, h, i); k/v [B,N,Hkv,d]. Returns (o_rows [R,d], lse_rows [R])."""
    q_rows = np.ascontiguousarray(q_rows, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    B, N, Hkv, d = k.shape
    R = rows.shape[0]
    if q_rows.shape != (R, d):
        raise ValueError("q_rows must be [len(rows), d]")
    o = np.empty((R, d), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    left, right = _window(window)
    rc = _lib().oracle_attn_rows_local_f64(_dptr(q_rows), 1, _dptr(k), _dptr(v), B, H, Hkv, N, d,
                                           int(bool(causal)), left, right, float(scale), R,
                                     rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                     _dptr(o), _dptr(lse))
    if rc:
        raise ValueError(f"oracle_attn_rows_f64 failed ({rc})")
    return o, lse


def attn_probs_f64(q: np.ndarray, k: np.ndarray, b: int, h: int, causal: bool, scale: float,
                   window=None):
    """Softmax probability matrix [N,N] of one (b, h); zeros where masked. Small N only."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    p = np.empty((N, N), dtype=np.float64)
    left, right = _window(window)
    rc = _lib().oracle_attn_probs_local_f64(_dptr(q), _dptr(k), B, H, Hkv, N, d, int(bool(causal)),
                                            left, right, float(scale), int(b), int(h), _dptr(p))
    if rc:
        raise ValueError(f"oracle_attn_probs_f64 failed ({rc})")
    return p


def attn_fwd(q_raw: np.ndarray, k_raw: np.ndarray, v_raw: np.ndarray, dtype: str, causal: bool,
             scale: float, descale=None, window=None):
    """Attention forward on the stored inputs exactly as handed to the GPU library:
    bit patterns of dtype `dtype` ("f16", "bf16" or "e4m3"); for e4m3, `descale` is the
    (q, k, v) per-tensor factors that multiply the decoded elements."""
    if dtype == "e4m3":
        if descale is None or len(descale) != 3:
            raise ValueError("e4m3 needs three descale factors")
        dq, dk, dv = (float(x) for x in descale)
    else:
        dq = dk = dv = 1.0
    return attn_fwd_f64(decode(q_raw, dtype, dq), decode(k_raw, dtype, dk), decode(v_raw, dtype, dv),
                        causal, scale, window)


def attn_rows(q_raw: np.ndarray, k_raw: np.ndarray, v_raw: np.ndarray, dtype: str, causal: bool,
              scale: float, rows: np.ndarray, descale=None, window=None):
    """Selected rows (b, h, i) of the forward on stored inputs, decoding only the query
    rows it needs. Returns (o_rows [R,d], lse_rows [R])."""
    if dtype == "e4m3":
        dq, dk, dv = (float(x) for x in descale)
    else:
        dq = dk = dv = 1.0
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    B, N, H, d = q_raw.shape
    q_sel = q_raw[rows[:, 0], rows[:, 2], rows[:, 1], :]
    return attn_rows_f64(decode(q_sel, dtype, dq), decode(k_raw, dtype, dk), decode(v_raw, dtype, dv),
                         H, rows, causal, scale, window)


# ---- block-sparse attention (attn_oracle.c) ----
# The block-sparse variant of the abstract of "FlashAttention: Fast and Memory-Efficient
# Exact Attention with IO-Awareness": key j is visible to query i iff
# mask[hm, i // block, j // block] != 0 (and j <= i when causal), hm = 0 for a mask
# shared by all heads, else the query head; a row with no visible key gives O = 0 and
# lse = -inf.

def _block_mask(mask, H: int, N: int, block: int) -> np.ndarray:
    mask = np.ascontiguousarray(mask, dtype=np.uint8)
    nb = (N + block - 1) // block
    if mask.ndim != 3 or mask.shape[1:] != (nb, nb) or mask.shape[0] not in (1, H):
        raise ValueError(f"block mask must be [1 or H, {nb}, {nb}] for N={N}, block={block}")
    return mask


def attn_fwd_block_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float,
                       mask, block: int = 64):
    """Block-sparse attention forward on fp64 inputs (layouts as attn_fwd_f64); mask is
    [mask_heads, nb, nb] (0 = block skipped). Returns (o, lse) in float64."""
    q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
    B, N, H, Hkv, d = _shape(q, k, v)
    mask = _block_mask(mask, H, N, block)
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    rc = _lib().oracle_attn_fwd_block_f64(_dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(lse), B, H, Hkv, N, d,
                                          int(bool(causal)), mask.ctypes.data, mask.shape[0], int(block),
                                          float(scale))
    if rc:
        raise ValueError(f"oracle_attn_fwd_block_f64 failed ({rc})")
    return o, lse


def attn_rows_block_f64(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, H: int, rows: np.ndarray,
                        causal: bool, scale: float, mask, block: int = 64):
    """Selected rows (b, h, i) of the block-sparse forward; q_rows [R,d] fp64."""
    q_rows = np.ascontiguousarray(q_rows, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    B, N, Hkv, d = k.shape
    mask = _block_mask(mask, H, N, block)
    R = rows.shape[0]
    if q_rows.shape != (R, d):
        raise ValueError("q_rows must be [len(rows), d]")
    o = np.empty((R, d), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    rc = _lib().oracle_attn_rows_block_f64(_dptr(q_rows), 1, _dptr(k), _dptr(v), B, H, Hkv, N, d,
                                           int(bool(causal)), mask.ctypes.data, mask.shape[0], int(block),
                                           float(scale), R, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                           _dptr(o), _dptr(lse))
    if rc:
        raise ValueError(f"oracle_attn_rows_block_f64 failed ({rc})")
    return o, lse


def attn_fwd_block(q_raw: np.ndarray, k_raw: np.ndarray, v_raw: np.ndarray, dtype: str, causal: bool,
                   scale: float, mask, block: int = 64):
    """Block-sparse forward on stored f16/bf16 inputs exactly as handed to the library."""
    return attn_fwd_block_f64(decode(q_raw, dtype), decode(k_raw, dtype), decode(v_raw, dtype), causal, scale,
                              mask, block)


def attn_rows_block(q_raw: np.ndarray, k_raw: np.ndarray, v_raw: np.ndarray, dtype: str, causal: bool,
                    scale: float, rows: np.ndarray, mask, block: int = 64):
    """Selected rows of the block-sparse forward on stored inputs."""
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    B, N, H, d = q_raw.shape
    q_sel = q_raw[rows[:, 0], rows[:, 2], rows[:, 1], :]
    return attn_rows_block_f64(decode(q_sel, dtype), decode(k_raw, dtype), decode(v_raw, dtype), H, rows, causal,
                               scale, mask, block)


# ---- block quantisation to e4m3 (fp8_quant_oracle.c) ----

def _u8p(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def _fp(a):
    assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """E4M3 codes (uint8) of float32 values: round to nearest even, saturating at 448."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    if _lib().oracle_e4m3_encode_array(_fp(y), y.size, _u8p(out)):
        raise ValueError("oracle_e4m3_encode_array rejected its arguments")
    return out


def fwht_f32(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform of every row (last axis, a power of two)
    in float32, butterfly stages h = 1, 2, ..., d/2."""
    y = np.array(x, dtype=np.float32, order="C", copy=True)
    d = y.shape[-1]
    if _lib().oracle_fwht_rows_f32(_fp(y), y.size // d, d):
        raise ValueError("oracle_fwht_rows_f32 rejected its arguments")
    return y


def block_exponent(amax: float) -> int:
    return int(_lib().oracle_block_exponent(float(amax)))


def block_quantize(x: np.ndarray, block_rows: int = 64, signs=None):
    """Block quantisation of x [B,N,Hx,d] (exact float values) to e4m3 with one
    power-of-two scale per block_rows x d slab of each (batch, head); with `signs` (d
    values +-1), rows are first replaced by (x * signs) H. Returns (codes uint8
    [B,N,Hx,d], scales uint8 E8M0 [B,Hx,ceil(N/block_rows)])."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    B, N, Hx, d = x.shape
    nb = (N + block_rows - 1) // block_rows
    codes = np.empty((B, N, Hx, d), dtype=np.uint8)
    scales = np.empty((B, Hx, nb), dtype=np.uint8)
    sg = None if signs is None else np.ascontiguousarray(signs, dtype=np.float32)
    rc = _lib().oracle_block_quantize_e4m3(_dptr(x), B, N, Hx, d, int(block_rows),
                                           _fp(sg) if sg is not None else None, _u8p(codes), _u8p(scales))
    if rc:
        raise ValueError(f"oracle_block_quantize_e4m3 failed ({rc})")
    return codes, scales


def block_dequantize(codes: np.ndarray, scales: np.ndarray, block_rows: int = 64) -> np.ndarray:
    """Exact values code * 2^(scale - 127) of block-quantised e4m3 data, float64."""
    B, N, Hx, d = codes.shape
    vals = decode(codes, "e4m3")
    rows = np.arange(N) // block_rows
    mult = np.ldexp(1.0, scales.astype(np.int64) - 127)          # [B, Hx, nb]
    return vals * mult[:, :, rows].transpose(0, 2, 1)[..., None]          # [B, N, Hx, 1]


# ---- gradient of the forward (attn_bwd_oracle.c) ----

def attn_bwd_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, causal: bool, scale: float,
                 window=None):
    """Analytic fp64 gradient of O = softmax(scale Q K^T [mask]) V for upstream dO (no
    gradient through lse). q, dout [B,N,H,d]; k, v [B,N,Hkv,d]. Returns (dq, dk, dv)."""
    q, k, v, dout = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, N, H, Hkv, d = _shape(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    left, right = _window(window)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    rc = _lib().oracle_attn_bwd_f64(_dptr(q), _dptr(k), _dptr(v), _dptr(dout), _dptr(dq), _dptr(dk), _dptr(dv),
                                    B, H, Hkv, N, d, int(bool(causal)), left, right, float(scale))
    if rc:
        raise ValueError(f"oracle_attn_bwd_f64 failed ({rc})")
    return dq, dk, dv


def attn_bwd_dq_rows_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, causal: bool,
                         scale: float, rows: np.ndarray, with_mag: bool = False):
    """dQ of the selected rows (b, h, i) only, [R, d] (same definition as attn_bwd_f64).
    With with_mag, also returns [R, 2, d]: sum_j |dS_ij||k_j| and sum_j P_ij |k_j|."""
    q, k, v, dout = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, N, H, Hkv, d = _shape(q, k, v)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    out = np.empty((rows.shape[0], d), dtype=np.float64)
    mag = np.empty((rows.shape[0], 2, d), dtype=np.float64) if with_mag else None
    rc = _lib().oracle_attn_bwd_dq_rows_f64(_dptr(q), _dptr(k), _dptr(v), _dptr(dout), B, H, Hkv, N, d,
                                            int(bool(causal)), float(scale), rows.shape[0],
                                            rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dptr(out),
                                            _dptr(mag) if with_mag else None)
    if rc:
        raise ValueError(f"oracle_attn_bwd_dq_rows_f64 failed ({rc})")
    return (out, mag) if with_mag else out


def attn_bwd_dkdv_rows_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, causal: bool,
                           scale: float, rows: np.ndarray, fwd=None, with_mag: bool = False):
    """dK and dV of the selected key rows (b, hk, j) only (hk a key/value head), each [R, d],
    summed over every query row that sees key j in every query head of hk's group (same
    definition as attn_bwd_f64). `fwd` = (o, lse) from attn_fwd_f64 on the same inputs,
    computed here when not given. With with_mag, also returns [R, 3, d]: sum_i |dS_ij||q_i|,
    sum_i P_ij w_i |q_i| (w_i = sum_t |dO_it O_it|) and sum_i P_ij |dO_i|."""
    q, k, v, dout = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v, dout))
    B, N, H, Hkv, d = _shape(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    o, lse = attn_fwd_f64(q, k, v, causal, scale) if fwd is None else fwd
    o = np.ascontiguousarray(o, dtype=np.float64)
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    if o.shape != q.shape or lse.shape != (B, H, N):
        raise ValueError("fwd must be (o [B,N,H,d], lse [B,H,N])")
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    R = rows.shape[0]
    dk = np.empty((R, d), dtype=np.float64)
    dv = np.empty((R, d), dtype=np.float64)
    mag = np.empty((R, 3, d), dtype=np.float64) if with_mag else None
    rc = _lib().oracle_attn_bwd_dkdv_rows_f64(_dptr(q), _dptr(k), _dptr(v), _dptr(dout), _dptr(o), _dptr(lse),
                                              B, H, Hkv, N, d, int(bool(causal)), float(scale), R,
                                              rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _dptr(dk),
                                              _dptr(dv), _dptr(mag) if with_mag else None)
    if rc:
        raise ValueError(f"oracle_attn_bwd_dkdv_rows_f64 failed ({rc})")
    return (dk, dv, mag) if with_mag else (dk, dv)


def attn_fwd_kv_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool, scale: float):
    """Rectangular forward: q [B,Nq,H,d] are the last Nq positions of a sequence whose keys
    k, v [B,Nk,Hkv,d] cover all Nk positions (decode); under the causal mask query i sees
    keys j <= Nk - Nq + i. Returns (o [B,Nq,H,d], lse [B,H,Nq])."""
    q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
    B, Nq, H, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k/v shape does not match q")
    o = np.empty_like(q)
    lse = np.empty((B, H, Nq), dtype=np.float64)
    rc = _lib().oracle_attn_fwd_kv_f64(_dptr(q), _dptr(k), _dptr(v), _dptr(o), _dptr(lse), B, H, Hkv, Nq, Nk, d,
                                       int(bool(causal)), float(scale))
    if rc:
        raise ValueError(f"oracle_attn_fwd_kv_f64 failed ({rc})")
    return o, lse
