"""Python binding of libfa.so (include/fa.h). Argument marshalling only: every step of
the attention forward runs in the library's gfx950 kernels; torch provides device
memory and the current stream. There is no fallback path: if the library is missing,
every call raises."""
from __future__ import annotations

import ctypes
import math
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_LAUNCH, FA_ERR_SCRATCH = 0, 1, 2, 3, 4
SPLITKV_STATIC_SCRATCH_BYTES = 32 << 20   # FA_SPLITKV_STATIC_SCRATCH_BYTES
FP8_BLOCK_ROWS = 64      # FA_FP8_BLOCK_ROWS
FA_DTYPE_F16, FA_DTYPE_BF16, FA_DTYPE_FP8_E4M3 = 0, 1, 2
DTYPE_NAMES = {"f16": FA_DTYPE_F16, "bf16": FA_DTYPE_BF16, "e4m3": FA_DTYPE_FP8_E4M3}

_lock = threading.Lock()
_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with exact_tiled_attention_03_amd.build.build()")
            L = ctypes.CDLL(LIB_PATH)
            c_int, c_float, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
            szp = ctypes.POINTER(ctypes.c_size_t)
            L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int,
                                 c_float, c_int, ctypes.POINTER(c_float), vp]
            L.fa_fwd.restype = c_int
            L.fa_fwd_local.argtypes = [vp, vp, vp, vp, vp] + [c_int] * 8 + [c_float, c_int,
                                                                            ctypes.POINTER(c_float), vp]
            L.fa_fwd_local.restype = c_int
            L.fa_fwd_block_sparse.argtypes = [vp] * 5 + [c_int] * 6 + [vp, c_int, c_float, c_int, vp]
            L.fa_fwd_block_sparse.restype = c_int
            L.fa_quantize_e4m3_block.argtypes = [vp, c_int, c_int, c_int, c_int, c_int, vp, vp, vp, vp]
            L.fa_quantize_e4m3_block.restype = c_int
            L.fa_fwd_fp8_block.argtypes = [vp] * 8 + [c_int] * 6 + [c_float, c_int, vp]
            L.fa_fwd_fp8_block.restype = c_int
            L.fa_bwd_workspace_bytes.argtypes = [c_int] * 3
            L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
            L.fa_bwd.argtypes = [vp] * 9 + [c_int] * 6 + [c_float, c_int, vp, ctypes.c_size_t, vp]
            L.fa_bwd.restype = c_int
            L.fa_fwd_splitkv_workspace_bytes.argtypes = [c_int] * 7
            L.fa_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
            L.fa_fwd_splitkv.argtypes = [vp] * 5 + [c_int] * 7 + [c_float, c_int, c_int, vp, ctypes.c_size_t, vp]
            L.fa_fwd_splitkv.restype = c_int
            L.fa_fwd_splitkv_static.argtypes = [vp] * 5 + [c_int] * 7 + [c_float, c_int, c_int, vp]
            L.fa_fwd_splitkv_static.restype = c_int
            L.fa_fwd_query.argtypes = [c_int] * 7 + [szp] * 5
            L.fa_fwd_query.restype = c_int
            L.fa_status_string.argtypes = [c_int]
            L.fa_status_string.restype = ctypes.c_char_p
            L.fa_version.argtypes = []
            L.fa_version.restype = c_int
            _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def version() -> int:
    return int(lib().fa_version())


def _check(status: int):
    if status != FA_OK:
        raise FaError(status, status_string(status))


def fa_fwd(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int, Hkv: int,
           N: int, d: int, causal: int, scale: float, dtype: int, descale=None, stream: int = 0) -> int:
    """Direct call of fa_fwd with raw pointers; returns the status code."""
    ds = (ctypes.c_float * 3)(*descale) if descale is not None else None
    return int(lib().fa_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Hkv, N, d, int(causal),
                            float(scale), int(dtype), ds, stream))


def fa_fwd_local(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int,
                 Hkv: int, N: int, d: int, causal: int, window_left: int, window_right: int,
                 scale: float, dtype: int, descale=None, stream: int = 0) -> int:
    """Direct call of fa_fwd_local (key window i-left <= j <= i+right, negative bound =
    unbounded) with raw pointers; returns the status code."""
    ds = (ctypes.c_float * 3)(*descale) if descale is not None else None
    return int(lib().fa_fwd_local(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Hkv, N, d, int(causal),
                                  int(window_left), int(window_right), float(scale), int(dtype), ds,
                                  stream))


def fa_quantize_e4m3_block(x_ptr: int, in_dtype: int, B: int, N: int, Hx: int, d: int, signs_ptr: int,
                           codes_ptr: int, scales_ptr: int, stream: int = 0) -> int:
    """Direct call of fa_quantize_e4m3_block with raw pointers; returns the status code."""
    return int(lib().fa_quantize_e4m3_block(x_ptr, int(in_dtype), B, N, Hx, d, signs_ptr or None, codes_ptr,
                                            scales_ptr, stream))


def fa_fwd_fp8_block(q_ptr: int, k_ptr: int, v_ptr: int, qs_ptr: int, ks_ptr: int, vs_ptr: int, o_ptr: int,
                     lse_ptr: int, B: int, H: int, Hkv: int, N: int, d: int, causal: int, scale: float,
                     qk_e4m3: int = 0, stream: int = 0) -> int:
    """Direct call of fa_fwd_fp8_block with raw pointers; returns the status code."""
    return int(lib().fa_fwd_fp8_block(q_ptr, k_ptr, v_ptr, qs_ptr, ks_ptr, vs_ptr, o_ptr, lse_ptr, B, H, Hkv,
                                      N, d, int(causal), float(scale), int(qk_e4m3), stream))


def fa_bwd_workspace_bytes(B: int, H: int, N: int) -> int:
    return int(lib().fa_bwd_workspace_bytes(B, H, N))


def fa_bwd(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, do_ptr: int, lse_ptr: int, dq_ptr: int, dk_ptr: int,
           dv_ptr: int, B: int, H: int, Hkv: int, N: int, d: int, causal: int, scale: float, dtype: int,
           ws_ptr: int, ws_bytes: int, stream: int = 0) -> int:
    """Direct call of fa_bwd with raw pointers; returns the status code."""
    return int(lib().fa_bwd(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr, B, H, Hkv, N, d,
                            int(causal), float(scale), int(dtype), ws_ptr, int(ws_bytes), stream))


def fa_fwd_splitkv_workspace_bytes(B: int, H: int, Hkv: int, Nq: int, Nk: int, d: int, num_splits: int = 0) -> int:
    return int(lib().fa_fwd_splitkv_workspace_bytes(B, H, Hkv, Nq, Nk, d, int(num_splits)))


def fa_fwd_splitkv(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int, Hkv: int, Nq: int,
                   Nk: int, d: int, causal: int, scale: float, dtype: int, num_splits: int, ws_ptr: int,
                   ws_bytes: int, stream: int = 0) -> int:
    """Direct call of fa_fwd_splitkv with raw pointers; returns the status code."""
    return int(lib().fa_fwd_splitkv(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Hkv, Nq, Nk, d, int(causal),
                                    float(scale), int(dtype), int(num_splits), ws_ptr, int(ws_bytes), stream))


def fa_fwd_splitkv_static(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int, Hkv: int,
                          Nq: int, Nk: int, d: int, causal: int, scale: float, dtype: int, num_splits: int,
                          stream: int = 0) -> int:
    """Direct call of fa_fwd_splitkv_static (no workspace, no allocation); returns the status code."""
    return int(lib().fa_fwd_splitkv_static(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Hkv, Nq, Nk, d, int(causal),
                                           float(scale), int(dtype), int(num_splits), stream))


def fa_fwd_query(B: int, H: int, Hkv: int, N: int, d: int, causal: int, dtype: int) -> dict:
    """Byte sizes of q, k/v, o, lse and the workspace (always 0); raises on bad sizes."""
    out = [ctypes.c_size_t(0) for _ in range(5)]
    _check(lib().fa_fwd_query(B, H, Hkv, N, d, int(causal), int(dtype), *[ctypes.byref(x) for x in out]))
    return dict(zip(("q", "kv", "o", "lse", "workspace"), (x.value for x in out)))


def _dtype_code(t, dtype):
    import torch
    if dtype is not None:
        if dtype not in DTYPE_NAMES:
            raise ValueError(f"dtype must be one of {sorted(DTYPE_NAMES)}")
        return DTYPE_NAMES[dtype]
    codes = {torch.float16: FA_DTYPE_F16, torch.bfloat16: FA_DTYPE_BF16, torch.float8_e4m3fn: FA_DTYPE_FP8_E4M3}
    if t.dtype not in codes:
        raise ValueError(f"unsupported element type {t.dtype} (float16, bfloat16 or float8_e4m3fn)")
    return codes[t.dtype]


def fwd(q, k, v, causal: bool = False, scale: float | None = None, descale=None, dtype: str | None = None,
        out=None, lse=None, stream=None, window=None):
    """Attention forward on device tensors.

    q [B,N,H,d], k and v [B,N,Hkv,d], contiguous, on one GPU; element type float16,
    bfloat16 or float8_e4m3fn (uint8 tensors with dtype="e4m3" are also accepted;
    e4m3 needs descale=(dq, dk, dv)). `window` = (left, right) restricts query i to
    keys i-left <= j <= i+right (negative: unbounded; calls fa_fwd_local). Returns
    (o [B,N,H,d], lse [B,H,N] float32);
    o has q's type for 16-bit inputs and bfloat16 for e4m3. Enqueues on the current
    stream (or `stream`) and returns without synchronising."""
    import torch
    code = _dtype_code(q, dtype)
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = torch.bfloat16 if code == FA_DTYPE_FP8_E4M3 else q.dtype
    if out is None:
        out = torch.empty((B, N, H, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    for t in (q, k, v, out, lse):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError("tensors must be contiguous and on the same device")
    if tuple(k.shape) != (B, N, Hkv, d) or tuple(v.shape) != (B, N, Hkv, d):
        raise ValueError("k and v must be [B,N,Hkv,d] matching q")
    _same_elem_type(q, (k, v), "q, k and v")
    if code == FA_DTYPE_FP8_E4M3 and q.element_size() != 1:
        raise ValueError("e4m3 inputs must be 1-byte tensors (float8_e4m3fn or uint8)")
    if code != FA_DTYPE_FP8_E4M3 and q.dtype != {FA_DTYPE_F16: torch.float16, FA_DTYPE_BF16: torch.bfloat16}[code]:
        raise ValueError(f"16-bit inputs must be float16 or bfloat16 matching dtype (got {q.dtype})")
    if tuple(out.shape) != (B, N, H, d) or out.dtype != out_dtype or tuple(lse.shape) != (B, H, N) \
            or lse.dtype != torch.float32:
        raise ValueError("out/lse have the wrong shape or type")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    if window is None:
        st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Hkv, N,
                    d, int(bool(causal)), scale, code, descale, stream)
    else:
        st = fa_fwd_local(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                          Hkv, N, d, int(bool(causal)), int(window[0]), int(window[1]), scale, code,
                          descale, stream)
    _check(st)
    return out, lse


SPARSE_BLOCK = 64   # FA_SPARSE_BLOCK: queries and keys per block of a block-sparse mask


def fa_fwd_block_sparse(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int, B: int, H: int, Hkv: int,
                        N: int, d: int, causal: int, mask_ptr: int, mask_heads: int, scale: float, dtype: int,
                        stream: int = 0) -> int:
    """Direct call of fa_fwd_block_sparse with raw pointers; returns the status code."""
    return int(lib().fa_fwd_block_sparse(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Hkv, N, d, int(causal),
                                         mask_ptr, int(mask_heads), float(scale), int(dtype), stream))


def fwd_block_sparse(q, k, v, block_mask, causal: bool = False, scale: float | None = None, out=None, lse=None,
                     stream=None):
    """Block-sparse attention forward on device tensors (float16 or bfloat16): query i of
    head h sees key j iff block_mask[hm, i // 64, j // 64] != 0 (hm = 0 for a mask of one
    head, else h; and j <= i when causal). block_mask is a contiguous uint8 device tensor
    [1 or H, nb, nb], nb = ceil(N / 64). Rows with no visible key get O = 0, lse = -inf.
    Returns (o [B,N,H,d], lse [B,H,N] float32) without synchronising."""
    import torch
    code = _dtype_code(q, None)
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    nb = (N + SPARSE_BLOCK - 1) // SPARSE_BLOCK
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    for t in (q, k, v, out, lse, block_mask):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError("tensors must be contiguous and on the same device")
    if block_mask.dtype != torch.uint8 or block_mask.dim() != 3 or tuple(block_mask.shape[1:]) != (nb, nb) \
            or block_mask.shape[0] not in (1, H):
        raise ValueError(f"block_mask must be uint8 [1 or {H}, {nb}, {nb}]")
    if tuple(k.shape) != (B, N, Hkv, d) or tuple(v.shape) != (B, N, Hkv, d):
        raise ValueError("k and v must be [B,N,Hkv,d] matching q")
    _same_elem_type(q, (k, v, out), "q, k, v and out")
    if tuple(out.shape) != (B, N, H, d) or tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("out/lse have the wrong shape or type")
    _check(fa_fwd_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Hkv,
                               N, d, int(bool(causal)), block_mask.data_ptr(), block_mask.shape[0], scale, code,
                               _stream(q, stream)))
    return out, lse


def _same_elem_type(ref, others, what: str):
    """Every tensor in `others` has ref's element type (the kernels size every read from it)."""
    for t in others:
        if t.dtype != ref.dtype:
            raise ValueError(f"{what} must share one element type (got {ref.dtype} and {t.dtype})")


def _stream(t, stream):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream if stream is None else stream


def quantize_e4m3_block(x, signs=None, codes=None, scales=None, stream=None):
    """Block quantisation of a float16/bfloat16 device tensor x [B,N,Hx,d] to e4m3 with
    one power-of-two scale per FP8_BLOCK_ROWS positions of each (batch, head); with
    `signs` (float32 device tensor of d values +-1), rows are rotated by (x * signs) H
    first. Returns (codes uint8 [B,N,Hx,d], scales uint8 E8M0 [B,Hx,nb])."""
    import torch
    B, N, Hx, d = x.shape
    if x.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError(f"x must be float16 or bfloat16 (got {x.dtype})")
    code = {torch.float16: FA_DTYPE_F16, torch.bfloat16: FA_DTYPE_BF16}[x.dtype]
    nb = (N + FP8_BLOCK_ROWS - 1) // FP8_BLOCK_ROWS
    if codes is None:
        codes = torch.empty((B, N, Hx, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, Hx, nb), dtype=torch.uint8, device=x.device)
    for t in (x, codes, scales) + ((signs,) if signs is not None else ()):
        if not t.is_contiguous() or t.device != x.device:
            raise ValueError("tensors must be contiguous and on the same device")
    if tuple(codes.shape) != (B, N, Hx, d) or codes.dtype != torch.uint8 or tuple(scales.shape) != (B, Hx, nb):
        raise ValueError("codes/scales have the wrong shape or type")
    if signs is not None and (tuple(signs.shape) != (d,) or signs.dtype != torch.float32):
        raise ValueError("signs must be a float32 tensor of d values")
    _check(fa_quantize_e4m3_block(x.data_ptr(), code, B, N, Hx, d, signs.data_ptr() if signs is not None else 0,
                                  codes.data_ptr(), scales.data_ptr(), _stream(x, stream)))
    return codes, scales


def fwd_fp8_block(q, k, v, q_scales, k_scales, v_scales, causal: bool = False, scale: float | None = None,
                  out=None, lse=None, stream=None, qk_e4m3: bool = False):
    """Attention forward on block-quantised e4m3 inputs (uint8 code tensors q [B,N,H,d],
    k and v [B,N,Hkv,d], with their E8M0 block scales). qk_e4m3: Q K^T on the e4m3 MFMA,
    for Q and K rotated by quantize_e4m3_block with signs (else exact bf16 products).
    Returns (o bfloat16, lse)."""
    import torch
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    nb = (N + FP8_BLOCK_ROWS - 1) // FP8_BLOCK_ROWS
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    for t in (q, k, v, q_scales, k_scales, v_scales, out, lse):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError("tensors must be contiguous and on the same device")
    if tuple(k.shape) != (B, N, Hkv, d) or tuple(v.shape) != (B, N, Hkv, d):
        raise ValueError("k and v must be [B,N,Hkv,d] matching q")
    if (tuple(q_scales.shape) != (B, H, nb) or tuple(k_scales.shape) != (B, Hkv, nb)
            or tuple(v_scales.shape) != (B, Hkv, nb)):
        raise ValueError("block scales must be [B,H,nb] (q) and [B,Hkv,nb] (k, v)")
    for t in (q, k, v, q_scales, k_scales, v_scales):
        if t.dtype != torch.uint8:
            raise ValueError("codes and block scales must be uint8 tensors")
    if tuple(out.shape) != (B, N, H, d) or out.dtype != torch.bfloat16 or tuple(lse.shape) != (B, H, N) \
            or lse.dtype != torch.float32:
        raise ValueError("out/lse have the wrong shape or type")
    _check(fa_fwd_fp8_block(q.data_ptr(), k.data_ptr(), v.data_ptr(), q_scales.data_ptr(), k_scales.data_ptr(),
                            v_scales.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Hkv, N, d, int(bool(causal)),
                            scale, int(bool(qk_e4m3)), _stream(q, stream)))
    return out, lse


def bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, dq=None, dk=None, dv=None,
        workspace=None, stream=None):
    """Gradient of the attention forward on device tensors: q, o, dout [B,N,H,d], k, v
    [B,N,Hkv,d] (float16 or bfloat16), lse [B,H,N] float32 as returned by fwd. Returns
    (dq, dk, dv). The D workspace (B*H*N float32) is allocated here unless given."""
    import torch
    code = _dtype_code(q, None)
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    nbytes = fa_bwd_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    for t in (q, k, v, o, lse, dout, dq, dk, dv, workspace):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError("tensors must be contiguous and on the same device")
    for t in (o, dout, dq):
        if tuple(t.shape) != (B, N, H, d) or t.dtype != q.dtype:
            raise ValueError("o, dout and dq must match q")
    for t in (k, v, dk, dv):
        if tuple(t.shape) != (B, N, Hkv, d) or t.dtype != q.dtype:
            raise ValueError("k, v, dk and dv must be [B,N,Hkv,d] of q's type")
    if tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be [B,H,N] float32")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must hold at least {nbytes} bytes")
    _check(fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                  dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d, int(bool(causal)), scale, code,
                  workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(q, stream)))
    return dq, dk, dv


def fwd_splitkv_static(q, k, v, out, lse, causal: bool = False, scale: float | None = None, num_splits: int = 0,
                       stream=None):
    """fwd_splitkv into caller-provided out [B,Nq,H,d] and lse [B,H,Nq] with the library's
    static scratch instead of a workspace: allocates nothing (for graph capture and serving
    loops). Calls that overlap on one GPU race. Returns (out, lse)."""
    code = _dtype_code(q, None)
    B, Nq, H, d = q.shape
    Hkv = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    for t in (q, k, v, out, lse):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError("tensors must be contiguous and on the same device")
    if k.dim() != 4 or tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B,Nk,Hkv,d] matching q")
    _same_elem_type(q, (k, v, out), "q, k, v and out")
    if tuple(out.shape) != (B, Nq, H, d) or tuple(lse.shape) != (B, H, Nq) or str(lse.dtype) != "torch.float32":
        raise ValueError("out/lse have the wrong shape or type")
    _check(fa_fwd_splitkv_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Hkv,
                                 Nq, k.shape[1], d, int(bool(causal)), scale, code, num_splits, _stream(q, stream)))
    return out, lse


def fwd_splitkv(q, k, v, causal: bool = False, scale: float | None = None, num_splits: int = 0, out=None, lse=None,
                workspace=None, stream=None):
    """Split-KV decode forward on device tensors: q [B,Nq,H,d] are the last Nq positions of
    the sequence whose keys k, v [B,Nk,Hkv,d] cover all Nk positions. Returns (o, lse [B,H,Nq])."""
    import torch
    code = _dtype_code(q, None)
    B, Nq, H, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    nbytes = fa_fwd_splitkv_workspace_bytes(B, H, Hkv, Nq, Nk, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 4) // 4, dtype=torch.float32, device=q.device)
    for t in (q, k, v, out, lse, workspace):
        if not t.is_contiguous() or t.device != q.device:
            raise ValueError("tensors must be contiguous and on the same device")
    if k.dim() != 4 or tuple(v.shape) != tuple(k.shape) or k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must be [B,Nk,Hkv,d] matching q")
    _same_elem_type(q, (k, v, out), "q, k, v and out")
    if tuple(out.shape) != (B, Nq, H, d) or tuple(lse.shape) != (B, H, Nq) or lse.dtype != torch.float32:
        raise ValueError("out/lse have the wrong shape or type")
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must hold at least {nbytes} bytes")
    _check(fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Hkv, Nq, Nk,
                          d, int(bool(causal)), scale, code, num_splits, workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(), _stream(q, stream)))
    return out, lse
