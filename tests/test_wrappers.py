"""Host-side argument checks of the Python binding (CPU only, no kernel launch): every
wrapper rejects mismatched shapes and element types with ValueError before it reaches the
library, because the kernels size every read from q's element type and the claimed sizes."""
import pytest
import torch

import exact_tiled_attention_03_amd as fa

B, N, H, HKV, D = 1, 64, 4, 2, 64


def t(shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def qkv(dtype=torch.bfloat16, k_shape=None, v_shape=None, k_dtype=None, v_dtype=None):
    q = t((B, N, H, D), dtype)
    k = t(k_shape or (B, N, HKV, D), k_dtype or dtype)
    v = t(v_shape or (B, N, HKV, D), v_dtype or dtype)
    return q, k, v


@pytest.mark.parametrize("kw", [
    dict(k_shape=(B, N - 1, HKV, D)),                  # shorter k
    dict(v_shape=(B, N, HKV, D // 2)),                 # narrower v
    dict(k_dtype=torch.float16),                       # 2-byte k of another type
    dict(k_dtype=torch.uint8),                         # 1-byte k with a 2-byte q
    dict(v_dtype=torch.float32),
])
def test_fwd_rejects_mismatched_kv(kw):
    with pytest.raises(ValueError):
        fa.fwd(*qkv(**kw))


def test_fwd_rejects_unknown_types():
    with pytest.raises(ValueError):
        fa.fwd(*qkv(torch.float32))
    with pytest.raises(ValueError):
        fa.fwd(*qkv(torch.float16), dtype="bf16")     # dtype string disagrees with the tensors
    with pytest.raises(ValueError):
        fa.fwd(*qkv(torch.bfloat16), dtype="e4m3", descale=(1.0, 1.0, 1.0))   # 2-byte codes
    with pytest.raises(ValueError):
        fa.fwd(*qkv(torch.bfloat16), dtype="fp4")


def test_fwd_rejects_bad_outputs():
    q, k, v = qkv()
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, out=t((B, N, H, D), torch.float16))
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, lse=t((B, H, N), torch.float16))
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, lse=t((B, N, H), torch.float32))


def test_block_sparse_rejects_mismatches():
    nb = (N + 63) // 64
    mask = torch.ones((1, nb, nb), dtype=torch.uint8)
    for kw in (dict(k_shape=(B, N, HKV + 1, D)), dict(k_dtype=torch.float16), dict(v_dtype=torch.uint8)):
        with pytest.raises(ValueError):
            fa.fwd_block_sparse(*qkv(**kw), mask)
    q, k, v = qkv()
    with pytest.raises(ValueError):
        fa.fwd_block_sparse(q, k, v, mask, out=t((B, N, H, D), torch.float16))
    with pytest.raises(ValueError):
        fa.fwd_block_sparse(q, k, v, mask.to(torch.int32))


def test_fp8_block_rejects_mismatches():
    nb = (N + 63) // 64
    q, k, v = qkv(torch.uint8)
    qs, ks, vs = t((B, H, nb), torch.uint8), t((B, HKV, nb), torch.uint8), t((B, HKV, nb), torch.uint8)
    with pytest.raises(ValueError):
        fa.fwd_fp8_block(q, t((B, N, HKV, D), torch.bfloat16), v, qs, ks, vs)
    with pytest.raises(ValueError):
        fa.fwd_fp8_block(q, k, v, qs, ks.to(torch.int16), vs)
    with pytest.raises(ValueError):
        fa.fwd_fp8_block(q, t((B, N - 1, HKV, D), torch.uint8), v, qs, ks, vs)
    with pytest.raises(ValueError):
        fa.fwd_fp8_block(q, k, v, qs, ks, vs, lse=t((B, H, N), torch.float16))


def test_bwd_rejects_mismatched_k():
    q, k, v = qkv()
    o, do = t((B, N, H, D)), t((B, N, H, D))
    lse = t((B, H, N), torch.float32)
    with pytest.raises(ValueError):
        fa.bwd(q, t((B, N - 1, HKV, D)), v, o, lse, do)           # shorter k
    with pytest.raises(ValueError):
        fa.bwd(q, t((B, N, HKV, D), torch.float16), v, o, lse, do)
    with pytest.raises(ValueError):
        fa.bwd(q, k, v, o, lse, do, workspace=t((1,), torch.float32))   # workspace too small


def test_splitkv_rejects_mismatches():
    q = t((B, 1, H, D))
    k = t((B, N, HKV, D))
    with pytest.raises(ValueError):
        fa.fwd_splitkv(q, k.to(torch.float16), k.to(torch.float16))
    with pytest.raises(ValueError):
        fa.fwd_splitkv(q, k, t((B, N - 1, HKV, D)))
    with pytest.raises(ValueError):
        fa.fwd_splitkv(q, k, k, workspace=t((1,), torch.float32))


def test_quantize_rejects_types():
    with pytest.raises(ValueError):
        fa.quantize_e4m3_block(t((B, N, H, D), torch.float32))
