"""The forward at the largest sizes the library accepts for its masks (GPU), on sampled
rows the oracle computes one by one.

* Dense causal GQA at N = 131072: 2048 key tiles per query tile, so the key offsets of
  the tile loop, the buffer extents (N rows of Hkv·d elements) and the longest-first
  schedule all run at a length far beyond the benchmarked ones.
* Block-sparse at N = 131072, the largest length whose mask row (2048 blocks of 64)
  fits the per-workgroup list, with a shared and a per-head mask, causal and not.
Tolerances as in the parity tests (bf16: |dO| <= 1e-2 max(1, |O_ref|), |dlse| <= 1e-3)."""
import sys

import numpy as np
import pytest
import torch

import exact_tiled_attention_03_amd as fa
import oracle
import synth_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

N_MAX = 131072


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rows(B, H, N, seed):
    rows = gu.sample_rows(B, H, N, n_random=24, seed=seed)
    extra = [(0, h, i) for h in range(H) for i in (N - 64, N - 65, N - 256, 65535, 65536)]
    return np.concatenate([rows, np.array(extra, dtype=np.int64)])


def _check(o, lse, inp, rows, causal, scale, mask, what):
    if mask is None:
        o_ref, lse_ref = oracle.attn_rows(inp["q"], inp["k"], inp["v"], "bf16", causal, scale, rows)
    else:
        o_ref, lse_ref = oracle.attn_rows_block(inp["q"], inp["k"], inp["v"], "bf16", causal, scale, rows, mask)
    o_g = o[rows[:, 0], rows[:, 2], rows[:, 1]].float().cpu().numpy().astype(np.float64)
    l_g = lse[rows[:, 0], rows[:, 1], rows[:, 2]].cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l_g), empty), f"{what}: rows with lse = -inf differ"
    assert np.all(o_g[empty] == 0.0), f"{what}: a row with no visible key is not zero"
    e = gu.compare(o_g[~empty], o_ref[~empty], l_g[~empty], lse_ref[~empty], "bf16", what)
    _log(f"[limits] {what}: max scaled dO {e[0]:.2e}, max dlse {e[2]:.2e}")


def test_dense_causal_gqa_at_131072():
    B, H, Hkv, N, d = 1, 4, 1, N_MAX, 128
    _log(f"[limits] dense causal B{B} H{H}/{Hkv} N{N} d{d}")
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, "bf16", seed=4100)
    scale = 1.0 / np.sqrt(d)
    o, lse = gu.run(inp, "bf16", True, scale)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(lse).all())
    _check(o, lse, inp, _rows(B, H, N, 4101), True, scale, None, "dense causal N=131072")


@pytest.mark.parametrize("causal,mask_heads", [(False, 1), (True, 2)])
def test_block_sparse_at_131072(causal, mask_heads):
    B, H, Hkv, N, d = 1, 2, 1, N_MAX, 128
    _log(f"[limits] block sparse causal={causal} mask_heads={mask_heads} N{N}")
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, "bf16", seed=4200)
    mask = synth_inputs.random_block_mask(mask_heads, N, 0.03, seed=4201 + mask_heads)
    assert mask.shape[1] == 2048
    mask[:, :, -1] = 1          # the last key block stays in every list (the list's last entry)
    scale = 1.0 / np.sqrt(d)
    q, k, v = (gu.to_dev(inp[x], "bf16") for x in "qkv")
    o, lse = fa.fwd_block_sparse(q, k, v, torch.from_numpy(mask).cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    _check(o, lse, inp, _rows(B, H, N, 4202), causal, scale, mask, f"block sparse N=131072 causal={causal}")
