"""Block-sparse attention through fa_fwd_block_sparse, against the fp64 oracle on the same
seeded inputs (GPU). The reading of the block-sparse variant named in the abstract of
"FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness": key j is
visible to query i of head h iff mask[hm, i // 64, j // 64] != 0 (hm = 0 for a shared
mask, else h), and j <= i under the causal flag; a row with no visible key gives O = 0
and lse = -inf. Random masks at 64-block granularity make the four 64-row query blocks
of a 256-query tile disagree, so one wavefront keeps a key tile that the other keeps
not; shapes span several tiles with ragged tails. Tolerances as in the dense parity
tests; rows with no visible key are compared exactly."""
import sys

import numpy as np
import pytest
import torch

import exact_tiled_attention_03_amd as fa
import oracle
import synth_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(inp, dtype, causal, scale, mask):
    q, k, v = (gu.to_dev(inp[x], dtype) for x in "qkv")
    m = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).cuda()
    o, lse = fa.fwd_block_sparse(q, k, v, m, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def _compare(o, o_ref, lse, lse_ref, dtype, what):
    """o [B,N,H,d] and lse [B,H,N]: rows with lse_ref = -inf must be exactly (0, -inf);
    the others are held to the dense parity bound."""
    o, o_ref = o.transpose(0, 2, 1, 3), o_ref.transpose(0, 2, 1, 3)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: rows with lse = -inf differ"
    assert np.all(o[empty] == 0.0), f"{what}: a row with no visible key is not zero"
    keep = ~empty
    return gu.compare(o[keep], o_ref[keep], lse[keep], lse_ref[keep], dtype, what)


CASES = [
    # dtype, B, H, Hkv, N, d, causal, mask_heads, kept share
    ("bf16", 1, 4, 2, 1000, 128, False, 1, 0.3),
    ("bf16", 1, 4, 2, 1000, 128, False, 4, 0.6),
    ("bf16", 1, 4, 2, 1000, 128, True, 4, 0.5),
    ("bf16", 2, 2, 2, 777, 128, True, 1, 0.3),
    ("bf16", 1, 2, 2, 1500, 128, False, 2, 0.1),
    ("bf16", 1, 8, 2, 2100, 64, True, 8, 0.2),
    ("bf16", 1, 2, 2, 65, 128, False, 2, 0.5),
    ("bf16", 1, 2, 2, 1, 128, False, 1, 1.0),
    ("bf16", 1, 2, 2, 300, 128, False, 2, 0.0),          # nothing kept: every row empty
    ("f16", 1, 3, 1, 700, 64, False, 3, 0.4),
    ("f16", 1, 2, 2, 513, 128, True, 2, 0.7),
    ("f16", 2, 4, 4, 256, 128, False, 1, 0.5),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_block_sparse_parity(case):
    dtype, B, H, Hkv, N, d, causal, heads, share = case
    _log(f"[block sparse] {case}")
    scale = 1.0 / np.sqrt(d)
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, dtype, seed=1200 + N + d + H)
    mask = synth_inputs.random_block_mask(heads, N, share, seed=1300 + N + heads)
    o, lse = gu.host(*_run(inp, dtype, causal, scale, mask))
    o_ref, lse_ref = oracle.attn_fwd_block(inp["q"], inp["k"], inp["v"], dtype, causal, scale, mask)
    _compare(o, o_ref, lse, lse_ref, dtype, str(case))


def test_empty_rows_under_the_causal_mask():
    """Query blocks that keep only key blocks after themselves see nothing under the
    causal mask (O = 0, lse = -inf); their neighbours keep the diagonal block."""
    B, H, Hkv, N, d = 1, 2, 2, 600, 128
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, "bf16", seed=77)
    nb = (N + 63) // 64
    mask = np.zeros((H, nb, nb), np.uint8)
    for qb in range(nb):
        if qb % 2:
            mask[:, qb, qb + 1:] = 1          # only later keys: empty under the mask
        else:
            mask[:, qb, qb] = 1
    o, lse = gu.host(*_run(inp, "bf16", True, 0.1, mask))
    o_ref, lse_ref = oracle.attn_fwd_block(inp["q"], inp["k"], inp["v"], "bf16", True, 0.1, mask)
    assert np.isneginf(lse_ref).any() and np.isfinite(lse_ref).any()
    _compare(o, o_ref, lse, lse_ref, "bf16", "empty rows under the causal mask")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_full_masks_are_the_dense_kernels(dtype):
    """A mask that keeps every block, and (with the causal flag) a lower-triangular block
    mask, visit the same key tiles in the same order as fa_fwd, so they agree with it
    bit for bit."""
    B, H, Hkv, N, d = 1, 4, 2, 1000, 128
    _log(f"[block sparse = dense] {dtype}")
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, dtype, seed=91)
    nb = (N + 63) // 64
    for causal, mask, what in ((False, np.ones((1, nb, nb), np.uint8), "all blocks = fa_fwd"),
                               (True, np.ones((H, nb, nb), np.uint8), "all blocks + causal = causal fa_fwd"),
                               (True, np.tril(np.ones((nb, nb), np.uint8))[None], "lower blocks + causal")):
        ref = gu.run(inp, dtype, causal, 0.1)
        o, lse = _run(inp, dtype, causal, 0.1, mask)
        assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16)), what
        assert torch.equal(lse, ref[1]), what


def test_block_sparse_workload_full_size():
    """The benchmark's block-sparse workload at full size (B1 H16 N16384 d128, one mask
    per head) in the launch configuration bench.py times, over every output element."""
    w = synth_inputs.WORKLOADS["block_sparse_bf16_b1_h16_n16384_d128"]
    _log(f"[block sparse workload] {w.name}")
    inp = synth_inputs.workload_inputs(w)
    mask = synth_inputs.workload_block_mask(w)
    o, lse = gu.host(*_run(inp, w.dtype, w.causal, w.scale, mask))
    o_ref, lse_ref = oracle.attn_fwd_block(inp["q"], inp["k"], inp["v"], w.dtype, w.causal, w.scale, mask)
    e = _compare(o, o_ref, lse, lse_ref, w.dtype, w.name)
    _log(f"[block sparse workload] every element: max scaled dO {e[0]:.2e}, max |dO| {e[1]:.2e}, "
         f"max dlse {e[2]:.2e}")
