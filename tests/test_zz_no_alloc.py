"""fa_fwd_splitkv_static (no workspace argument, no allocation: the library's per-GPU
static scratch) against fa_fwd_splitkv with a caller workspace, through the C ABI: two
calls in a row, the second with a smaller input, each bit-identical to the workspace
entry point on the same inputs and within the bf16 tolerance of the fp64 oracle."""
import sys

import numpy as np
import pytest
import torch

import exact_tiled_attention_03_amd as fa
import oracle
import synth_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # B, H, Hkv, Nq, Nk, d, causal, num_splits (0: the library's plan)
    (4, 32, 8, 1, 16384, 128, False, 0),
    (2, 8, 2, 3, 700, 64, True, 5),
]


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _call_both(case, seed):
    B, H, Hkv, Nq, Nk, d, causal, splits = case
    inp = synth_inputs.make_decode_inputs(B, H, Hkv, Nq, Nk, d, "bf16", seed)
    q, k, v = (gu.to_dev(inp[x], "bf16") for x in "qkv")
    scale = 1.0 / np.sqrt(d)
    o_ref = torch.empty_like(q)
    lse_ref = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    nbytes = fa.fa_fwd_splitkv_workspace_bytes(B, H, Hkv, Nq, Nk, d, splits)
    assert 0 < nbytes <= fa.SPLITKV_STATIC_SCRATCH_BYTES
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream().cuda_stream
    st = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ref.data_ptr(), lse_ref.data_ptr(), B, H,
                           Hkv, Nq, Nk, d, int(causal), scale, fa.FA_DTYPE_BF16, splits, ws.data_ptr(), nbytes, stream)
    assert st == fa.FA_OK, fa.status_string(st)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=q.device)
    st = fa.fa_fwd_splitkv_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Hkv,
                                  Nq, Nk, d, int(causal), scale, fa.FA_DTYPE_BF16, splits, stream)
    assert st == fa.FA_OK, fa.status_string(st)
    torch.cuda.synchronize()
    return inp, (o, lse), (o_ref, lse_ref), scale


def test_static_scratch_matches_workspace_entry_point_twice():
    for n, case in enumerate(CASES):
        _log(f"[no-alloc] call {n + 1}: {case}")
        inp, (o, lse), (o_ref, lse_ref), scale = _call_both(case, seed=1700 + n)
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), f"call {n + 1}: o differs"
        assert torch.equal(lse, lse_ref), f"call {n + 1}: lse differs"
        causal = case[6]
        ro, rl = oracle.attn_fwd_kv_f64(*(oracle.decode(inp[x], "bf16") for x in "qkv"), causal, scale)
        e = gu.compare(*gu.host(o, lse)[:1], ro, gu.host(o, lse)[1], rl, "bf16", f"no-alloc call {n + 1}")
        _log(f"[no-alloc] call {n + 1}: bit-identical to fa_fwd_splitkv; max scaled dO vs oracle {e[0]:.2e}, "
             f"max dlse {e[2]:.2e}")


def test_static_scratch_refuses_oversized_requests():
    q = torch.zeros((1, 1, 32, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1 << 17, 8, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((1, 32, 1), dtype=torch.float32, device="cuda")
    st = fa.fa_fwd_splitkv_static(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 32, 8,
                                  1, 1 << 17, 128, 0, 0.088, fa.FA_DTYPE_BF16, 4096, 0)
    assert st == fa.FA_ERR_SCRATCH
