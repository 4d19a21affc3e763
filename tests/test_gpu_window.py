"""Key-window (sliding-window / local) attention through fa_fwd_local, against the fp64
oracle on the same seeded inputs (GPU). Key j is visible to query i iff
i - left <= j <= i + right (negative side: unbounded), intersected with the causal mask;
this is the reading of the sliding-window patterns that the page "FlashAttention: The
Algorithm That Made Long-Context AI Possible" names (section "Why context lengths exploded
after 2022"). Shapes span several 256-query and 64-key tiles with ragged tails; windows
are placed on both sides of tile boundaries, narrower than a wavefront's 32 queries and
wider than the sequence. Tolerances as in the unwindowed parity tests."""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


CASES = [
    # dtype, B, H, Hkv, N, d, causal, (left, right)
    ("bf16", 1, 4, 2, 1000, 128, True, (255, -1)),
    ("bf16", 1, 4, 2, 1000, 128, True, (256, -1)),
    ("bf16", 1, 2, 2, 1000, 128, True, (63, -1)),
    ("bf16", 1, 2, 2, 1000, 128, True, (64, -1)),
    ("bf16", 1, 2, 2, 700, 128, True, (0, -1)),
    ("bf16", 1, 2, 2, 700, 128, True, (5, 9)),            # right bound under the mask: no effect
    ("bf16", 2, 4, 2, 900, 128, False, (100, 100)),
    ("bf16", 1, 2, 1, 900, 128, False, (0, 0)),
    ("bf16", 1, 2, 2, 900, 128, False, (300, 5)),
    ("bf16", 1, 2, 2, 900, 128, False, (5, 300)),
    ("bf16", 1, 2, 2, 900, 128, False, (-1, 70)),
    ("bf16", 1, 2, 2, 900, 128, False, (70, -1)),
    ("bf16", 1, 2, 2, 900, 128, False, (17, 31)),
    ("bf16", 1, 8, 2, 1500, 128, True, (511, -1)),
    ("f16", 1, 3, 1, 777, 64, False, (129, 33)),
    ("f16", 1, 2, 2, 777, 64, True, (200, -1)),
    ("f16", 2, 2, 2, 513, 128, False, (1, 1)),
    ("bf16", 1, 2, 2, 333, 64, False, (400, 400)),        # wider than the sequence
    ("bf16", 1, 2, 2, 1, 128, True, (3, -1)),
    ("bf16", 1, 2, 2, 2, 128, False, (0, 0)),
    ("bf16", 1, 2, 2, 3, 64, False, (1, 0)),
    ("bf16", 1, 2, 2, 129, 128, False, (0, 64)),
    # windows wide enough that workgroups have a masked left edge, a range of tiles inside
    # every query's band (the unmasked step body) and a masked right edge or diagonal
    ("bf16", 1, 2, 2, 1300, 128, False, (300, 300)),
    ("bf16", 1, 2, 1, 1217, 128, True, (700, -1)),
    ("f16", 1, 2, 1, 1100, 64, True, (700, -1)),
    ("f16", 1, 2, 2, 1000, 128, False, (450, 200)),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)).replace(" ", ""))
def test_window_full_parity(case):
    dtype, B, H, Hkv, N, d, causal, window = case
    _log(f"[window] {case}")
    scale = 1.0 / np.sqrt(d)
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, dtype, seed=900 + N + d + H + window[0])
    o, lse = gu.host(*gu.run(inp, dtype, causal, scale, window))
    o_ref, lse_ref = oracle.attn_fwd(inp["q"], inp["k"], inp["v"], dtype, causal, scale, window=window)
    gu.compare(o, o_ref, lse, lse_ref, dtype, str(case))


FP8_CASES = [
    # B, H, Hkv, N, d, causal, window
    (1, 2, 2, 700, 128, True, (200, -1)),
    (1, 2, 1, 600, 128, False, (64, 64)),
    (1, 2, 2, 333, 64, False, (0, 40)),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "-".join(map(str, c)).replace(" ", ""))
def test_window_fp8_parity(case):
    B, H, Hkv, N, d, causal, window = case
    _log(f"[window fp8] {case}")
    scale = 1.0 / np.sqrt(d)
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, "e4m3", seed=950 + N, outlier_frac=1e-3)
    o, lse = gu.host(*gu.run(inp, "e4m3", causal, scale, window))
    o_ref, lse_ref = oracle.attn_fwd(inp["q"], inp["k"], inp["v"], "e4m3", causal, scale, inp["descale"],
                                     window=window)
    bound = gu.fp8_quantization_bound(inp, causal, scale, o_ref, window)
    few = gu.fp8_exempt_elements(*(oracle.decode(inp[x], "e4m3", s_) for x, s_ in zip("qkv", inp["descale"])), causal,
                             scale, o_ref, window)
    e = gu.compare(o, o_ref, lse, lse_ref, "e4m3", str(case), extra_bound=bound, extra_rows=few)
    _log(f"[window fp8] {case}: {e[3]} of {o.size} elements within the derived bound only "
         f"({int(few.sum())} elements outside the stated regime)")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "e4m3"])
def test_unbounded_windows_are_the_unwindowed_kernels(dtype):
    """(-1, -1) is fa_fwd itself, (-1, 0) without the flag is the causal mask, and a
    window that reaches every key (left = N - 1, which runs the band kernel) repeats the
    unmasked kernel's arithmetic tile for tile: all three agree bit for bit."""
    B, H, Hkv, N, d = 1, 4, 2, 700, 128
    _log(f"[window reductions] {dtype}")
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, dtype, seed=31)
    full = gu.run(inp, dtype, False, 0.1)
    causal = gu.run(inp, dtype, True, 0.1)
    for window, ref, what in (((-1, -1), full, "(-1,-1) = fa_fwd"), ((-1, 0), causal, "(-1,0) = causal"),
                              ((N - 1, N - 1), full, "band covering everything = full"),
                              ((N - 1, -1), full, "band, left side only, covering everything = full")):
        o, lse = gu.run(inp, dtype, False, 0.1, window)
        assert torch.equal(o.view(torch.int16) if o.dtype != torch.float32 else o,
                           ref[0].view(torch.int16) if ref[0].dtype != torch.float32 else ref[0]), what
        assert torch.equal(lse, ref[1]), what


def test_zero_query_gives_local_means():
    """Q = 0: each row is the mean of the V rows inside its window, lse = ln(count)."""
    B, N, H, Hkv, d = 1, 1100, 2, 1, 128
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, "bf16", seed=79)
    inp["q"] = np.zeros_like(inp["q"])
    v = oracle.decode(inp["v"], "bf16")[0, :, 0, :]
    csum = np.concatenate([np.zeros((1, d)), np.cumsum(v, axis=0)])
    for causal, (left, right) in ((True, (300, -1)), (False, (40, 90))):
        o, lse = gu.host(*gu.run(inp, "bf16", causal, 0.1, (left, right)))
        i = np.arange(N)
        lo = np.maximum(0, i - left)
        hi = i if causal else np.minimum(N - 1, i + right)
        cnt = hi - lo + 1
        ref = (csum[hi + 1] - csum[lo]) / cnt[:, None]
        for h in range(H):
            gu.compare(o[0, :, h, :], ref, lse[0, h], np.log(cnt), "bf16", f"Q=0 window causal={causal}")
