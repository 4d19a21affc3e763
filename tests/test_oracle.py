"""The oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
import synth_inputs
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=[p.__name__ for p in pins.ALL_PINS])
def test_pin(pin):
    pin()


def test_rows_match_full_forward():
    rng = np.random.default_rng(5)
    for causal in (False, True):
        B, N, H, Hkv, d = 2, 45, 4, 2, 16
        q = rng.standard_normal((B, N, H, d))
        k = rng.standard_normal((B, N, Hkv, d))
        v = rng.standard_normal((B, N, Hkv, d))
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.25)
        rows = np.array([[0, 0, 0], [1, 3, 44], [0, 2, 17], [1, 1, 1]])
        orow, lrow = oracle.attn_rows_f64(q[rows[:, 0], rows[:, 2], rows[:, 1]], k, v, H, rows, causal, 0.25)
        for r, (b, h, i) in enumerate(rows):
            assert np.array_equal(orow[r], o[b, i, h]) and lrow[r] == lse[b, h, i]


def test_stored_input_entry_decodes_like_manual():
    inp = synth_inputs.make_inputs(1, 2, 1, 16, 8, "bf16", 7)
    o, lse = oracle.attn_fwd(inp["q"], inp["k"], inp["v"], "bf16", True, 0.3)
    q, k, v = (oracle.decode(inp[x], "bf16") for x in "qkv")
    o2, lse2 = oracle.attn_fwd_f64(q, k, v, True, 0.3)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    e = synth_inputs.make_inputs(1, 2, 2, 16, 8, "e4m3", 8, outlier_frac=0.05)
    o, lse = oracle.attn_fwd(e["q"], e["k"], e["v"], "e4m3", False, 0.3, e["descale"])
    q, k, v = (oracle.decode(e[x], "e4m3", s) for x, s in zip("qkv", e["descale"]))
    o2, lse2 = oracle.attn_fwd_f64(q, k, v, False, 0.3)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_oracle_rejects_bad_shapes():
    q = np.zeros((1, 4, 3, 8)); k = np.zeros((1, 4, 2, 8))
    with pytest.raises(ValueError):
        oracle.attn_fwd_f64(q, k, k, False, 1.0)   # H % Hkv != 0


def test_bwd_dq_rows_match_full_gradient():
    rng = np.random.default_rng(6)
    for causal in (False, True):
        B, N, H, Hkv, d = 2, 33, 4, 2, 8
        q, k, v, g = (rng.standard_normal(s) for s in ((B, N, H, d), (B, N, Hkv, d), (B, N, Hkv, d), (B, N, H, d)))
        dq, _, _ = oracle.attn_bwd_f64(q, k, v, g, causal, 0.4)
        rows = np.array([[0, 0, 0], [1, 3, 32], [0, 2, 17], [1, 1, 5]])
        dqr = oracle.attn_bwd_dq_rows_f64(q, k, v, g, causal, 0.4, rows)
        for r, (b, h, i) in enumerate(rows):
            assert np.allclose(dqr[r], dq[b, i, h], rtol=1e-13, atol=1e-15)
