"""Gradient of the attention forward (fa_bwd) against the fp64 oracle's analytic gradient
on the same seeded inputs (GPU). The forward's o and lse come from fa_fwd on the GPU, as
in training; the oracle differentiates its own exact forward. Bound, per element: twice
the rounding bound derived in gpu_util.bwd_error_bound (storage-type rounding of P, dS and
the outputs, and of O inside D = <dO, O>), plus 1e-5 for float32 accumulation."""
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


def _run(case, seed):
    dtype, B, H, Hkv, N, d, causal = case
    scale = 1.0 / np.sqrt(d)
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, dtype, seed=seed)
    dout = synth_inputs.make_dout(B, N, H, d, dtype, seed=seed + 7)
    q, k, v = (gu.to_dev(inp[x], dtype) for x in "qkv")
    do = gu.to_dev(dout, dtype)
    o, lse = fa.fwd(q, k, v, causal=causal, scale=scale)
    grads = fa.bwd(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    bounds, ref = gu.bwd_error_bound(*(oracle.decode(inp[x], dtype) for x in "qkv"), oracle.decode(dout, dtype),
                                     causal, scale, dtype)
    return grads, ref, bounds


def _check(grads, ref, bounds, what):
    ratios = []
    for g, r, bd, name in zip(grads, ref, bounds, ("dq", "dk", "dv")):
        g = g.float().cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        err = np.abs(g - r)
        lim = 2.0 * bd + 1e-5
        ratio = float(np.max(err / lim)) if r.size else 0.0
        ratios.append(ratio)
        assert ratio <= 1.0, (f"{what} {name}: {int((err > lim).sum())} elements over the bound, max err/bound "
                              f"{ratio:.2f}, max |dg| {err.max():.3e}")
    return ratios


CASES = [
    # dtype, B, H, Hkv, N, d, causal
    ("bf16", 1, 2, 2, 128, 128, False),
    ("bf16", 1, 2, 2, 128, 128, True),
    ("bf16", 2, 4, 2, 300, 128, False),
    ("bf16", 2, 4, 2, 300, 128, True),
    ("f16", 1, 2, 2, 257, 128, True),
    ("f16", 1, 3, 1, 200, 64, False),
    ("bf16", 1, 4, 1, 333, 64, True),
    ("bf16", 1, 8, 2, 1024, 128, True),
    ("bf16", 1, 2, 2, 640, 64, False),
] + [("bf16", 1, 2, 2, n, d, c) for n in (1, 3, 17, 64, 65, 129) for d in (64, 128) for c in (False, True)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_bwd_parity(case):
    _log(f"[bwd] {case}")
    grads, ref, bounds = _run(case, seed=600 + case[4] + case[5])
    e = _check(grads, ref, bounds, str(case))
    _log(f"[bwd] {case}: err/bound dq {e[0]:.2f} dk {e[1]:.2f} dv {e[2]:.2f}")


def test_bwd_deterministic():
    case = ("bf16", 2, 4, 2, 300, 128, True)
    dtype, B, H, Hkv, N, d, causal = case
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, dtype, seed=5)
    q, k, v = (gu.to_dev(inp[x], dtype) for x in "qkv")
    do = gu.to_dev(synth_inputs.make_dout(B, N, H, d, dtype, seed=6), dtype)
    o, lse = fa.fwd(q, k, v, causal=causal)
    g1 = fa.bwd(q, k, v, o, lse, do, causal=causal)
    g2 = fa.bwd(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_bwd_gqa_equals_repeated_heads():
    """dK, dV of a shared K/V head equal the sums over its query heads of the gradients
    with K and V repeated per head (up to rounding of the per-head terms)."""
    dtype, B, H, Hkv, N, d = "bf16", 1, 4, 2, 200, 128
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, dtype, seed=9)
    q, k, v = (gu.to_dev(inp[x], dtype) for x in "qkv")
    do = gu.to_dev(synth_inputs.make_dout(B, N, H, d, dtype, seed=10), dtype)
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    kr = k.repeat_interleave(H // Hkv, dim=2).contiguous()
    vr = v.repeat_interleave(H // Hkv, dim=2).contiguous()
    o2, lse2 = fa.fwd(q, kr, vr, causal=True)
    dq2, dk2, dv2 = fa.bwd(q, kr, vr, o2, lse2, do, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq.view(torch.int16), dq2.view(torch.int16)), "dq is per query head"
    for g, g2 in ((dk, dk2), (dv, dv2)):
        s2 = g2.float().view(B, N, Hkv, H // Hkv, d).sum(dim=3)
        err = (g.float() - s2).abs().max().item()
        assert err <= 2e-2 * (s2.abs().max().item() + 1e-6), err


def _row_bounds(q, k, v, dout, rows, causal, scale, dtype):
    """The bound of gpu_util.bwd_error_bound for dq of single rows (b, h, i), in numpy."""
    u = gu.UNIT_ROUNDOFF[dtype]
    H, Hkv = q.shape[2], k.shape[2]
    out = []
    for b, h, i in rows:
        hk = h // (H // Hkv)
        n = i + 1 if causal else k.shape[1]
        K, V = k[b, :n, hk], v[b, :n, hk]
        s_ = scale * (K @ q[b, i, h])
        p = np.exp(s_ - s_.max())
        p /= p.sum()
        dp = V @ dout[b, i, h]
        o = p @ V
        ds = p * (dp - p @ dp)
        dD = u * np.sum(np.abs(dout[b, i, h]) * np.abs(o))
        out.append(scale * (u * np.abs(ds) @ np.abs(K) + dD * (p @ np.abs(K))))
    return np.array(out)


@pytest.mark.parametrize("name", [n for n, w in synth_inputs.WORKLOADS.items() if w.backward])
def test_bwd_workload_full_size(name):
    """The gradient workloads at full size, in the launch configuration the benchmark
    times: whole (batch, head) slices against the oracle for the multi-head shape; for the
    causal grouped-query shape, dq on sampled rows and, over all positions, the exact
    identities sum_j dk_j = 0 and sum_j dv_j = sum over the group of sum_i dO_i."""
    w = synth_inputs.WORKLOADS[name]
    _log(f"[bwd workload] {name}")
    inp = synth_inputs.workload_inputs(w)
    dout = synth_inputs.make_dout(w.B, w.N, w.H, w.d, w.dtype, w.seed + 100)
    q, k, v = (gu.to_dev(inp[x], w.dtype) for x in "qkv")
    do = gu.to_dev(dout, w.dtype)
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t.float()).all())
    g = w.H // w.Hkv
    if not w.causal and g == 1:
        for b, h in ((0, 0), (w.B - 1, w.H - 1)):
            sl = lambda a: np.ascontiguousarray(oracle.decode(a[b:b + 1, :, h:h + 1], w.dtype))
            bounds, ref = gu.bwd_error_bound(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(dout), w.causal, w.scale,
                                             w.dtype)
            got = [t[b:b + 1, :, h:h + 1] for t in (dq, dk, dv)]
            e = _check(got, ref, bounds, f"{name} b{b} h{h}")
            _log(f"[bwd workload] b{b} h{h}: err/bound dq {e[0]:.2f} dk {e[1]:.2f} dv {e[2]:.2f}")
        return
    rows = gu.sample_rows(w.B, w.H, w.N, n_random=24, seed=w.seed)
    qd, kd, vd, dd = (oracle.decode(a, w.dtype) for a in (inp["q"], inp["k"], inp["v"], dout))
    ref = oracle.attn_bwd_dq_rows_f64(qd, kd, vd, dd, w.causal, w.scale, rows)
    bound = _row_bounds(qd, kd, vd, dd, rows, w.causal, w.scale, w.dtype)
    got = dq[rows[:, 0], rows[:, 2], rows[:, 1]].float().cpu().numpy().astype(np.float64)
    ratio = float(np.max(np.abs(got - ref) / (2 * bound + 1e-5)))
    _log(f"[bwd workload] dq sampled rows: err/bound {ratio:.2f}")
    assert ratio <= 1.0
    dkf, dvf = dk.double(), dv.double()
    sk = dkf.sum(dim=1).abs().max().item()
    assert sk <= 2e-2 * dkf.abs().sum(dim=1).max().item(), f"sum_j dk_j = {sk:.3e}"
    dos = do.double().view(w.B, w.N, w.Hkv, g, w.d).sum(dim=(1, 3))
    sv = (dvf.sum(dim=1) - dos).abs().max().item()
    assert sv <= 2e-2 * dvf.abs().sum(dim=1).max().item(), f"sum_j dv_j - sum_i dO_i = {sv:.3e}"
    _log(f"[bwd workload] |sum dk| {sk:.2e}, |sum dv - sum dO| {sv:.2e}")
