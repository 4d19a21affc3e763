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


def _unit_forward(qd, kd, vd, causal, scale, units):
    """The oracle's forward (o, lse) on the query heads of the (b, kv-head) units, placed in
    full-size arrays (zeros elsewhere; only those rows are read)."""
    B, N, H, d = qd.shape
    g = H // kd.shape[2]
    o = np.zeros_like(qd)
    lse = np.zeros((B, H, N))
    for b, hk in units:
        hs = slice(hk * g, (hk + 1) * g)
        ou, lu = oracle.attn_fwd_f64(np.ascontiguousarray(qd[b:b + 1, :, hs]), np.ascontiguousarray(kd[b:b + 1, :, hk:hk + 1]),
                                     np.ascontiguousarray(vd[b:b + 1, :, hk:hk + 1]), causal, scale)
        o[b, :, hs], lse[b, hs] = ou[0], lu[0]
    return o, lse


def _check_rows(name, got, ref, bound):
    err = np.abs(got - ref)
    lim = 2.0 * bound + 1e-5
    ratio = float(np.max(err / lim)) if ref.size else 0.0
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    assert ratio <= 1.0, f"{name}: {int((err > lim).sum())} elements over the bound, max err/bound {ratio:.2f}"
    return ratio


@pytest.mark.parametrize("name", [n for n, w in synth_inputs.WORKLOADS.items() if w.backward])
def test_bwd_workload_full_size(name):
    """The gradient workloads at full size, in the launch configuration the benchmark
    times, element by element against the oracle within twice the derived rounding bound
    (gpu_util.bwd_error_bound, from the oracle's absolute-value sums): every key row of dK
    and dV for whole (batch, K/V head) units, every row of dQ for those units' query
    heads, and, in every (batch, head) slice, the dQ rows on both sides of each query- and
    key-tile boundary plus random rows."""
    w = synth_inputs.WORKLOADS[name]
    _log(f"[bwd workload] {name}")
    inp = synth_inputs.workload_inputs(w)
    dout = synth_inputs.make_dout(w.B, w.N, w.H, w.d, w.dtype, w.seed + 100)
    q, k, v = (gu.to_dev(inp[x], w.dtype) for x in "qkv")
    do = gu.to_dev(dout, w.dtype)
    o, lse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    dq, dk, dv = (t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv))
    del q, k, v, do, o, lse
    u = gu.UNIT_ROUNDOFF[w.dtype]
    g = w.H // w.Hkv
    qd, kd, vd, dd = (oracle.decode(a, w.dtype) for a in (inp["q"], inp["k"], inp["v"], dout))
    rng = np.random.default_rng(w.seed)
    # (b, kv-head) units checked whole: one for the grouped shape (each of its keys sums over
    # 4 x 8192 query rows), eight for the multi-head shape
    units = [(w.B - 1, w.Hkv - 1)] if g > 1 else sorted(
        {(0, 0), (w.B - 1, w.Hkv - 1)} | {(int(rng.integers(w.B)), int(rng.integers(w.Hkv))) for _ in range(6)})
    fo, flse = _unit_forward(qd, kd, vd, w.causal, w.scale, units)
    # dK, dV: every key row of each unit
    krows = np.array([[b, hk, j] for b, hk in units for j in range(w.N)], dtype=np.int64)
    rk, rv, mk = oracle.attn_bwd_dkdv_rows_f64(qd, kd, vd, dd, w.causal, w.scale, krows, (fo, flse), with_mag=True)
    sel = (krows[:, 0], krows[:, 2], krows[:, 1])
    ek = _check_rows(f"{name} dk", dk[sel], rk, w.scale * u * (mk[:, 0] + mk[:, 1]) + u * np.abs(rk))
    ev = _check_rows(f"{name} dv", dv[sel], rv, u * mk[:, 2] + u * np.abs(rv))
    # dQ: every row of the units' query heads, tile-boundary rows of every slice, random rows
    edge = sorted({i for t in (gu.KEY_TILE, gu.QUERY_TILE) for x in range(0, w.N + 1, t) for i in (x - 1, x)
                   if 0 <= i < w.N} if w.N <= 4096 else
                  {i for x in range(0, w.N + 1, gu.QUERY_TILE) for i in (x - 1, x) if 0 <= i < w.N})
    qrows = {(b, h, i) for b, hk in units for h in (range(hk * g, (hk + 1) * g) if g == 1 else (hk * g,))
             for i in range(w.N)}
    qrows |= {(b, h, i) for b in range(w.B) for h in range(w.H) for i in edge}
    qrows |= {tuple(r) for r in gu.sample_rows(w.B, w.H, w.N, n_random=64, seed=w.seed).tolist()}
    qrows = np.array(sorted(qrows), dtype=np.int64)
    rq, mq = oracle.attn_bwd_dq_rows_f64(qd, kd, vd, dd, w.causal, w.scale, qrows, with_mag=True)
    o_rows, _ = oracle.attn_rows_f64(qd[qrows[:, 0], qrows[:, 2], qrows[:, 1]], kd, vd, w.H, qrows, w.causal,
                                     w.scale)
    dD = u * np.sum(np.abs(dd[qrows[:, 0], qrows[:, 2], qrows[:, 1]] * o_rows), axis=1)
    eq = _check_rows(f"{name} dq", dq[qrows[:, 0], qrows[:, 2], qrows[:, 1]], rq,
                     w.scale * (u * mq[:, 0] + dD[:, None] * mq[:, 1]) + u * np.abs(rq))
    _log(f"[bwd workload] {name}: {len(krows)} dK/dV rows of units {units} and {len(qrows)} dQ rows, every element; "
         f"err/bound dq {eq:.2f} dk {ek:.2f} dv {ev:.2f}")
