"""Pins of the fp64 oracle against facts that do not come from the oracle itself:
brute force in 50-digit arithmetic, an independent library implementation, closed
forms, invariants of softmax attention and the storage-format definitions.

The pages describe attention as S = Q K^T, O = softmax(S) V (section "The quadratic
bottleneck in standard attention" of "FlashAttention: The Algorithm That Made
Long-Context AI Possible") and state that the tiled method is exact (abstract of
"FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness"). They
print no worked example, so every pin here is derived from that definition.

Each pin is a function that raises AssertionError on failure. The same battery runs
against deliberately broken copies of the oracle (test_oracle_mutants.py) to show
that a plausible mistake anywhere in it fails at least one pin.
"""
from __future__ import annotations

import json
import math
import os

import mpmath
import numpy as np
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _qkv(rng, B, N, H, Hkv, d):
    return (rng.standard_normal((B, N, H, d)), rng.standard_normal((B, N, Hkv, d)),
            rng.standard_normal((B, N, Hkv, d)))


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: max scaled error {err:.3e} > {tol:.1e}"


# P1 -- brute force in 50 significant digits on tiny inputs.
def pin_mpmath_bruteforce():
    rng = np.random.default_rng(11)
    mpmath.mp.dps = 50
    cases = [(1, 1, 1, 1, False), (2, 1, 3, 4, True), (2, 2, 5, 8, False), (2, 1, 8, 4, True),
             (1, 1, 17, 8, False), (2, 2, 2, 1, True), (4, 2, 6, 3, True)]
    for H, Hkv, N, d, causal in cases:
        q, k, v = _qkv(rng, 1, N, H, Hkv, d)
        scale = 0.37
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, scale)
        for h in range(H):
            hk = h // (H // Hkv)
            for i in range(N):
                J = range(i + 1) if causal else range(N)
                s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[0, i, h, t]) * mpmath.mpf(k[0, j, hk, t])
                                                     for t in range(d)) for j in J]
                L = mpmath.log(mpmath.fsum(mpmath.exp(x) for x in s))
                w = [mpmath.exp(x - L) for x in s]
                ref_o = [float(mpmath.fsum(w[n] * mpmath.mpf(v[0, j, hk, t]) for n, j in enumerate(J)))
                         for t in range(d)]
                _close(o[0, i, h], ref_o, 1e-13, f"mpmath O (H{H} Hkv{Hkv} N{N} d{d} c{causal}) h{h} i{i}")
                _close(lse[0, h, i], float(L), 1e-13, f"mpmath lse h{h} i{i}")


def _sdpa_lse(q, k, causal, scale, H, Hkv):
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(H // Hkv, dim=1)
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * scale
    if causal:
        N = q.shape[1]
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    return torch.logsumexp(s, dim=-1).numpy()


# P2 -- an independent library implementation (torch CPU scaled_dot_product_attention, float64).
def pin_torch_sdpa():
    rng = np.random.default_rng(12)
    for B, H, Hkv, N, d, causal in [(1, 2, 2, 128, 64, False), (2, 4, 2, 67, 16, True),
                                    (1, 4, 1, 33, 8, False), (1, 2, 2, 130, 128, True)]:
        q, k, v = _qkv(rng, B, N, H, Hkv, d)
        scale = 1.0 / math.sqrt(d)
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, scale)
        t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
        ref = F.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=causal, scale=scale,
                                             enable_gqa=(H != Hkv)).permute(0, 2, 1, 3).numpy()
        _close(o, ref, 1e-12, f"sdpa O B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
        _close(lse, _sdpa_lse(q, k, causal, scale, H, Hkv), 1e-12, "logsumexp of scores")


# P3 -- Q = 0: every score is 0, so O_i is the mean of the visible V rows and lse_i = ln|J_i|.
def pin_zero_query():
    rng = np.random.default_rng(13)
    for causal in (False, True):
        B, N, H, Hkv, d = 2, 37, 4, 2, 8
        _, k, v = _qkv(rng, B, N, H, Hkv, d)
        q = np.zeros((B, N, H, d))
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.7)
        for h in range(H):
            hk = h // (H // Hkv)
            if causal:
                ref = np.cumsum(v[:, :, hk, :], axis=1) / np.arange(1, N + 1)[None, :, None]
                ref_lse = np.log(np.arange(1, N + 1))[None, :].repeat(B, 0)
            else:
                ref = np.repeat(v[:, :, hk, :].mean(axis=1, keepdims=True), N, axis=1)
                ref_lse = np.full((B, N), math.log(N))
            _close(o[:, :, h, :], ref, 1e-13, f"Q=0 mean of V (causal={causal}) h{h}")
            _close(lse[:, h, :], ref_lse, 1e-13, f"Q=0 lse=ln|J| (causal={causal})")


# P4 -- one key: O = V_0 and lse = scale * <q, k_0>.
def pin_single_key():
    rng = np.random.default_rng(14)
    q, k, v = _qkv(rng, 3, 1, 4, 2, 5)
    for causal in (False, True):
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.3)
        for h in range(4):
            hk = h // 2
            _close(o[:, 0, h, :], v[:, 0, hk, :], 1e-15, "N=1 O=V0")
            _close(lse[:, h, 0], 0.3 * np.einsum("bt,bt->b", q[:, 0, h, :], k[:, 0, hk, :]), 1e-14,
                   "N=1 lse=scale*q.k")


# P5 -- two keys: weights are logistic functions of the score difference.
def pin_two_keys():
    rng = np.random.default_rng(15)
    q, k, v = _qkv(rng, 1, 2, 1, 1, 6)
    scale = 0.45
    o, lse = oracle.attn_fwd_f64(q, k, v, False, scale)
    s = [scale * float(np.dot(q[0, 0, 0], k[0, j, 0])) for j in range(2)]
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))
    ref = sig(s[0] - s[1]) * v[0, 0, 0] + sig(s[1] - s[0]) * v[0, 1, 0]
    _close(o[0, 0, 0], ref, 1e-14, "two-key logistic form")
    _close(lse[0, 0, 0], np.logaddexp(s[0], s[1]), 1e-14, "two-key lse=logaddexp")
    # causal: the first query sees only key 0
    o, lse = oracle.attn_fwd_f64(q, k, v, True, scale)
    _close(o[0, 0, 0], v[0, 0, 0], 1e-15, "causal row 0 sees key 0 only")
    _close(lse[0, 0, 0], s[0], 1e-14, "causal row 0 lse")


# P6 -- rows of P sum to one and are nonnegative: constant V gives a constant output
# and O is affine in V.
def pin_affine_in_v():
    rng = np.random.default_rng(16)
    B, N, H, Hkv, d = 2, 29, 2, 1, 7
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    for causal in (False, True):
        c = rng.standard_normal(d)
        o, _ = oracle.attn_fwd_f64(q, k, np.broadcast_to(c, v.shape).copy(), causal, 0.5)
        _close(o, np.broadcast_to(c, o.shape), 1e-14, "constant V")
        o1, l1 = oracle.attn_fwd_f64(q, k, v, causal, 0.5)
        o2, l2 = oracle.attn_fwd_f64(q, k, 2.5 * v - 1.25, causal, 0.5)
        _close(o2, 2.5 * o1 - 1.25, 1e-13, "O(aV+b)=aO(V)+b")
        _close(l2, l1, 0.0, "lse does not depend on V")


# P7 -- probability rows: nonnegative, sum to one, zero above the diagonal when causal,
# and the output is those rows applied to V.
def pin_probability_rows():
    rng = np.random.default_rng(17)
    B, N, H, Hkv, d = 1, 23, 2, 2, 4
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    for causal in (False, True):
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.8)
        for h in range(H):
            p = oracle.attn_probs_f64(q, k, 0, h, causal, 0.8)
            assert np.all(p >= 0), "negative probability"
            _close(p.sum(axis=1), np.ones(N), 1e-14, "rows sum to 1")
            if causal:
                assert np.all(np.triu(p, 1) == 0), "mass above the diagonal"
            _close(o[0, :, h, :], p @ v[0, :, h, :], 1e-13, "O = P V")
            s = 0.8 * q[0, :, h, :] @ k[0, :, h, :].T
            with np.errstate(divide="ignore"):
                _close(np.where(p > 0, np.log(np.where(p > 0, p, 1)) + lse[0, h, :, None], 0),
                       np.where(p > 0, s, 0), 1e-12, "P_ij = exp(s_ij - lse_i)")


# P8 -- without the mask, permuting key/value rows together changes nothing.
def pin_key_permutation():
    rng = np.random.default_rng(18)
    B, N, H, Hkv, d = 2, 41, 4, 2, 6
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    o, lse = oracle.attn_fwd_f64(q, k, v, False, 0.6)
    perm = rng.permutation(N)
    o2, lse2 = oracle.attn_fwd_f64(q, k[:, perm], v[:, perm], False, 0.6)
    _close(o2, o, 1e-13, "key permutation O")
    _close(lse2, lse, 1e-13, "key permutation lse")


# P9 -- adding w to every key shifts every score of row i by scale*<q_i, w>: O is
# unchanged and lse_i moves by exactly that amount.
def pin_key_shift():
    rng = np.random.default_rng(19)
    B, N, H, Hkv, d = 1, 31, 2, 1, 5
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    w = rng.standard_normal(d)
    for causal in (False, True):
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.9)
        o2, lse2 = oracle.attn_fwd_f64(q, k + w, v, causal, 0.9)
        _close(o2, o, 1e-12, "key shift O")
        shift = 0.9 * np.einsum("bnhd,d->bhn", q, w)
        _close(lse2, lse + shift, 1e-12, "key shift lse")


# P10 -- grouped-query attention equals multi-head attention with each K/V head
# repeated for its group of query heads (query head h reads K/V head h // (H/Hkv)).
def pin_gqa_repeat():
    rng = np.random.default_rng(20)
    B, N, H, Hkv, d = 2, 19, 6, 2, 4
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    for causal in (False, True):
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.5)
        kr = np.repeat(k, H // Hkv, axis=2)
        vr = np.repeat(v, H // Hkv, axis=2)
        o2, lse2 = oracle.attn_fwd_f64(q, kr, vr, causal, 0.5)
        _close(o, o2, 0.0, "GQA = repeated MHA (O)")
        _close(lse, lse2, 0.0, "GQA = repeated MHA (lse)")


# P11 -- under the mask, row i equals unmasked attention over keys 0..i.
def pin_causal_prefix():
    rng = np.random.default_rng(21)
    B, N, H, Hkv, d = 1, 17, 2, 2, 4
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    o, lse = oracle.attn_fwd_f64(q, k, v, True, 0.7)
    for i in (0, 1, 5, 16):
        qq = np.repeat(q[:, i:i + 1], i + 1, axis=1)
        o2, lse2 = oracle.attn_fwd_f64(qq, k[:, :i + 1], v[:, :i + 1], False, 0.7)
        _close(o2[:, 0], o[:, i], 1e-13, f"causal row {i} = prefix attention (O)")
        _close(lse2[:, :, 0], lse[:, :, i], 1e-13, f"causal row {i} = prefix attention (lse)")


# P12 -- splitting the keys into two sets: lse merges by logaddexp and O merges with
# weights exp(lse_part - lse).
def pin_split_merge():
    rng = np.random.default_rng(22)
    B, N, H, Hkv, d = 1, 24, 2, 1, 6
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    o, lse = oracle.attn_fwd_f64(q, k, v, False, 0.55)
    a = 10
    # queries attend separately to keys [0,a) and [a,N): pad each part to N rows by
    # evaluating each query against the part (rows of q are independent)
    def part(ks, vs):
        n = ks.shape[1]
        oo = np.empty((B, N, H, d))
        ll = np.empty((B, H, N))
        for i in range(N):
            qq = np.repeat(q[:, i:i + 1], n, axis=1)
            o_, l_ = oracle.attn_fwd_f64(qq, ks, vs, False, 0.55)
            oo[:, i] = o_[:, 0]
            ll[:, :, i] = l_[:, :, 0]
        return oo, ll
    oa, la = part(k[:, :a], v[:, :a])
    ob, lb = part(k[:, a:], v[:, a:])
    lm = np.logaddexp(la, lb)
    _close(lm, lse, 1e-13, "lse = logaddexp(lse_A, lse_B)")
    wa = np.exp(la - lm).transpose(0, 2, 1)[..., None]
    wb = np.exp(lb - lm).transpose(0, 2, 1)[..., None]
    _close(wa * oa + wb * ob, o, 1e-13, "O = sum of parts weighted by exp(lse_part - lse)")


# P13 -- large score gaps: the output is the value row of the best key and lse the best
# score; scores of magnitude ~1e3 stay finite (the row maximum is subtracted).
def pin_hardmax_and_range():
    rng = np.random.default_rng(23)
    B, N, H, Hkv, d = 1, 9, 1, 1, 3
    k = rng.standard_normal((B, N, Hkv, d))
    v = rng.standard_normal((B, N, Hkv, d))
    q = np.zeros((B, N, H, d))
    best = 4
    k[0, best, 0] = np.array([50.0, 0.0, 0.0])
    k[0, :best, 0, 0] = np.linspace(-5, 5, best)
    k[0, best + 1:, 0, 0] = np.linspace(-5, 9, N - best - 1)
    q[0, :, 0] = np.array([1.0, 0.0, 0.0])
    o, lse = oracle.attn_fwd_f64(q, k, v, False, 1.0)
    _close(o[0, :, 0], np.repeat(v[0, best:best + 1, 0], N, axis=0), 1e-15, "hardmax O")
    assert np.all(np.abs(lse[0, 0] - 50.0) < 1e-13), "hardmax lse = best score"
    for mag in (300.0, 1000.0):
        o, lse = oracle.attn_fwd_f64(q, k * (mag / 50.0), v, True, 1.0)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), f"non-finite at score magnitude {mag}"
        _close(o[0, best:, 0], np.repeat(v[0, best:best + 1, 0], N - best, axis=0), 1e-15,
               f"hardmax under the mask at magnitude {mag}")


# P14 -- storage formats decode to the values their definitions give, checked against
# independent decoders (numpy binary16, torch bfloat16 and float8_e4m3fn).
def pin_decoders():
    codes16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = oracle.decode(codes16, "f16")
    ref = codes16.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(f16[fin], ref[fin]), "f16 decode"
    assert np.array_equal(np.isnan(f16), np.isnan(ref)) and np.array_equal(np.isinf(f16), np.isinf(ref))
    bf = oracle.decode(codes16, "bf16")
    refb = torch.from_numpy(codes16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(refb)
    assert np.array_equal(bf[fin], refb[fin]), "bf16 decode"
    assert np.array_equal(np.isnan(bf), np.isnan(refb)) and np.array_equal(np.isinf(bf), np.isinf(refb))
    codes8 = np.arange(256, dtype=np.uint16).astype(np.uint8)
    e = oracle.decode(codes8, "e4m3")
    refe = torch.from_numpy(codes8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    fin = np.isfinite(refe)
    assert np.array_equal(e[fin], refe[fin]), "e4m3 decode"
    assert np.array_equal(np.isnan(e), np.isnan(refe)), "e4m3 NaN codes"
    # definition points of OCP E4M3: largest finite, smallest normal, smallest subnormal
    assert e[0x7E] == 448.0 and e[0x08] == 2.0 ** -6 and e[0x01] == 2.0 ** -9 and e[0xFE] == -448.0
    assert oracle.decode(np.array([0x38], np.uint8), "e4m3", 0.25)[0] == 0.25, "descale multiplies"


# Closed-form fixtures derived by hand (tests/golden/*.json, each with its derivation).
def pin_golden_fixtures():
    for name in sorted(os.listdir(GOLDEN)):
        if not name.endswith(".json"):
            continue
        with open(os.path.join(GOLDEN, name)) as f:
            fx = json.load(f)
        q = np.array(fx["q"], dtype=np.float64)
        k = np.array(fx["k"], dtype=np.float64)
        v = np.array(fx["v"], dtype=np.float64)
        scale = fx["scale"] if isinstance(fx["scale"], float) else eval(fx["scale"], {"math": math})
        o, lse = oracle.attn_fwd_f64(q, k, v, fx["causal"], scale, fx.get("window"))
        _close(o, np.array(fx["o"]), fx["tol"], f"golden {name} O")
        _close(lse, np.array(fx["lse"]), fx["tol"], f"golden {name} lse")


# Key windows. The long-context page names sliding-window patterns (section "Why
# context lengths exploded after 2022") without defining them; the reading pinned here
# keeps key j for query i iff i - left <= j <= i + right (negative bound: unbounded),
# intersected with the causal mask.
def _window_mask(N, causal, left, right):
    """Boolean [N, N] visibility built from the offset matrix j - i (an implementation
    independent of the oracle's per-row range arithmetic)."""
    off = np.subtract.outer(np.arange(N), np.arange(N)).T       # off[i, j] = j - i
    keep = np.ones((N, N), dtype=bool)
    if causal:
        keep &= off <= 0
    if left >= 0:
        keep &= off >= -left
    if right >= 0:
        keep &= off <= right
    return keep


WINDOW_CASES = [(False, 0, 0), (False, 1, 2), (False, 2, 1), (False, 3, -1), (False, -1, 4),
                (True, 2, -1), (True, 0, 3), (True, 5, 7), (False, 40, 40), (True, -1, -1)]


# P15 -- windows against brute force in 50 digits and against torch's attention with an
# explicit boolean mask (float64, CPU).
def pin_window_bruteforce_and_sdpa():
    rng = np.random.default_rng(31)
    mpmath.mp.dps = 50
    N, H, Hkv, d = 9, 2, 1, 3
    q, k, v = _qkv(rng, 1, N, H, Hkv, d)
    for causal, left, right in WINDOW_CASES:
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.6, (left, right))
        keep = _window_mask(N, causal, left, right)
        for h in range(H):
            for i in range(N):
                J = [j for j in range(N) if keep[i, j]]
                s = [mpmath.mpf(0.6) * mpmath.fsum(mpmath.mpf(q[0, i, h, t]) * mpmath.mpf(k[0, j, 0, t])
                                                   for t in range(d)) for j in J]
                L = mpmath.log(mpmath.fsum(mpmath.exp(x) for x in s))
                ref = [float(mpmath.fsum(mpmath.exp(x - L) * mpmath.mpf(v[0, j, 0, t]) for x, j in zip(s, J)))
                       for t in range(d)]
                _close(o[0, i, h], ref, 1e-13, f"window ({causal},{left},{right}) mpmath O h{h} i{i}")
                _close(lse[0, h, i], float(L), 1e-13, f"window ({causal},{left},{right}) mpmath lse")
    B, N, H, Hkv, d = 2, 70, 4, 2, 16
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    for causal, left, right in WINDOW_CASES:
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.25, (left, right))
        mask = torch.from_numpy(_window_mask(N, causal, left, right))
        ref = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=mask, scale=0.25,
                                             enable_gqa=True).permute(0, 2, 1, 3).numpy()
        _close(o, ref, 1e-12, f"window ({causal},{left},{right}) vs sdpa with mask")


# P16 -- windows in closed form: with Q = 0 row i is the mean of its visible V rows and
# lse_i = ln(count); a window of width zero gives O_i = V_i and lse_i = scale <q_i, k_i>.
def pin_window_closed_forms():
    rng = np.random.default_rng(32)
    B, N, H, Hkv, d = 1, 23, 2, 1, 5
    _, k, v = _qkv(rng, B, N, H, Hkv, d)
    q0 = np.zeros((B, N, H, d))
    for causal, left, right in WINDOW_CASES:
        o, lse = oracle.attn_fwd_f64(q0, k, v, causal, 0.9, (left, right))
        keep = _window_mask(N, causal, left, right).astype(np.float64)
        count = keep.sum(axis=1)
        for h in range(H):
            _close(o[0, :, h], keep @ v[0, :, 0] / count[:, None], 1e-13,
                   f"window ({causal},{left},{right}) Q=0 local mean")
            _close(lse[0, h], np.log(count), 1e-13, f"window ({causal},{left},{right}) Q=0 ln(count)")
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    for causal in (False, True):
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.4, (0, 0))
        for h in range(H):
            _close(o[0, :, h], v[0, :, 0], 1e-15, "window (0,0): O_i = V_i")
            _close(lse[0, h], 0.4 * np.einsum("nt,nt->n", q[0, :, h], k[0, :, 0]), 1e-14,
                   "window (0,0): lse_i = scale <q_i, k_i>")


# P17 -- windows reduce to the unwindowed cases: a window wider than the sequence is
# the full (or causal) attention, and right = 0 without the mask is the causal mask.
def pin_window_reductions():
    rng = np.random.default_rng(33)
    B, N, H, Hkv, d = 1, 31, 2, 2, 4
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    for causal in (False, True):
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.5)
        for w in ((N, N), (N - 1, N - 1), (-1, -1), (10 * N, -1)):
            o2, lse2 = oracle.attn_fwd_f64(q, k, v, causal, 0.5, w)
            assert np.array_equal(o, o2) and np.array_equal(lse, lse2), f"wide window {w} (causal={causal})"
    oc, lc = oracle.attn_fwd_f64(q, k, v, True, 0.5)
    o2, l2 = oracle.attn_fwd_f64(q, k, v, False, 0.5, (-1, 0))
    assert np.array_equal(oc, o2) and np.array_equal(lc, l2), "right = 0 is the causal mask"
    # a causal window is a row-wise suffix of the causal prefix: row i with left = L is
    # the unmasked attention of query i over keys max(0, i-L) .. i
    L = 4
    o, lse = oracle.attn_fwd_f64(q, k, v, True, 0.5, (L, -1))
    for i in (0, 3, 4, 17, 30):
        lo = max(0, i - L)
        n = i + 1 - lo
        o2, l2 = oracle.attn_fwd_f64(np.repeat(q[:, i:i + 1], n, axis=1), k[:, lo:i + 1], v[:, lo:i + 1],
                                     False, 0.5)
        _close(o2[:, 0], o[:, i], 1e-13, f"causal window row {i} = slice attention (O)")
        _close(l2[:, :, 0], lse[:, :, i], 1e-13, f"causal window row {i} = slice attention (lse)")


# Block-sparse attention (the block-sparse FlashAttention of the abstract of
# "FlashAttention: Fast and Memory-Efficient Exact Attention with IO-Awareness", which
# the pages name without defining). Reading pinned here: key j is visible to query i iff
# mask[hm, i // block, j // block] != 0 (and j <= i when causal); a row with no visible
# key gives O = 0 and lse = -inf.
def _block_element_mask(mask, h, N, block, causal):
    """Boolean [N, N] visibility expanded from the block mask with np.kron (independent of
    the oracle's per-key index arithmetic)."""
    m = mask[0 if mask.shape[0] == 1 else h].astype(bool)
    keep = np.kron(m, np.ones((block, block), dtype=bool))[:N, :N]
    if causal:
        keep &= np.tril(np.ones((N, N), dtype=bool))
    return keep


# P26 -- block masks against brute force in 50 digits and against torch's attention with
# an explicit boolean mask (float64, CPU); rows with no visible key give O = 0, lse = -inf.
def pin_block_sparse_bruteforce_and_sdpa():
    rng = np.random.default_rng(41)
    mpmath.mp.dps = 50
    N, H, Hkv, d, block = 10, 2, 1, 3, 3               # nb = 4, ragged last block
    q, k, v = _qkv(rng, 1, N, H, Hkv, d)
    mask = (rng.random((H, 4, 4)) < 0.5).astype(np.uint8)
    mask[0, 1, :] = 0                                  # an empty block row in head 0
    for causal in (False, True):
        o, lse = oracle.attn_fwd_block_f64(q, k, v, causal, 0.6, mask, block)
        for h in range(H):
            keep = _block_element_mask(mask, h, N, block, causal)
            for i in range(N):
                J = [j for j in range(N) if keep[i, j]]
                if not J:
                    assert np.all(o[0, i, h] == 0.0) and lse[0, h, i] == -np.inf, f"empty row {h},{i}"
                    continue
                s = [mpmath.mpf(0.6) * mpmath.fsum(mpmath.mpf(q[0, i, h, t]) * mpmath.mpf(k[0, j, 0, t])
                                                   for t in range(d)) for j in J]
                L = mpmath.log(mpmath.fsum(mpmath.exp(x) for x in s))
                ref = [float(mpmath.fsum(mpmath.exp(x - L) * mpmath.mpf(v[0, j, 0, t]) for x, j in zip(s, J)))
                       for t in range(d)]
                _close(o[0, i, h], ref, 1e-13, f"block mask (causal={causal}) mpmath O h{h} i{i}")
                _close(lse[0, h, i], float(L), 1e-13, f"block mask (causal={causal}) mpmath lse")
    B, N, H, Hkv, d, block = 2, 150, 4, 2, 16, 64      # nb = 3
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
    for heads in (1, H):
        mask = (rng.random((heads, 3, 3)) < 0.6).astype(np.uint8)
        mask[:, :, 0] = 1                              # every row sees key block 0: no empty rows
        for causal in (False, True):
            o, lse = oracle.attn_fwd_block_f64(q, k, v, causal, 0.25, mask, block)
            emask = torch.from_numpy(np.stack([_block_element_mask(mask, h, N, block, causal) for h in range(H)]))
            ref = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=emask, scale=0.25,
                                                 enable_gqa=True).permute(0, 2, 1, 3).numpy()
            _close(o, ref, 1e-12, f"block mask heads={heads} causal={causal} vs sdpa with mask")
            ref_lse = np.stack([_sdpa_lse_masked(q[:, :, h], k[:, :, h // (H // Hkv)], emask[h].numpy(), 0.25)
                                for h in range(H)], axis=1)
            _close(lse, ref_lse, 1e-12, f"block mask heads={heads} causal={causal} lse")


def _sdpa_lse_masked(qh, kh, keep, scale):
    """ln sum_j exp(scale <q_i, k_j>) over the visible keys, via torch.logsumexp."""
    s = scale * torch.einsum("bid,bjd->bij", torch.from_numpy(qh), torch.from_numpy(kh))
    s = s.masked_fill(~torch.from_numpy(keep), -float("inf"))
    return torch.logsumexp(s, dim=-1).numpy()


# P27 -- block masks reduce to the dense cases: an all-ones mask is the full (or causal)
# attention, a lower-triangular block mask with the causal flag is the causal mask, and
# a block-diagonal mask is independent attention inside each block (bit-identical: the
# same sums in the same order); with Q = 0 a row is the mean of its visible V rows.
def pin_block_sparse_reductions():
    rng = np.random.default_rng(42)
    B, N, H, Hkv, d, block = 1, 100, 2, 1, 8, 16       # nb = 7
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    nb = 7
    for causal in (False, True):
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.5)
        o2, l2 = oracle.attn_fwd_block_f64(q, k, v, causal, 0.5, np.ones((1, nb, nb), np.uint8), block)
        assert np.array_equal(o, o2) and np.array_equal(lse, l2), f"all-ones mask (causal={causal})"
    oc, lc = oracle.attn_fwd_f64(q, k, v, True, 0.5)
    o2, l2 = oracle.attn_fwd_block_f64(q, k, v, True, 0.5, np.tril(np.ones((nb, nb), np.uint8))[None], block)
    assert np.array_equal(oc, o2) and np.array_equal(lc, l2), "lower-triangular block mask + causal"
    o, lse = oracle.attn_fwd_block_f64(q, k, v, False, 0.5, np.eye(nb, dtype=np.uint8)[None], block)
    for qb in range(nb):
        lo, hi = qb * block, min(N, (qb + 1) * block)
        o2, l2 = oracle.attn_fwd_f64(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], False, 0.5)
        assert np.array_equal(o[:, lo:hi], o2) and np.array_equal(lse[:, :, lo:hi], l2), f"diagonal block {qb}"
    mask = (rng.random((H, nb, nb)) < 0.4).astype(np.uint8)
    q0 = np.zeros_like(q)
    for causal in (False, True):
        o, lse = oracle.attn_fwd_block_f64(q0, k, v, causal, 0.9, mask, block)
        for h in range(H):
            keep = _block_element_mask(mask, h, N, block, causal).astype(np.float64)
            count = keep.sum(axis=1)
            seen = count > 0
            _close(o[0, seen, h], (keep @ v[0, :, 0])[seen] / count[seen, None], 1e-13,
                   f"block mask Q=0 local mean (causal={causal}) h{h}")
            _close(lse[0, h, seen], np.log(count[seen]), 1e-13, f"block mask Q=0 ln(count) h{h}")
            assert np.all(o[0, ~seen, h] == 0.0) and np.all(lse[0, h, ~seen] == -np.inf), "empty rows"


# Block quantisation to e4m3 and incoherent processing. The abstract of "FlashAttention-3:
# Fast and Accurate Attention with Asynchrony and Low-precision" names both without
# defining them; the readings pinned here: one power-of-two scale per 64-row slab of each
# (batch, head), codes by round-to-nearest-even, rotation (x * s) H with H Sylvester-Hadamard.
def _e4m3_values():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# P18 -- the e4m3 encoder against torch's float8_e4m3fn cast and against brute force
# nearest-value search, including every tie and the saturation and sign rules.
def pin_e4m3_encode():
    vals = _e4m3_values()
    fin = np.isfinite(vals)
    grid = np.unique(vals[fin])                                   # sorted finite values
    mids = (grid[:-1] + grid[1:]) / 2                             # exact ties (in float32 too)
    rng = np.random.default_rng(41)
    ys = np.concatenate([grid, mids, rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
                         np.ldexp(rng.uniform(-1, 1, 5000), rng.integers(-12, 9, 5000))]).astype(np.float32)
    codes = oracle.e4m3_encode(ys)
    ref = torch.from_numpy(ys).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref), f"e4m3 encode vs torch: {int((codes != ref).sum())} differ"
    # brute force: the decoded code is a nearest finite value; at a tie its fraction is even
    dec = vals[codes]
    dist = np.abs(dec - ys.astype(np.float64))
    best = np.min(np.abs(grid[None, :] - ys.astype(np.float64)[:, None]), axis=1)
    assert np.all(dist == best), "e4m3 encode is not nearest"
    tie = np.isin(ys.astype(np.float64), mids)
    assert np.all((codes[tie] & 1) == 0), "e4m3 ties go to the even code"
    sat = oracle.e4m3_encode(np.array([448.0, 460.0, 1e6, -500.0, np.inf, -np.inf], np.float32))
    assert list(sat) == [0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE], f"saturation {sat}"
    special = oracle.e4m3_encode(np.array([0.0, -0.0, np.nan, 2.0 ** -10, -(2.0 ** -10) * 1.5], np.float32))
    assert list(special) == [0x00, 0x80, 0x7F, 0x00, 0x81], f"zero/NaN/subnormal {special}"


# P19 -- the fast Walsh-Hadamard transform against the Sylvester-Hadamard matrix of
# scipy (fp64 product), H H = d I exactly on small integers, and Parseval.
def pin_fwht():
    import scipy.linalg
    rng = np.random.default_rng(42)
    for d in (1, 2, 8, 64, 128):
        H = scipy.linalg.hadamard(d).astype(np.float64)
        x = rng.standard_normal((7, d)).astype(np.float32)
        y = oracle.fwht_f32(x)
        ref = x.astype(np.float64) @ H
        assert np.max(np.abs(y - ref)) <= 8 * d * 2.0 ** -24 * np.max(np.abs(x)) * np.log2(max(d, 2)), f"fwht d={d}"
        xi = rng.integers(-8, 9, (5, d)).astype(np.float32)
        assert np.array_equal(oracle.fwht_f32(oracle.fwht_f32(xi)), d * xi), f"H H = d I (d={d})"
        assert np.array_equal(oracle.fwht_f32(xi), (xi.astype(np.float64) @ H).astype(np.float32)), \
            f"exact on integers (d={d})"
        assert abs(np.sum(ref ** 2) - d * np.sum(x.astype(np.float64) ** 2)) < 1e-6 * d * np.sum(x ** 2) + 1e-9


# P20 -- block quantisation: the scale exponent is the smallest that fits the slab's
# largest magnitude under 448 (floored at -127, 0 for a zero slab), every code is the
# e4m3 rounding of the (rotated) value times 2^-e, and ragged tails form their own slab.
def pin_block_quantize():
    rng = np.random.default_rng(43)
    vals = _e4m3_values()
    grid = np.unique(vals[np.isfinite(vals)])
    B, N, Hx, d, br = 2, 150, 3, 64, 64
    x = (rng.standard_normal((B, N, Hx, d)) * np.exp(rng.uniform(-3, 3, (B, 1, Hx, 1)))).astype(np.float32)
    x[0, 64:128, 1] = 0.0                                        # an all-zero slab
    x[1, 0:64, 0] = 0.0
    x[1, 5, 0, 7] = 448.0                                        # amax exactly 448: e = 0
    x[1, 64:128, 2] *= 2.0 ** -140 / np.abs(x[1, 64:128, 2]).max()   # tiny slab: e floored
    signs = np.where(rng.random(d) < 0.5, -1.0, 1.0).astype(np.float32)
    import scipy.linalg
    H = scipy.linalg.hadamard(d).astype(np.float64)
    for sg in (None, signs):
        codes, scales = oracle.block_quantize(x.astype(np.float64), br, sg)
        nb = (N + br - 1) // br
        assert scales.shape == (B, Hx, nb)
        y = x.astype(np.float64) if sg is None else (x.astype(np.float64) * sg) @ H
        for b in range(B):
            for h in range(Hx):
                for k in range(nb):
                    slab = y[b, k * br:(k + 1) * br, h]
                    amax = np.max(np.abs(slab))
                    e = int(scales[b, h, k]) - 127
                    if amax == 0:
                        assert e == 0 and np.all(codes[b, k * br:(k + 1) * br, h] & 0x7F == 0), "zero slab"
                        continue
                    if e > -127:
                        assert amax * 2.0 ** -e <= 448 < amax * 2.0 ** -(e - 1), f"exponent b{b} h{h} k{k}"
                    else:
                        assert amax * 2.0 ** 127 <= 448, "floored exponent"
                    dec = vals[codes[b, k * br:(k + 1) * br, h]] * 2.0 ** e
                    # nearest e4m3 value after exact scaling (float32 rounding of the rotation
                    # moves a value by at most a few float32 ulps)
                    z = slab * 2.0 ** -e
                    best = np.min(np.abs(grid[None, :] - z.reshape(-1)[:, None]), axis=1).reshape(z.shape)
                    slack = 64 * 2.0 ** -24 * np.abs(z) + (0 if sg is None else 1e-6 * np.max(np.abs(z)))
                    assert np.all(np.abs(dec * 2.0 ** -e - z) <= best + slack), f"codes b{b} h{h} k{k}"
    assert int(oracle.block_quantize(x.astype(np.float64), br)[1][1, 0, 0]) == 127, "amax 448 -> e = 0"
    assert int(oracle.block_quantize(x.astype(np.float64), br)[1][1, 2, 1]) == 0, "tiny slab -> e = -127"


# P21 -- incoherent processing leaves attention unchanged: rotating Q and K by s H and
# dividing the score scale by d gives the same output and lse (fp64, unquantised).
def pin_rotation_identity():
    import scipy.linalg
    rng = np.random.default_rng(44)
    for d in (64, 128):
        q, k, v = _qkv(rng, 2, 40, 4, 2, d)
        s = np.where(rng.random(d) < 0.5, -1.0, 1.0)
        H = scipy.linalg.hadamard(d).astype(np.float64)
        for causal in (False, True):
            o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.3)
            o2, lse2 = oracle.attn_fwd_f64((q * s) @ H, (k * s) @ H, v, causal, 0.3 / d)
            _close(o2, o, 1e-12, f"rotated attention O (d={d})")
            _close(lse2, lse, 1e-12, f"rotated attention lse (d={d})")


# Gradients. The pages report training throughput but print no backward algorithm; the
# oracle's gradient is the analytic derivative of the forward definition for an upstream
# dO (no gradient through lse).
def _loss(q, k, v, g, causal, scale, window=None):
    """L = sum(O * g) with O from a direct numpy evaluation of the definition (masked
    softmax of the scaled scores times V), independent of the oracle's code."""
    B, N, H, d = q.shape
    kr = np.repeat(k, H // k.shape[2], axis=2)
    vr = np.repeat(v, H // v.shape[2], axis=2)
    s = np.einsum("bihd,bjhd->bhij", q, kr) * scale
    keep = _window_mask(N, causal, *(window if window is not None else (-1, -1)))
    s = np.where(keep, s, -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    p /= p.sum(axis=-1, keepdims=True)
    return float(np.sum(np.einsum("bhij,bjhd->bihd", p, vr) * g))


# P22 -- central finite differences of L = sum(O * dO) in every coordinate of tiny inputs.
def pin_bwd_finite_differences():
    rng = np.random.default_rng(51)
    for causal, window in ((False, None), (True, None), (False, (1, 2))):
        B, N, H, Hkv, d = 1, 5, 2, 1, 3
        q, k, v = _qkv(rng, B, N, H, Hkv, d)
        g = rng.standard_normal(q.shape)
        dq, dk, dv = oracle.attn_bwd_f64(q, k, v, g, causal, 0.7, window)
        h = 1e-6
        for x, dx, name in ((q, dq, "dq"), (k, dk, "dk"), (v, dv, "dv")):
            fd = np.empty_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                lp = _loss(q, k, v, g, causal, 0.7, window)
                x[idx] = old - h
                lm = _loss(q, k, v, g, causal, 0.7, window)
                x[idx] = old
                fd[idx] = (lp - lm) / (2 * h)
            assert np.max(np.abs(fd - dx)) <= 1e-7 * max(1.0, np.max(np.abs(dx))), \
                f"{name} vs finite differences (causal={causal}, window={window})"


# P23 -- torch float64 autograd of scaled_dot_product_attention (an independent library).
def pin_bwd_torch_autograd():
    rng = np.random.default_rng(52)
    for B, H, Hkv, N, d, causal, window in ((1, 2, 2, 40, 16, False, None), (2, 4, 2, 37, 8, True, None),
                                             (1, 4, 1, 50, 8, False, (6, 3)), (1, 2, 2, 45, 8, True, (10, -1))):
        q, k, v = _qkv(rng, B, N, H, Hkv, d)
        g = rng.standard_normal(q.shape)
        dq, dk, dv = oracle.attn_bwd_f64(q, k, v, g, causal, 0.3, window)
        t = lambda x: torch.from_numpy(x.copy()).permute(0, 2, 1, 3).requires_grad_(True)
        tq, tk, tv = t(q), t(k), t(v)
        if window is None:
            o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.3, enable_gqa=(H != Hkv))
        else:
            mask = torch.from_numpy(_window_mask(N, causal, *window))
            o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.3, enable_gqa=(H != Hkv))
        o.backward(torch.from_numpy(g).permute(0, 2, 1, 3))
        for mine, ref, name in ((dq, tq.grad, "dq"), (dk, tk.grad, "dk"), (dv, tv.grad, "dv")):
            _close(mine, ref.permute(0, 2, 1, 3).numpy(), 1e-11, f"{name} vs torch autograd (B{B} H{H}/{Hkv} N{N})")


# P24 -- exact invariants: the dS rows sum to zero, so sum_j dK_j = 0; the P rows sum to
# one, so sum_j dV_j = sum over the group's query heads of sum_i dO_i; a window of width
# zero makes every P row one-hot, so dQ = dK = 0 and dV_j = sum over the group of dO_j.
def pin_bwd_invariants():
    rng = np.random.default_rng(53)
    B, N, H, Hkv, d = 2, 30, 4, 2, 6
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    g = rng.standard_normal(q.shape)
    gs = g.reshape(B, N, Hkv, H // Hkv, d).sum(axis=3)               # group sums of dO per position
    for causal in (False, True):
        dq, dk, dv = oracle.attn_bwd_f64(q, k, v, g, causal, 0.45)
        assert np.max(np.abs(dk.sum(axis=1))) < 1e-12, "sum_j dK_j = 0"
        _close(dv.sum(axis=1), gs.sum(axis=1), 1e-12, "sum_j dV_j = sum_i dO_i")
    dq, dk, dv = oracle.attn_bwd_f64(q, k, v, g, False, 0.45, (0, 0))
    assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk)) < 1e-15, "one-hot P: dQ = dK = 0"
    _close(dv, gs, 1e-14, "one-hot P: dV_j = group sum of dO_j")


# Decode / split-KV. The pages name work-centric and split decode schedules (the Lean
# Attention and Stream-K titles in the reference lists) without defining them; the reading:
# Nq queries are the last Nq positions of a sequence of Nk keys.
# P25 -- the rectangular forward equals the last Nq rows of the square forward over Nk
# positions (causal and not), reduces to it at Nq = Nk, and matches torch's float64 SDPA
# with an explicit bottom-right mask.
def pin_decode_rectangular():
    rng = np.random.default_rng(61)
    for B, H, Hkv, Nq, Nk, d in ((1, 4, 2, 1, 50, 8), (2, 2, 1, 7, 40, 16), (1, 2, 2, 13, 13, 4)):
        q_full, k, v = _qkv(rng, B, Nk, H, Hkv, d)
        q = np.ascontiguousarray(q_full[:, Nk - Nq:])
        for causal in (False, True):
            o, lse = oracle.attn_fwd_kv_f64(q, k, v, causal, 0.35)
            of, lf = oracle.attn_fwd_f64(q_full, k, v, causal, 0.35)
            _close(o, of[:, Nk - Nq:], 1e-13, f"decode O = last rows of square (Nq{Nq} Nk{Nk} c{causal})")
            _close(lse, lf[:, :, Nk - Nq:], 1e-13, "decode lse = last rows of square")
            keep = np.ones((Nq, Nk), dtype=bool)
            if causal:
                keep = np.arange(Nk)[None, :] <= (Nk - Nq + np.arange(Nq))[:, None]
            t = lambda x: torch.from_numpy(x).permute(0, 2, 1, 3)
            ref = F.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=torch.from_numpy(keep), scale=0.35,
                                                 enable_gqa=(H != Hkv)).permute(0, 2, 1, 3).numpy()
            _close(o, ref, 1e-12, "decode vs sdpa with bottom-right mask")


# P28 -- row selection: the single-row entry points (used to check full-size outputs one
# row at a time) return exactly the rows of the whole-tensor functions, which the other
# pins tie to the definition: plain, causal, key windows, block masks (shared and per-head,
# causal, empty rows), and the stored-input entries that decode only the selected queries.
def pin_row_selection():
    rng = np.random.default_rng(45)
    B, N, H, Hkv, d = 2, 70, 4, 2, 8
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    rows = np.array([[b, h, i] for b in range(B) for h in range(H) for i in range(N)])
    rows = rows[rng.permutation(len(rows))[:160]]           # shuffled: output order follows rows
    qr = q[rows[:, 0], rows[:, 2], rows[:, 1]]
    for causal in (False, True):
        for window in (None, (5, -1), (3, 9), (-1, 0), (0, 0), (-1, 12)):
            o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.3, window)
            orow, lrow = oracle.attn_rows_f64(qr, k, v, H, rows, causal, 0.3, window)
            assert np.array_equal(orow, o[rows[:, 0], rows[:, 2], rows[:, 1]]), f"rows o causal={causal} w={window}"
            assert np.array_equal(lrow, lse[rows[:, 0], rows[:, 1], rows[:, 2]]), f"rows lse causal={causal} w={window}"
    nb = (N + 15) // 16
    shared = (rng.random((1, nb, nb)) < 0.5).astype(np.uint8)
    shared[0, 2, :] = 0                                      # an empty block row
    per_head = (rng.random((H, nb, nb)) < 0.4).astype(np.uint8)
    for mask in (shared, per_head):
        for causal in (False, True):
            o, lse = oracle.attn_fwd_block_f64(q, k, v, causal, 0.3, mask, 16)
            orow, lrow = oracle.attn_rows_block_f64(qr, k, v, H, rows, causal, 0.3, mask, 16)
            assert np.array_equal(orow, o[rows[:, 0], rows[:, 2], rows[:, 1]]), f"block rows o causal={causal}"
            assert np.array_equal(lrow, lse[rows[:, 0], rows[:, 1], rows[:, 2]]), f"block rows lse causal={causal}"
            assert np.any(np.isneginf(lse)) or mask is per_head, "the empty block row is exercised"
    # stored-input entries (bit patterns), including the e4m3 descales
    raw = {x: np.asarray(torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
                         ).view(np.uint16) for x, a in zip("qkv", (q, k, v))}
    for causal, window in ((False, None), (True, (6, -1))):
        o, lse = oracle.attn_fwd(raw["q"], raw["k"], raw["v"], "bf16", causal, 0.3, window=window)
        orow, lrow = oracle.attn_rows(raw["q"], raw["k"], raw["v"], "bf16", causal, 0.3, rows, window=window)
        assert np.array_equal(orow, o[rows[:, 0], rows[:, 2], rows[:, 1]]), "stored-input rows"
        assert np.array_equal(lrow, lse[rows[:, 0], rows[:, 1], rows[:, 2]]), "stored-input rows lse"
    mask64 = (rng.random((H, 2, 2)) < 0.7).astype(np.uint8)
    o, lse = oracle.attn_fwd_block(raw["q"], raw["k"], raw["v"], "bf16", True, 0.3, mask64)
    orow, lrow = oracle.attn_rows_block(raw["q"], raw["k"], raw["v"], "bf16", True, 0.3, rows, mask64)
    assert np.array_equal(orow, o[rows[:, 0], rows[:, 2], rows[:, 1]]), "stored-input block rows"
    assert np.array_equal(lrow, lse[rows[:, 0], rows[:, 1], rows[:, 2]]), "stored-input block rows lse"
    e8 = {x: rng.integers(0, 256, (B, N, hh, d)).astype(np.uint8) for x, hh in zip("qkv", (H, Hkv, Hkv))}
    for x in e8:
        e8[x][(e8[x] & 0x7F) == 0x7F] = 0                    # no NaN codes
    ds = (0.01, 0.02, 0.5)
    o, lse = oracle.attn_fwd(e8["q"], e8["k"], e8["v"], "e4m3", False, 0.3, ds)
    orow, lrow = oracle.attn_rows(e8["q"], e8["k"], e8["v"], "e4m3", False, 0.3, rows, ds)
    assert np.array_equal(orow, o[rows[:, 0], rows[:, 2], rows[:, 1]]), "e4m3 rows"


# P29 -- block dequantisation: every value equals its code's e4m3 value (torch's
# float8_e4m3fn decode) times 2^(byte - 127) of its 64-row block, expanded with np.repeat;
# and a round trip through block_quantize stays within half an e4m3 step of the input
# (after the block's power-of-two scaling), for normal and subnormal codes.
def pin_block_dequantize():
    rng = np.random.default_rng(46)
    B, N, Hx, d, br = 2, 150, 3, 32, 64
    nb = (N + br - 1) // br
    codes = rng.integers(0, 256, (B, N, Hx, d)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3F                     # no NaN codes
    scales = rng.integers(100, 150, (B, Hx, nb)).astype(np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mult = np.repeat(np.exp2(scales.astype(np.float64) - 127.0), br, axis=2)[:, :, :N]    # [B, Hx, N]
    ref = vals * np.transpose(mult, (0, 2, 1))[..., None]
    got = oracle.block_dequantize(codes, scales, br)
    assert got.shape == ref.shape and np.array_equal(got, ref), "block_dequantize vs repeat expansion"
    x = rng.standard_normal((B, N, Hx, d)) * np.exp(rng.uniform(-6, 6, (B, 1, Hx, 1)))
    x[0, :, 0, :4] *= 1e-3                                   # values in the subnormal range of their block
    c, sc = oracle.block_quantize(x, br)
    y = oracle.block_dequantize(c, sc, br)
    e = np.transpose(np.repeat(sc.astype(np.float64) - 127.0, br, axis=2)[:, :, :N], (0, 2, 1))[..., None]
    z = np.abs(x) * np.exp2(-e)                               # scaled magnitudes, <= 448
    assert np.all(z <= 448.0), "scaled values fit e4m3"
    half = np.where(z >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(z, 2.0 ** -6))) - 4), 2.0 ** -10)
    err = np.abs(y - x) * np.exp2(-e)
    assert np.all(err <= half * (1 + 1e-12)), f"round trip beyond half an e4m3 step ({(err > half).sum()})"
    assert np.any(err > 0.9 * half), "the bound is reached (a tight check)"


# P30 -- gradient rows: the selected-row gradient entry points (dQ rows; dK and dV of key
# rows, which take the forward's O and lse) equal the whole-tensor gradient of
# attn_bwd_f64, pinned by P22-P24; their absolute-value sums equal a numpy evaluation of
# the same sums from the probability matrix.
def pin_bwd_rows():
    rng = np.random.default_rng(47)
    B, N, H, Hkv, d = 2, 41, 4, 2, 8
    q, k, v = _qkv(rng, B, N, H, Hkv, d)
    g = rng.standard_normal((B, N, H, d))
    g_ = H // Hkv
    for causal in (False, True):
        dq, dk, dv = oracle.attn_bwd_f64(q, k, v, g, causal, 0.4)
        o, lse = oracle.attn_fwd_f64(q, k, v, causal, 0.4)
        qrows = np.array([[b, h, i] for b in range(B) for h in range(H) for i in range(N)])[::3]
        dqr, qmag = oracle.attn_bwd_dq_rows_f64(q, k, v, g, causal, 0.4, qrows, with_mag=True)
        _close(dqr, dq[qrows[:, 0], qrows[:, 2], qrows[:, 1]], 1e-13, f"dq rows causal={causal}")
        krows = np.array([[b, hk, j] for b in range(B) for hk in range(Hkv) for j in range(N)])[::-2]
        dkr, dvr, kmag = oracle.attn_bwd_dkdv_rows_f64(q, k, v, g, causal, 0.4, krows, (o, lse), with_mag=True)
        _close(dkr, dk[krows[:, 0], krows[:, 2], krows[:, 1]], 1e-13, f"dk rows causal={causal}")
        _close(dvr, dv[krows[:, 0], krows[:, 2], krows[:, 1]], 1e-13, f"dv rows causal={causal}")
        dkr2, dvr2 = oracle.attn_bwd_dkdv_rows_f64(q, k, v, g, causal, 0.4, krows)
        assert np.array_equal(dkr, dkr2) and np.array_equal(dvr, dvr2), "fwd computed inside"
        for b in range(B):
            for h in range(H):
                hk = h // g_
                P = oracle.attn_probs_f64(q, k, b, h, causal, 0.4)
                dS = P * (g[b, :, h] @ v[b, :, hk].T - np.sum(g[b, :, h] * o[b, :, h], axis=1)[:, None])
                w = np.sum(np.abs(g[b, :, h] * o[b, :, h]), axis=1)
                sel = (qrows[:, 0] == b) & (qrows[:, 1] == h)
                i = qrows[sel, 2]
                _close(qmag[sel, 0], np.abs(dS[i]) @ np.abs(k[b, :, hk]), 1e-12, "dq |dS||k|")
                _close(qmag[sel, 1], P[i] @ np.abs(k[b, :, hk]), 1e-12, "dq P|k|")
        for r, (b, hk, j) in enumerate(krows):
            m = np.zeros((3, d))
            for h in range(hk * g_, (hk + 1) * g_):
                P = oracle.attn_probs_f64(q, k, b, h, causal, 0.4)
                dS = P * (g[b, :, h] @ v[b, :, hk].T - np.sum(g[b, :, h] * o[b, :, h], axis=1)[:, None])
                w = np.sum(np.abs(g[b, :, h] * o[b, :, h]), axis=1)
                m[0] += np.abs(dS[:, j]) @ np.abs(q[b, :, h])
                m[1] += (P[:, j] * w) @ np.abs(q[b, :, h])
                m[2] += P[:, j] @ np.abs(g[b, :, h])
            _close(kmag[r], m, 1e-12, "dk/dv magnitude sums")


ALL_PINS = [pin_mpmath_bruteforce, pin_torch_sdpa, pin_zero_query, pin_single_key, pin_two_keys,
            pin_affine_in_v, pin_probability_rows, pin_key_permutation, pin_key_shift, pin_gqa_repeat,
            pin_causal_prefix, pin_split_merge, pin_hardmax_and_range, pin_decoders, pin_golden_fixtures,
            pin_window_bruteforce_and_sdpa, pin_window_closed_forms, pin_window_reductions,
            pin_e4m3_encode, pin_fwht, pin_block_quantize, pin_rotation_identity,
            pin_bwd_finite_differences, pin_bwd_torch_autograd, pin_bwd_invariants, pin_decode_rectangular,
            pin_block_sparse_bruteforce_and_sdpa, pin_block_sparse_reductions, pin_row_selection,
            pin_block_dequantize, pin_bwd_rows]
