"""The library inside HIP graphs and on a non-default stream (GPU): forward (plain,
key-window, block-sparse, per-tensor e4m3, block-scaled e4m3 in both Q K^T modes), the
block quantiser, gradient, split-KV decode and its allocation-free variant are captured
once into a torch CUDA graph (hipGraph) with preallocated
outputs and workspaces, replayed several times with eager work in between, and every
replay must equal the eager result bit for bit. The kernels enqueue no memset and
allocate nothing, so capture needs no special path."""
import numpy as np
import pytest
import torch

import exact_tiled_attention_03_amd as fa
import synth_inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t


def test_graph_replays_match_eager():
    B, H, Hkv, N, d = 1, 4, 2, 300, 128
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, "bf16", seed=21)
    q, k, v = (gu.to_dev(inp[x], "bf16") for x in "qkv")
    do = gu.to_dev(synth_inputs.make_dout(B, N, H, d, "bf16", 22), "bf16")
    dec = synth_inputs.make_decode_inputs(2, 8, 2, 2, 500, d, "bf16", 23)
    dq_, dk_, dv_ = (gu.to_dev(dec[x], "bf16") for x in "qkv")

    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N) // 4, device="cuda")
    od = torch.empty_like(dq_)
    lsed = torch.empty(2, 8, 2, device="cuda")
    wsd = torch.empty(fa.fa_fwd_splitkv_workspace_bytes(2, 8, 2, 2, 500, d, 4) // 4, device="cuda")
    ow, lsew = torch.empty_like(q), torch.empty(B, H, N, device="cuda")
    os_, lses = torch.empty_like(q), torch.empty(B, H, N, device="cuda")
    bmask = torch.from_numpy(synth_inputs.random_block_mask(H, N, 0.5, seed=24)).cuda()

    def work():
        fa.fwd(q, k, v, causal=True, out=o, lse=lse)
        fa.bwd(q, k, v, o, lse, do, causal=True, dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws)
        fa.fwd_splitkv(dq_, dk_, dv_, causal=True, num_splits=4, out=od, lse=lsed, workspace=wsd)
        fa.fwd(q, k, v, causal=True, window=(100, -1), out=ow, lse=lsew)
        fa.fwd_block_sparse(q, k, v, bmask, causal=False, out=os_, lse=lses)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, lse, *grads, od, lsed, ow, lsew, os_, lses)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        for t in (o, lse, *grads, od, lsed, ow, lsew, os_, lses):
            t.fill_(float("nan")) if t.dtype == torch.float32 else t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        names = ("o", "lse", "dq", "dk", "dv", "o_dec", "lse_dec", "o_win", "lse_win", "o_sparse", "lse_sparse")
        for name, a, b in zip(names, (o, lse, *grads, od, lsed, ow, lsew, os_, lses), eager):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: {name} differs from eager"
        _ = (q.float() * 2).sum().item()         # unrelated eager work between replays


def test_non_default_stream():
    B, H, Hkv, N, d = 2, 4, 4, 200, 64
    inp = synth_inputs.make_inputs(B, H, Hkv, N, d, "f16", seed=24)
    q, k, v = (gu.to_dev(inp[x], "f16") for x in "qkv")
    ref_o, ref_l = fa.fwd(q, k, v)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.fwd(q, k, v)                 # enqueued on s (the current stream)
    s.synchronize()
    assert torch.equal(_bits(o), _bits(ref_o)) and torch.equal(lse, ref_l)


def test_graph_replays_match_eager_e4m3_and_static_scratch():
    """The e4m3 paths (per-tensor forward, block quantiser, block-scaled forward with Q K^T
    on the bf16 and on the e4m3 MFMA) and the allocation-free split-KV entry point, captured
    and replayed like the test above."""
    B, H, Hkv, N, d = 1, 4, 2, 300, 128
    e8 = synth_inputs.make_inputs(B, H, Hkv, N, d, "e4m3", seed=31, outlier_frac=1e-3)
    q8, k8, v8 = (torch.from_numpy(np.ascontiguousarray(e8[x])).cuda() for x in "qkv")
    bf = synth_inputs.make_inputs(B, H, Hkv, N, d, "bf16", seed=32)
    qb, kb, vb = (gu.to_dev(bf[x], "bf16") for x in "qkv")
    signs = torch.from_numpy(synth_inputs.random_signs(d, 33)).cuda()
    dec = synth_inputs.make_decode_inputs(2, 8, 2, 2, 500, d, "bf16", 34)
    dq_, dk_, dv_ = (gu.to_dev(dec[x], "bf16") for x in "qkv")

    o8 = torch.empty(B, N, H, d, dtype=torch.bfloat16, device="cuda")
    l8 = torch.empty(B, H, N, device="cuda")
    qz = [fa.quantize_e4m3_block(x, sg) for x, sg in ((qb, signs), (kb, signs), (vb, None))]
    (qc, qs), (kc, ks), (vc, vs) = qz
    ob0, lb0 = torch.empty_like(o8), torch.empty_like(l8)
    ob1, lb1 = torch.empty_like(o8), torch.empty_like(l8)
    od = torch.empty_like(dq_)
    ld = torch.empty(2, 8, 2, device="cuda")
    outs = (o8, l8, qc, qs, kc, ks, vc, vs, ob0, lb0, ob1, lb1, od, ld)

    def work():
        fa.fwd(q8, k8, v8, scale=1.0 / np.sqrt(d), descale=e8["descale"], dtype="e4m3", out=o8, lse=l8)
        for (x, sg), (c, sc) in zip(((qb, signs), (kb, signs), (vb, None)), qz):
            fa.quantize_e4m3_block(x, sg, codes=c, scales=sc)
        fa.fwd_fp8_block(qc, kc, vc, qs, ks, vs, causal=True, scale=1.0 / np.sqrt(d) / d, out=ob0, lse=lb0)
        fa.fwd_fp8_block(qc, kc, vc, qs, ks, vs, causal=True, scale=1.0 / np.sqrt(d) / d, out=ob1, lse=lb1,
                         qk_e4m3=True)
        fa.fwd_splitkv_static(dq_, dk_, dv_, od, ld, causal=True, num_splits=4)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    names = ("o_e4m3", "lse_e4m3", "q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales",
             "o_block", "lse_block", "o_block_qk8", "lse_block_qk8", "o_static", "lse_static")
    for rep in range(3):
        for t in outs:
            if t.dtype == torch.float32:
                t.fill_(float("nan"))
            else:
                t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, eager):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep}: {name} differs from eager"
        _ = (qb.float() * 2).sum().item()        # unrelated eager work between replays
