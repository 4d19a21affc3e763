"""The library's environment switches (GPU): FA_LOG=1 names every launched kernel with its
template arguments and grid on stderr, and FA_FORCE_VARIANT=fp8_block_qk=bf16|e4m3 overrides
the qk_e4m3 argument of fa_fwd_fp8_block. Each case runs in a child process, because the
library reads the environment once."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SNIPPET = r"""
import sys, torch
sys.path.insert(0, {root!r})
import exact_tiled_attention_03_amd as fa
g = torch.Generator().manual_seed(0)
q, k, v = (torch.randn(1, 300, 4, 128, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
if {what!r} == "fwd":
    fa.fwd(q, k, v, causal=True)
else:
    signs = (torch.randint(0, 2, (128,), generator=g) * 2 - 1).float().cuda()
    (qc, qs), (kc, ks), (vc, vs) = (fa.quantize_e4m3_block(x, s) for x, s in ((q, signs), (k, signs), (v, None)))
    o, lse = fa.fwd_fp8_block(qc, kc, vc, qs, ks, vs, causal=False, scale=1.0 / 128 ** 1.5, qk_e4m3=True)
    assert bool(torch.isfinite(o.float()).all())
torch.cuda.synchronize()
print("done", flush=True)
"""


def _run(what, **env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, "-c", SNIPPET.format(root=ROOT, what=what)], env=e, cwd=ROOT,
                       capture_output=True, text=True, timeout=240)
    print(r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-2000:]
    return [l for l in r.stderr.splitlines() if l.startswith("fa: ")]


def test_fa_log_names_the_launch():
    lines = _run("fwd", FA_LOG="1")
    assert len(lines) == 1, lines
    assert lines[0].startswith("fa: fa_fwd_overlap_kernel [") and "D = 128" in lines[0] and "grid 8 block 512" in lines[0], lines


def test_fa_log_off_by_default():
    assert _run("fwd", FA_LOG="0") == []


@pytest.mark.parametrize("force,kernel", [(None, "fa_fwd_e4m3qk_kernel"), ("fp8_block_qk=bf16", "fa_fwd_fp8_kernel"),
                                          ("fp8_block_qk=e4m3", "fa_fwd_e4m3qk_kernel")])
def test_force_variant_fp8_block_qk(force, kernel):
    env = {"FA_LOG": "1"}
    if force:
        env["FA_FORCE_VARIANT"] = force
    lines = _run("fp8", **env)
    assert sum(l.startswith("fa: quantize_e4m3_block_kernel") for l in lines) == 3, lines
    attn = [l for l in lines if not l.startswith("fa: quantize")]
    assert len(attn) == 1 and attn[0].startswith(f"fa: {kernel} ["), lines
