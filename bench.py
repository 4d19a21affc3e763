"""Benchmark of the attention forward hot path on one MI355X.

A step is one attention forward (one fa_fwd launch through the C ABI, fa_fwd_local for
a key-window workload, fa_fwd_block_sparse for a block-sparse one) over the whole
workload, inputs resident in HBM. Prints one JSON line with TFLOP/s counted as
4*B*H*N^2*d (halved under the causal mask; for a key window or a block mask, 4*B*d times
the visible (query, key) pairs over the heads), the roofline of the kernel (achieved
TFLOP/s from HIP events on the launch stream against the dense bf16/f16 MFMA peak) and
the fp64 CPU oracle timed on the host cores on a bounded sample of the same workload.
The default workload is causal grouped-query attention, bf16, B4 Hq32 Hkv8 N8192 d128.
The timed steps run as 5 event-timed windows; the roofline uses their median (the min is
reported too), and the driver's current shader clock is sampled during them.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --mode copy      # plain device copy of known size, for counter scaling
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth_inputs  # noqa: E402

DEFAULT_WORKLOAD = "gqa_causal_bf16_b4_h32_kv8_n8192_d128"
WINDOWS = 5          # the timed steps are split into this many event-timed windows
# Dense MFMA peak of MI355X: 256 CUs x 4 SIMDs x 2.4 GHz x (1024 bf16/f16 or 2048 fp8 FLOP/clk/SIMD)
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "e4m3": 5033.2}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
METRIC = "attention fwd TFLOP/s (4*B*H*N^2*d, causal halved) and % MFMA peak, bf16 d=128"


def source_hash(path: str) -> str:
    return hashlib.sha256(open(os.path.join(ROOT, path), "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per step from the committed rocprofv3 counter summary, if it was taken on
    the current sources of every kernel the step runs; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get("workloads", {}).get(workload)
    if not entry:
        return None
    try:
        if any(source_hash(path) != sha for path, sha in entry.get("kernel_sources", {}).items()):
            return None
    except OSError:
        return None
    return entry.get("hbm_bytes_per_launch")


def to_dev(bits, dtype):
    if dtype == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(bits)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def cpu_baseline(w: synth_inputs.Workload, inp: dict, budget_s: float = 12.0):
    """The fp64 oracle on a bounded sample: whole (batch, GQA group) slices of the same
    inputs, in order, until about budget_s seconds of wall time on the host cores (for a
    block-quantised workload: the oracle's block quantisation of the slice, then attention
    on the dequantised values)."""
    import oracle
    dq, dk, dv = inp["descale"] if inp["descale"] else (1.0, 1.0, 1.0)
    signs = synth_inputs.random_signs(w.d, w.seed) if w.fp8_block else None

    if w.backward:
        dout = synth_inputs.make_dout(w.B, w.N, w.H, w.d, w.dtype, w.seed + 100)

    if w.decode_nq:
        t0 = time.perf_counter()
        bs = 0
        while bs < w.B and time.perf_counter() - t0 < budget_s:
            sl = lambda n: oracle.decode(np.ascontiguousarray(inp[n][bs:bs + 1]), w.dtype)
            oracle.attn_fwd_kv_f64(sl("q"), sl("k"), sl("v"), w.causal, w.scale)
            bs += 1
        el = time.perf_counter() - t0
        fl = w.flops * bs / w.B
        return {"value": fl / el / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
                "cpu_model": cpu_model(),
                "sample": f"first {bs} of {w.B} batches of {w.name} ({fl / 1e9:.2f} GFLOP, {el:.1f} s in fp64)"}

    def prep(x, sg):
        if not w.fp8_block:
            return x
        return oracle.block_dequantize(*oracle.block_quantize(x, 64, sg))
    g = w.H // w.Hkv
    per_head = w.flops / (w.B * w.H)
    bmask = synth_inputs.workload_block_mask(w) if w.sparse_density else None
    heads, elapsed, flops = 0, 0.0, 0.0
    for b in range(w.B):
        if elapsed >= budget_s:
            break
        q = oracle.decode(inp["q"][b:b + 1], w.dtype, dq)
        k = oracle.decode(inp["k"][b:b + 1], w.dtype, dk)
        v = oracle.decode(inp["v"][b:b + 1], w.dtype, dv)
        for hk in range(w.Hkv):
            if elapsed >= budget_s:
                break
            t0 = time.perf_counter()
            qs = prep(np.ascontiguousarray(q[:, :, hk * g:(hk + 1) * g]), signs)
            ks = prep(np.ascontiguousarray(k[:, :, hk:hk + 1]), signs)
            vs = prep(np.ascontiguousarray(v[:, :, hk:hk + 1]), None)
            if w.backward:
                ds = oracle.decode(dout[b:b + 1, :, hk * g:(hk + 1) * g], w.dtype)
                oracle.attn_bwd_f64(qs, ks, vs, ds, w.causal, w.scale)
            elif bmask is not None:
                mh = bmask[hk * g:(hk + 1) * g]
                oracle.attn_fwd_block_f64(qs, ks, vs, w.causal, w.scale, mh)
            else:
                oracle.attn_fwd_f64(qs, ks, vs, w.causal, w.scale / (w.d if w.fp8_block else 1), w.window)
            elapsed += time.perf_counter() - t0
            heads += g
            flops += (4.0 * w.d * synth_inputs.block_mask_pairs(mh, w.N, w.causal, g) if bmask is not None
                      else per_head * g)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {heads} of {w.B * w.H} (batch, head) slices of {w.name} in memory order, "
                      f"whole slices ({flops / 1e9:.1f} GFLOP, {elapsed:.1f} s in fp64)"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class ClockSampler:
    """Samples the GPU shader clock from the driver's sysfs files while running (the
    current DPM level of pp_dpm_sclk, else hwmon freq1_input), every ~10 ms on a host
    thread. The samples are the driver's reported current clock, not a counter."""

    def __init__(self):
        import glob
        import threading
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.hwmon = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/freq1_input"))
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def read(self):
        for p in self.paths:
            try:
                for line in open(p):
                    if "*" in line:
                        return float(line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", ""))
            except (OSError, ValueError, IndexError):
                continue
        for p in self.hwmon:
            try:
                return float(open(p).read()) / 1e6
            except (OSError, ValueError):
                continue
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self.read()
            if v is not None:
                self.samples.append(v)
            self._stop.wait(0.01)

    def __enter__(self):
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        a = np.array(self.samples)
        src = "pp_dpm_sclk" if self.paths else "hwmon freq1_input"
        return {"median_MHz": float(np.median(a)), "min_MHz": float(a.min()), "max_MHz": float(a.max()),
                "samples": int(a.size), "source": f"driver sysfs {src} (current level, sampled every ~10 ms)"}


def run_copy():
    """A plain device copy of known size: the reference for the HBM counters' scale, and
    the copy rate this machine reaches, the practical ceiling of the HBM-bound kernels."""
    n = 1 << 28  # 2^28 float32 = 1 GiB read, 1 GiB written per copy
    x = torch.ones(n, device="cuda", dtype=torch.float32)
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    timed = 20
    e0.record(stream)
    for _ in range(timed):
        y.copy_(x)
    e1.record(stream)
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / timed * 1e-3
    print(json.dumps({"mode": "copy", "bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
                      "launches": 5 + timed, "ms_per_copy": s * 1e3,
                      "TBps_moved": 2 * n * 4 / s / 1e12}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(synth_inputs.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", default="attn", choices=["attn", "copy"])
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention forward here is a single-GPU kernel "
              "library with no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy":
        run_copy()
        return

    import exact_tiled_attention_03_amd as fa

    w = synth_inputs.WORKLOADS[args.workload]
    inp = synth_inputs.workload_inputs(w)
    q, k, v = (to_dev(inp[x], w.dtype) for x in "qkv")
    dt = w.dtype if w.dtype == "e4m3" else None
    stream = torch.cuda.current_stream()
    quant = None
    if w.fp8_block:
        # block quantisation (Q and K rotated) on the GPU, timed on its own; the step is
        # the attention on the quantised codes, as for the per-tensor e4m3 workload
        signs = torch.from_numpy(synth_inputs.random_signs(w.d, w.seed)).cuda()
        qz = [fa.quantize_e4m3_block(x, sg) for x, sg in ((q, signs), (k, signs), (v, None))]
        reps = 20
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for (x, sg), (c, sc) in zip(((q, signs), (k, signs), (v, None)), qz):
                fa.quantize_e4m3_block(x, sg, codes=c, scales=sc)
        e1.record(stream)
        torch.cuda.synchronize()
        q_ms = e0.elapsed_time(e1) / reps
        nbytes = sum(x.numel() * 3 + sc.numel() for x, (c, sc) in zip((q, k, v), qz))
        quant = {"kernel": "quantize_e4m3_block (q, k, v)", "ms": round(q_ms, 5),
                 "bytes": nbytes, "achieved_GBps": round(nbytes / (q_ms * 1e-3) / 1e9, 1), "peak_GBps": 8000.0,
                 "frac": round(nbytes / (q_ms * 1e-3) / 1e9 / 8000.0, 4)}
        (qc, qs), (kc, ks), (vc, vs) = qz

        def step(o=None, lse=None):
            return fa.fwd_fp8_block(qc, kc, vc, qs, ks, vs, causal=w.causal, scale=w.scale / w.d, out=o, lse=lse,
                                    qk_e4m3=True)
    elif w.decode_nq:
        # split-KV decode: a step is one fa_fwd_splitkv call (partials + merge)
        nbytes = fa.fa_fwd_splitkv_workspace_bytes(w.B, w.H, w.Hkv, w.decode_nq, w.N, w.d, 0)
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")

        def step(o=None, lse=None):
            return fa.fwd_splitkv(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=ws)
    elif w.sparse_density:
        # block-sparse: a step is one fa_fwd_block_sparse call; the mask is resident
        bmask = torch.from_numpy(synth_inputs.workload_block_mask(w)).cuda()

        def step(o=None, lse=None):
            return fa.fwd_block_sparse(q, k, v, bmask, causal=w.causal, scale=w.scale, out=o, lse=lse)
    elif w.backward:
        # the gradient pass: the forward's o and lse are computed once, outside the timed
        # region; a step is one fa_bwd call (three launches)
        fo, flse = fa.fwd(q, k, v, causal=w.causal, scale=w.scale)
        dout = to_dev(synth_inputs.make_dout(w.B, w.N, w.H, w.d, w.dtype, w.seed + 100), w.dtype)
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
        ws = torch.empty(fa.fa_bwd_workspace_bytes(w.B, w.H, w.N) // 4, dtype=torch.float32, device="cuda")

        def step(o=None, lse=None):
            fa.bwd(q, k, v, fo, flse, dout, causal=w.causal, scale=w.scale, dq=grads[0], dk=grads[1], dv=grads[2],
                   workspace=ws)
            return grads[0], flse
    else:
        def step(o=None, lse=None):
            return fa.fwd(q, k, v, causal=w.causal, scale=w.scale, descale=inp["descale"], dtype=dt, out=o,
                          lse=lse, window=w.window)
    o, lse = step()
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all()), "non-finite output"

    for _ in range(args.warmup):
        step(o, lse)
    # the K timed steps run as WINDOWS consecutive windows, each bracketed by HIP events on
    # the launch stream; the wall clock covers all K
    nwin = max(1, min(WINDOWS, args.steps))
    sizes = [args.steps // nwin + (1 if i < args.steps % nwin else 0) for i in range(nwin)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nwin + 1)]
    torch.cuda.synchronize()
    with ClockSampler() as clocks:
        t0 = time.perf_counter()
        evs[0].record(stream)
        for i, n in enumerate(sizes):
            for _ in range(n):
                step(o, lse)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    win_ms = [evs[i].elapsed_time(evs[i + 1]) / n for i, n in enumerate(sizes)]
    kernel_ms = float(np.median(win_ms))

    ms_per_step = wall * 1e3 / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (kernel_ms * 1e-3) / 1e12
    cdt = "e4m3" if w.fp8_block else w.dtype
    peak = PEAK_TFLOPS[cdt]
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": measured_traffic(w.name), "kernel_ms": round(kernel_ms, 5),
            "kernel_ms_min": round(min(win_ms), 5), "window_ms": [round(x, 5) for x in win_ms],
            "timing": f"median (and min) over {nwin} event-timed windows of the {args.steps} timed steps",
            "achieved_at_min": round(w.flops / (min(win_ms) * 1e-3) / 1e12, 2)}
    if w.decode_nq:
        # decode reads every K/V element once: HBM-bound; algorithmic bytes = Q + K + V + O + lse
        el = 2
        alg = (w.B * w.decode_nq * w.H * w.d * el * 2 + 2 * w.B * w.N * w.Hkv * w.d * el + 4 * w.B * w.H * w.decode_nq)
        gbps = alg / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s",
                "frac": round(gbps / 8000.0, 4), "traffic": measured_traffic(w.name), "kernel_ms": round(kernel_ms, 5),
                "kernel_ms_min": round(min(win_ms), 5), "window_ms": [round(x, 5) for x in win_ms],
                "algorithmic_bytes": alg}
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cdt,
        "data": "synthetic (seeded N(0,1) inputs)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   **({"pass": "backward (dq, dk, dv; FLOP = 2.5x forward)"} if w.backward else {}),
                   **({"Nq": w.decode_nq, "Nk": w.N, "pass": "split-KV decode"} if w.decode_nq else {}),
                   "causal": w.causal, "scale": w.scale, "flop_per_step": w.flops,
                   **({"window": list(w.window)} if w.window else {}),
                   **({"block_sparse": {"block": synth_inputs.SPARSE_BLOCK, "mask_heads": w.H,
                                        "kept_blocks": round(float(synth_inputs.workload_block_mask(w).mean()), 4),
                                        "pattern": "local + global + random key blocks per 256-query group"}}
                      if w.sparse_density else {}),
                   **({"fp8": "block scales (64 rows, E8M0), Hadamard-rotated q/k, Q K^T on the e4m3 MFMA"}
                      if w.fp8_block else {})},
        "roofline": roof,
        "sclk": clocks.summary(),
    }
    if quant:
        out["quantize"] = quant
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
