"""Benchmark of the attention forward hot path on one MI355X.

A step is one attn_fwd call over the headline workload (B=1, H=32,
Sq=Skv=8192, d=128, bf16, non-causal), inputs resident in HBM.  The JSON line
reports whole-job TFLOP/s (4*B*H*Sq*Skv*d flop per step), the prefill
kernel's roofline (MFMA bf16 peak), the median and minimum step, the fp64
CPU oracle timed on every row of the same workload (also the reference of
the headline's parity record; sampled rows for the other forward workloads),
and, under "workloads", the other shapes: the
causal 8K run, the 2K d=64 causal run, varlen grouped-query prefill,
sliding-window attention with sinks at 32K tokens, split-KV decode over a
contiguous and a paged cache (HBM roofline), and the backward pass of the
8K shape (useful TFLOP/s, counted as 2.5 times the forward's).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E, published
METRIC = "attention fwd TFLOP/s (% bf16 MFMA peak) prefill; decode HBM GB/s (% peak)"
HEADLINE = "mha_s8192_d128"
PROFILES = os.path.join(ROOT, "profiles")


# the sources each measured workload's kernels are built from: a counter
# summary under profiles/ is used only while these files are unchanged
KERNEL_SOURCES = {
    "mha_s8192_d128": ("attn_prefill_pp.hip", "attn_common.h", "attn_internal.h"),
    "decode_gqa_s16384_d128": ("attn_decode_bf16.hip", "attn_combine.hip", "attn_common.h", "attn_internal.h"),
    "bwd_mha_s8192_d128": ("attn_backward.hip", "attn_common.h", "attn_internal.h"),
}


def kernel_source_sha(workload: str = HEADLINE) -> str:
    h = hashlib.sha256()
    for name in sorted(KERNEL_SOURCES[workload]):
        with open(os.path.join(ROOT, "exact_attention_09_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def provenance(wl) -> dict:
    """What identifies this measurement without the repository's history:
    the hashes of the kernel sources the profiles are keyed to, of the
    library that ran, and the input recipe."""
    from exact_attention_09_amd import synth
    lib = os.path.join(ROOT, "exact_attention_09_amd", "libattn09.so")
    h = hashlib.sha256()
    with open(lib, "rb") as f:
        for chunk in iter(lambda: f.read(1 << 20), b""):
            h.update(chunk)
    return {"kernel_source_sha16": {w: kernel_source_sha(w) for w in sorted(KERNEL_SOURCES)},
            "library_sha16": h.hexdigest()[:16],
            "inputs": (f"synth.normal_tensor, seed 1000 * {wl.wid} + tensor id (q {synth.TENSOR_Q}, k {synth.TENSOR_K}, "
                       f"v {synth.TENSOR_V}), bf16 of N(0, 1)")}


def read_traffic(workload: str):
    """HBM bytes per launch measured by rocprofv3 counters for the current
    kernel sources, or None when the summary is missing or stale."""
    path = os.path.join(PROFILES, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha(workload):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_steps(fn, steps: int, warmup: int, stream):
    """Warm up, then time `steps` calls back to back: wall clock between two
    device synchronisations, and HIP events on the launch stream at every step
    boundary (mean over the region, plus the median and minimum step)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mid = steps // 2
    median = per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])
    return {"wall_ms_per_step": 1e3 * wall / steps, "event_ms_mean": ev[0].elapsed_time(ev[steps]) / steps,
            "event_ms_median": median, "event_ms_min": per[0]}


def run_workload(name: str, steps: int, warmup: int, inputs=None, keep_outputs: bool = False):
    import numpy as np
    import torch

    import exact_attention_09_amd as ea
    from exact_attention_09_amd.workloads import WORKLOADS, to_device
    wl = WORKLOADS[name]
    x = inputs if inputs is not None else wl.make_inputs()
    q, k, v = (to_device(x[t], wl.dtype) for t in ("q", "k", "v"))
    cu = torch.from_numpy(x["cu_seqlens"]).cuda() if x["cu_seqlens"] is not None else None
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device)
    ws = None
    ns = 0
    if wl.Sq == 1 and not wl.varlen:
        ns = wl.num_splits or ea.attn_decode_num_splits(wl.B, wl.Hkv, wl.Skv)
        ws = torch.empty(ea.attn_workspace_bytes(wl.B, wl.H, wl.d, ns), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    if wl.paged:
        bt = torch.from_numpy(x["block_table"]).cuda()
        sl = torch.from_numpy(x["seqlens_k"]).cuda()
        lse = torch.empty((wl.B, wl.H), dtype=torch.float32, device=q.device)

        def step():
            ea.attn_fwd_paged(q, k, v, bt, sl, o, lse, scale=wl.scale, num_splits=ns, workspace=ws,
                              stream=stream.cuda_stream)
    elif wl.backward:
        dout = to_device(x["dout"], wl.dtype)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bws = torch.empty(ea.attn_bwd_workspace_bytes(1 if wl.varlen else wl.B, wl.H, wl.Sq), dtype=torch.uint8,
                          device="cuda")
        if wl.window > 0 or wl.sinks:
            sk = torch.from_numpy(x["sinks"]).cuda() if wl.sinks else None
            ds = torch.empty(wl.H, dtype=torch.float32, device="cuda") if wl.sinks else None
            # o, lse of the forward, untimed
            ea.attn_fwd_window_sink(q, k, v, o, lse, window=wl.window, sinks=sk, scale=wl.scale, cu_seqlens=cu)

            def step():
                ea.attn_bwd_window_sink(q, k, v, o, lse, dout, window=wl.window, sinks=sk, scale=wl.scale,
                                        cu_seqlens=cu, dq=dq, dk=dk, dv=dv, dsinks=ds, workspace=bws,
                                        stream=stream.cuda_stream)
        else:
            # o, lse of the forward, untimed
            ea.attn_fwd(q, k, v, o, lse, causal=wl.causal, scale=wl.scale, cu_seqlens=cu)

            def step():
                ea.attn_bwd(q, k, v, o, lse, dout, causal=wl.causal, scale=wl.scale, cu_seqlens=cu, dq=dq, dk=dk,
                            dv=dv, workspace=bws, stream=stream.cuda_stream)
    elif wl.window > 0 or wl.sinks:
        sk = torch.from_numpy(x["sinks"]).cuda() if wl.sinks else None

        def step():
            ea.attn_fwd_window_sink(q, k, v, o, lse, window=wl.window, sinks=sk, scale=wl.scale, cu_seqlens=cu,
                                    num_splits=ns, workspace=ws, stream=stream.cuda_stream)
    else:
        def step():
            ea.attn_fwd_ex(q, k, v, o, lse, causal=wl.causal, scale=wl.scale, cu_seqlens=cu, num_splits=ns,
                           workspace=ws, stream=stream.cuda_stream)

    t = time_steps(step, steps, warmup, stream)
    if keep_outputs and not wl.backward:
        # the last step's outputs, for the parity record
        t["outputs"] = (o.float().cpu().numpy(), lse.cpu().numpy())
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return wl, ns, t


def cpu_threads() -> int:
    """Host threads for the oracle: the cores, at most 16 (a GPU machine allots 16
    CPUs to each GPU)."""
    return max(1, min(16, os.cpu_count() or 1))


def parity_record(o, lse, o_ref, lse_ref, rows_compared: int) -> dict:
    """max |dO| (raw and against the bf16-rounded oracle), elements above
    1e-2, max |dLSE|, with positions (indices into the compared rows)."""
    import numpy as np
    o = np.asarray(o, np.float64)
    o_ref = np.asarray(o_ref, np.float64).reshape(o.shape)
    lse = np.asarray(lse, np.float64).reshape(-1)
    lse_ref = np.asarray(lse_ref, np.float64).reshape(-1)
    err = np.abs(o - o_ref)
    i = np.unravel_index(int(np.argmax(err)), err.shape)
    f = np.ascontiguousarray(o_ref.astype(np.float32)).view(np.uint32).astype(np.uint64)
    rb = (((f + 0x7FFF + ((f >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    fin = np.isfinite(lse_ref)
    same_inf = bool(np.array_equal(np.isneginf(lse), np.isneginf(lse_ref)))
    lerr = np.abs(lse[fin] - lse_ref[fin]) if fin.any() else np.zeros(1)
    j = int(np.argmax(lerr))
    return {"rows": int(rows_compared), "max_dO": float(err[i]), "argmax": [int(x) for x in i],
            "max_dO_vs_bf16_ref": float(np.abs(o - rb).max()), "n_over_1e-2": int((err > 1e-2).sum()),
            "max_dLSE": float(lerr[j]), "argmax_lse": int(np.flatnonzero(fin)[j]) if fin.any() else -1,
            "empty_rows_match": same_inf}


def cpu_baseline(name: str, inputs, gpu_out, threads: int):
    """The oracle as it stands on every query row of the headline workload
    (every key of each row), on the host cores, timed; its output is also the
    reference for the headline's parity record."""
    import numpy as np

    import oracle
    from exact_attention_09_amd.workloads import WORKLOADS, host_f32
    wl = WORKLOADS[name]
    q, k, v = (host_f32(inputs[t], wl.dtype) for t in ("q", "k", "v"))
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attention(q, k, v, wl.scale, wl.causal, nthreads=threads)
    dt = time.perf_counter() - t0
    n = wl.B * wl.H * wl.Sq
    flops = wl.flops()
    base = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(),
            "sample": f"all {n} query rows of {name} (all {wl.Skv} keys each, fp64 naive), {dt:.1f} s",
            "threads_note": "at most 16 threads: a GPU box allots 16 CPUs to each GPU"}
    parity = parity_record(gpu_out[0], gpu_out[1], o_ref, lse_ref, n) if gpu_out is not None else None
    return base, parity


def sampled_parity(name: str, gpu_out, threads: int, n_rows: int = 2048):
    """Parity of another forward workload's last GPU step on seeded sample
    rows (every row when there are few), for the record."""
    import numpy as np

    import oracle
    from exact_attention_09_amd.workloads import WORKLOADS, host_f32
    wl = WORKLOADS[name]
    x = wl.make_inputs()
    q, k, v = (host_f32(x[t], wl.dtype) for t in ("q", "k", "v"))
    o, lse = gpu_out
    kw = {}
    if wl.window > 0 or wl.sinks:
        kw = {"window": wl.window, "sinks": x["sinks"]}
    rng = np.random.default_rng(1000 + wl.wid)
    if wl.varlen:
        cu = x["cu_seqlens"]
        q, k, v = q[0], k[0], v[0]
        total = wl.H * wl.total_tokens
        flat = np.arange(total) if total <= n_rows else rng.choice(total, n_rows, replace=False)
        hh, tt = flat // wl.total_tokens, flat % wl.total_tokens
        bb = np.searchsorted(cu, tt, side="right") - 1
        rows = np.stack([bb, hh, tt - cu[bb]], axis=1).astype(np.int64)
        o_ref, lse_ref = oracle.attention(q, k, v, wl.scale, wl.causal, cu_seqlens=cu, rows=rows, nthreads=threads,
                                          **kw)
        og, lg = o[0, hh, tt], lse[0, hh, tt]
    else:
        total = wl.B * wl.H * wl.Sq
        flat = np.arange(total) if total <= n_rows else rng.choice(total, n_rows, replace=False)
        b, h, i = flat // (wl.H * wl.Sq), (flat // wl.Sq) % wl.H, flat % wl.Sq
        rows = np.stack([b, h, i], axis=1).astype(np.int64)
        o_ref, lse_ref = oracle.attention(q, k, v, wl.scale, wl.causal, rows=rows, nthreads=threads, **kw)
        og, lg = o[b, h, i], lse[b, h, i]
    return parity_record(og, lg, o_ref, lse_ref, len(rows))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--quick", action="store_true", help="headline workload only, no CPU baseline")
    ap.add_argument("--workload", default=HEADLINE, help="time only this workload (profiling runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="first run one plain device copy of MIB MiB (scale for HBM byte counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; the attention forward shards over "
              "(batch, head) with no exchange, so there is no multi-GPU run to time", file=sys.stderr)
        return 2

    import torch

    import exact_attention_09_amd as ea
    from exact_attention_09_amd.workloads import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    ea.load_library()

    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"# calibration copy of {n} bytes done", file=sys.stderr, flush=True)
        del src, dst
        torch.cuda.empty_cache()

    if args.workload != HEADLINE:
        wl, ns, t = run_workload(args.workload, args.steps, args.warmup)
        print(json.dumps({"workload": args.workload, "timing": t}), flush=True)
        return 0

    wl = WORKLOADS[HEADLINE]
    inputs = wl.make_inputs()
    print(f"# timing {HEADLINE}", file=sys.stderr, flush=True)
    _, _, t = run_workload(HEADLINE, args.steps, args.warmup, inputs, keep_outputs=not args.quick)
    flops = wl.flops()
    value = flops / (t["wall_ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (t["event_ms_mean"] * 1e-3) / 1e12
    traffic = read_traffic(HEADLINE)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(t["wall_ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "B": wl.B, "H": wl.H, "Hkv": wl.Hkv, "Sq": wl.Sq, "Skv": wl.Skv,
                   "d": wl.d, "causal": wl.causal, "layout": "BHSD", "inputs": "N(0,1) seeded"},
        "median_ms": round(t["event_ms_median"], 4), "min_ms": round(t["event_ms_min"], 4),
        "mean_ms": round(t["event_ms_mean"], 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "prefill_pp_kernel<128,false,false,false,false>",
                     "launch_ms_mean": round(t["event_ms_mean"], 4),
                     "frac_at_median": round(flops / (t["event_ms_median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "provenance": provenance(wl),
    }
    workloads = {}
    outputs = {}
    if not args.quick:
        for name in ("mha_causal_s8192_d128", "mha_causal_s2048_d64", "varlen_gqa_causal_d128",
                     "swa_sink_s32768_d128", "decode_gqa_s16384_d128", "decode_paged_gqa_s16384_d128",
                     "bwd_mha_s8192_d128", "bwd_mha_causal_s8192_d128", "bwd_varlen_gqa_causal_d128",
                     "bwd_swa_sink_s8192_d128"):
            print(f"# timing {name}", file=sys.stderr, flush=True)
            w, ns, tt = run_workload(name, args.steps, args.warmup, keep_outputs=not WORKLOADS[name].paged)
            if "outputs" in tt:
                outputs[name] = tt.pop("outputs")
            entry = {"ms_per_step": round(tt["wall_ms_per_step"], 4), "launch_ms_mean": round(tt["event_ms_mean"], 4),
                     "median_ms": round(tt["event_ms_median"], 4), "min_ms": round(tt["event_ms_min"], 4)}
            if w.Sq == 1 and not w.varlen:
                gbps = w.bytes(ns) / (tt["event_ms_mean"] * 1e-3) / 1e9
                entry.update({"GB/s": round(gbps, 1), "frac_hbm": round(gbps / PEAK_HBM_GBPS, 4),
                              "num_splits": ns, "bytes_per_step": w.bytes(ns)})
            else:
                tf = w.flops() / (tt["event_ms_mean"] * 1e-3) / 1e12
                entry.update({"TFLOP/s": round(tf, 2), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4),
                              "flops_per_step": w.flops()})
            workloads[name] = entry
        # the CPU leg: the oracle on every headline row (timed), which is also
        # the headline's parity reference, then sampled parity of the other
        # forward workloads' last steps
        print("# cpu baseline", file=sys.stderr, flush=True)
        threads = cpu_threads()
        base, parity = cpu_baseline(HEADLINE, inputs, t.get("outputs"), threads)
        line["cpu_baseline"] = base
        line["parity"] = {HEADLINE: parity}
        for name, out in outputs.items():
            print(f"# parity {name}", file=sys.stderr, flush=True)
            line["parity"][name] = sampled_parity(name, out, threads)
    else:
        line["cpu_baseline"] = None
    line["workloads"] = workloads
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
