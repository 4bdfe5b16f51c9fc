"""Benchmark: fused linear-cross-entropy forward+backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one lce_forward_backward call (every step of the method: label
count, logits tiles with the online log-sum-exp, per-row NLL and chunk sums,
dlogits, grad_hidden = G W, FP32 grad_weight = G^T h and grad_bias, the final
bf16 casts; outputs the loss and the three gradients, as the pages' loss
function does) over the whole workload, with inputs, outputs and workspace
resident in HBM before the timed region starts. Prints ONE JSON line.

Default workload: the Qwen3-8B-shaped head at one GPU's share of a 1M-token
sequence (N=131072 rows, H=4096, V=151936, bias, Zipf(1.1) labels, 2% ignored,
chunk_rows=256, sum reduction), seeded synthetic inputs (lce_inputs recipe).

The JSON line also carries:
  roofline      the dominant kernel's throughput from HIP events the library
                records around each launch during the timed steps, against the
                MI355X dense bf16 MFMA peak; `traffic` is the HBM bytes per
                launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE counters
                (profiles/<kernel>_<workload>_traffic.md), reported only while
                the kernel source still has the hash recorded there;
  cpu_baseline  the float64 CPU oracle timed on a bounded row sample of the
                same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0
METRIC = "fused linear-CE fwd+bwd tokens/sec on 1 MI355X; % of bf16 MFMA peak"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles for the library's per-launch trace."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            self.arr[i] = ev
        self.n = n

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[a], self.arr[b])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(self.arr[i])


def make_traces(lib_mod, events: HipEvents, steps: int, cap: int):
    traces = []
    for s in range(steps):
        t = lib_mod.LceTrace()
        t.events = ctypes.cast(ctypes.byref(events.arr, ctypes.sizeof(ctypes.c_void_p) * 2 * cap * s),
                               ctypes.POINTER(ctypes.c_void_p))
        kinds = (ctypes.c_int32 * cap)()
        dims = (ctypes.c_int64 * (3 * cap))()
        t.kinds = ctypes.cast(kinds, ctypes.POINTER(ctypes.c_int32))
        t.dims = ctypes.cast(dims, ctypes.POINTER(ctypes.c_int64))
        t.capacity = cap
        t.count = 0
        traces.append((t, kinds, dims, s))
    return traces


def step_times(events: HipEvents, traces, cap: int) -> list:
    """Per-step device time: first launch's start event to the last launch's end event."""
    out = []
    for t, _, _, s in traces:
        if t.count > 0:
            out.append(events.elapsed_ms(2 * cap * s, 2 * cap * s + 2 * (t.count - 1) + 1))
    return out


def matmul_roof(torch, dev, H: int, V: int, rows: int = 16384, reps: int = 5) -> dict:
    """torch.matmul (the vendor bf16 GEMM) on the forward logits shape of one row group."""
    a = torch.randn(rows, H, device=dev).to(torch.bfloat16)
    b = torch.randn(H, V, device=dev).to(torch.bfloat16)      # contiguous right operand
    c = torch.matmul(a, b)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / reps
    del a, b, c
    return {"shape": [rows, H, V], "ms": ms, "tflops": 2.0 * rows * H * V / (ms * 1e-3) / 1e12,
            "what": "torch.matmul bf16, [rows,H] x [H,V], same shape as one row group's logits product"}


def summarize_traces(lib_mod, events: HipEvents, traces, cap: int) -> dict:
    per = {}
    for t, kinds, dims, s in traces:
        for i in range(t.count):
            k = lib_mod.KERNEL_KINDS[kinds[i]]
            base = 2 * cap * s + 2 * i
            ms = events.elapsed_ms(base, base + 1)
            m, n, kk = dims[3 * i], dims[3 * i + 1], dims[3 * i + 2]
            e = per.setdefault(k, {"ms": 0.0, "launches": 0, "flops": 0.0})
            e["ms"] += ms
            e["launches"] += 1
            e["flops"] += 2.0 * m * n * kk
    steps = max(1, len(traces))
    out = {}
    for k, e in per.items():
        out[k] = {
            "ms_per_step": e["ms"] / steps,
            "launches_per_step": e["launches"] / steps,
            "avg_launch_ms": e["ms"] / e["launches"],
            "tflops": (e["flops"] / (e["ms"] * 1e-3) / 1e12) if e["flops"] > 0 and e["ms"] > 0 else None,
        }
    return out


def cpu_baseline(inp, w, rows: int) -> dict:
    """The float64 oracle as it stands, on the first `rows` rows at full H, V."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import lce_oracle as O
    h = inp.hidden_f32()[:rows]
    y = inp.labels[:rows]
    wf = inp.weight_f32()
    bf = inp.bias_f32()
    t0 = time.perf_counter()
    O.forward_backward(h, wf, bf, y, reduction=w.reduction, chunk_rows=w.chunk_rows)
    dt = time.perf_counter() - t0
    threads = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = int(max(threads)) if threads else (os.cpu_count() or 1)
    return {"value": rows / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {rows} rows of {w.name} at full H={w.hidden}, V={w.vocab}: float64 forward + "
                      f"grad_hidden, grad_weight, grad_bias ({dt:.1f} s)",
            "seconds": dt}


KERNEL_SOURCE = os.path.join(ROOT, "chunked_lm_head_lce_amd", "csrc", "lce_kernels.hip")


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary, or None when there is none or the kernel source changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.startswith("- "):
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    with open(KERNEL_SOURCE, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != digest or "hbm_bytes_per_launch" not in fields:
        return None
    return float(fields["hbm_bytes_per_launch"])


def memory_sweep(torch, lce, dev) -> dict:
    """Peak extra HBM and step time of lce_forward_backward against N at the
    Qwen3-4B / 8B head shapes, beside a plain eager PyTorch loss (F.linear +
    F.cross_entropy + autograd, [N, V] logits) where it fits in 200 GB;
    then chunk_rows and rows_in_flight sweeps at N=32768, H=4096. Inputs are
    seeded on the device (hidden ~ N(0,1), weight ~ 0.02 N(0,1), labels
    uniform, 2% ignored), all bf16."""
    import torch.nn.functional as F
    V = 151936

    def inputs(N, H):
        g = torch.Generator(device=dev)
        g.manual_seed(0)
        h = torch.randn(N, H, device=dev, generator=g).to(torch.bfloat16)
        w = (0.02 * torch.randn(V, H, device=dev, generator=g)).to(torch.bfloat16)
        y = torch.randint(0, V, (N,), device=dev, generator=g)
        y[torch.randperm(N, device=dev, generator=g)[: N // 50]] = -100
        return h, w, y

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        r = fn()
        b.record()
        torch.cuda.synchronize()
        return r, a.elapsed_time(b)

    def lib_run(h, w, y, **kw):
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        out, ms = timed(lambda: lce.lce_forward_backward(h, w, None, y, want_lse=False, **kw))
        outs = sum(t.numel() * t.element_size() for t in (out.loss, out.n_valid, out.status, out.grad_hidden,
                                                          out.grad_weight) if t is not None)
        extra = torch.cuda.max_memory_allocated(dev) - base - outs
        del out
        return extra / 1e9, ms

    def eager_run(h, w, y):
        hh = h.detach().clone().requires_grad_(True)
        ww = w.detach().clone().requires_grad_(True)
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)

        def step():
            hh.grad = None
            ww.grad = None
            loss = F.cross_entropy(F.linear(hh, ww).float(), y, ignore_index=-100, reduction="sum")
            loss.backward()
            return loss
        _, ms = timed(step)
        grads = hh.grad.numel() * 2 + ww.grad.numel() * 2
        extra = torch.cuda.max_memory_allocated(dev) - base - grads
        del hh, ww
        return extra / 1e9, ms

    rows = []
    for H in (2560, 4096):
        for N in (8192, 32768, 65536, 131072, 163840):
            h, w, y = inputs(N, H)
            lib_gb, lib_ms = lib_run(h, w, y)
            rec = {"hidden": H, "n_rows": N, "lib_extra_gb": lib_gb, "lib_ms": lib_ms,
                   "logits_fp32_gb": 4.0 * N * V / 1e9}
            if 16.0 * N * V <= 200e9:
                eg, ems = eager_run(h, w, y)
                rec.update({"eager_extra_gb": eg, "eager_ms": ems})
            else:
                rec.update({"eager_extra_gb": None, "eager_ms": None,
                            "eager_note": "not run: predicted > 200 GB ([N,V] logits in bf16 and fp32 with grads)"})
            log(f"[sweep] H={H} N={N}: library {lib_gb:.1f} GB {lib_ms:.0f} ms; eager {rec['eager_extra_gb']}")
            rows.append(rec)
            del h, w, y
            torch.cuda.empty_cache()
    h, w, y = inputs(32768, 4096)
    chunks = []
    for c in (128, 256, 512, 1024, 2048):
        gb, ms = lib_run(h, w, y, chunk_rows=c)
        chunks.append({"chunk_rows": c, "lib_extra_gb": gb, "lib_ms": ms})
    groups = []
    for g in (4096, 8192, 16384, 32768):
        gb, ms = lib_run(h, w, y, rows_in_flight=g)
        groups.append({"rows_in_flight": g, "lib_extra_gb": gb, "lib_ms": ms})
    return {"metric": "peak extra HBM (GB) and fwd+bwd time (ms) vs N; library vs eager [N,V] logits",
            "vocab": V, "rows": rows, "chunk_rows_sweep_n32768_h4096": chunks,
            "rows_in_flight_sweep_n32768_h4096": groups}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen3_8b_1m_shard")
    ap.add_argument("--rows-in-flight", type=int, default=0)
    ap.add_argument("--fwd-steps", type=int, default=3)
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--memory-sweep", action="store_true",
                    help="instead of the benchmark: peak extra HBM and time vs N, library vs eager, and "
                         "chunk_rows / rows_in_flight sweeps (one JSON line)")
    ap.add_argument("--no-matmul-roof", action="store_true",
                    help="skip timing torch.matmul on the logits shape (context for the roofline)")
    ap.add_argument("--copy-gib", type=float, default=0.0,
                    help="also run one plain device-to-device copy of this many GiB (a kernel of known "
                         "traffic, used to calibrate the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: the loss shards by rows with no exchange inside the kernels, "
              f"so a run on {args.gpus} GPUs is not provided; run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    import chunked_lm_head_lce_amd as lce
    from chunked_lm_head_lce_amd import _lib
    from lce_inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.memory_sweep:
        print(json.dumps(memory_sweep(torch, lce, dev)), flush=True)
        return 0
    log(f"[bench] generating {w.name} inputs (N={w.n_rows}, H={w.hidden}, V={w.vocab})")
    t0 = time.perf_counter()
    inp = make_inputs(w)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s")

    import numpy as np

    def dev_bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    hd, wd = dev_bits(inp.hidden_bits), dev_bits(inp.weight_bits)
    bd = None if inp.bias_bits is None else dev_bits(inp.bias_bits)
    yd = torch.from_numpy(inp.labels).to(dev)
    torch.cuda.synchronize()
    base_bytes = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)

    rif = args.rows_in_flight or None
    # The call the pages' loss function makes: the loss and the gradients
    # (per-row lse is an optional diagnostic output of the library and is
    # not asked for; ignored rows then need no work at all).
    kw = dict(chunk_rows=w.chunk_rows, reduction=w.reduction, rows_in_flight=rif, want_f32=False, want_lse=False)
    log("[bench] first call")
    out = lce.lce_forward_backward(hd, wd, bd, yd, **kw)
    torch.cuda.synchronize()
    out.check()
    ws = torch.empty(out.workspace_bytes, dtype=torch.uint8, device=dev)
    out_bytes = sum(t.numel() * t.element_size() for t in (out.loss, out.lse, out.n_valid, out.status,
                                                             out.grad_hidden, out.grad_weight, out.grad_bias)
                    if t is not None)
    for _ in range(args.warmup):
        lce.lce_forward_backward(hd, wd, bd, yd, workspace=ws, out=out, **kw)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    cap = 256
    events = HipEvents(2 * cap * args.steps)
    traces = make_traces(_lib, events, args.steps, cap)
    stream = torch.cuda.current_stream(dev)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for t, _, _, _ in traces:
        lce.lce_forward_backward(hd, wd, bd, yd, workspace=ws, out=out, trace=t, **kw)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_step = start.elapsed_time(stop) / args.steps
    out.check()
    log(f"[bench] timed {args.steps} steps: {ms_step:.2f} ms/step (wall {wall:.2f}s)")
    kernels = summarize_traces(_lib, events, traces, cap)
    per_step = sorted(step_times(events, traces, cap))
    peak_extra = torch.cuda.max_memory_allocated(dev) - base_bytes - out_bytes

    # forward only
    ms_fwd = None
    if args.fwd_steps > 0:
        fout = lce.lce_forward(hd, wd, bd, yd, chunk_rows=w.chunk_rows, reduction=w.reduction)
        torch.cuda.synchronize()
        fws = torch.empty(fout.workspace_bytes, dtype=torch.uint8, device=dev)
        s2, e2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s2.record(stream)
        for _ in range(args.fwd_steps):
            lce.lce_forward(hd, wd, bd, yd, chunk_rows=w.chunk_rows, reduction=w.reduction, workspace=fws,
                            out=fout)
        e2.record(stream)
        torch.cuda.synchronize()
        ms_fwd = s2.elapsed_time(e2) / args.fwd_steps
    events.close()
    roof = None
    if not args.no_matmul_roof:
        roof = matmul_roof(torch, dev, w.hidden, w.vocab)
        log(f"[bench] torch.matmul on the logits shape: {roof['tflops']:.0f} TFLOP/s")
    if args.copy_gib > 0:
        nbytes = int(args.copy_gib * (1 << 30))
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {nbytes} bytes device to device (counter calibration)")
        del src, dst

    N, H, V = w.n_rows, w.hidden, w.vocab
    tok_s = N / (ms_step * 1e-3)
    pct = 6.0 * N * H * V / (ms_step * 1e-3) / (PEAK_BF16_TFLOPS * 1e12)
    pct_fwd = 2.0 * N * H * V / (ms_fwd * 1e-3) / (PEAK_BF16_TFLOPS * 1e12) if ms_fwd else None

    dom_name = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dom = kernels[dom_name]
    achieved = dom["tflops"] or 0.0
    # achieved counts the launch's whole product shape (every row of the row
    # group, ignored ones too: the 6 N H V convention of the headline); the
    # products run on the labelled rows only, n_valid / N of that work
    n_valid = int(out.n_valid.item())
    roofline = {"bound": "mfma", "kernel": dom_name, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(dom_name, w.name), "traffic_unit": "bytes/launch",
                "avg_launch_ms": dom["avg_launch_ms"], "launches_per_step": dom["launches_per_step"],
                "executed_frac": n_valid / N,
                "achieved_executed": achieved * n_valid / N}

    cpu = None
    if not args.no_cpu_baseline:
        rows = min(args.cpu_rows, N)
        log(f"[bench] cpu baseline: oracle on {rows} rows")
        cpu = cpu_baseline(inp, w, rows)
        log(f"[bench] cpu baseline {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    rec = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "n_rows": N, "hidden": H, "vocab": V, "bias": w.bias_std is not None,
                   "labels": w.labels + (f"({w.zipf_s})" if w.labels == "zipf" else ""),
                   "ignored_rows": w.n_ignored, "chunk_rows": w.chunk_rows, "reduction": w.reduction,
                   "rows_in_flight": rif or 16384, "parallelism": "single GPU",
                   "outputs": "loss, grad_hidden, grad_weight, grad_bias (bf16; FP32 accumulation)"},
        "pct_peak_bf16": pct,
        "step_ms_min": per_step[0] if per_step else None,
        "step_ms_median": per_step[len(per_step) // 2] if per_step else None,
        "vendor_gemm_same_shape": roof,
        "fwd_tokens_per_s": N / (ms_fwd * 1e-3) if ms_fwd else None, "fwd_ms": ms_fwd,
        "fwd_pct_peak_bf16": pct_fwd,
        "peak_extra_hbm_gb": peak_extra / 1e9, "full_logits_fp32_gb": 4.0 * N * V / 1e9,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "loss": float(out.loss.item()), "n_valid": n_valid,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
