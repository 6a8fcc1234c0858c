"""Decode-attention benchmark on one MI355X: decode µs/step and achieved HBM GB/s.

One step = one full decode call (split kernel + merge kernel when the plan has
more than one split) over one batch of synthetic input already resident in HBM.
The KV cache is rotated over enough device copies that every step reads it cold
(at least 512 MiB between reuses: twice the 256 MiB Infinity Cache).

Printed: one JSON line with the metric, the whole-step throughput (unique K+V
bytes / step time), the dominant kernel's roofline (its own launch durations
timed with HIP events on the stream it runs on), the float64 CPU oracle's
throughput on a bounded sample of the same workload and, for single-sequence
decode workloads, the KV-length curve the metric is stated over (32 heads,
S = 4k .. 128k and 131073 tokens; "sweep").

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--kv fp8] [--no-sweep] [--no-cpu-baseline] [--graph]
  python bench.py --workload prefill_bf16_h32_n4096_causal   # the prefill kernel (TFLOP/s, matrix-core roofline)
  python bench.py --copy-probe BYTES   # a plain device copy, to scale rocprof byte counters
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

METRIC = "decode µs/step + achieved HBM GB/s (fraction of peak), KV 4k→128k"
PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
COLD_BYTES = 512 << 20      # bytes touched between reuses of one KV copy
DEFAULT_WORKLOAD = "decode_bf16_h32_s4096"
SPLIT_KERNELS = {1: "split_valu_kernel", 2: "split_mfma_kernel"}  # by fd_plan.kernel
SWEEP = (4096, 8192, 16384, 32768, 65536, 131072, 131073)


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


# The sources each timed kernel and its launch are built from (a counter profile is
# tied to them): the kernel, the shared device code and, for the planner that sets
# the grid and the split stride, the C-ABI layer and its header.
_CSRC = "decode_attention_13_amd/csrc/"
_COMMON = (_CSRC + "fd_device.h", _CSRC + "fd_internal.h", _CSRC + "fd_api.hip", "include/fd.h")
KERNEL_SOURCES = {
    "split_valu_kernel": (_CSRC + "fd_split_valu.hip",) + _COMMON,
    "split_mfma_kernel": (_CSRC + "fd_split_mfma.hip",) + _COMMON,
    "prefill_kernel": (_CSRC + "fd_prefill.hip",) + _COMMON,
}


def kernel_source_hash(kernel: str) -> str:
    """Hash of one kernel's HIP sources: a committed counter profile is used only while it matches."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel: str, workload: str) -> dict | None:
    """HBM bytes per launch of a kernel from the committed rocprofv3 --pmc summary."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash(kernel):
        return None  # the kernel changed since the counters were taken
    return t


class Case:
    """A workload placed in device memory with rotated KV copies and its C-ABI arguments."""

    def __init__(self, w, chunk: int = 0, kernel: str = "auto", data: dict | None = None, kv: str = "native",
                 merge: str = "auto", launch: str = "auto"):
        import torch

        import decode_attention_13_amd as fd
        from decode_attention_13_amd import binding

        self.w = w
        self.fd = fd
        self.lib = fd.lib()
        dev = torch.device("cuda:0")
        if data is None:
            log(f"generating {w.name}")
            data = w.make()
        self.fp8 = kv == "fp8"
        if self.fp8:
            from decode_attention_13_amd.inputs import with_fp8_kv
            data = with_fp8_kv(data)
        d = data
        self.d = d
        forced = chunk or kernel != "auto" or merge != "auto" or launch != "auto"
        self.opt = fd.options(force_chunk=chunk, kernel=kernel, merge=merge, launch=launch) if forced else None
        qdt = inputs_dtype(w.dtype)
        esize = 1 if self.fp8 else torch.tensor([], dtype=qdt).element_size()
        self.dtype_code = binding.FD_DTYPE_KV_E4M3[qdt] if self.fp8 else binding.FD_DTYPE[qdt]
        self.dtype_name = f"{w.dtype}_kv_e4m3" if self.fp8 else w.dtype
        if w.kind == "single":
            self.kv_bytes = 2 * w.S * w.Hkv * 128 * esize
            self.units = w.S * w.Hkv
            self.plan = fd.decode_plan(w.H, w.Hkv, w.S, self.dtype_code, 0, self.opt)
            self.q = d["q"].to(dev)
            srcs = (d["k"], d["v"])
        else:
            self.total = d["total_kv"]
            self.kv_bytes = 2 * self.total * w.Hkv * 128 * esize
            self.units = self.total * w.Hkv
            self.plan = fd.paged_plan(w.B, w.H, w.Hkv, self.dtype_code, w.page_size, d["max_seq_len"], self.total, 0,
                                      self.opt)
            self.q = d["q"].to(dev)
            self.table = d["block_table"].to(dev)
            self.lens = d["seq_lens"].to(dev)
            srcs = (d["k_cache"], d["v_cache"])
        self.copies = max(1, math.ceil(COLD_BYTES / self.kv_bytes))
        kd, vd = srcs[0].to(dev), srcs[1].to(dev)
        self.kv = [(kd, vd)] + [(kd.clone(), vd.clone()) for _ in range(self.copies - 1)]
        self.o = torch.empty_like(self.q)
        self.ws = fd.new_workspace(self.plan["workspace_bytes"], dev)
        self.stream = torch.cuda.current_stream()
        log(f"{w.name}: plan {self.plan}, {self.copies} KV copies of {self.kv_bytes / 1e6:.1f} MB")

    def step(self, i: int, opt=None, stream=None) -> None:
        import ctypes
        k, v = self.kv[i % self.copies]
        st = self.stream.cuda_stream if stream is None else stream.cuda_stream
        o = opt if opt is not None else self.opt
        optp = ctypes.byref(o) if o is not None else None
        w = self.w
        if w.kind == "single" and self.fp8:
            rc = self.lib.fd_decode_fp8kv(self.q.data_ptr(), k.data_ptr(), v.data_ptr(), self.o.data_ptr(), w.H, w.Hkv,
                                          w.S, 128, self.dtype_code, self.d["scale"], self.d["k_scale"],
                                          self.d["v_scale"], self.ws.data_ptr(), self.ws.numel(), optp,
                                          st)
        elif w.kind == "single":
            rc = self.lib.fd_decode(self.q.data_ptr(), k.data_ptr(), v.data_ptr(), self.o.data_ptr(), w.H, w.Hkv, w.S,
                                    128, self.dtype_code, self.d["scale"], self.ws.data_ptr(),
                                    self.ws.numel(), optp, st)
        elif self.fp8:
            rc = self.lib.fd_paged_decode_fp8kv(self.q.data_ptr(), k.data_ptr(), v.data_ptr(), self.table.data_ptr(),
                                                self.lens.data_ptr(), w.page_size, self.o.data_ptr(), self.d["scale"],
                                                self.d["k_scale"], self.d["v_scale"], w.B, w.H, w.Hkv, 128,
                                                self.d["num_pages"], self.d["max_blocks"], self.d["max_seq_len"],
                                                self.total, self.dtype_code, self.ws.data_ptr(), self.ws.numel(),
                                                optp, st)
        else:
            rc = self.lib.fd_paged_decode(self.q.data_ptr(), k.data_ptr(), v.data_ptr(), self.table.data_ptr(),
                                          self.lens.data_ptr(), w.page_size, self.o.data_ptr(), self.d["scale"], w.B,
                                          w.H, w.Hkv, 128, self.d["num_pages"], self.d["max_blocks"],
                                          self.d["max_seq_len"], self.total, self.dtype_code, self.ws.data_ptr(),
                                          self.ws.numel(), optp, st)
        if rc != 0:
            raise RuntimeError(f"{self.lib.fd_status_string(rc).decode()}: {self.lib.fd_last_error().decode()}")


def inputs_dtype(name: str):
    from decode_attention_13_amd.inputs import DTYPES
    return DTYPES[name]


def time_graph(case: Case, steps: int) -> dict:
    """The step captured in a HIP graph (torch.cuda.graph): one captured step per
    rotated KV copy, the graph replayed back to back; wall time per step."""
    import torch

    n = case.copies
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for i in range(n):
            case.step(i, stream=cap)
    reps = max(1, steps // n)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    return {"us_per_step": round((time.perf_counter() - t0) / (reps * n) * 1e6, 3), "steps": reps * n,
            "steps_per_replay": n}


def time_steps(case: Case, steps: int, warmup: int) -> dict:
    """Whole-step wall time over exactly `steps` steps, then the split kernel alone
    (its start and end stamped by the dispatch itself, on the launch stream) over
    another `steps` steps that follow `warmup` untimed ones."""
    import torch

    for i in range(warmup):
        case.step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        case.step(i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps

    begins = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for ev in begins + ends:  # torch creates the underlying hipEvent_t on first record
        ev.record()
        assert ev.cuda_event, "event handle not materialised"
    base = case.opt
    opts = [case.fd.options(force_num_splits=base.force_num_splits if base else 0,
                            force_chunk=base.force_chunk if base else 0,
                            kernel=base.force_kernel if base else 0,
                            merge=base.force_merge if base else 0,
                            launch=base.force_launch if base else 0,
                            split_begin_event=begins[i], split_end_event=ends[i]) for i in range(steps)]
    torch.cuda.synchronize()
    for i in range(warmup):  # back to steady state after the synchronisations
        case.step(i)
    for i in range(steps):
        case.step(i, opts[i])
    torch.cuda.synchronize()
    split_ms = [b.elapsed_time(e) for b, e in zip(begins, ends)]
    split_ms.sort()
    return {"wall_s": wall, "split_mean_s": sum(split_ms) / len(split_ms) / 1e3,
            "split_median_s": split_ms[len(split_ms) // 2] / 1e3}


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it: model name, family, model and stepping."""
    info = {}
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if not line.strip():
                    break  # the first processor's block
                k, _, v = line.partition(":")
                info[k.strip()] = v.strip()
    except OSError:
        pass
    name = info.get("model name", "unknown")
    ids = ", ".join(f"{k} {info[k]}" for k in ("cpu family", "model", "stepping") if k in info)
    return f"{name} ({ids})" if ids else name


def host_cores() -> int:
    """Cores this process may run on (its affinity mask)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _oracle_step_single(d, fp8: bool) -> float:
    """Wall time of one whole oracle decode step (every head) of a contiguous workload."""
    import oracle
    t0 = time.perf_counter()
    if fp8:
        oracle.decode_attention_e4m3(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], d["scale"])
    else:
        oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"])
    return time.perf_counter() - t0


def cpu_baseline(w, budget_s: float = 12.0, fp8: bool = False) -> dict:
    """The float64 oracle as it stands, timed on this host with its BLAS threads set
    to the cores of this process (the E4M3 form of the oracle when the cache is FP8).

    Workloads whose whole step takes under a few seconds (the 512-token fp32 and the
    4k bf16 decodes) are timed as whole steps, median of 3 after one untimed run;
    larger ones over a bounded sample of heads or sequences. The 512-token fp32
    decode is also timed on one thread."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from decode_attention_13_amd.inputs import WORKLOADS
    threads = host_cores()
    with threadpool_limits(limits=threads):
        out = _cpu_baseline(w, budget_s, fp8, np, oracle)
    small = WORKLOADS["decode_f32_h8_s512"]
    ds = small.make()
    _oracle_step_single(ds, False)
    with threadpool_limits(limits=1):
        one = sorted(_oracle_step_single(ds, False) for _ in range(3))[1]
    out.update({"cores": threads, "cpu": cpu_model(),
                "single_thread": {"workload": small.name, "us_per_step": round(one * 1e6, 1),
                                  "value": round(small.kv_bytes() / one / 1e9, 4), "unit": "GB/s", "cores": 1}})
    return out


def _cpu_baseline(w, budget_s, fp8, np, oracle) -> dict:
    d = w.make()
    if fp8:
        from decode_attention_13_amd.inputs import with_fp8_kv
        d = with_fp8_kv(d)
    kv_bytes = 2 * _kv_elems(w, d) if fp8 else w.kv_bytes()  # E4M3: one byte per element
    if w.kind == "single" and w.S * w.H <= 4096 * 32:
        _oracle_step_single(d, fp8)
        runs = sorted(_oracle_step_single(d, fp8) for _ in range(3))
        step_s = runs[1]
        return {"value": round(kv_bytes / step_s / 1e9, 4), "unit": "GB/s", "kind": "oracle",
                "sample": f"whole steps of {w.name}, median of 3 ({', '.join(f'{r * 1e3:.1f}' for r in runs)} ms)",
                "us_per_step": round(step_s * 1e6, 1)}
    if w.kind == "single":
        heads = list(range(w.H))
        n_done = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            h = heads[n_done % len(heads)]
            if fp8:
                oracle.decode_attention_e4m3(d["q"], d["k"], d["v"], d["k_scale"], d["v_scale"], d["scale"],
                                             heads=[h])
            else:
                oracle.decode_attention(d["q"], d["k"], d["v"], d["scale"], heads=[h])
            n_done += 1
        el = time.perf_counter() - t0
        sample = f"{n_done} single-head decodes of {w.name} (S={w.S}), {el:.1f} s"
        step_s = el / n_done * w.H
    else:
        lens = d["seq_lens"].numpy()
        n_done, tokens_done = 0, 0
        rng = np.random.default_rng(0)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            b = int(rng.integers(w.B))
            pairs = [(b, h) for h in range(w.H)]
            if fp8:
                oracle.paged_decode_attention_e4m3(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                                   d["seq_lens"], d["page_size"], d["k_scale"], d["v_scale"],
                                                   d["scale"], pairs=pairs)
            else:
                oracle.paged_decode_attention(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                                              d["page_size"], d["scale"], pairs=pairs)
            n_done += 1
            tokens_done += int(lens[b])
        el = time.perf_counter() - t0
        sample = f"{n_done} whole sequences (all {w.H} heads) of {w.name}, {el:.1f} s"
        step_s = el / tokens_done * float(lens.sum())
    return {"value": round(kv_bytes / step_s / 1e9, 4), "unit": "GB/s", "kind": "oracle",
            "sample": sample, "us_per_step": round(step_s * 1e6, 1)}


def _kv_elems(w, d) -> int:
    """K (or V) elements of a workload."""
    return (w.S if w.kind == "single" else int(d["total_kv"])) * w.Hkv * 128


PREFILL_METRIC = "prefill attention TFLOP/s (useful flops: 4 * D per visible query-key pair and head)"
PEAK_TFLOPS_16BIT = 2500.0  # MI355X dense bf16 / f16 matrix-core peak


def bench_prefill(args) -> dict:
    """One step = one fd_prefill call over the whole prompt batch (inputs resident in HBM)."""
    import ctypes

    import torch

    import decode_attention_13_amd as fd
    from decode_attention_13_amd.inputs import PREFILL_WORKLOADS
    w = PREFILL_WORKLOADS[args.workload]
    log(f"generating {w.name}")
    d = w.make()
    dev = torch.device("cuda:0")
    q, k, v = d["q"].to(dev), d["k"].to(dev), d["v"].to(dev)
    o = torch.empty_like(q)
    lib = fd.lib()
    code = fd.binding.FD_DTYPE[q.dtype]
    stream = torch.cuda.current_stream()
    # bf16: the workspace of the f16-V path (the f16 copy of V and its flags), allocated once
    ws_bytes = 0 if args.no_workspace else fd.prefill_workspace_size(w.B, w.N, w.Hkv, q.dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ws_ptr = ws.data_ptr() if ws_bytes else None

    def step(opt=None):
        rc = lib.fd_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), w.B, w.N, w.H, w.Hkv, 128, code,
                            d["scale"], int(w.causal), ws_ptr, ws_bytes, ctypes.byref(opt) if opt is not None else None,
                            stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"{lib.fd_status_string(rc).decode()}: {lib.fd_last_error().decode()}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    begins = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for ev in begins + ends:
        ev.record()
    opts = [fd.options(split_begin_event=begins[i], split_end_event=ends[i]) for i in range(args.steps)]
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    for i in range(args.steps):
        step(opts[i])
    torch.cuda.synchronize()
    ks = sorted(b.elapsed_time(e) / 1e3 for b, e in zip(begins, ends))
    k_mean = sum(ks) / len(ks)
    flops = w.flops()
    # the committed counters are those of the default path (for bf16, the f16-V kernel)
    traffic = None if (args.no_workspace and w.dtype == "bf16") else load_traffic("prefill_kernel", w.name)
    line = {
        "metric": PREFILL_METRIC,
        "value": round(flops / step_s / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N": w.N, "H": w.H, "Hkv": w.Hkv, "D": 128, "causal": w.causal,
                   "flops": flops, "parallelism": "single GPU",
                   "pv": ("f16 MFMAs on an f16 copy of V (workspace)" if ws_bytes else
                          "bf16 MFMAs, P split in two" if w.dtype == "bf16" else "f16 MFMAs")},
        "roofline": {"bound": "mfma", "achieved": round(flops / k_mean / 1e12, 2), "peak": PEAK_TFLOPS_16BIT,
                     "unit": "TFLOP/s", "frac": round(flops / k_mean / 1e12 / PEAK_TFLOPS_16BIT, 4),
                     "traffic": (round(traffic["bytes_per_launch"]) if traffic else None),
                     "kernel": "prefill_kernel", "kernel_us_mean": round(k_mean * 1e6, 3),
                     "kernel_us_median": round(ks[len(ks) // 2] * 1e6, 3), "flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline_prefill(w, d)
    return line


def cpu_baseline_prefill(w, d, budget_s: float = 12.0) -> dict:
    """The float64 oracle's prefill, one (sequence, head) at a time, over a bounded sample."""
    from threadpoolctl import threadpool_limits

    import oracle
    threads = host_cores()
    with threadpool_limits(limits=threads):
        return _cpu_baseline_prefill(w, d, budget_s, threads, oracle)


def _cpu_baseline_prefill(w, d, budget_s, threads, oracle) -> dict:
    n_done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b, h = divmod(n_done % (w.B * w.H), w.H)
        oracle.prefill_attention(d["q"], d["k"], d["v"], d["scale"], w.causal, heads=[h], batches=[b])
        n_done += 1
    el = time.perf_counter() - t0
    per_head = w.flops() / (w.B * w.H)
    return {"value": round(per_head * n_done / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "cpu": cpu_model(),
            "kind": "oracle",
            "sample": f"{n_done} (sequence, head) prefills of {w.name} (N={w.N}), {el:.1f} s"}


def copy_probe(nbytes: int, steps: int) -> None:
    """A plain device-to-device copy of known size (for scaling FETCH_SIZE/WRITE_SIZE)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "steps": steps}))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--chunk", type=int, default=0, help="force tokens per split (multiple of 64)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"], help="force the split kernel")
    ap.add_argument("--merge", default="auto", choices=["auto", "kernel", "fused"],
                    help="force how split partials are merged (merge kernel, or the last workgroups)")
    ap.add_argument("--launch", default="auto", choices=["auto", "grid", "persistent"],
                    help="paged workloads: a workgroup per item, or one per resident slot claiming items")
    ap.add_argument("--kv", default="native", choices=["native", "fp8"],
                    help="cache storage: the workload's dtype, or FP8 E4M3 codes with per-tensor scales")
    ap.add_argument("--sweep", action="store_true",
                    help="time the pages' KV-length sweep (4k..128k) also for a paged workload")
    ap.add_argument("--no-sweep", action="store_true", help="skip the KV-length sweep")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph (field \"graph\")")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workspace", action="store_true",
                    help="prefill, bf16: pass no workspace (P.V on bf16 MFMAs with the split P)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library and this benchmark run on one GPU)",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return 0

    from decode_attention_13_amd.inputs import CHOICE_WORKLOADS, PREFILL_WORKLOADS, WORKLOADS, sweep_workload
    if args.workload in PREFILL_WORKLOADS:
        print(json.dumps(bench_prefill(args)), flush=True)
        return 0
    w = WORKLOADS[args.workload] if args.workload in WORKLOADS else CHOICE_WORKLOADS[args.workload]
    case = Case(w, args.chunk, args.kernel, kv=args.kv, merge=args.merge, launch=args.launch)
    split_kernel = SPLIT_KERNELS[case.plan["kernel"]]
    wl_name = w.name + ("_kv_e4m3" if case.fp8 else "")
    t = time_steps(case, args.steps, args.warmup)
    step_s = t["wall_s"]
    split_s = t["split_mean_s"]
    achieved = case.kv_bytes / split_s / 1e9
    traffic = load_traffic(split_kernel, wl_name)
    line = {
        "metric": METRIC,
        "value": round(case.kv_bytes / step_s / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 6),
        "us_per_step": round(step_s * 1e6, 3),
        "frac_of_peak": round(case.kv_bytes / step_s / 1e9 / PEAK_GBPS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype_name,
        "data": "synthetic",
        "config": {"workload": wl_name, "kv_bytes": case.kv_bytes, "plan": case.plan, "kv_copies": case.copies,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4),
                     "traffic": (round(traffic["bytes_per_launch"]) if traffic else None),
                     "kernel": split_kernel, "kernel_us_mean": round(split_s * 1e6, 3),
                     "kernel_us_median": round(t["split_median_s"] * 1e6, 3),
                     "bytes_per_launch": case.kv_bytes,
                     "bytes_per_unit": case.kv_bytes // case.units, "units_per_launch": case.units},
    }
    if args.graph:
        line["graph"] = time_graph(case, args.steps)
        log(f"graph replay: {line['graph']}")
    case_fp8 = case.fp8
    del case
    torch.cuda.empty_cache()
    if (args.sweep or w.kind == "single") and not args.no_sweep:
        sweep = []
        for S in SWEEP:
            c = Case(sweep_workload(S), kv=args.kv)
            ts = time_steps(c, max(20, args.steps // 4), 5)
            sweep.append({"S": S, "us_per_step": round(ts["wall_s"] * 1e6, 2),
                          "GBps": round(c.kv_bytes / ts["wall_s"] / 1e9, 1),
                          "split_kernel_GBps": round(c.kv_bytes / ts["split_mean_s"] / 1e9, 1)})
            log(f"sweep S={S}: {sweep[-1]}")
            del c
            torch.cuda.empty_cache()
        line["sweep"] = sweep
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(w, fp8=case_fp8)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
