#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--only]

One step = one decode-attention call over a batch: the split-KV partial
kernel and the log-sum-exp reduction (pa_decode_partial + pa_reduce, which is
exactly what pa_decode launches).  Inputs are seeded synthetic workloads that
are already resident in HBM when the timed region starts; `value` comes from
back-to-back steps, and `cold_call_ms` gives per-call times with L2 and the
MALL flushed before each call (a 1 GiB rewrite outside the timed interval).
The partial
kernel, the dominant one, is also timed on its own with HIP events on the
stream it is launched on; its algorithmic KV-read bytes per launch divided by
that average duration give the achieved HBM bandwidth reported against the
8 TB/s MI355X peak.

Prints ONE JSON line on stdout.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn tokens/s + achieved KV-read HBM GB/s (% of MI355X peak), 1 GPU"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
DEFAULT_CONFIG = "ragged_gqa_bf16"   # the largest single-GPU workload
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "decode_attention_paged_amd", "csrc")

# the sources each partial kernel is compiled from (its file and the headers it includes)
KERNEL_SOURCES = {
    "mha": ("pa_mha.hip", "pa_device.h", "pa_launch.h", "pa_merge.h"),
    "gqa": ("pa_gqa.hip", "pa_sched.hip", "pa_device.h", "pa_launch.h", "pa_merge.h"),
    "mla": ("pa_mla.hip", "pa_device.h", "pa_launch.h"),
}


def kernel_family(inp) -> str:
    """Which partial kernel serves the workload (the library's own dispatch rule)."""
    if inp.kind == "mla":
        return "mla"
    cols = inp.num_q_heads // inp.num_kv_heads * inp.q_len   # MFMA columns: (row, head) pairs
    if (inp.dtype == "bf16" and inp.head_dim in (64, 128) and inp.block_size in (16, 32)
            and 2 <= cols <= 16):
        return "gqa"
    return "mha"


def kernel_source_hash(family: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _profile_value(path: str, key: str, family: str):
    """`key: <number>` from a committed profile summary, if still current.

    The summary holds a line `kernel_source_sha256: <hash>`; its figures are
    used only when the hash matches today's kernel sources.
    """
    if not os.path.exists(path):
        return None
    text = open(path).read()
    mh = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    mb = re.search(key + r":\s*([0-9.eE+]+)", text)
    if not mh or not mb or mh.group(1) != kernel_source_hash(family):
        return None
    return float(mb.group(1))


def load_traffic(workload: str, family: str):
    """HBM bytes per launch (profiles/pmc_<workload>.md), if still current."""
    return _profile_value(os.path.join(PROFILES, f"pmc_{workload}.md"), "hbm_bytes_per_launch",
                          family)


def load_mfma_busy(workload: str, family: str):
    """Fraction of the kernel's CU cycles the matrix cores were busy
    (profiles/mfma_<workload>.md, from SQ_VALU_MFMA_BUSY_CYCLES), if still current."""
    return _profile_value(os.path.join(PROFILES, f"mfma_{workload}.md"), "mfma_busy_frac", family)


def progress(msg: str) -> None:
    """One line of progress on stderr (stdout carries only the JSON result)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--only", action="store_true",
                    help="time only --config (no other workloads, no CPU baseline)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration under rocprofv3)")
    return ap.parse_args()


class Case:
    """One workload on the device with prebound library calls."""

    def __init__(self, name: str):
        import torch

        import decode_attention_paged_amd as pa
        from decode_attention_paged_amd import _lib
        from workloads import make_config
        from workloads.device import to_device, torch_dtype

        self.name = name
        self.inp = inp = make_config(name, poison=False)
        self.t = to_device(inp, "cuda", poison=False)
        self.mla = inp.kind == "mla"
        self.family = kernel_family(inp)
        self.shape = pa.make_shape(
            batch=inp.batch, num_q_heads=inp.num_q_heads, num_kv_heads=inp.num_kv_heads,
            head_dim=inp.head_dim, head_dim_v=inp.head_dim_v, block_size=inp.block_size,
            max_blocks_per_seq=inp.max_blocks_per_seq, num_blocks=inp.num_blocks,
            max_context_len=inp.max_context_len, scale=inp.scale, dtype=torch_dtype(inp.dtype),
            q_len=inp.q_len, kv_dtype=torch_dtype(inp.kv_dtype) if inp.kv_dtype else 0,
            k_scale=inp.k_scale, v_scale=inp.v_scale)
        self.S = pa.choose_num_splits(self.shape, 0, self.mla)
        nbytes = pa.workspace_size(self.shape, self.S, self.mla)
        # zero-filled: the fused reduction's arrival counters start at 0
        self.ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        rows = (inp.batch, inp.num_q_heads) if inp.q_len == 1 else (inp.batch, inp.q_len, inp.num_q_heads)
        self.out = torch.empty(rows + (inp.head_dim_v,), dtype=torch_dtype(inp.dtype), device="cuda")
        self.lse = torch.empty(rows, dtype=torch.float32, device="cuda")
        lib = _lib.load()
        P = ctypes.c_void_p
        stream = P(torch.cuda.current_stream().cuda_stream)
        sh = ctypes.byref(self.shape)
        t = self.t
        ws, wsb = P(self.ws.data_ptr()), self.ws.numel()
        out, lse = P(self.out.data_ptr()), P(self.lse.data_ptr())
        bt, ctx = P(t["block_table"].data_ptr()), P(t["context_lens"].data_ptr())
        q = P(t["q"].data_ptr())
        # A decode call is one launch when the splits merge inside the partial
        # kernel (MHA/GQA with small per-unit partials), else the partial
        # kernel and the reduction (pa_decode_launches says which).  Two-launch
        # calls are made here as the two calls they consist of, so that each
        # kernel can be timed alone.
        self.launches = pa.decode_launches(self.shape, self.S, self.mla)
        self.fused = self.launches == 1
        if self.mla:
            kv = P(t["kv_cache"].data_ptr())
            self._partial = (lib.pa_decode_mla_partial,
                             (sh, q, kv, bt, ctx, self.S, out, lse, ws, wsb, stream))
        else:
            k, v = P(t["k_cache"].data_ptr()), P(t["v_cache"].data_ptr())
            if self.fused:
                self._partial = (lib.pa_decode,
                                 (sh, q, k, v, bt, ctx, self.S, out, lse, ws, wsb, stream))
            else:
                self._partial = (lib.pa_decode_partial,
                                 (sh, q, k, v, bt, ctx, self.S, out, lse, ws, wsb, stream))
        self._reduce = None if self.fused else (
            lib.pa_reduce, (sh, ctx, self.S, int(self.mla), ws, wsb, out, lse, stream))
        self.kv_bytes = inp.kv_bytes_read()
        self.tokens = int(inp.context_lens.astype("int64").sum())

    def partial(self):
        fn, args = self._partial
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"partial step failed with status {st}")

    def reduce(self):
        if self._reduce is None:
            return
        fn, args = self._reduce
        st = fn(*args)
        if st != 0:
            raise RuntimeError(f"reduce step failed with status {st}")

    def step(self):
        self.partial()
        self.reduce()

    def flops(self) -> float:
        i = self.inp
        # (query row, context token) pairs: row j of q_len sees ctx - q_len + 1 + j tokens
        pairs = sum(max(0, int(c) - i.q_len + 1 + j) for c in i.context_lens for j in range(i.q_len))
        return 2.0 * pairs * i.num_q_heads * (i.head_dim + i.head_dim_v)

    def _loop(self, fn, steps: int):
        """Average ms per call of `fn` over `steps` back-to-back calls.

        HIP events on the launch stream bracket the whole loop; nothing else is
        enqueued between the calls, so for a single-launch `fn` this is that
        kernel's average launch duration.  Also returns host wall time.
        """
        import torch

        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall * 1e3 / steps

    def time(self, steps: int, warmup: int):
        """Time `steps` whole steps (the timed region), then each kernel alone."""
        import torch

        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        ev_ms, wall_ms = self._loop(self.step, steps)
        r = dict(ms_per_step=wall_ms, ev_ms_per_step=ev_ms)
        if self.fused:
            r["partial_ms"] = ev_ms          # one launch per step
            r["reduce_ms"] = 0.0
        else:
            r["partial_ms"], _ = self._loop(self.partial, steps)
            r["reduce_ms"], _ = self._loop(self.reduce, steps)
        return r

    def cold(self, calls: int, flush_bytes: int = 1 << 30):
        """Per-call times with L2 and the 256 MB MALL flushed before each call.

        A 1 GiB buffer is rewritten before every call (outside the timed
        interval); HIP events on the launch stream bracket the call alone.
        Returns (median, p10, p90) in ms.
        """
        import torch

        flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
        evs = []
        for i in range(calls):
            flush.fill_(float(i))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            self.step()
            e1.record()
            evs.append((e0, e1))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in evs)
        del flush
        torch.cuda.empty_cache()
        q = lambda f: t[min(len(t) - 1, int(f * len(t)))]
        return q(0.5), q(0.1), q(0.9)

    def roofline(self, partial_ms: float):
        """The partial kernel against the HBM roofline: algorithmic KV bytes per
        launch over its average launch duration, and counter-measured traffic."""
        achieved = self.kv_bytes / (partial_ms * 1e-3) / 1e9
        traffic = load_traffic(self.name, self.family)
        rf = {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "traffic_over_algorithmic": None if traffic is None else round(traffic / self.kv_bytes, 4),
            "kernel": (f"{self.family} split-KV kernel with fused reduction" if self.fused
                       else f"{self.family} partial step: unit-order launch + partial kernel "
                            "(the reduction is a third launch)" if self.launches == 3
                       else f"{self.family} partial kernel (the reduction is a second launch)"),
            "algorithmic_bytes_per_launch": self.kv_bytes,
            "avg_launch_ms": round(partial_ms, 5),
        }
        if self.mla:
            tflops = self.flops() / (partial_ms * 1e-3) / 1e12
            rf["mfma"] = {
                "achieved_tflops": round(tflops, 1),
                "peak_tflops": PEAK_BF16_TFLOPS,
                "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                "flops_per_launch": self.flops(),
                "busy_frac_counter": load_mfma_busy(self.name, self.family),
            }
        return rf

    def summary(self, r):
        frac = (self.kv_bytes / (r["partial_ms"] * 1e-3) / 1e9) / PEAK_HBM_GBS
        d = dict(
            workload=self.inp.meta.get("desc", self.name),
            num_splits=self.S,
            kernel=self.family,
            ms_per_step=round(r["ms_per_step"], 5),
            ev_ms_per_step=round(r["ev_ms_per_step"], 5),
            tokens_per_s=round(self.inp.batch * self.inp.q_len / (r["ms_per_step"] * 1e-3), 1),
            q_len=self.inp.q_len,
            partial_ms=round(r["partial_ms"], 5),
            reduce_ms=round(r["reduce_ms"], 5),
            kv_bytes=self.kv_bytes,
            kv_gbps_partial=round(self.kv_bytes / (r["partial_ms"] * 1e-3) / 1e9, 1),
            kv_gbps_step=round(self.kv_bytes / (r["ms_per_step"] * 1e-3) / 1e9, 1),
            frac_of_peak_partial=round(frac, 4),
        )
        if "cold_ms" in r:
            med, p10, p90 = r["cold_ms"]
            d["cold_call_ms"] = {"median": round(med, 5), "p10": round(p10, 5), "p90": round(p90, 5)}
            d["cold_kv_gbps"] = round(self.kv_bytes / (med * 1e-3) / 1e9, 1)
        d["kv_tokens_per_s"] = round(self.tokens / (r["ms_per_step"] * 1e-3), 1)
        d["roofline"] = self.roofline(r["partial_ms"])
        return d

    def free(self):
        import torch

        self.t.clear()
        del self.ws, self.out, self.lse
        torch.cuda.empty_cache()


def stream_reference(nbytes: int = 4 << 30, reps: int = 5):
    """Measured bandwidth of plain device streams beside the 8 TB/s peak: the
    library's streaming-read probe over 4 GiB (the KV gather's load form; 16x
    the 256 MB MALL, so it reads HBM), and a 4 GiB device-to-device copy
    (reads and writes 4 GiB), timed with HIP events."""
    import torch

    import decode_attention_paged_amd as pa

    src = torch.ones(nbytes // 4, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    t_read = timed(lambda: pa.stream_read(src, sink))
    t_copy = timed(lambda: dst.copy_(src))
    del src, dst, sink
    torch.cuda.empty_cache()
    return {"read_gbps": round(nbytes / t_read / 1e9, 1),
            "copy_gbps": round(2 * nbytes / t_copy / 1e9, 1),
            "bytes": nbytes,
            "kind": "pa_stream_read (128-bit non-temporal loads, read only) and torch copy_ "
                    "(read + write) over 4 GiB, HIP events"}


def cpu_baseline(inp, min_s: float = 10.0, max_s: float = 30.0):
    """The float64 oracle, as it stands, on a bounded sample of the workload.

    Sequences of the batch are decoded one at a time (all heads), cycling
    through the batch until at least `min_s` seconds of CPU work are done.
    """
    from threadpoolctl import threadpool_info

    import oracle

    bt = inp.compact_block_table()
    done, toks = 0, 0
    t0 = time.perf_counter()
    while True:
        b = done % inp.batch
        one_q = inp.q[b:b + 1]
        if inp.kind == "mla":
            oracle.paged_decode_mla(one_q, inp.c_pages, bt[b:b + 1], inp.context_lens[b:b + 1],
                                    inp.scale, dv=inp.head_dim_v, dtype=inp.dtype)
        else:
            oracle.paged_decode(one_q, inp.k_pages, inp.v_pages, bt[b:b + 1],
                                inp.context_lens[b:b + 1], inp.scale, dtype=inp.dtype)
        done += 1
        toks += int(inp.context_lens[b])
        el = time.perf_counter() - t0
        if el >= min_s or el >= max_s:
            break
    dt = time.perf_counter() - t0
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    bytes_per_tok = inp.kv_bytes_read() / max(1, int(inp.context_lens.sum()))
    return {
        "value": round(done / dt, 3),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} sequence decodes (cycling the batch of {inp.batch}; all "
                  f"{inp.num_q_heads} heads; {toks} context tokens) in {dt:.1f} s, float64 NumPy",
        "kv_gbps": round(toks * bytes_per_tok / dt / 1e9, 4),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        sys.exit(2)

    import torch

    from workloads import CONFIG_ORDER

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    progress(f"{args.config}: drawing inputs")
    main_case = Case(args.config)
    progress(f"{args.config}: timing {args.steps} steps")
    r = main_case.time(args.steps, args.warmup)
    if not args.only:
        r["cold_ms"] = main_case.cold(min(args.steps, 50))
    main_sum = main_case.summary(r)
    inp = main_case.inp

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    roofline = main_case.roofline(r["partial_ms"])
    main_case.free()
    if not args.only:
        ref = stream_reference()
        roofline["measured_stream"] = ref
        roofline["frac_of_measured_read"] = round(roofline["achieved"] / ref["read_gbps"], 4)

    per_config = {}
    if not args.only:
        for name in CONFIG_ORDER:
            if name == args.config:
                per_config[name] = main_sum
                continue
            progress(f"{name}: drawing inputs and timing")
            c = Case(name)
            rr = c.time(max(20, args.steps // 4), max(5, args.warmup // 2))
            rr["cold_ms"] = c.cold(20)
            per_config[name] = c.summary(rr)
            c.free()
            del c

    cpu = None
    if not args.only and not args.no_cpu:
        progress("CPU oracle baseline")
        cpu = cpu_baseline(inp)

    line = {
        "metric": METRIC,
        "value": round(inp.batch / (r["ms_per_step"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": inp.dtype,
        "data": "synthetic (seeded N(0,1) q/K/V, shuffled page tables; see workloads/)",
        "config": {
            "workload": f"{args.config}: {inp.meta.get('desc', '')}",
            "batch": inp.batch,
            "num_q_heads": inp.num_q_heads,
            "num_kv_heads": inp.num_kv_heads,
            "head_dim": inp.head_dim,
            "block_size": inp.block_size,
            "context_tokens": main_case.tokens,
            "num_splits": main_case.S,
            "parallelism": "single GPU",
        },
        "kv_gbps_step": main_sum["kv_gbps_step"],
        "kv_tokens_per_s": main_sum["kv_tokens_per_s"],
        "cold_call_ms": main_sum.get("cold_call_ms"),
        "kv_frac_of_peak_step": round(main_sum["kv_gbps_step"] / PEAK_HBM_GBS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_config": per_config,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
