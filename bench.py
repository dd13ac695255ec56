"""Benchmark: one step = moe_permute + moe_unpermute over one batch (the whole path).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3]
                    [--ep N --ep-rank R --ep-layout contiguous] [--no-sweep]

The headline workload is the largest single-GPU shape, DeepSeek-V3-shaped:
N=16384 tokens, hidden 7168 bf16, 256 experts, topk 8, Zipf(1.2) routing with
empty experts.  With ``--ep N`` the step is one expert-parallel rank's share:
the local-expert permute (moe_permute_local, rank R's experts of an N-way
split) and the unpermute of its output (moe_unpermute_local: remote slots
skipped).

Prints ONE JSON line.  ``value`` is whole-step achieved HBM bandwidth:
algorithmic bytes of permute + unpermute (each input read once, each output
written once) divided by the measured time per step, with every input already
resident in HBM.  Buffer sets rotate so that the bytes touched between two
visits of one set are at least six times the 256 MB last-level (Infinity)
cache (fewer sets still showed some reuse through that cache).

``roofline`` is for the dominant kernel of the step, timed with HIP events on
the stream the kernels run on; ``traffic`` carries the HBM bytes per launch
measured with rocprofv3 counters when the committed counter summary matches
the current kernel source (else null).  ``cpu_baseline`` times the CPU oracle
on a bounded sample of the same workload on this host.  ``sweep`` (plain
headline runs only) carries the µs-per-step curve against tokens from the
same process: the Mixtral- and Qwen3-shaped steps, tiny, and the decode sizes
N = 1, 4, 16, 64, 256 through one scratch preallocated for N = 256.
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "permute+unpermute achieved HBM GB/s (% of peak) and µs/call vs tokens"
HBM_PEAK_GBPS = 8000.0
LLC_BYTES = 256 << 20
LLC_ROTATION = 6  # bytes touched between two visits of a buffer set >= 6x the last-level cache
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "mixture_experts_token_amd", "csrc")


def algorithmic_bytes(w, local=None, id_bytes: int = 4, quant_groups: int = 0) -> dict:
    """Bytes the method must move: each input read once, each output written once.

    local: None for the plain permute, else (tokens_read, local_rows,
    num_local_experts) of a local-expert permute -- only tokens with a local
    row are read, only local rows are written (and read back by the
    unpermute, with their weights); every token still gets an output row.
    quant_groups > 0: the permute reads bf16 rows and writes one fp8 byte per
    element plus quant_groups float scales per permuted row.
    """
    import workloads as W

    b = W.ELEMENT_BYTES[w.hidden_dtype]
    if quant_groups:
        n, h, r, e = w.num_tokens, w.hidden_size, w.num_rows, w.num_experts
        by = W.ELEMENT_BYTES[w.output_dtype]
        t_read, m, nl = local if local is not None else (n, r, e)
        permute = t_read * h * 2 + m * (h + 4 * quant_groups) + id_bytes * r + 4 * r + 4 * m + 8 * (nl + 1)
        if local is not None:
            permute += 4 * e
        unpermute = m * h * by + 4 * r + 4 * m + n * h * by
        return {"permute": permute, "unpermute": unpermute, "total": permute + unpermute}
    by = W.ELEMENT_BYTES[w.output_dtype]
    n, h, r, e = w.num_tokens, w.hidden_size, w.num_rows, w.num_experts
    if local is None:
        permute = n * h * b + r * h * b + id_bytes * r + 8 * r + 8 * (e + 1)
        if w.hidden_dtype == "fp8_e4m3":
            permute += 4 * n + 4 * r
        unpermute = r * h * by + 4 * r + 4 * r + n * h * by
    else:
        t_read, m, nl = local
        permute = t_read * h * b + m * h * b + id_bytes * r + 4 * e + 4 * r + 4 * m + 8 * (nl + 1)
        if w.hidden_dtype == "fp8_e4m3":
            permute += 4 * t_read + 4 * m
        unpermute = m * h * by + 4 * r + 4 * m + n * h * by
    return {"permute": permute, "unpermute": unpermute, "total": permute + unpermute}


# Sources whose kernels a counter summary measured: a summary stays valid while
# these files are unchanged.
DIGEST_FILES = {
    "permute": ["moe_permute_device.h", "moe_permute_wave.hip", "moe_permute_fused.hip", "moe_permute_coarse.hip",
                "moe_permute_staged.hip", "moe_permute_rows.hip", "moe_permute_launch.hip", "moe_launch.h",
                "moe_plan.h"],
    "unpermute": ["moe_unpermute.hip", "moe_launch.h", "moe_plan.h"],
    "gemm": ["moe_gemm_kernels.hip", "moe_gemm_skinny.hip", "moe_gemm_device.h", "moe_launch.h", "moe_plan.h"],
}


def kernel_source_digest(op: str = "permute") -> str:
    """SHA-256 over the sources of `op`'s kernels (what the counters were taken on)."""
    h = hashlib.sha256()
    for name in sorted(DIGEST_FILES[op]):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def load_traffic(workload: str, op: str):
    """HBM bytes per call of `op` (summed over its kernels) and the kernel names, from
    the committed rocprofv3 counter summary -- only if it matches the current source."""
    path = os.path.join(PROFILES, "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None, None
    try:
        rec = json.load(open(path))
    except Exception:
        return None, None
    entry = rec.get("ops", {}).get(op)
    if not entry:
        return None, None
    kernels = entry.get("kernels")
    if entry.get("kernel_source_sha256", rec.get("kernel_source_sha256")) != kernel_source_digest(op):
        return None, kernels
    return entry.get("hbm_bytes_per_call"), kernels


def load_probe():
    """libhbm_probe.so (streaming-ceiling kernels built beside the library), or None."""
    import ctypes

    path = os.path.join(ROOT, "mixture_experts_token_amd", "libhbm_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    for fn in (lib.hbm_probe_fanout, lib.hbm_probe_reduce):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                       ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.hbm_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p]
    lib.hbm_probe_write.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.hbm_probe_read.restype = lib.hbm_probe_write.restype = ctypes.c_int
    lib.hbm_probe_fanout_source.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int, ctypes.c_int64, ctypes.c_void_p]
    lib.hbm_probe_fanout_source.restype = ctypes.c_int
    return lib


def copy_calibration(mib: int, dev) -> None:
    """A plain elementwise copy kernel (negation) over a fresh mib-MiB float32
    buffer, 5 times: its known traffic scales the rocprofv3 byte counters."""
    import torch

    src = torch.ones((mib << 20) // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize(dev)
    del src, dst


# Output width of the expert GEMM per workload: the gate and up projections of
# the expert MLP side by side (2 x the expert intermediate size).
GEMM_N = {"tiny": 256, "mixtral": 2 * 14336, "qwen3": 2 * 768, "dsv3": 2 * 2048, "decode": 2 * 2048}
MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_gemm(args, w, ids_np, dev) -> int:
    """One line for the grouped GEMM over the permuted rows (moe_grouped_gemm_bf16)."""
    import numpy as np
    import torch

    from mixture_experts_token_amd import binding

    n, k, e = args.gemm_n or GEMM_N[w.name], w.hidden_size, w.num_experts
    counts = np.bincount(ids_np.reshape(-1), minlength=e)
    off = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)).to(dev)
    rows = int(counts.sum())
    gen = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn((rows, k), device=dev, generator=gen).to(torch.bfloat16)
    wts = (torch.randn((e, n, k), device=dev, generator=gen) * k**-0.5).to(torch.bfloat16)
    y = torch.empty((rows, n), dtype=torch.bfloat16, device=dev)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, dev)
    flops = 2.0 * rows * n * k
    used = int((counts > 0).sum())
    nbytes = rows * k * 2 + used * n * k * 2 + rows * n * 2  # rows, weights of experts with rows, output
    for _ in range(args.warmup):
        binding.moe_grouped_gemm_bf16(x, wts, off, y)
    torch.cuda.synchronize(dev)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        binding.moe_grouped_gemm_bf16(x, wts, off, y)
    end.record()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    us = start.elapsed_time(end) * 1e3 / args.steps
    tflops = flops / (us * 1e-6) / 1e12
    traffic, kernels = load_traffic("%s_gemm" % w.name, "gemm")
    # The bound is the roof the shape hits first: below the ridge point
    # (peak FLOP/s over peak bytes/s) the weights' HBM traffic limits it.
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    gbps = nbytes / (us * 1e-6) / 1e9
    if flops / nbytes >= ridge:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    line = {
        "metric": "grouped GEMM over permuted rows, achieved TFLOP/s (bf16 in, fp32 accumulate)",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name + "_expert_gemm", "rows": rows, "n": n, "k": k, "num_experts": e,
                   "experts_with_rows": used, "routing": w.routing, "parallelism": "single GPU"},
        "us_per_call": round(us, 3), "flops_per_call": flops, "algorithmic_bytes_per_call": nbytes,
        "hbm_GBps_at_algorithmic_bytes": round(gbps, 1),
        "arithmetic_intensity_flop_per_byte": round(flops / nbytes, 1),
        "wall_s_timed_region": round(wall, 4),
        "roofline": dict(roof, traffic=traffic,
                         kernel=" + ".join(kernels) if kernels else "grouped_gemm_bf16_kernel",
                         algorithmic_flops_per_launch=flops, algorithmic_bytes_per_launch=nbytes,
                         avg_launch_us=round(us, 3)),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline(inputs_host, w, budget_s: float = 10.0, max_reps: int = 50, local=None, emap=None) -> dict:
    """The CPU oracle (single thread) on full steps of the workload until ~budget_s."""
    import oracle

    x, ids, wts, y = inputs_host
    nbytes = algorithmic_bytes(w, local)["total"]
    reps, t0 = 0, time.perf_counter()
    while True:
        if local is None:
            p = oracle.permute(x, ids, w.num_experts)
        else:
            p = oracle.permute_local(x, ids, w.num_experts, emap, local[2])
        oracle.unpermute(y, wts, p["inv_permuted_idx"], w.output_dtype)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            break
    return {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d full %s steps (N=%d permute + unpermute) in %.1f s, single-threaded C oracle; "
                      "host has %d cores" % (reps, w.name, w.num_tokens, el, len(os.sched_getaffinity(0)))}


def run_workload(args, w, dev) -> dict:
    """Time args.steps steps of workload w (permute + unpermute) and return the bench line."""
    import numpy as np
    import torch

    import workloads as W
    from mixture_experts_token_amd import binding

    ids_np, wts_np = W.make_routing(w, seed=0)
    local, emap_np, emap, n_off = None, None, None, w.num_experts + 1
    if args.ep > 1:
        emap_np, n_local = W.expert_map_for(w.num_experts, args.ep, args.ep_rank, args.ep_layout)
        is_local = emap_np[ids_np] >= 0
        local = (int(is_local.any(axis=1).sum()), int(is_local.sum()), n_local)
        emap = torch.from_numpy(emap_np).to(dev)
        n_off = n_local + 1
    quant = args.quant == "fp8"
    if quant:
        from dataclasses import replace as dc_replace

        w = dc_replace(w, hidden_dtype="bf16")  # the quantiser reads bf16 rows
        if args.group and (w.hidden_size % args.group or args.group & (args.group - 1)):
            raise SystemExit("--group must be a power of two dividing the hidden size")
    quant_groups = (w.hidden_size // args.group if args.group else 1) if quant else 0
    nb = algorithmic_bytes(w, local, 8 if args.ids == "int64" else 4, quant_groups)

    ids = torch.from_numpy(ids_np.astype(np.int64) if args.ids == "int64" else ids_np).to(dev)
    wts = torch.from_numpy(wts_np).to(dev)
    x0, scale0 = W.make_hidden(w, seed=0, device=dev)
    y0 = W.make_expert_output(w, seed=0, device=dev)
    hdt = x0.dtype
    step_footprint = nb["total"]
    nsets = args.sets or min(64, max(1, math.ceil(LLC_ROTATION * LLC_BYTES / step_footprint)))
    sets = []
    for i in range(nsets):
        sets.append({
            "x": x0 if i == 0 else x0.clone(),
            "scale": scale0,
            "y": y0 if i == 0 else y0.clone(),
            "xp": torch.empty((w.num_rows, w.hidden_size), dtype=torch.uint8 if quant else hdt, device=dev),
            "sp": (torch.empty((w.num_rows, quant_groups), dtype=torch.float32, device=dev) if quant else
                   None if scale0 is None else torch.empty(w.num_rows, dtype=torch.float32, device=dev)),
            "off": torch.empty(n_off, dtype=torch.int64, device=dev),
            "perm": torch.empty(w.num_rows, dtype=torch.int32, device=dev),
            "inv": torch.empty(w.num_rows, dtype=torch.int32, device=dev),
            "out": torch.empty((w.num_tokens, w.hidden_size), dtype=y0.dtype, device=dev),
        })
    if local is None:
        ws_bytes = binding.moe_permute_workspace_size(w.num_tokens, w.topk, w.num_experts)
    else:
        ws_bytes = binding.moe_permute_local_workspace_size(w.num_tokens, w.topk, w.num_experts, local[2])
    ws = torch.empty(max(16, ws_bytes), dtype=torch.uint8, device=dev)

    # Kernels go to torch's current stream (the capture stream while a graph is recorded).
    def permute(s):
        wsp = s.get("ws", ws)
        if quant:
            binding.moe_permute_quant_fp8(s["x"], ids, w.num_experts, s["xp"], s["sp"], s["off"], s["perm"], s["inv"],
                                          wsp, group_size=args.group, expert_map=emap,
                                          num_local_experts=local[2] if local is not None else 0)
        elif local is None:
            binding.moe_permute(s["x"], ids, w.num_experts, s["xp"], s["off"], s["perm"], s["inv"], wsp,
                                token_scale=s["scale"], permuted_scale=s["sp"])
        else:
            binding.moe_permute_local(s["x"], ids, w.num_experts, emap, local[2], s["xp"], s["off"], s["perm"],
                                      s["inv"], wsp, token_scale=s["scale"], permuted_scale=s["sp"])

    def unpermute(s):
        (binding.moe_unpermute if local is None else binding.moe_unpermute_local)(s["y"], wts, s["inv"], s["out"])

    def step(i):
        permute(sets[i % nsets])
        unpermute(sets[i % nsets])

    def timed(body, k):
        """Time k calls of body(i) between HIP events on the current stream; returns us per call."""
        if args.graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(k):
                    body(i)
            g.replay()
            torch.cuda.synchronize(dev)
            run = g.replay
        else:
            def run():
                for i in range(k):
                    body(i)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        start.record()
        run()
        end.record()
        torch.cuda.synchronize(dev)
        return start.elapsed_time(end) * 1e3 / k, time.perf_counter() - t0

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, dev)

    for i in range(args.warmup):
        s = sets[i % nsets]
        permute(s)
        unpermute(s)
    torch.cuda.synchronize(dev)

    k = args.steps
    # Timed region: exactly K steps (permute + unpermute), nothing else between the kernels.
    us_step, wall = timed(step, k)
    ms_step = us_step / 1e3
    value = nb["total"] / (ms_step * 1e-3) / 1e9

    # Per-operation durations: K back-to-back calls of one operation (same buffer
    # rotation) between one pair of HIP events on the kernels' stream.
    perm_avg, _ = timed(lambda i: permute(sets[i % nsets]), k)
    unperm_avg, _ = timed(lambda i: unpermute(sets[i % nsets]), k)
    # Same-run streaming ceiling for each operation's byte mix: plain fan-out and
    # reduce kernels (no index work, contiguous destinations) over the same
    # rotating buffers; the fastest of 1/2/4/8 vectors per lane with
    # non-temporal or plain stores counts.
    ceiling = None
    # the probes model the full fan-out / fan-in of unchanged rows only
    probe = load_probe() if local is None and not quant else None
    if probe is not None:
        dev_index = dev.index if dev.index is not None else 0
        xrow = w.hidden_size * W.ELEMENT_BYTES[w.hidden_dtype]
        yrow = w.hidden_size * W.ELEMENT_BYTES[w.output_dtype]

        def probe_fan(i, variant):
            s = sets[i % nsets]
            rc = probe.hbm_probe_fanout(s["x"].data_ptr(), s["xp"].data_ptr(), w.num_tokens, xrow, w.topk, variant,
                                        torch._C._cuda_getCurrentRawStream(dev_index))
            assert rc == 0, rc

        def probe_red(i, variant):
            s = sets[i % nsets]
            rc = probe.hbm_probe_reduce(s["y"].data_ptr(), s["out"].data_ptr(), w.num_tokens, yrow, w.topk, variant,
                                        torch._C._cuda_getCurrentRawStream(dev_index))
            assert rc == 0, rc

        fan_us = min(timed(lambda i: probe_fan(i, v), k)[0] for v in range(8))
        red_us = min(timed(lambda i: probe_red(i, v), k)[0] for v in range(8))
        fan_bytes = (1 + w.topk) * w.num_tokens * xrow
        red_bytes = (1 + w.topk) * w.num_tokens * yrow
        step_ceiling = (fan_bytes + red_bytes) / ((fan_us + red_us) * 1e-6) / 1e9
        ceiling = {"kind": "same-run streaming probe: same byte mix, no index work, contiguous destinations",
                   "permute_GBps": round(fan_bytes / (fan_us * 1e-6) / 1e9, 1),
                   "unpermute_GBps": round(red_bytes / (red_us * 1e-6) / 1e9, 1),
                   "step_GBps": round(step_ceiling, 1),
                   "pct_of_step_ceiling": round(100 * value / step_ceiling, 2)}
        if args.direction_split:
            # Each operation's bytes split into their two directions, each timed
            # alone (read-only and write-only probes, fastest variant), beside
            # the mixed probe and the operation itself.
            def probe_dir(i, read, buf, rows, row_bytes, variant):
                s = sets[i % nsets]
                stream = torch._C._cuda_getCurrentRawStream(dev_index)
                if read:
                    rc = probe.hbm_probe_read(s[buf].data_ptr(), s["xp"].data_ptr(), rows, row_bytes, variant, stream)
                else:
                    rc = probe.hbm_probe_write(s[buf].data_ptr(), rows, row_bytes, variant, stream)
                assert rc == 0, rc

            def fastest(read, buf, rows, row_bytes):
                return min(timed(lambda i: probe_dir(i, read, buf, rows, row_bytes, v), k)[0]
                           for v in ((0, 2, 4, 6) if read else range(8)))

            def split(read_buf, read_rows, read_row, write_buf, write_rows, write_row, mixed_us, op_us):
                r_us = fastest(True, read_buf, read_rows, read_row)
                w_us = fastest(False, write_buf, write_rows, write_row)
                return {"read_bytes": read_rows * read_row, "read_alone_us": round(r_us, 3),
                        "write_bytes": write_rows * write_row, "write_alone_us": round(w_us, 3),
                        "sum_alone_us": round(r_us + w_us, 3), "mixed_probe_us": round(mixed_us, 3),
                        "operation_us": round(op_us, 3)}

            def fan_source(i, source_rows):
                s = sets[i % nsets]
                rc = probe.hbm_probe_fanout_source(s["x"].data_ptr(), s["xp"].data_ptr(), w.num_tokens, xrow,
                                                   w.topk, source_rows, torch._C._cuda_getCurrentRawStream(dev_index))
                assert rc == 0, rc

            ceiling["direction_split"] = {
                "permute": split("x", w.num_tokens, xrow, "xp", w.num_rows, xrow, fan_us, perm_avg),
                "unpermute": split("y", w.num_rows, yrow, "out", w.num_tokens, yrow, red_us, unperm_avg)}
            # the fan-out's writes with no reads, and with reads of a few rows
            # that stay in L2 (64) or in the last-level cache (2048)
            ceiling["direction_split"]["permute"]["fanout_writes_by_source_rows_us"] = {
                str(sr): round(timed(lambda i: fan_source(i, sr), k)[0], 3)
                for sr in (0, 64, 2048) if sr <= w.num_tokens}
        torch.cuda.synchronize(dev)

    # The same steps with every output buffer and the workspace allocated per
    # call through torch's caching allocator (what a caller without
    # preallocated scratch does); eager launches only.
    alloc_cmp = None
    if args.alloc_per_call and not args.graph:
        def step_alloc(i):
            s = dict(sets[i % nsets])
            for key in ("xp", "sp", "off", "perm", "inv", "out"):
                if s[key] is not None:
                    s[key] = torch.empty_like(s[key])
            s["ws"] = torch.empty(max(16, ws_bytes), dtype=torch.uint8, device=dev)
            permute(s)
            unpermute(s)

        for i in range(args.warmup):
            step_alloc(i)
        us_alloc, _ = timed(step_alloc, k)
        alloc_cmp = {"kind": "outputs and workspace allocated per call (torch.empty), eager",
                     "us_per_step": round(us_alloc, 3),
                     "reuse_saves_pct": round(100 * (us_alloc - us_step) / us_alloc, 2)}

    tiny = torch.zeros(1, device=dev)
    floor_args = args.graph
    launch_floor_us = timed(lambda i: tiny.add_(1.0), k)[0] if floor_args else None

    if unperm_avg >= perm_avg:
        dom, dom_us, dom_bytes = "unpermute", unperm_avg, nb["unpermute"]
    else:
        dom, dom_us, dom_bytes = "permute", perm_avg, nb["permute"]
    profile_key = w.name if local is None else "%s_ep%d_r%d" % (w.name, args.ep, args.ep_rank)
    if quant:
        profile_key += "_fp8" + ("_g%d" % args.group if args.group else "")
    traffic, kernels = load_traffic(profile_key, dom)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": " + ".join(kernels) if kernels else "moe_" + dom,
                "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 3)}

    cpu = None
    if not args.no_cpu_baseline:
        to_np = lambda t: (t.view(torch.int16).cpu().numpy().view("uint16") if t.dtype == torch.bfloat16  # noqa
                           else t.cpu().numpy())
        cpu = None if quant else cpu_baseline((to_np(x0), ids_np, wts_np, to_np(y0)), w, local=local, emap=emap_np)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": k,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8_e4m3": "fp8_e4m3"}[w.hidden_dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "num_tokens": w.num_tokens, "hidden_size": w.hidden_size,
                   "num_experts": w.num_experts, "topk": w.topk, "hidden_dtype": w.hidden_dtype,
                   "output_dtype": w.output_dtype, "routing": w.routing, "ids_dtype": args.ids,
                   "quantise": None if not quant else {"to": "fp8_e4m3fn", "group": args.group or w.hidden_size},
                   "buffer_sets": nsets,
                   "parallelism": "single GPU" if local is None else
                   "one expert-parallel rank's share on a single GPU",
                   **({} if local is None else {"expert_parallel": {
                       "ep_size": args.ep, "rank": args.ep_rank, "layout": args.ep_layout,
                       "local_experts": local[2], "tokens_read": local[0], "local_rows": local[1]}})},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "us_per_step": round(ms_step * 1e3, 3),
        "permute_us": round(perm_avg, 3),
        "launch_floor_us": None if launch_floor_us is None else round(launch_floor_us, 3),
        "timing": "hip_graph_replay" if args.graph else "eager_launches",
        "unpermute_us": round(unperm_avg, 3),
        "permute_GBps": round(nb["permute"] / (perm_avg * 1e-6) / 1e9, 1),
        "unpermute_GBps": round(nb["unpermute"] / (unperm_avg * 1e-6) / 1e9, 1),
        "algorithmic_bytes_per_step": nb["total"],
        "algorithmic_bytes_per_op": {"permute": nb["permute"], "unpermute": nb["unpermute"]},
        "wall_s_timed_region": round(wall, 4),
        "ceiling": ceiling,
        **({} if alloc_cmp is None else {"alloc_per_call": alloc_cmp}),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    return line


SWEEP_EAGER = ("mixtral", "qwen3")  # large shapes: eager launches, rotating buffer sets
SWEEP_MIN_STEPS = 100


def sweep_enabled(args) -> bool:
    """The sweep rides along with a plain headline line (no expert map, quantiser or id-type variant)."""
    return (not args.no_sweep and args.ep == 1 and args.quant == "none" and args.ids == "int32" and not args.gemm
            and not args.tokens and not args.alloc_per_call)


def run_sweep(args, dev, skip: str) -> dict:
    """µs per step against tokens, every workload other than the headline's, timed in this process.

    The large shapes run like the headline (eager launches, rotating buffer
    sets, same-run streaming ceiling); tiny and the decode sizes are latency
    bound and are timed as HIP graph replays beside the same-run launch floor
    (graph replay of a one-element kernel).  The decode sweep reuses one set of
    buffers preallocated for N=256 (MoEPermuteScratch) in the order 1, 4, 16,
    64, 256, and also reports eager steps with those buffers against eager
    steps that allocate every output and the workspace per call.
    """
    import copy

    import torch

    import workloads as W

    steps = max(args.steps, SWEEP_MIN_STEPS)
    warmup = max(args.warmup, 10)
    out = {"steps_per_entry": steps, "entries": []}

    def entry(line, graph):
        return {"workload": line["config"]["workload"], "num_tokens": line["config"]["num_tokens"],
                "timing": "hip_graph_replay" if graph else "eager_launches",
                "us_per_step": line["us_per_step"], "GBps": line["value"],
                "pct_of_hbm_peak": line["pct_of_hbm_peak"], "permute_us": line["permute_us"],
                "unpermute_us": line["unpermute_us"], "launch_floor_us": line["launch_floor_us"],
                "pct_of_step_ceiling": (line["ceiling"] or {}).get("pct_of_step_ceiling")}

    for name in SWEEP_EAGER + ("tiny",):
        if name == skip:
            continue
        a = copy.copy(args)
        a.steps, a.warmup, a.no_cpu_baseline, a.sets, a.copy_calibration = steps, warmup, True, None, 0
        a.graph = name == "tiny"
        line = run_workload(a, W.WORKLOADS[name], dev)
        out["entries"].append(entry(line, a.graph))
        torch.cuda.empty_cache()
    out["entries"].extend(decode_sweep(dev, steps, warmup))
    return out


def decode_sweep(dev, steps: int, warmup: int) -> list:
    """Decode sizes N = 1, 4, 16, 64, 256 through one MoEPermuteScratch sized for N = 256."""
    import torch

    import workloads as W
    from mixture_experts_token_amd import binding

    base = W.WORKLOADS["decode"]
    n_max = max(W.DECODE_SWEEP)
    scratch = binding.MoEPermuteScratch(n_max, base.topk, base.num_experts, dev, hidden_size=base.hidden_size,
                                        hidden_dtype=torch.uint8, with_scale=True)
    out_buf = torch.empty((n_max, base.hidden_size), dtype=torch.bfloat16, device=dev)
    tiny = torch.zeros(1, device=dev)

    def timed(body, k, graph):
        if graph:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(k):
                    body(i)
            g.replay()
            torch.cuda.synchronize(dev)
            run = g.replay
        else:
            def run():
                for i in range(k):
                    body(i)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        start.record()
        run()
        end.record()
        torch.cuda.synchronize(dev)
        return start.elapsed_time(end) * 1e3 / k

    res = []
    for n in W.DECODE_SWEEP:
        w = base.with_tokens(n)
        ids_np, wts_np = W.make_routing(w, seed=0)
        ids = torch.from_numpy(ids_np).to(dev)
        wts = torch.from_numpy(wts_np).to(dev)
        x, scale = W.make_hidden(w, seed=0, device=dev)
        y = W.make_expert_output(w, seed=0, device=dev)
        out = out_buf[:n]
        nb = algorithmic_bytes(w)
        held = {}

        def permute(i):
            held["p"] = scratch.permute(x, ids, token_scale=scale)

        def unpermute(i):
            binding.moe_unpermute(y, wts, held["p"]["inv_permuted_idx"], out)

        def step(i):
            permute(i)
            unpermute(i)

        def step_alloc(i):
            xp = torch.empty((n * w.topk, w.hidden_size), dtype=torch.uint8, device=dev)
            sp = torch.empty(n * w.topk, dtype=torch.float32, device=dev)
            off = torch.empty(w.num_experts + 1, dtype=torch.int64, device=dev)
            perm = torch.empty(n * w.topk, dtype=torch.int32, device=dev)
            inv = torch.empty(n * w.topk, dtype=torch.int32, device=dev)
            ws = torch.empty(max(16, binding.moe_permute_workspace_size(n, w.topk, w.num_experts)),
                             dtype=torch.uint8, device=dev)
            o = torch.empty((n, w.hidden_size), dtype=torch.bfloat16, device=dev)
            binding.moe_permute(x, ids, w.num_experts, xp, off, perm, inv, ws, token_scale=scale, permuted_scale=sp)
            binding.moe_unpermute(y, wts, inv, o)

        for i in range(warmup):
            step(i)
            step_alloc(i)
        torch.cuda.synchronize(dev)
        us = timed(step, steps, True)
        p_us = timed(permute, steps, True)
        u_us = timed(unpermute, steps, True)
        floor = timed(lambda i: tiny.add_(1.0), steps, True)
        eager = timed(step, steps, False)
        eager_alloc = timed(step_alloc, steps, False)
        gbps = nb["total"] / (us * 1e-6) / 1e9
        res.append({"workload": "decode", "num_tokens": n, "timing": "hip_graph_replay",
                    "us_per_step": round(us, 3), "GBps": round(gbps, 1),
                    "pct_of_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2), "permute_us": round(p_us, 3),
                    "unpermute_us": round(u_us, 3), "launch_floor_us": round(floor, 3),
                    "pct_of_step_ceiling": None, "scratch": "one MoEPermuteScratch for N=256, reused",
                    "eager_us_per_step_reused": round(eager, 3),
                    "eager_us_per_step_alloc_per_call": round(eager_alloc, 3)})
    return res



def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3",
                    help="headline workload (default: the largest single-GPU shape, DeepSeek-V3-shaped)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the token sweep (the other workloads and the decode sizes, timed in the same run)")
    ap.add_argument("--tokens", type=int, default=None, help="override the workload's token count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--direction-split", action="store_true",
                    help="also time each operation's reads alone and writes alone (streaming probes)")
    ap.add_argument("--sets", type=int, default=None, help="buffer sets to rotate (default: enough to beat the LLC)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before timing, run a plain elementwise copy kernel (negation) over a fresh MIB-MiB "
                         "float32 buffer 5 times; its known traffic scales rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K steps (and each per-operation batch) in a HIP graph and time its replay")
    ap.add_argument("--ep", type=int, default=1, help="expert-parallel ranks: time one rank's local-expert step")
    ap.add_argument("--ep-rank", type=int, default=0)
    ap.add_argument("--ep-layout", default="contiguous", choices=["contiguous", "round_robin", "shuffled"])
    ap.add_argument("--quant", default="none", choices=["none", "fp8"],
                    help="fp8: the permute quantises bf16 rows to E4M3FN codes + scales on the way "
                         "(moe_permute_quant_fp8)")
    ap.add_argument("--group", type=int, default=0, help="quantisation group size in elements (0: per token)")
    ap.add_argument("--gemm", action="store_true",
                    help="time the grouped GEMM over the permuted rows instead (moe_grouped_gemm_bf16)")
    ap.add_argument("--gemm-n", type=int, default=0, help="GEMM output width (default: 2 x expert intermediate)")
    ap.add_argument("--alloc-per-call", action="store_true",
                    help="also time the same K steps with every output and the workspace allocated per call "
                         "(torch.empty, eager only), the pattern preallocated scratch replaces")
    ap.add_argument("--ids", default="int32", choices=["int32", "int64"],
                    help="expert id type handed to the permute (int64 is read directly, no cast pass)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(the path shards by token or by expert, see the design notes)" % args.gpus, file=sys.stderr)
        return 2

    import torch

    import workloads as W
    from mixture_experts_token_amd import binding

    binding.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.workload]
    if args.tokens:
        w = w.with_tokens(args.tokens)
    if args.gemm:
        ids_np, _ = W.make_routing(w, seed=0)
        return bench_gemm(args, w, ids_np, dev)
    line = run_workload(args, w, dev)
    if sweep_enabled(args):
        torch.cuda.empty_cache()
        line["sweep"] = run_sweep(args, dev, skip=w.name)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
