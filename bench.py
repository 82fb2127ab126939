"""Benchmark: gated causal attention prefill at S=8192, D=256, bf16 on one MI355X.

One step = one full pass of the hot path over the workload: the key/value
prologue and the attention kernel (query norm + RoPE, scores, online softmax,
context, sigmoid gate), i.e. one ``attn_prefill_gated`` call.  Inputs are
seeded synthetic tensors resident in HBM before the timed region.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints one JSON line.  ``value`` is algorithmic TFLOP/s of the whole step
(4*D FLOPs per visible (row, key, query head) triple), from one event pair
around the K steps.  ``roofline`` is for the dominant kernel (attention),
timed with the library's HIP events around each of its launches on the launch
stream; the other kernels get events only with ``--time-all-kernels`` and the
steps one each only with ``--step-spread``, since every event costs the stream
a few microseconds.  ``cpu_baseline`` times the CPU oracle on a bounded row sample
of the same workload.

A packed-batch workload (``--workload c6_varlen_16x128_2048``) runs its
sequences in one ``attn_prefill_gated_batch`` call per step; its CPU baseline
samples the longest sequence.  The shared-prefix workload (``--workload
c8_shared_4096_16x128_512``) runs its branches in one
``attn_prefill_shared_batch`` call per step over a prefix cache filled once
before the timing; its CPU baseline and parity sample the longest branch.

``--mode copy`` runs only a plain device copy of known size (used to scale the
HBM byte counters of a ``rocprofv3 --pmc`` run).  ``--mode gemm`` times the
vendor library's bf16 GEMM (torch.matmul, 8192^3, random N(0,1) operands) on
the same box: the matrix-core rate a tuned library reaches under this box's
power limit, as context for the attention kernel's ``roofline``.  ``--mode
mfma`` runs the library's calibration kernel (back-to-back bf16 MFMAs on
pseudo-random operands, one wave per SIMD on every compute unit) and reports
the shader clock and matrix-core rate the device sustains under that load.
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

PEAK_BF16_TFLOPS = 2500.0         # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attention.json")
TRAFFIC_WEIGHTS_FILE = os.path.join(ROOT, "profiles", "traffic_weights.json")
KERNEL_SOURCE = os.path.join(ROOT, "gated_gqa_causal_amd", "csrc", "kernels.hip")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """sha256 prefix of the kernels' sources (kernels.hip and the headers it
    builds from: the parameter blocks and the work schedule)."""
    h = hashlib.sha256()
    for name in ("kernels.hip", "kernels.h", "schedule.h"):
        with open(os.path.join(os.path.dirname(KERNEL_SOURCE), name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, path: str = TRAFFIC_FILE):
    """HBM bytes per launch of a kernel (the attention kernel, or the weights
    kernel) on a workload, from a committed PMC summary ({"workloads": {key:
    {"kernel_source_sha256_16": ..., "bytes_per_launch": ...}}}, the key being
    the workload name and the flags that change what runs, e.g.
    "c3_prefix_t8192_qb1024 --cached"), or None when there is no record or
    the kernel source changed since its counters were taken."""
    try:
        with open(path) as f:
            rec = json.load(f).get("workloads", {}).get(workload)
    except (OSError, ValueError, AttributeError):
        return None
    if not rec or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def kernel_algorithmic(p, rows: int, keys: int, new_keys: int, flops: float, weights: bool,
                       fp8_cache: bool = False) -> dict:
    """Algorithmic work of one launch of each kernel of a step: FLOPs for the
    attention kernel, bytes that must cross HBM at least once for every kernel.

    rows: query rows of the step; keys: keys the attention walks (T, or a
    packed batch's total); new_keys: keys the key prologue prepares (all of
    them, or the window's when the prefix comes from a cache); flops: the
    step's algorithmic FLOPs (4 D per visible (row, key, query head));
    fp8_cache: the key prologue writes e4m3 cache rows with one fp32 scale
    each, and kv_widen turns the cache's keys 0..keys-1 into bf16 tiles."""
    Hq, Hkv, D = p.n_q_heads, p.n_kv_heads, p.head_dim
    half_rot = p.rotary_dim // 2
    out_b = rows * Hq * D * 2
    att_read = (rows * Hq * 2 * D * 2                  # q|gate rows
                + 2 * Hkv * keys * D * 2               # prepared keys and transposed values
                + 2 * rows * half_rot * 4)             # cos/sin rows of the query positions
    rec = {"attention": {"flop": flops, "read_bytes": att_read, "write_bytes": out_b},
           "kv_prologue": {"read_bytes": 2 * new_keys * Hkv * D * 2 + 2 * new_keys * half_rot * 4 + D * 2,
                           "write_bytes": 2 * new_keys * Hkv * D * 2}}
    if fp8_cache:
        rec["kv_prologue"]["write_bytes"] = 2 * new_keys * Hkv * (D + 4)
        rec["kv_widen"] = {"read_bytes": 2 * keys * Hkv * (D + 4), "write_bytes": 2 * keys * Hkv * D * 2}
    if p.mask is not None:
        S = p.rows
        W = (S + 31) // 32
        # The causal part of each row, in whole 32-key words: mask_pack reads
        # those bytes and writes a bit word for every key word plus one flag per
        # (64-row block, key word); the attention kernel reads the causal words.
        causal_words = sum(i // 32 + 1 for i in range(S))
        rec["mask_pack"] = {"read_bytes": 32 * causal_words, "write_bytes": S * W * 4 + ((S + 63) // 64) * W}
        rec["attention"]["read_bytes"] += 4 * causal_words
    if weights:
        rec["weights"] = {"read_bytes": rows * Hq * D * 2 + Hkv * keys * D * 2 + rows * Hq * 8,
                          "write_bytes": rows * Hq * keys * 2}
    return rec


def cpu_info():
    """(CPU model name, logical CPUs this process may run on)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        avail = os.cpu_count() or 1
    return model, avail


def cpu_baseline(p, rows_target: int, threads: int):
    """The oracle on a bounded row sample of the workload: its key prologue
    (every key, all KV heads) and the attention of every `stride`-th row
    ending at the last, all heads, spread over `threads` host threads.
    Returns (the cpu_baseline record, the sampled rows, their oracle outputs)."""
    import numpy as np
    import oracle
    orc = oracle.get()
    stride = max(1, p.rows // rows_target)
    rows = np.arange(p.rows - 1, -1, -stride, dtype=np.int32)[::-1].copy()

    def pair_flops(rr):
        # 4 D FLOPs per visible (row, key, query head), as in the GPU's figure.
        pos = p.q_base + rr.astype(np.int64)
        if p.mask is not None:
            m = np.asarray(p.mask)[rr] != 0
            vis = (m & (np.arange(p.T)[None, :] <= pos[:, None])).sum()
        elif not p.causal:
            vis = rr.size * p.T
        else:
            vis = (pos + 1).sum()
        return 4.0 * p.head_dim * p.n_q_heads * float(vis)

    t0 = time.perf_counter()
    kp = orc.prepare_keys(p)
    t_keys = time.perf_counter() - t0
    want = orc.attention(p, rows=rows, kp=kp, threads=threads)
    dt = time.perf_counter() - t0
    flops = pair_flops(rows)
    # One thread over a fixed subset (the last 64 rows, all heads).
    last = np.arange(max(0, p.rows - 64), p.rows, dtype=np.int32)
    t1 = time.perf_counter()
    orc.attention(p, rows=last, kp=kp, threads=1)
    dt1 = time.perf_counter() - t1
    model, avail = cpu_info()
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "cores_available": avail, "cpu_model": model,
           "cores_note": "the oracle's rows spread over at most 16 threads, the host share of one GPU",
           "sample": f"{rows.size} query rows (every {stride}th, ending at the last row) x "
                     f"{p.n_q_heads} heads of {p.name}, after the key prologue over all {p.T} keys "
                     f"({t_keys:.2f} s, single-threaded, inside the timing); {dt:.2f} s wall, "
                     f"{flops / 1e9:.1f} GFLOP",
           "one_thread": {"value": pair_flops(last) / dt1 / 1e12, "unit": "TFLOP/s",
                          "sample": f"the last {last.size} rows x {p.n_q_heads} heads (keys prepared "
                                    f"beforehand), {dt1:.2f} s wall"}}
    return rec, rows, want


class TimingEvents:
    """HIP events created with hipEventDisableSystemFence, through the HIP
    runtime torch loaded: timing-only events whose recording neither writes
    back nor invalidates the caches (torch's events carry a system-scope
    fence, which at this step size adds tens of microseconds to each step)."""

    def __init__(self, n: int):
        import ctypes
        import torch
        self.ct = ctypes
        self.hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), ctypes.c_uint(0x20000000)) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i: int, stream):
        if self.hip.hipEventRecord(self.ev[i], self.ct.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed(self, i: int, j: int) -> float:
        ms = self.ct.c_float(0.0)
        if self.hip.hipEventSynchronize(self.ev[j]) != 0 or \
                self.hip.hipEventElapsedTime(self.ct.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def device_peak():
    """Compute units and peak shader clock the device reports, and the dense
    bf16 MFMA rate they give (4 SIMDs x 1024 FLOP per clock per compute unit)."""
    import torch
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    mhz = None
    try:
        import ctypes
        # The HIP runtime torch loaded (a second runtime in the process would
        # not share its device state); hipDeviceAttributeClockRate = 5, kHz.
        hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        val = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) == 0 and val.value > 0:
            mhz = val.value / 1000.0
    except (OSError, AttributeError):
        pass
    return {"compute_units": cus, "peak_sclk_mhz": mhz,
            "tflops": None if mhz is None else round(cus * 4 * 1024 * mhz * 1e6 / 1e12, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c2_dense_s8192_g4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--mode", choices=["attention", "copy", "gemm", "mfma"], default="attention")
    ap.add_argument("--cached", action="store_true",
                    help="prefix workloads: keys before q_base come from a prepared K/V cache "
                         "(attn_prefill_append); only the window's keys are prepared per step")
    ap.add_argument("--fp8-cache", action="store_true",
                    help="as --cached, with the fp8 (e4m3 rows, fp32 row scales) cache "
                         "(attn_prefill_append_fp8): each step encodes the window's keys and "
                         "widens the whole cache before the attention kernel")
    ap.add_argument("--weights", action="store_true",
                    help="each step also writes the normalised bf16 attention weights [rows][Hq][T] "
                         "(attn_prefill_weights)")
    ap.add_argument("--step-spread", action="store_true",
                    help="record an event between consecutive steps and report the per-step median/p10/p90 "
                         "(each event costs the stream a few microseconds)")
    ap.add_argument("--time-all-kernels", action="store_true",
                    help="library events around every kernel (kv prologue, mask pack too), not only the "
                         "attention (and weights) kernel")
    ap.add_argument("--preheat-ms", type=float, default=250.0,
                    help="after the W warmup steps, run untimed steps until this much time has passed "
                         "since the first one: the GPU takes 30-60 ms of load to leave its idle clocks")
    ap.add_argument("--no-spread", action="store_true",
                    help="skip the second run of K steps that gives the per-step median/p10/p90")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB scrub buffer between timed steps (outside each step's events)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the path would shard by KV head or by query rows with no exchange, but the "
              "library and this benchmark run on one GPU.", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import gated_gqa_causal_amd as ga
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.mode == "copy":
        nbytes = 1 << 30
        src = torch.empty(nbytes // 2, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read_per_copy": nbytes,
                          "bytes_written_per_copy": nbytes, "copies": args.steps}), flush=True)
        return

    if args.mode == "mfma":
        ga.attn_mfma_clock_probe(2000)                 # warm the clocks
        mhz, tf = ga.attn_mfma_clock_probe(40000)
        print(json.dumps({"mode": "mfma", "op": "v_mfma_f32_32x32x16_bf16", "operands": "uniform [-1,1) bf16",
                          "shader_mhz": round(mhz), "tflops": round(tf, 1)}), flush=True)
        return

    if args.mode == "gemm":
        n = 8192
        g = torch.Generator(device=dev)
        g.manual_seed(0)
        a = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        b = torch.randn((n, n), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
        c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
        for _ in range(max(args.warmup, 1)):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"mode": "gemm", "m": n, "n": n, "k": n, "dtype": "bf16", "ms": round(ms, 5),
                          "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)}), flush=True)
        return

    t0 = time.perf_counter()
    batch = shared = None
    if args.workload in synth.SHARED_CONFIGS:
        # Branches of one shared prefix: p stands for the longest branch (a window
        # over prefix + branch) where one problem is needed.
        shared = synth.config_shared(args.workload)
        p = max(shared.branches, key=lambda q: q.rows)
        log(f"workload {args.workload}: prefix {shared.P} tokens, {len(shared.branches)} branches, "
            f"{shared.total} new tokens (lengths {min(shared.lens)}..{max(shared.lens)}), Hq={p.n_q_heads} "
            f"Hkv={p.n_kv_heads}; generated in {time.perf_counter() - t0:.1f}s")
    elif args.workload in synth.BATCH_CONFIGS:
        # A packed batch: p stands for its longest sequence where one problem is
        # needed (shapes, the CPU baseline's sample).
        batch = synth.config_batch(args.workload)
        p = max(batch.seqs, key=lambda q: q.T)
        log(f"workload {args.workload}: {len(batch.seqs)} sequences, {batch.total} tokens "
            f"(lengths {min(batch.lens)}..{max(batch.lens)}), Hq={p.n_q_heads} Hkv={p.n_kv_heads}; "
            f"generated in {time.perf_counter() - t0:.1f}s")
    else:
        p = synth.config_problem(args.workload)
        log(f"workload {args.workload}: T={p.T} q_base={p.q_base} Hq={p.n_q_heads} Hkv={p.n_kv_heads} "
            f"mask={'yes' if p.mask is not None else 'no'}; generated in {time.perf_counter() - t0:.1f}s")

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    src = batch if batch is not None else shared if shared is not None else p
    qg, k, v = dev_bf16(src.qg), dev_bf16(src.k), dev_bf16(src.v)
    wq, wk = dev_bf16(p.q_norm_w), dev_bf16(p.k_norm_w)
    cos = torch.from_numpy(p.cos).to(dev)
    sin = torch.from_numpy(p.sin).to(dev)
    mask = None if p.mask is None else torch.from_numpy(p.mask).to(dev)
    rows = batch.total if batch is not None else shared.total if shared is not None else p.rows
    out = torch.empty((rows, p.n_q_heads * 256), dtype=torch.bfloat16, device=dev)
    # A batch's sequences each start on a 32-key tile of the workspace.
    cap = sum((L + 31) // 32 * 32 for L in batch.lens) if batch is not None else p.T
    if shared is not None:
        # positions up to the prefix plus the longest branch; every branch's own
        # keys on 32-key tiles of the workspace
        cap = max(shared.P + max(shared.lens), sum((L + 31) // 32 * 32 for L in shared.lens))
    ctx = ga.Context(p.n_q_heads, p.n_kv_heads, cap, p.rms_eps)
    stream = torch.cuda.current_stream()

    cache = None
    fp8 = bool(args.fp8_cache)
    if args.cached or fp8:
        if not p.q_base or mask is not None or not p.causal:
            raise SystemExit("--cached / --fp8-cache need a prefix workload (q_base > 0, causal, unmasked)")
        cache = ctx.kv_cache_fp8() if fp8 else ctx.kv_cache()
        append = ctx.prefill_append_fp8 if fp8 else ctx.prefill_append
        qb = p.q_base
        # The prefix's keys, prepared once outside the timing (their query rows are
        # not part of this workload: a zero qg block stands in for them).
        zero_qg = torch.zeros((qb,) + tuple(qg.shape[1:]), dtype=torch.bfloat16, device=dev)
        append(zero_qg, k[:qb], v[:qb], wq, wk, cos, sin, qb, 0, cache)
        k_new, v_new = k[qb:], v[qb:]

    shared_cache = None
    if shared is not None:
        if args.cached or fp8:
            raise SystemExit("--cached / --fp8-cache do not apply to a shared-prefix workload")
        # The prefix's keys, prepared once outside the timing into the cache the
        # branches read (its query rows are not part of this workload).
        shared_cache = ctx.kv_cache()
        pre = shared.prefix
        zero_qg = torch.zeros((shared.P,) + tuple(qg.shape[1:]), dtype=torch.bfloat16, device=dev)
        ctx.prefill_append(zero_qg, dev_bf16(pre.k), dev_bf16(pre.v), wq, wk, cos, sin, shared.P, 0, shared_cache)

    wbuf = None
    if args.weights:
        if batch is not None or cache is not None or shared is not None:
            raise SystemExit("--weights covers the single-sequence passes (gated, prefix, masked, bidirectional)")
        wbuf = torch.empty((rows, p.n_q_heads, p.T), dtype=torch.bfloat16, device=dev)
        wkind = 2 if mask is not None else 3 if not p.causal else 1 if p.q_base else 0

    def step():
        if wbuf is not None:
            ctx.prefill_weights(qg, k, v, wq, wk, cos, sin, kind=wkind, q_base=p.q_base, mask=mask, out=out,
                                weights=wbuf, stream=stream)
        elif batch is not None:
            ctx.prefill_gated_batch(qg, k, v, wq, wk, cos, sin, batch.lens, out=out, stream=stream)
        elif shared is not None:
            ctx.prefill_shared_batch(qg, k, v, wq, wk, cos, sin, shared.P, shared_cache, shared.lens, out=out,
                                     stream=stream)
        elif cache is not None:
            append(qg, k_new, v_new, wq, wk, cos, sin, p.T, p.q_base, cache, out=out, stream=stream)
        elif not p.causal:
            ctx.prefill_bidirectional(qg, k, v, wq, wk, cos, sin, out=out, stream=stream)
        elif mask is not None:
            ctx.prefill_masked(qg, k, v, wq, wk, cos, sin, mask, out=out, stream=stream)
        elif p.q_base:
            ctx.prefill_prefix(qg, k, v, wq, wk, cos, sin, p.q_base, out=out, stream=stream)
        else:
            ctx.prefill_gated(qg, k, v, wq, wk, cos, sin, out=out, stream=stream)

    tw = time.perf_counter()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # Pre-heat: from idle the shader clock ramps up over 30-60 ms of load (c2:
    # 0.49 ms per step in the first 20 steps after the warmup, 0.458 from the
    # 60th on), so untimed steps run on until preheat_ms have passed; the
    # timed steps then measure the steady state.
    pre_steps = 0
    while (time.perf_counter() - tw) * 1e3 < args.preheat_ms:
        for _ in range(10):
            step()
        pre_steps += 10
        torch.cuda.synchronize()
    preheat = {"steps": pre_steps, "ms": round((time.perf_counter() - tw) * 1e3, 1)}
    log(f"warmup {args.warmup} done, pre-heat {pre_steps} more steps ({preheat['ms']} ms since the first)")

    # Library events (a few microseconds of stream time each) only around the
    # kernels the JSON line needs: the attention kernel for `roofline`, the
    # weights kernel for `weights_roofline`; --time-all-kernels adds the rest.
    timed = [ga.ATTN_KERNEL_ATTENTION] + ([ga.ATTN_KERNEL_WEIGHTS] if args.weights else [])
    ctx.set_timing(True, kernels=None if args.time_all_kernels else timed)
    # One event pair around the K steps; --step-spread adds one event between
    # consecutive steps (per-step median/p10/p90); with --cold a 512 MiB scrub
    # write runs between steps, outside each step's event pair.
    ev = lambda: torch.cuda.Event(enable_timing=True)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None
    step_ms = None
    torch.cuda.synchronize()
    if scrub is None:
        marks = [ev() for _ in range(args.steps + 1 if args.step_spread else 2)]
        marks[0].record(stream)
        for i in range(args.steps):
            step()
            if args.step_spread:
                marks[i + 1].record(stream)
        if not args.step_spread:
            marks[1].record(stream)
        torch.cuda.synchronize()
        total_ms = marks[0].elapsed_time(marks[-1])
        if args.step_spread:
            step_ms = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
    else:
        pairs = [(ev(), ev()) for _ in range(args.steps)]
        for i in range(args.steps):
            scrub.fill_(i & 255)
            pairs[i][0].record(stream)
            step()
            pairs[i][1].record(stream)
        torch.cuda.synchronize()
        step_ms = [a.elapsed_time(b) for a, b in pairs]
        total_ms = sum(step_ms)
    attn_ms, attn_n = ctx.read_timing(ga.ATTN_KERNEL_ATTENTION)
    pro_ms, pro_n = ctx.read_timing(ga.ATTN_KERNEL_KV_PROLOGUE)
    mp_ms, mp_n = ctx.read_timing(ga.ATTN_KERNEL_MASK_PACK)
    w_ms, w_n = ctx.read_timing(ga.ATTN_KERNEL_WEIGHTS)
    ctx.set_timing(False)
    spread = None
    if step_ms is None and not args.no_spread:
        # The per-step spread from a second run of K steps with a timing-only
        # event between consecutive steps (so these steps are not the ones
        # `value` is computed from), straight after the timed steps, before
        # any host work lets the GPU idle and its clock drop.
        te = TimingEvents(args.steps + 1)
        te.record(0, stream)
        for i in range(args.steps):
            step()
            te.record(i + 1, stream)
        torch.cuda.synchronize()
        sp = [te.elapsed(i, i + 1) for i in range(args.steps)]
        te.close()
        spread = {"median": round(float(np.median(sp)), 5), "p10": round(float(np.percentile(sp, 10)), 5),
                  "p90": round(float(np.percentile(sp, 90)), 5),
                  "from": "a second run of K steps, a timing-only event between consecutive steps"}
    out_bits = out.view(torch.int16).cpu().numpy().view(np.uint16)
    bit_exact = None
    if batch is not None:
        # The longest sequence's rows of the timed launch (parity below), and the
        # bit-exact check: they equal that sequence's own launch.
        si = batch.seqs.index(p)
        s0 = int(sum(batch.lens[:si]))
        out_bits = out_bits[s0:s0 + p.T]
        alone = ctx.prefill_gated(dev_bf16(p.qg), dev_bf16(p.k), dev_bf16(p.v), wq, wk, cos, sin, stream=stream)
        torch.cuda.synchronize()
        bit_exact = {f"sequence_{si}_equals_its_own_launch": bool(torch.equal(alone, out[s0:s0 + p.T]))}
    if shared is not None:
        # The longest branch's rows of the timed launch (parity below), and the
        # bit-exact check: they equal that branch's own prefix window over prefix + branch.
        bi = shared.branches.index(p)
        b0 = int(sum(shared.lens[:bi]))
        out_bits = out_bits[b0:b0 + p.rows]
        win = ctx.prefill_prefix(dev_bf16(p.qg), dev_bf16(p.k), dev_bf16(p.v), wq, wk, cos, sin, p.q_base,
                                 stream=stream)
        torch.cuda.synchronize()
        bit_exact = {f"branch_{bi}_equals_its_own_window_pass":
                     bool(torch.equal(win, out[b0:b0 + p.rows]))}
    if (not args.no_cpu_baseline and batch is None and cache is None and wbuf is None and mask is None
            and p.causal and p.rows >= 2048):
        # The bit-exact index check on the benchmark's own inputs: a prefix
        # window over the last rows (q_base a multiple of 128) equals the same
        # rows of the timed pass.
        qb = p.q_base + (p.rows // 2) // 128 * 128
        win = ctx.prefill_prefix(qg[qb - p.q_base:], k, v, wq, wk, cos, sin, qb, stream=stream)
        torch.cuda.synchronize()
        bit_exact = {f"prefix_window_from_{qb}_equals_the_pass": bool(torch.equal(win, out[qb - p.q_base:]))}
    ms_per_step = total_ms / args.steps
    traffic_key = " ".join([args.workload] + [f for f, on in (("--cached", args.cached),
                                                              ("--fp8-cache", args.fp8_cache),
                                                              ("--weights", args.weights)) if on])
    flops = batch.flops() if batch is not None else shared.flops() if shared is not None else p.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    attn_avg_ms = attn_ms / max(attn_n, 1)
    achieved = flops / (attn_avg_ms * 1e-3) / 1e12
    log(f"timed {args.steps} steps: {ms_per_step:.4f} ms/step; attention {attn_avg_ms:.4f} ms"
        + (f", kv prologue {pro_ms / pro_n:.4f} ms" if pro_n else "")
        + (f", mask pack {mp_ms / mp_n:.4f} ms" if mp_n else "")
        + (f", weights {w_ms / max(w_n, 1):.4f} ms" if w_n else ""))

    rec = {
        "metric": "gated causal attention prefill TFLOP/s and ms at S=8192, D=256 bf16",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload,
                   "tokens": batch.total if batch is not None else shared.total if shared is not None else p.T,
                   "q_base": p.q_base, "n_q_heads": p.n_q_heads,
                   "n_kv_heads": p.n_kv_heads, "head_dim": p.head_dim, "rotary_dim": p.rotary_dim,
                   "masked": p.mask is not None, "causal": p.causal,
                   "cached_prefix": bool(args.cached or args.fp8_cache), "fp8_cache": fp8,
                   "weights": bool(args.weights),
                   "seed": (synth.BATCH_CONFIGS[args.workload]["seed"] if batch is not None else
                            synth.SHARED_CONFIGS[args.workload]["seed"] if shared is not None else p.seed),
                   "algorithmic_gflop": round(flops / 1e9, 3)},
        "step_ms": None if step_ms is None else {
            "median": round(float(np.median(step_ms)), 5),
            "p10": round(float(np.percentile(step_ms, 10)), 5),
            "p90": round(float(np.percentile(step_ms, 90)), 5),
            "caches": "cold (512 MiB scrub between steps)" if args.cold else "warm"},
        "timing_events": "library events around " + ("every kernel" if args.time_all_kernels else
                                                     " and ".join(["attention"] + (["weights"] if args.weights else [])))
                         + (", one bench event per step" if step_ms is not None else ", one pair around the steps"),
        "kernels_ms": {"attention": round(attn_avg_ms, 5),
                       "kv_prologue": round(pro_ms / pro_n, 5) if pro_n else None,
                       "mask_pack": round(mp_ms / max(mp_n, 1), 5) if mp_n else None,
                       "weights": round(w_ms / max(w_n, 1), 5) if w_n else None},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(traffic_key)},
        "peak_from_device": device_peak(),
        "warmup_preheat": preheat,
    }
    if spread is not None:
        rec["step_ms"] = spread
    if w_n:
        # Weights kernel: bf16 weights written, plus the queries, keys and row
        # statistics it reads once.
        wbytes = (rows * p.n_q_heads * p.T * 2 + rows * p.n_q_heads * 256 * 2
                  + p.n_kv_heads * p.T * 256 * 2 + rows * p.n_q_heads * 8)
        w_gbs = wbytes / (w_ms / w_n * 1e-3) / 1e9
        rec["weights_roofline"] = {"bound": "hbm", "achieved": round(w_gbs, 1), "peak": PEAK_HBM_GBS,
                                   "unit": "GB/s", "frac": round(w_gbs / PEAK_HBM_GBS, 4),
                                   "traffic": measured_traffic(traffic_key, TRAFFIC_WEIGHTS_FILE),
                                   "bytes_per_launch": wbytes}
    keys = batch.total if batch is not None else p.T
    new_keys = keys - p.q_base if cache is not None else keys
    if shared is not None:
        # the prefix's keys (read from the cache) and every branch's own
        keys, new_keys = shared.P + shared.total, shared.total
    rec["kernels_algorithmic"] = kernel_algorithmic(p, rows, keys, new_keys, flops, bool(w_n), fp8)
    if batch is not None:
        rec["config"]["sequences"] = len(batch.seqs)
        rec["config"]["seq_lens"] = batch.lens
    if shared is not None:
        rec["config"]["q_base"] = 0
        rec["config"]["prefix_len"] = shared.P
        rec["config"]["branches"] = len(shared.branches)
        rec["config"]["branch_lens"] = shared.lens
    ctx.close()
    rec["parity"] = None
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, cpu_info()[1])
        log(f"cpu baseline: oracle on {args.cpu_rows} rows, {threads} threads")
        rec["cpu_baseline"], rows_s, want = cpu_baseline(p, args.cpu_rows, threads)
        if out_bits is not None:
            # The timed pass's output on the oracle's sampled rows: the contract
            # bound and the deviation in quanta of each row-head's scale.
            sys.path.insert(0, os.path.join(ROOT, "tests"))
            from gpu_util import QUANTA_RMS_MAX, parity_record
            pr = parity_record(p.name, out_bits[rows_s], want, p.n_q_heads)
            rec["parity"] = {"rows_vs_oracle": int(rows_s.size), "elements": pr["elements"],
                             "contract_bound_violations": pr["bound_violations"],
                             "worst_bound_frac": pr["worst_bound_frac"],
                             "row_quanta_rms_max": pr["rms_quanta_max"], "row_quanta_rms_limit": QUANTA_RMS_MAX,
                             "elem_quanta_max": pr["elem_quanta_max"], "elem_outliers": pr["elem_outliers"],
                             "quanta_hist": pr["hist"], "identical": pr["identical"],
                             "bit_exact": bit_exact}
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
