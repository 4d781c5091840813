"""Benchmark of the paged-KV attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-prefill]

One step is one pass of the hot path over the Llama-3-8B-shaped decode
batch: kv_cache_write of the 256 new tokens (bf16), the split-K decode
partition kernel and the merge kernel, with the 3.4 GB cache resident in HBM.
The chunked-prefill kernel (16 sequences x 256 new tokens, window 4096) is
timed in the same run and reported under "prefill".

The line printed last is one JSON object: the step's algorithmic KV bytes per
second ("value"), the decode partition kernel against the HBM roofline
(timed with HIP events on the launch stream), and the fp64 oracle timed on the
host ("cpu_baseline").  Also reported: the same prefill call over an INT8
pool ("prefill_int8"), the smaller decode workloads (tiny fp32, Qwen2.5-1.5B
shaped bf16, INT8 KV; back to back and after a cache flush: "decode_shapes"),
and the slot-mapping and block-copy kernels ("block_ops").  Every timed
configuration is checked against the oracle on sampled outputs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode attn: KV GB/s & % of HBM peak; prefill-chunk % MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
PROFILES = os.path.join(ROOT, "profiles")


class Regions:
    """roctx profiler regions: with `rocprofv3 --selected-regions` only the
    timed loops (and the calibration copy) are profiled, not input generation.
    Without a profiler attached the calls do nothing."""

    def __init__(self):
        import ctypes
        self.lib = None
        for name in ("librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so"):
            try:
                self.lib = ctypes.CDLL(name)
                break
            except OSError:
                continue

    def resume(self):
        if self.lib is not None:
            self.lib.roctxProfilerResume(0)

    def pause(self):
        if self.lib is not None:
            self.lib.roctxProfilerPause(0)


REGIONS = None


def kernel_source_hash(name: str) -> str:
    p = os.path.join(ROOT, "paged_kv_cache_235_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def read_traffic(tag: str, source: str):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on the current kernel source (profiles/<tag>.traffic.txt)."""
    path = os.path.join(PROFILES, f"{tag}.traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != kernel_source_hash(source):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ decode step
def decode_bytes(case):
    """Algorithmic bytes of one decode call: K and V of every visible key once
    per KV head (the GQA group shares the read), the block-table entries, Q
    and the fp32 output."""
    e = {"f32": 4, "bf16": 2, "i8": 1}[case.kv_dtype]
    lens = case.seq_lens.astype(np.int64)
    eff = np.minimum(lens, case.window) if case.window > 0 else lens
    kv = int(eff.sum()) * case.num_kv_heads * case.head_dim * e * 2
    if case.kv_dtype == "i8":
        kv += int(eff.sum()) * case.num_kv_heads * 2 * 2
    table = int((-(-lens // case.block_size)).sum()) * 4
    q = case.num_seqs * case.num_q_heads * case.head_dim * (4 if case.in_dtype == "f32" else 2)
    out = case.num_seqs * case.num_q_heads * case.head_dim * 4
    return {"kv": kv, "table": table, "q": q, "out": out}


def write_bytes(num_tokens, num_kv_heads, head_dim, esz=2):
    # read K and V, write them into the pools, read the slot ids
    return 2 * 2 * num_tokens * num_kv_heads * head_dim * esz + 4 * num_tokens


def partition_sweep(args, torch, pkv, tl, case, pools, bt, lens, q, sizes, check, ref, part_bytes):
    """The same resident decode batch at other split-K partition sizes (a choice
    the caller makes): the partition kernel's time between the library's events
    on the launch stream, the whole call's time, and a check of each size's
    output on the sampled sequences."""
    dev = q.device
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    res = {}
    for P in sizes:
        w = pkv.decode_workspace(case.num_seqs, case.num_q_heads, case.head_dim, case.max_blocks_per_seq,
                                 case.block_size, P, device=dev)

        def call(e=None):
            if e:
                pkv.set_decode_start_event(e[1])
                pkv.set_decode_split_event(e[2])
                e[0].record()
            pkv.paged_attention_decode(q, pools["k"], pools["v"], bt, lens, case.softmax_scale, partition_size=P,
                                       k_scale=pools["ks"], v_scale=pools["vs"], out=out, workspace=w)
            if e:
                e[3].record()
                pkv.set_decode_start_event(None)
                pkv.set_decode_split_event(None)

        for _ in range(args.warmup):
            call()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for e in ev:
            call(e)
        torch.cuda.synchronize()
        part_us = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
        call_us = float(np.mean([e[0].elapsed_time(e[3]) for e in ev])) * 1e3
        err = tl.assert_close(out[check], ref, "bf16", f"partition size {P}")
        gbs = part_bytes / (part_us * 1e-6) / 1e9
        res[str(P)] = {"partition_us": round(part_us, 1), "call_us": round(call_us, 1), "GB/s": round(gbs, 1),
                       "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "max_abs_err_sampled": float(err)}
    return res


def bench_decode(args, torch, pkv, workloads, tl):
    dev = torch.device("cuda", 0)
    case = workloads.llama_decode()
    print(f"[bench] decode setup: {case.num_seqs} seqs, {int(case.seq_lens.sum())} tokens, "
          f"{case.num_blocks} blocks", flush=True)
    pools = tl.alloc_pools(case, dev)
    tl.write_tokens(case, pools, dev, "all")      # the step rewrites its new tokens with the same values
    bt, lens, _ = tl.tables(case, dev)
    q = case.q(dev)
    new_k = case.kv_at("k", case.new_tokens(), dev)
    new_v = case.kv_at("v", case.new_tokens(), dev)
    new_slots = torch.from_numpy(case.new_slots()).to(dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    workspace = pkv.decode_workspace(case.num_seqs, case.num_q_heads, case.head_dim, case.max_blocks_per_seq,
                                     case.block_size, case.partition_size, device=dev)
    ws_bytes = workspace.numel()
    torch.cuda.synchronize()
    print(f"[bench] decode setup done; workspace {ws_bytes / 2**20:.1f} MiB", flush=True)

    def step(ev=None):
        # ev: after-start, after-write, before-partition (library), after-partition (library), end
        if ev:
            ev[0].record()
        pkv.kv_cache_write(new_k, new_v, new_slots, pools["k"], pools["v"])
        if ev:
            ev[1].record()
            pkv.set_decode_start_event(ev[2])
            pkv.set_decode_split_event(ev[3])
        pkv.paged_attention_decode(q, pools["k"], pools["v"], bt, lens, case.softmax_scale,
                                   partition_size=case.partition_size, out=out, workspace=workspace)
        if ev:
            pkv.set_decode_start_event(None)
            pkv.set_decode_split_event(None)
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps: nothing but the step's own launches between the two events
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    REGIONS.resume()
    start.record()
    for i in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    # the same number of steps again with events between the launches, for the
    # per-kernel breakdown (the markers themselves add a little to each step)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    REGIONS.pause()
    t_write = np.array([e[0].elapsed_time(e[1]) for e in evs])
    t_gap = np.array([e[1].elapsed_time(e[2]) for e in evs])       # between the write and the partition kernel
    t_part = np.array([e[2].elapsed_time(e[3]) for e in evs])
    t_merge = np.array([e[3].elapsed_time(e[4]) for e in evs])
    t_call = np.array([e[2].elapsed_time(e[4]) for e in evs])      # the decode call: partition + merge
    t_step = np.array([e[0].elapsed_time(e[4]) for e in evs])

    # correctness of the timed configuration, on a sample of sequences
    check = sorted({int(np.argmax(case.seq_lens)), int(np.argmin(case.seq_lens)), 7, 100, 200})
    sub = case.subset(check)
    from oracle.cases import build_cache, expected_outputs
    ref = expected_outputs(sub, cache=build_cache(sub, device=dev))
    err = tl.assert_close(out[check], ref, "bf16", "bench decode")

    b = decode_bytes(case)
    wb = write_bytes(case.num_seqs, case.num_kv_heads, case.head_dim)
    step_bytes = sum(b.values()) + wb
    part_bytes = b["kv"] + b["table"] + b["q"]
    part_s = float(np.mean(t_part)) / 1e3
    achieved = part_bytes / part_s / 1e9
    call_s = float(np.mean(t_call)) / 1e3
    call_achieved = part_bytes / call_s / 1e9
    sweep = None
    if not args.no_extra:
        sweep = partition_sweep(args, torch, pkv, tl, case, pools, bt, lens, q, (512, 1024, 2048), check, ref,
                                part_bytes)
    return {
        "partition_size_sweep": sweep,
        "case": case,
        "pools": pools,
        "out": out,
        "ms_per_step": total_ms / args.steps,
        "wall_ms_per_step": wall * 1e3 / args.steps,
        "step_bytes": step_bytes,
        "breakdown_us": {"kv_cache_write": float(np.mean(t_write)) * 1e3,
                         "write_to_partition_gap": float(np.mean(t_gap)) * 1e3,
                         "decode_partition": float(np.mean(t_part)) * 1e3,
                         "decode_merge": float(np.mean(t_merge)) * 1e3,
                         "decode_call": float(np.mean(t_call)) * 1e3,
                         "step_median": float(np.median(t_step)) * 1e3,
                         "step_p10": float(np.percentile(t_step, 10)) * 1e3,
                         "step_p90": float(np.percentile(t_step, 90)) * 1e3},
        "bytes": b,
        # the step's cache write on its own: read and write of the 256 new K/V vectors
        "kv_cache_write": {"us": round(float(np.mean(t_write)) * 1e3, 2), "bytes": wb,
                           "GB/s": round(wb / (float(np.mean(t_write)) / 1e3) / 1e9, 1)},
        "roofline": {"kernel": "decode_partition_kernel<bf16, D=128, G=4>", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic("decode_llama3_8b_shaped", "decode.hip"),
                     "algorithmic_bytes_per_launch": part_bytes},
        # the whole decode call (partition kernel + merge kernel, from the event
        # before the partition kernel to the one after the call), same bytes
        "roofline_call": {"what": "paged_attention_decode call: partition + merge kernels", "bound": "hbm",
                          "achieved": round(call_achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": round(call_achieved / HBM_PEAK_GBS, 4), "us": round(call_s * 1e6, 1),
                          "algorithmic_bytes_per_call": part_bytes},
        "max_abs_err": float(err),
    }


def full_output_parity(tl, out, ref):
    """Every output element of the timed decode call against the oracle: the
    the benchmark spec tolerances asserted, the worst errors reported."""
    g = out.detach().float().cpu().double().numpy().reshape(ref.shape)
    err = np.abs(g - ref)
    dim = ref.shape[-1]
    e = err.reshape(-1, dim).max(1)
    r = np.abs(ref).reshape(-1, dim).max(1)
    rel = float((e[r > 0] / r[r > 0]).max()) if (r > 0).any() else 0.0
    tl.assert_close(out, ref, "bf16", "whole Llama-shaped decode output")
    return {"rows": int(ref.shape[0] * ref.shape[1]), "max_abs_err": float(err.max()),
            "max_per_vector_rel_err": rel, "tolerance": {"abs": tl.ABS_BF16, "per_vector_rel": tl.REL_BF16}}


def run_metadata(torch):
    """ROCm version, GPU, library source hash (and git revision where a checkout
    is present), and the seed of every workload the line reports."""
    import subprocess
    rocm = None
    for path in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        try:
            rocm = open(path).read().strip()
            break
        except OSError:
            continue
    props = torch.cuda.get_device_properties(0)
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_235_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        h.update(name.encode())
        h.update(open(os.path.join(csrc, name), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "pagedkv.h"), "rb").read())
    rev = None
    try:
        rev = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                             timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        pass
    return {"rocm": rocm, "torch": torch.__version__, "gpu": props.name,
            "gcn_arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
            "library_source_sha256_16": h.hexdigest()[:16], "git_rev": rev,
            "seeds": {"llama3-8b-decode": 3, "prefill-window": 5, "qwen2.5-1.5b-decode": 2,
                      "int8-kv-decode": 4, "tiny-fp32-decode": 1, "mixed-step": 6,
                      "kv_cache_write_at_scale": 11}}


def host_cpu():
    """Host CPU model and logical core count (the oracle runs on one of them)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "logical_cores": os.cpu_count()}


def cpu_baseline(case, torch, dev):
    """The fp64 oracle (single-threaded C) on the whole decode step: K/V come
    from the seeded generator (run on the GPU, copied to the host), the
    oracle writes its own host pool; only gather + attention are timed."""
    import oracle
    from oracle.cases import build_cache, to_numpy
    cache = build_cache(case, device=dev)
    q = to_numpy(case.q())
    t0 = time.perf_counter()
    ref = oracle.decode(cache, q, case.in_dtype, case.seq_lens, case.block_tables, case.softmax_scale,
                        case.window)
    dt = time.perf_counter() - t0
    kv = decode_bytes(case)
    step_bytes = sum(kv.values()) + write_bytes(case.num_seqs, case.num_kv_heads, case.head_dim)
    return {"value": round(step_bytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3), "host": host_cpu(),
            "sample": f"the whole decode step: all {case.num_seqs} sequences, "
                      f"{int(case.seq_lens.sum())} context tokens, gather + two-pass fp64 attention "
                      f"on one host thread"}, ref


# ------------------------------------------------------------------ prefill
def prefill_flops(case):
    """Algorithmic flops: 4 * D per visible (query row, key) pair per query head."""
    total = 0
    for s in range(case.num_seqs):
        L, C = int(case.seq_lens[s]), int(case.new_lens[s])
        p = np.arange(L - C, L, dtype=np.int64)
        vis = p + 1 if case.window <= 0 else np.minimum(p + 1, case.window)
        total += int(vis.sum())
    return 4 * case.head_dim * case.num_q_heads * total


def bench_prefill(args, torch, pkv, workloads, tl, kv_dtype="bf16"):
    dev = torch.device("cuda", 0)
    case = workloads.prefill_window()
    if kv_dtype == "i8":
        import dataclasses
        case = dataclasses.replace(case, kv_dtype="i8", outliers=0.01)
    pools = tl.alloc_pools(case, dev)
    tl.write_tokens(case, pools, dev, "all")      # the chunk's own tokens are rewritten before each call
    bt, lens, cu = tl.tables(case, dev)
    q = case.q(dev)
    new_k = case.kv_at("k", case.new_tokens(), dev)
    new_v = case.kv_at("v", case.new_tokens(), dev)
    new_slots = torch.from_numpy(case.new_slots()).to(dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)

    def call():
        pkv.paged_attention_prefill_chunk(q, cu, lens, pools["k"], pools["v"], bt, case.max_q_len,
                                          case.softmax_scale, sliding_window=case.window, out=out,
                                          k_scale=pools["ks"], v_scale=pools["vs"])

    pkv.kv_cache_write(new_k, new_v, new_slots, pools["k"], pools["v"], pools["ks"], pools["vs"])
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    REGIONS.resume()
    for e in evs:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    REGIONS.pause()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    check = [0, int(np.argmax(case.seq_lens)), int(np.argmin(case.seq_lens))]
    sub = case.subset(sorted(set(check)))
    from oracle.cases import build_cache, expected_outputs
    ref = expected_outputs(sub, cache=build_cache(sub, device=dev))
    cu_np = case.cu_q_lens
    rows = np.concatenate([np.arange(cu_np[s], cu_np[s + 1]) for s in sorted(set(check))])
    err = tl.assert_close(out[torch.from_numpy(rows).to(dev)], ref, "bf16", "bench prefill")
    fl = prefill_flops(case)
    sec = float(np.mean(t)) / 1e3
    tf = fl / sec / 1e12
    kern = "prefill_ring_kernel<W=8> (bf16 pool, head_dim 128)" if kv_dtype == "bf16" else "prefill_pipe_kernel<D=128, 8 waves, INT8>"
    return {"workload": "chunked prefill: 16 sequences x 256 new tokens on 1024..16384-token paged "
                        f"contexts, 32 q / 8 kv heads, head_dim 128, {kv_dtype} pool, causal + window 4096",
            "us_per_call": round(sec * 1e6, 2), "us_p10": round(float(np.percentile(t, 10)) * 1e3, 2),
            "us_p90": round(float(np.percentile(t, 90)) * 1e3, 2),
            "roofline": {"kernel": kern, "bound": "mfma", "achieved": round(tf, 1),
                         "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                         "traffic": read_traffic("prefill_window" if kv_dtype == "bf16" else "prefill_window_int8",
                                                 "prefill.hip"),
                         "algorithmic_flops_per_launch": fl},
            "max_abs_err": float(err)}


# ------------------------------------------------------------------ INT8 at the large batch
def bench_decode_int8_large(args, torch, pkv, workloads, tl):
    """The Llama-3-8B-shaped decode batch over an INT8 pool (K/V written through
    the quantising cache write): the partition kernel's time and its algorithmic
    bytes (codes + fp16 scales) per second, next to the bf16 figure."""
    import dataclasses
    dev = torch.device("cuda", 0)
    case = dataclasses.replace(workloads.llama_decode(), kv_dtype="i8")
    pools = tl.alloc_pools(case, dev)
    tl.write_tokens(case, pools, dev, "all")
    bt, lens, _ = tl.tables(case, dev)
    q = case.q(dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    workspace = pkv.decode_workspace(case.num_seqs, case.num_q_heads, case.head_dim, case.max_blocks_per_seq,
                                     case.block_size, case.partition_size, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]

    def call(e=None):
        if e:
            pkv.set_decode_start_event(e[0])
            pkv.set_decode_split_event(e[1])
        pkv.paged_attention_decode(q, pools["k"], pools["v"], bt, lens, case.softmax_scale,
                                   partition_size=case.partition_size, k_scale=pools["ks"], v_scale=pools["vs"],
                                   out=out, workspace=workspace)
        if e:
            pkv.set_decode_start_event(None)
            pkv.set_decode_split_event(None)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    REGIONS.resume()
    for e in ev:
        call(e)
    torch.cuda.synchronize()
    REGIONS.pause()
    us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
    check = sorted({int(np.argmax(case.seq_lens)), int(np.argmin(case.seq_lens)), 7})
    sub = case.subset(check)
    from oracle.cases import build_cache, expected_outputs
    ref = expected_outputs(sub, cache=build_cache(sub, device=dev))
    err = tl.assert_close(out[check], ref, "bf16", "int8 large decode")
    b = decode_bytes(case)
    part_bytes = b["kv"] + b["table"] + b["q"]
    sweep = partition_sweep(args, torch, pkv, tl, case, pools, bt, lens, q, (512, 1024, 2048), check, ref,
                            part_bytes)
    del pools
    torch.cuda.empty_cache()
    return {"workload": "Llama-3-8B-shaped decode batch (256 seqs, 840,545 tokens) over an INT8 pool",
            "partition_us": round(us, 1), "algorithmic_bytes_per_launch": part_bytes,
            "GB/s": round(part_bytes / (us / 1e6) / 1e9, 1),
            "frac_of_hbm_peak": round(part_bytes / (us / 1e6) / 1e9 / HBM_PEAK_GBS, 4),
            "max_abs_err_sampled": float(err), "partition_size_sweep": sweep}


# ------------------------------------------------------------------ mixed step
def bench_mixed(args, torch, pkv, workloads, tl):
    """A serving step mixing 16 prefill chunks (256 tokens each) with 240 decode
    rows, window 4096: one prefill-kernel launch over the whole batch, against
    two launches on the same pool (prefill kernel over the chunks, decode kernel
    over the decode rows), on one stream and on two streams that may overlap.
    Sampled rows of each are checked against the oracle."""
    dev = torch.device("cuda", 0)
    case = workloads.mixed_step()
    pools = tl.alloc_pools(case, dev)
    tl.write_tokens(case, pools, dev, "all")
    bt, lens, cu = tl.tables(case, dev)
    q = case.q(dev)
    npf = int((case.new_lens > 1).sum())
    rows_pf = int(case.cu_q_lens[npf])
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    out2 = torch.empty(q.shape, dtype=torch.float32, device=dev)
    out3 = torch.empty(q.shape, dtype=torch.float32, device=dev)
    workspace = pkv.decode_workspace(case.num_seqs - npf, case.num_q_heads, case.head_dim, case.max_blocks_per_seq,
                                     case.block_size, 512, device=dev)
    cu_pf = cu[:npf + 1].contiguous()

    def one():
        pkv.paged_attention_prefill_chunk(q, cu, lens, pools["k"], pools["v"], bt, case.max_q_len,
                                          case.softmax_scale, sliding_window=case.window, out=out)

    def two():
        pkv.paged_attention_prefill_chunk(q[:rows_pf], cu_pf, lens[:npf], pools["k"], pools["v"], bt[:npf],
                                          case.max_q_len, case.softmax_scale, sliding_window=case.window,
                                          out=out2[:rows_pf])
        pkv.paged_attention_decode(q[rows_pf:], pools["k"], pools["v"], bt[npf:], lens[npf:], case.softmax_scale,
                                   sliding_window=case.window, partition_size=512, out=out2[rows_pf:],
                                   workspace=workspace)

    s_a, s_b = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)    # default priority

    def two_streams():
        # the same two launches on two streams, free to run at the same time
        cur = torch.cuda.current_stream(dev)
        e0 = torch.cuda.Event()
        e0.record(cur)
        s_a.wait_event(e0)
        s_b.wait_event(e0)
        with torch.cuda.stream(s_b):
            pkv.paged_attention_decode(q[rows_pf:], pools["k"], pools["v"], bt[npf:], lens[npf:], case.softmax_scale,
                                       sliding_window=case.window, partition_size=512, out=out3[rows_pf:],
                                       workspace=workspace)
        with torch.cuda.stream(s_a):
            pkv.paged_attention_prefill_chunk(q[:rows_pf], cu_pf, lens[:npf], pools["k"], pools["v"], bt[:npf],
                                              case.max_q_len, case.softmax_scale, sliding_window=case.window,
                                              out=out3[:rows_pf])
        cur.wait_stream(s_a)
        cur.wait_stream(s_b)

    res = {"workload": "mixed serving step: 16 prefill chunks of 256 tokens on 1024..16384-token contexts + "
                       "240 decode rows on clipped log-normal contexts (median 2048), 32 q / 8 kv heads, "
                       "head_dim 128, bf16, window 4096",
           "algorithmic_flops": prefill_flops(case)}
    for name, fn in (("one_launch_prefill_kernel", one), ("two_launches_prefill_plus_decode", two),
                     ("two_launches_on_two_streams", two_streams)):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        REGIONS.resume()
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        REGIONS.pause()
        us = float(np.mean([a.elapsed_time(b) for a, b in ev])) * 1e3
        res[name] = {"us_per_step": round(us, 2), "TFLOP/s": round(res["algorithmic_flops"] / (us / 1e6) / 1e12, 1)}
    # both paths against the oracle on sampled rows (decode over the matching prefix)
    import oracle
    from oracle.cases import build_cache, to_numpy
    picks = [0, 9, 16, 100, case.num_seqs - 1]
    sub = case.subset(picks)
    cache = build_cache(sub, device=dev)
    qs = to_numpy(sub.q(dev))
    err = 0.0
    for si, s_ in enumerate(picks):
        L, C = int(case.seq_lens[s_]), int(case.new_lens[s_])
        for i in sorted({0, C - 1}):
            row = int(sub.cu_q_lens[si]) + i
            ref = oracle.decode(cache, qs[row:row + 1], "bf16", np.array([L - C + i + 1], np.int32),
                                sub.block_tables[si:si + 1], sub.softmax_scale, sub.window)
            r = int(case.cu_q_lens[s_]) + i
            err = max(err, tl.assert_close(out[r:r + 1], ref, "bf16", "mixed one launch"),
                      tl.assert_close(out2[r:r + 1], ref, "bf16", "mixed two launches"),
                      tl.assert_close(out3[r:r + 1], ref, "bf16", "mixed two streams"))
    res["two_streams_equal_one_stream"] = bool(torch.equal(out2, out3))
    res["max_abs_err_sampled"] = float(err)
    del pools
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ other decode shapes
def back_to_back_us(torch, fn, n):
    """GPU time per call of n calls queued back to back: the GPU is held by a
    spin kernel while the host queues them, so host launch cost is not timed."""
    torch.cuda._sleep(20_000_000)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / n


def bench_decode_shapes(args, torch, pkv, workloads, tl):
    """The smaller decode workloads at several partition sizes: calls back to
    back (their K/V, a few MB, stay in the 256 MB last-level cache: 'warm') and
    one at a time after a 1 GiB write that evicts them ('cold', from HBM).  Each
    configuration is checked against the oracle."""
    from oracle.cases import expected_outputs
    dev = torch.device("cuda", 0)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    res = {}
    for name, make in (("tiny fp32 decode (4 seqs, 4 q / 2 kv, D 64)", workloads.tiny_fp32_decode),
                       ("Qwen2.5-1.5B-shaped bf16 decode (8 seqs, 12 q / 2 kv, D 128)", workloads.qwen_decode),
                       ("INT8-KV decode (64 seqs, Qwen2.5-1.5B shapes, 1% x8 outliers)", workloads.int8_decode)):
        case = make()
        pools = tl.alloc_pools(case, dev)
        tl.write_tokens(case, pools, dev, "all")
        bt, lens, _ = tl.tables(case, dev)
        q = case.q(dev)
        out = torch.empty(q.shape, dtype=torch.float32, device=dev)
        from oracle.cases import build_cache
        ref = expected_outputs(case, cache=build_cache(case, device=dev))
        by = decode_bytes(case)
        nbytes = sum(by.values())
        entry = {"workload": name, "context_tokens": int(case.seq_lens.sum()), "algorithmic_bytes": nbytes,
                 "by_partition_size": {}}
        for part in (0, 64, 128, 256, 512):
            workspace = pkv.decode_workspace(case.num_seqs, case.num_q_heads, case.head_dim,
                                             case.max_blocks_per_seq, case.block_size, part, device=dev)

            def call():
                pkv.paged_attention_decode(q, pools["k"], pools["v"], bt, lens, case.softmax_scale,
                                           sliding_window=case.window, partition_size=part,
                                           k_scale=pools["ks"], v_scale=pools["vs"], out=out, workspace=workspace)

            for _ in range(args.warmup):
                call()
            torch.cuda.synchronize()
            n = max(args.steps, 20)
            REGIONS.resume()
            warm = back_to_back_us(torch, call, n)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for a, b in ev:                       # cold: the cache evicted first
                flush.fill_(1.0)
                a.record()
                call()
                b.record()
            torch.cuda.synchronize()
            REGIONS.pause()
            cold = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
            err = tl.assert_close(out, ref, "f32" if case.kv_dtype == "f32" else "bf16", f"{name} P={part}")
            entry["by_partition_size"][part] = {
                "warm_us": round(warm, 2), "warm_GB/s": round(nbytes / (warm / 1e6) / 1e9, 1),
                "cold_us_median": round(cold, 2), "cold_GB/s": round(nbytes / (cold / 1e6) / 1e9, 1),
                "max_abs_err": float(err)}
        best = min(entry["by_partition_size"], key=lambda k: entry["by_partition_size"][k]["cold_us_median"])
        entry["best_partition_size_cold"] = best
        entry["best_cold_frac_of_hbm_peak"] = round(
            entry["by_partition_size"][best]["cold_GB/s"] / HBM_PEAK_GBS, 4)
        res[case.name] = entry
        del pools
    del flush
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ block bookkeeping kernels
def bench_block_ops(args, torch, pkv, workloads):
    """Device slot mapping for the two large steps, and a burst of block copies
    (copy on write of 256 shared Llama-shaped blocks: 8 kv heads x 16 x 128 bf16)."""
    dev = torch.device("cuda", 0)
    res = {}
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    for tag, case in (("llama3-8b decode step (256 rows)", workloads.llama_decode()),
                      ("window-4096 prefill step (4096 rows)", workloads.prefill_window())):
        k_pool = torch.empty((case.num_blocks, 1, 16, 64), dtype=torch.bfloat16, device=dev)   # shape only
        cu, lens, bt = t(case.cu_q_lens), t(case.seq_lens), t(case.block_tables)
        out = torch.empty(int(case.cu_q_lens[-1]), dtype=torch.int32, device=dev)
        for _ in range(args.warmup):
            pkv.build_slot_mapping(cu, lens, bt, k_pool, out=out)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        REGIONS.resume()
        for a, b in ev:
            a.record()
            pkv.build_slot_mapping(cu, lens, bt, k_pool, out=out)
            b.record()
        torch.cuda.synchronize()
        warm = back_to_back_us(torch, lambda: pkv.build_slot_mapping(cu, lens, bt, k_pool, out=out), args.steps)
        REGIONS.pause()
        assert np.array_equal(out.cpu().numpy(), case.new_slots()), tag
        us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
        res["slot_mapping: " + tag] = {"us_median_one_call": round(us, 2), "us_back_to_back": round(warm, 2)}
    nb, pairs = 4096, 256
    shape = (nb, 8, 16, 128)
    k = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    v = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    perm = np.random.default_rng(0).permutation(nb).astype(np.int32)
    src, dst = t(perm[:pairs]), t(perm[pairs:2 * pairs])
    for _ in range(args.warmup):
        pkv.kv_cache_copy_blocks(src, dst, k, v)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    REGIONS.resume()
    for a, b in ev:
        a.record()
        pkv.kv_cache_copy_blocks(src, dst, k, v)
        b.record()
    torch.cuda.synchronize()
    warm = back_to_back_us(torch, lambda: pkv.kv_cache_copy_blocks(src, dst, k, v), args.steps)
    REGIONS.pause()
    us = float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e3
    moved = 2 * 2 * pairs * 8 * 16 * 128 * 2           # K and V, read and written
    res["copy_blocks: 256 Llama-shaped blocks"] = {"us_median_one_call": round(us, 2),
                                                    "us_back_to_back": round(warm, 2), "bytes": moved,
                                                    "GB/s_back_to_back": round(moved / (warm / 1e6) / 1e9, 1)}
    return res


def calibrate_copy(torch):
    """A plain elementwise copy of known size (negation, so the kernel is easy to
    pick out by name), for scaling rocprofv3 byte counters: each launch reads
    and writes exactly 1 GiB."""
    dev = torch.device("cuda", 0)
    n = 1 << 28                      # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    REGIONS.resume()
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    REGIONS.pause()
    print(f"[bench] calibration copy: 3 launches, each {n * 4} bytes read and {n * 4} written", flush=True)


def bench_kv_write(args, torch, pkv):
    """kv_cache_write at sizes where bandwidth, not launch latency, decides: the
    window-4096 prefill step's 4096 new tokens and a 65536-token batch, as bf16
    copies and as INT8 quantising writes, Llama-shaped heads (8 KV heads,
    head_dim 128), slots on shuffled blocks.  Algorithmic bytes: the bf16 K and
    V read once, the pool bytes (and fp16 scales) written once."""
    dev = torch.device("cuda", 0)
    hkv, d, bs = 8, 128, 16
    g = torch.Generator(device=dev).manual_seed(11)
    res = {}
    for n in (4096, 65536):
        nb = n // bs
        k = torch.randn((n, hkv, d), device=dev, dtype=torch.float32, generator=g).to(torch.bfloat16)
        v = torch.randn((n, hkv, d), device=dev, dtype=torch.float32, generator=g).to(torch.bfloat16)
        perm = torch.randperm(nb, device=dev, generator=g).to(torch.int32)
        slots = (perm[:, None] * bs + torch.arange(bs, device=dev, dtype=torch.int32)[None, :]).reshape(-1)
        for kv in ("bf16", "i8"):
            if kv == "bf16":
                kp = torch.empty((nb, hkv, bs, d), dtype=torch.bfloat16, device=dev)
                vp = torch.empty_like(kp)
                ks = vs = None
                wbytes = 2 * n * hkv * d * 2
            else:
                kp = torch.empty((nb, hkv, bs, d), dtype=torch.int8, device=dev)
                vp = torch.empty_like(kp)
                ks = torch.empty((nb, hkv, bs), dtype=torch.float16, device=dev)
                vs = torch.empty_like(ks)
                wbytes = 2 * n * hkv * (d + 2)
            nbytes = 2 * n * hkv * d * 2 + wbytes
            call = lambda: pkv.kv_cache_write(k, v, slots, kp, vp, ks, vs)
            for _ in range(args.warmup):
                call()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
            for a_, b_ in ev:
                a_.record()
                call()
                b_.record()
            torch.cuda.synchronize()
            us = float(np.median([a_.elapsed_time(b_) for a_, b_ in ev])) * 1e3
            res[f"{kv} pool, {n} tokens"] = {"us_median": round(us, 2), "bytes": nbytes,
                                             "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del k, v, kp, vp, ks, vs
    torch.cuda.empty_cache()
    return res


def measured_peaks(torch):
    """What this GPU reaches, beside the published peaks the roofline fractions
    are quoted against.  The measurement kernels of include/pkv_probe.h: a
    streaming read of 4 GiB (far past the 256 MiB last-level cache; every
    16-byte chunk read once, four loads in flight per thread, in grid-stride
    order and in a contiguous span per workgroup) and bf16 MFMA
    chains with no memory traffic; best over a few grid sizes.  torch's copy
    and GEMM are given as library reference points.  Each rate is the mean over
    back-to-back launches between two events, after untimed launches."""
    import ctypes
    from paged_kv_cache_235_amd import _build
    plib = ctypes.CDLL(_build.PROBE_LIB_PATH)
    for f in (plib.pkv_probe_stream_read, plib.pkv_probe_stream_read_spans):
        f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    plib.pkv_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                         ctypes.c_void_p]
    dev = torch.device("cuda", 0)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def seconds(fn, reps):
        for _ in range(2):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps / 1e3

    def call(rc):
        if rc != 0:
            raise RuntimeError(f"probe launch failed ({rc})")

    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    threads = 256
    read, spans = {}, {}
    for grid in (2048, 4096, 8192, 16384, 32768):
        sink = torch.empty(grid * threads, dtype=torch.int32, device=dev)
        for fn, res in ((plib.pkv_probe_stream_read, read), (plib.pkv_probe_stream_read_spans, spans)):
            t = seconds(lambda: call(fn(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                        ctypes.c_void_p(sink.data_ptr()), grid, stream)), 10)
            res[grid] = nbytes / t / 1e9
    out = torch.empty_like(buf)
    t_copy = seconds(lambda: out.copy_(buf), 10)
    del buf, out
    mfma = {}
    iters = 10000
    for grid in (512, 1024):
        sink = torch.empty(grid * threads, dtype=torch.float32, device=dev)
        t = seconds(lambda: call(plib.pkv_probe_mfma_bf16(ctypes.c_void_p(sink.data_ptr()), iters, grid, 1,
                                                          stream)), 5)
        mfma[grid] = grid * 4 * iters * 4 * 32768 / t / 1e12
    m = 8192
    g = torch.Generator(device=dev).manual_seed(0)
    a_ = torch.randn(m, m, device=dev, dtype=torch.bfloat16, generator=g)
    b_ = torch.randn(m, m, device=dev, dtype=torch.bfloat16, generator=g)
    c_ = torch.empty(m, m, device=dev, dtype=torch.bfloat16)
    t_mm = seconds(lambda: torch.matmul(a_, b_, out=c_), 20)
    del a_, b_, c_
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(max(max(read.values()), max(spans.values())), 1),
            "hbm_read_GBps_by_grid": {str(k): round(v, 1) for k, v in read.items()},
            "hbm_read_spans_GBps_by_grid": {str(k): round(v, 1) for k, v in spans.items()},
            "bf16_mfma_TFLOPs": round(max(mfma.values()), 1),
            "bf16_mfma_TFLOPs_by_grid": {str(k): round(v, 1) for k, v in mfma.items()},
            "torch_copy_GBps": round(2 * nbytes / t_copy / 1e9, 1),
            "torch_bf16_gemm_8192_TFLOPs": round(2 * m ** 3 / t_mm / 1e12, 1),
            "how": "pkv_probe_stream_read (grid-stride order) and pkv_probe_stream_read_spans (a contiguous "
                   "span per workgroup) over 4 GiB, the best of both orders and all grids; pkv_probe_mfma_bf16 "
                   "(10000 rounds of 4 MFMA chains per wave), best grid; torch copy_ of 4 GiB (read + write) and "
                   "torch.matmul of two 8192^2 bf16 matrices for reference"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the smaller decode shapes, the block kernels and the measured peaks")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (scale for rocprofv3 byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged-attention path here has no multi-GPU "
              "mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    global REGIONS
    REGIONS = Regions()
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import paged_kv_cache_235_amd as pkv
    import workloads
    import pkv_testlib as tl

    pkv.load_library()
    if args.calibrate_copy:
        calibrate_copy(torch)
    d = bench_decode(args, torch, pkv, workloads, tl)
    print(f"[bench] decode: {d['ms_per_step'] * 1e3:.1f} us/step, partition "
          f"{d['breakdown_us']['decode_partition']:.1f} us = {d['roofline']['achieved']:.0f} GB/s", flush=True)
    case = d.pop("case")
    d.pop("pools")
    torch.cuda.empty_cache()
    pre = pre8 = None
    if not args.no_prefill:
        try:
            pre = bench_prefill(args, torch, pkv, workloads, tl)
            print(f"[bench] prefill: {pre['us_per_call']:.1f} us = {pre['roofline']['achieved']:.0f} TFLOP/s",
                  flush=True)
        except pkv.PagedKVError as e:
            pre = {"error": str(e)}
        torch.cuda.empty_cache()
        try:
            pre8 = bench_prefill(args, torch, pkv, workloads, tl, kv_dtype="i8")
            print(f"[bench] prefill INT8: {pre8['us_per_call']:.1f} us = {pre8['roofline']['achieved']:.0f} TFLOP/s",
                  flush=True)
        except pkv.PagedKVError as e:
            pre8 = {"error": str(e)}
        torch.cuda.empty_cache()
    shapes = blocks = mixed = i8big = kvw = None
    if not args.no_extra:
        i8big = bench_decode_int8_large(args, torch, pkv, workloads, tl)
        print(f"[bench] INT8 Llama-shaped decode: {i8big}", flush=True)
        mixed = bench_mixed(args, torch, pkv, workloads, tl)
        print(f"[bench] mixed step: {mixed}", flush=True)
        shapes = bench_decode_shapes(args, torch, pkv, workloads, tl)
        for k_, v_ in shapes.items():
            b_ = v_["best_partition_size_cold"]
            print(f"[bench] {k_}: best partition {b_}: {v_['by_partition_size'][b_]}", flush=True)
        blocks = bench_block_ops(args, torch, pkv, workloads)
        print(f"[bench] block ops: {blocks}", flush=True)
        kvw = bench_kv_write(args, torch, pkv)
        print(f"[bench] kv_cache_write at scale: {kvw}", flush=True)
    peaks = None
    if not args.no_extra:
        peaks = measured_peaks(torch)
        print(f"[bench] measured peaks: {peaks}", flush=True)
        r = d["roofline"]
        r["measured_peak"] = peaks["hbm_read_GBps"]
        r["frac_of_measured"] = round(r["achieved"] / peaks["hbm_read_GBps"], 4)
        for p_ in (pre, pre8):
            if p_ and "roofline" in p_:
                p_["roofline"]["measured_peak"] = peaks["bf16_mfma_TFLOPs"]
                p_["roofline"]["frac_of_measured"] = round(p_["roofline"]["achieved"] / peaks["bf16_mfma_TFLOPs"], 4)
    cpu = None
    full_parity = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle, one thread)...", flush=True)
        cpu, ref_all = cpu_baseline(case, torch, torch.device("cuda", 0))
        print(f"[bench] cpu baseline: {cpu['seconds']} s", flush=True)
        # the timed decode output of the whole batch against the oracle's
        full_parity = full_output_parity(tl, d["out"], ref_all)
        print(f"[bench] whole decode output vs oracle: {full_parity}", flush=True)
    d.pop("out")
    value = d["step_bytes"] / (d["ms_per_step"] / 1e3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; K/V/Q ~ N(0,1) by Irwin-Hall, clipped log-normal context lengths, "
                "shuffled physical blocks)",
        "config": {"workload": "Llama-3-8B-shaped decode step: kv_cache_write of 256 new tokens + split-K "
                               "paged decode (512-token partitions) + merge",
                   "batch": case.num_seqs, "q_heads": case.num_q_heads, "kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "block_size": case.block_size, "kv_dtype": case.kv_dtype,
                   "context_tokens": int(case.seq_lens.sum()), "context_len_min": int(case.seq_lens.min()),
                   "context_len_max": int(case.seq_lens.max()), "num_blocks": case.num_blocks,
                   "partition_size": case.partition_size},
        "roofline": d["roofline"],
        "roofline_call": d["roofline_call"],
        "cpu_baseline": cpu,
        "full_output_parity": full_parity,
        "run": run_metadata(torch),
        "breakdown_us": d["breakdown_us"],
        "decode_partition_size_sweep": d["partition_size_sweep"],
        "kv_cache_write": d["kv_cache_write"],
        "algorithmic_bytes": d["bytes"],
        "max_abs_err_sampled": d["max_abs_err"],
        "prefill": pre,
        "prefill_int8": pre8,
        "decode_int8_llama_shaped": i8big,
        "mixed_step": mixed,
        "decode_shapes": shapes,
        "block_ops": blocks,
        "kv_cache_write_at_scale": kvw,
        "measured_peaks": peaks,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
