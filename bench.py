"""Benchmark: paged decode attention on one MI355X.

A step is one pass of the whole hot path over one batch: ``pa_decode`` (block
table gather, logits, online softmax, P.V, GQA sharing, split-context
partials) and, when the context is split, ``pa_reduce`` (log-sum-exp merge and
store).  Inputs are resident in HBM before the timed region starts.

Default workload: 70B-style GQA decode -- 64 sequences, 64 query heads over 8
KV heads, head_dim 128, bf16 KV, every context 4096 tokens, 16-token blocks,
shuffled block tables.  Prints one JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--config 2]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


DECODE_SOURCES = ("pa_decode.hip", "pa_common.h", "pa_internal.h", "pa_units.h")


def kernel_source_hash() -> str:
    """Hash of the code the decode kernel is compiled from (comments and blank
    lines left out), to tell whether stored counters still apply."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_365_amd", "csrc")
    for name in DECODE_SOURCES:
        text = open(os.path.join(csrc, name), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())
        h.update(name.encode())
        h.update(code.encode())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, partition: int):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "pa_decode_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash():
        return None
    if entry.get("partition_size") != partition:
        return None
    return entry.get("hbm_bytes_per_launch")


def decode_kernel_bytes(w, partition: int, query_tokens: int = 1, key_bytes=None) -> int:
    """Algorithmic bytes one pa_decode (or pa_verify_decode) launch must move: K and
    V rows of every live token (2 * H_kv * d * element bytes per token), q, live
    block-table entries and context lengths, plus the output rows when it writes
    them itself (unsplit).  Split-context partials are not algorithmic and are not
    counted."""
    from paged_kv_cache_365_amd.workloads import ELEM_BYTES
    e = ELEM_BYTES[w.dtype]
    bs = w.block_size
    live = int(((w.context_lens.astype("int64") + bs - 1) // bs).sum())  # table entries read
    qo = query_tokens * w.num_seqs * w.num_q_heads * w.head_dim * e
    scales = {1: 4, 0.25: 8}.get(key_bytes, 0) * w.num_kv_heads * w.head_dim
    return (w.kv_bytes_logical(key_bytes) + qo * (1 if partition else 2) + 4 * live +
            4 * w.num_seqs + scales)


def _oracle_pass(w, min_seconds, max_seconds, threads, verify_q=None, k8=None, k2=None):
    """Whole passes of the fp64 oracle over every sequence of the workload, with
    ``threads`` BLAS threads, until about ``min_seconds`` have elapsed (bounded by
    ``max_seconds``; the last pass may stop early).  Returns (sequences, seconds)."""
    import oracle
    from oracle import quantized_kv
    from threadpoolctl import threadpool_limits
    B = w.num_seqs
    with threadpool_limits(threads):
        t0 = time.perf_counter()
        done_seqs = 0
        while time.perf_counter() - t0 < min_seconds:
            for s in range(B):
                if k2 is not None:
                    qs = w.q[s:s + 1, None] if verify_q is None else verify_q[s:s + 1]
                    quantized_kv.paged_decode_k2(qs, k2[0], w.v_pool, w.block_tables[s:s + 1],
                                                 w.context_lens[s:s + 1], w.scale, k2[1], k2[2],
                                                 w.dtype)
                elif k8 is not None:
                    qs = w.q[s:s + 1, None] if verify_q is None else verify_q[s:s + 1]
                    quantized_kv.paged_decode_k8(qs, k8[0], w.v_pool, w.block_tables[s:s + 1],
                                                 w.context_lens[s:s + 1], w.scale, k8[1], w.dtype)
                elif verify_q is None:
                    oracle.paged_decode(w.q[s:s + 1], w.k_pool, w.v_pool, w.block_tables[s:s + 1],
                                        w.context_lens[s:s + 1], w.scale, w.dtype)
                else:
                    oracle.paged_verify(verify_q[s:s + 1], w.k_pool, w.v_pool,
                                        w.block_tables[s:s + 1], w.context_lens[s:s + 1],
                                        w.scale, w.dtype)
                done_seqs += 1
                if time.perf_counter() - t0 > max_seconds:
                    break
        return done_seqs, time.perf_counter() - t0


def cpu_baseline(w, min_seconds: float = 8.0, max_seconds: float = 25.0, verify_q=None,
                 k8=None, k2=None):
    """The fp64 oracle on the same workload, timed twice: with BLAS threads set to
    every host core this process may use (the reported value), and with one
    thread.  ``verify_q`` [B][T][H_q][d]: time the verify oracle over that draft
    instead; ``k8`` = (codes, scales): the int8-key oracle; ``k2`` = (words,
    steps, zero points): the 2-bit-key oracle."""
    B = w.num_seqs
    T = 1 if verify_q is None else verify_q.shape[1]
    key_bytes = 1 if k8 is not None else (0.25 if k2 is not None else None)
    nbytes = w.algorithmic_bytes(query_tokens=T, key_bytes=key_bytes)
    cores = len(os.sched_getaffinity(0))
    legs = {}
    for name, threads in (("all_cores", cores), ("one_thread", 1)):
        done, dt = _oracle_pass(w, min_seconds, max_seconds, threads, verify_q, k8, k2)
        legs[name] = {
            "value": round(nbytes * done / B / dt / 1e9, 4), "cores": threads,
            "tokens_per_s": round(done * T / dt, 3),
            "sample": f"{done} sequences ({done / B:.2f} passes over all {B} sequences x "
                      f"{w.num_q_heads} heads of the workload), numpy float64, BLAS threads "
                      f"{threads}, {dt:.1f} s"}
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    host = {"cpu_count": os.cpu_count(), "affinity": cores, "cpu_model": model}
    rec = dict(legs["all_cores"])
    rec.update({"unit": "GB/s", "kind": "oracle", "host": host, "one_thread": legs["one_thread"]})
    return rec


def copy_bandwidth(torch, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """Read+write GB/s of a plain device copy (context for the roofline)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del src, dst
    return 2 * nbytes / dt / 1e9


def time_launches(torch, stream, fn, reps: int = 20) -> float:
    """Mean seconds of one fn() launch over ``reps`` back-to-back launches
    (HIP events on the launch stream)."""
    fn()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e-3


def achievable(torch, pa, w, d, stream, nbytes: int = 1 << 30) -> dict:
    """Read rates measured in the same run: a plain streaming read of ``nbytes``
    (pa_probe_read) and, for 16-bit pools of 16-token blocks, the K/V tile reads
    of the decode call with nothing computed (pa_probe_read_tiles)."""
    out = {}
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(2048 * 4, dtype=torch.int32, device="cuda")
    t = time_launches(torch, stream, lambda: pa.pa_probe_read(src, sink, stream))
    out["stream_read_gbps"] = round(nbytes / t / 1e9, 1)
    out["stream_read_bytes"] = nbytes
    del src
    if w.dtype in ("f16", "bf16") and w.block_size == 16:
        sink = torch.empty(w.num_seqs * w.num_kv_heads * 8, dtype=torch.int32, device="cuda")
        t = time_launches(torch, stream, lambda: pa.pa_probe_read_tiles(
            d.k_pool, d.v_pool, d.block_tables, d.context_lens, d.max_context_len, sink, stream))
        out["decode_tile_reads_gbps"] = round(w.kv_bytes_logical() / t / 1e9, 1)
        out["decode_tile_reads_us"] = round(t * 1e6, 2)
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="workload index 0..4 (default: 70B GQA 4K)")
    ap.add_argument("--partition", type=int, default=None, help="override the partition size")
    ap.add_argument("--tuned", action="store_true",
                    help="use the tuned partition size even where the workload names its own")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--block-size", type=int, default=16, choices=(16, 8),
                    help="tokens per physical block (8: the smaller blocks the pages mention "
                         "for 70B models)")
    ap.add_argument("--longest-first", action="store_true",
                    help="order the batch by context length, longest first, as a scheduler "
                         "would with pa_bm_sort_longest_first (the workload is otherwise as drawn)")
    ap.add_argument("--kv", choices=("native", "k8", "k2"), default="native",
                    help="k8: int8 keys with per-channel scales (pa_decode_k8); k2: 2-bit keys "
                         "with per-channel steps and zero points (pa_decode_k2); values in the "
                         "workload's 16-bit type")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="time pa_decode_shared_prefix (+ pa_reduce): the prefix every table "
                         "starts with computed once per KV head for the whole batch "
                         "(shared-prefix workload; the partition size must divide the prefix)")
    ap.add_argument("--verify", type=int, default=0, metavar="T",
                    help="time the speculative-decoding verify call over a T-token draft "
                         "(pa_verify_decode) instead of single-token decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-achievable", action="store_true",
                    help="skip the read probes (streaming read, the decode's tile reads)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB device copy first (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              f"(the decode path is single-GPU; split by sequence or KV head it needs no exchange)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from paged_kv_cache_365_amd import pa, tuning
    from paged_kv_cache_365_amd import workloads as wl
    from paged_kv_cache_365_amd.device import upload

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pa.load()

    log(f"generating workload {args.config}")
    w = wl.make_config(args.config, args.seed, block_size=args.block_size)
    if args.longest_first:
        import dataclasses
        order = np.argsort(-w.context_lens.astype(np.int64), kind="stable")
        w = dataclasses.replace(w, q=w.q[order], block_tables=w.block_tables[order],
                                context_lens=w.context_lens[order])
    P = tuning.partition_for(w, own=not args.tuned) if args.partition is None else args.partition
    prefix_tokens = w.prefix_blocks * w.block_size
    if args.shared_prefix and (not prefix_tokens or P <= 0 or prefix_tokens % P or args.verify or
                               args.kv != "native"):
        print("--shared-prefix needs a workload with a shared prefix, a partition size that "
              "divides it, one query token and the native KV type", file=sys.stderr)
        return 2
    d = upload(w, "cuda")
    T = max(args.verify, 1)
    B, Hq, D = d.q.shape
    k8 = args.kv == "k8"
    k2 = args.kv == "k2"
    key_bytes = 1 if k8 else (0.25 if k2 else None)
    if (k8 or k2) and w.dtype not in ("f16", "bf16"):
        print(f"--kv {args.kv} needs a 16-bit workload", file=sys.stderr)
        return 2
    if k2:
        words, k2_step, k2_zero = wl.k2_inputs(w, 4343 + args.config,
                                               outlier_columns=10 if args.config == 2 else 0)
        k2_pool = torch.from_numpy(words.view(np.int32)).to("cuda")
        k2_step_t = torch.from_numpy(k2_step).to("cuda")
        k2_zero_t = torch.from_numpy(k2_zero).to("cuda")
    if k8:
        codes, kscale = wl.k8_inputs(w, 4242 + args.config,
                                     outlier_columns=10 if args.config == 2 else 0)
        k8_pool = torch.from_numpy(codes).to("cuda")
        k8_scale = torch.from_numpy(kscale).to("cuda")
    if args.verify or k8 or k2:
        from paged_kv_cache_365_amd.device import to_torch
        q_np = wl.normal(np.random.default_rng(7), (B, T, Hq, D), w.dtype)
        qv = to_torch(q_np, w.dtype, "cuda")
        out = torch.empty_like(qv)
        ws = None
        if P:
            n = pa.pa_decode_workspace_bytes(B, T * Hq, D, d.max_context_len, P)
            ws = torch.empty(n // 4, dtype=torch.float32, device="cuda")
    else:
        out = torch.empty_like(d.q)
        ws = pa.workspace_for(d.q, d.k_pool, d.max_context_len, P)
    stream = torch.cuda.current_stream()
    log(f"{w.name}: B={B} Hq={Hq} Hkv={w.num_kv_heads} d={D} dtype={w.dtype} "
        f"maxlen={w.max_context_len} partition={P}")

    copy_gbps = None
    if args.copy_calibration:
        copy_gbps = copy_bandwidth(torch)
        log(f"device copy: {copy_gbps:.0f} GB/s (read+write)")

    def step(ev=None):
        """One pass of the hot path; ``ev`` = events (before decode, after decode,
        after reduce)."""
        if ev is not None:
            ev[0].record(stream)
        if k2:
            pa.pa_decode_k2(qv, k2_pool, d.v_pool, k2_step_t, k2_zero_t, d.block_tables,
                            d.context_lens, d.max_context_len, d.scale, P, ws, None if P else out,
                            stream)
        elif k8:
            pa.pa_decode_k8(qv, k8_pool, d.v_pool, k8_scale, d.block_tables, d.context_lens,
                            d.max_context_len, d.scale, P, ws, None if P else out, stream)
        elif args.shared_prefix:
            pa.pa_decode_shared_prefix(d.q, d.k_pool, d.v_pool, d.block_tables, d.context_lens,
                                       d.max_context_len, d.scale, prefix_tokens, P, ws, stream)
        elif args.verify:
            pa.pa_verify_decode(qv, d.k_pool, d.v_pool, d.block_tables, d.context_lens,
                                d.max_context_len, d.scale, P, ws, None if P else out, stream)
        else:
            pa.pa_decode(d.q, d.k_pool, d.v_pool, d.block_tables, d.context_lens,
                         d.max_context_len, d.scale, P, ws, None if P else out, stream)
        if ev is not None:
            ev[1].record(stream)
        if P:
            pa.pa_reduce(ws, d.context_lens, B, T * Hq, D, d.max_context_len, P, out, stream)
            if ev is not None:
                ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    # Timed region: K back-to-back steps between two HIP events on the launch
    # stream (an event pair around every launch would itself add several
    # microseconds between kernels).
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    device_ms_per_step = t_start.elapsed_time(t_end) / args.steps
    log(f"timed {args.steps} steps in {wall * 1e3:.2f} ms "
        f"(device {device_ms_per_step * 1e3:.2f} us/step)")

    # Second pass of K steps with an event pair around every launch: the
    # distribution of single-launch durations (p10 / median / p90), and for a
    # split step, which is two kernels, the decode launch's own mean.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
              for _ in range(args.steps)]
    for k in range(args.steps):
        step(events[k])
    torch.cuda.synchronize()
    launch_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    launch_pct = {f"p{q}": round(float(np.percentile(launch_ms, q)) * 1e3, 2) for q in (10, 50, 90)}
    if P:
        decode_ms = float(np.mean(launch_ms))
        reduce_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
        duration_source = "HIP events around each pa_decode launch (second pass of K steps)"
    else:
        # a step is exactly one launch of the decode kernel
        decode_ms = device_ms_per_step
        reduce_ms = 0.0
        duration_source = "HIP events bracketing the K timed launches"

    ms_per_step = wall * 1e3 / args.steps
    alg = w.algorithmic_bytes(query_tokens=T, key_bytes=key_bytes)
    value = alg / (ms_per_step * 1e-3) / 1e9
    kbytes = decode_kernel_bytes(w, P, T, key_bytes)
    achieved = kbytes / (decode_ms * 1e-3) / 1e9
    workload = (w.name + ("-k8" if k8 else "") + ("-k2" if k2 else "") +
                (f"-verify{T}" if args.verify else "") + ("-sp" if args.shared_prefix else ""))
    traffic = stored_traffic(workload, P)

    rec = {
        "metric": "paged decode-attention KV GB/s and % of HBM peak; tokens/s at 70B-GQA 4K",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"i8k-{w.dtype}" if k8 else (f"u2k-{w.dtype}" if k2 else w.dtype),
        "accum_dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": workload, "num_seqs": B, "query_tokens": T, "num_q_heads": Hq, "num_kv_heads": w.num_kv_heads,
            "head_dim": D, "max_context_len": w.max_context_len, "block_size": w.block_size,
            "partition_size": P, "pool_blocks": w.num_blocks,
            "batch_order": "longest-first" if args.longest_first else "as drawn", "seed": args.seed if args.seed is not None else 1000 + args.config,
        },
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(B * T / (ms_per_step * 1e-3), 1),
        "algorithmic_bytes_per_step": alg,
        "device_us_per_step": round(device_ms_per_step * 1e3, 2),
        "decode_us": round(decode_ms * 1e3, 2),
        "reduce_us": round(reduce_ms * 1e3, 2),
        "decode_launch_us": launch_pct,
        "roofline": {
            "kernel": ("pa_decode_k8" if k8 else "pa_decode_k2" if k2 else
                       "pa_verify_decode" if args.verify else
                       "pa_decode_shared_prefix" if args.shared_prefix else "pa_decode"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kbytes,
            "duration_source": duration_source,
        },
    }
    if workload.startswith("70b"):
        # one call is one attention layer; LLaMA-2 70B has 80 of them (the KV
        # Cache section of "LLM推理优化实战：从KV Cache到Speculative Decoding，
        # 把延迟打下来" sizes its cache with that count), so this is the
        # attention-only decode rate of the whole model
        rec["attention_tokens_per_s_80_layers"] = round(B * T / (80 * ms_per_step * 1e-3), 1)
    if w.prefix_blocks:
        # shared blocks counted once: the bytes a step must take from memory
        rec["unique_bytes_per_step"] = w.algorithmic_bytes(unique=True, query_tokens=T)
        rec["unique_gbps"] = round(rec["unique_bytes_per_step"] / (ms_per_step * 1e-3) / 1e9, 2)
    if copy_gbps is not None:
        rec["device_copy_gbps"] = round(copy_gbps, 1)
    if not args.no_achievable:
        ach = achievable(torch, pa, w, d, stream)
        if "decode_tile_reads_gbps" in ach and not (k8 or k2):
            # the decode kernel's own KV rate against the same reads with no compute
            kv_rate = w.kv_bytes_logical() / (decode_ms * 1e-3) / 1e9
            ach["decode_over_tile_reads"] = round(kv_rate / ach["decode_tile_reads_gbps"], 4)
        rec["roofline"]["achievable"] = ach
        log(f"achievable: {ach}")
    del d, out, ws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host (cpu_baseline)")
        rec["cpu_baseline"] = cpu_baseline(w, verify_q=q_np if args.verify else None,
                                           k8=(codes, kscale) if k8 else None,
                                           k2=(words, k2_step, k2_zero) if k2 else None)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
