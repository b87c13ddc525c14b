#!/usr/bin/env python3
"""Benchmark of one decode step of paged attention on one MI355X.

A step is the whole hot path for one layer over one batch: copy-on-write block copies (when the
workload has any), the slot-mapped write of every sequence's new token and decode attention
through the block tables. By default the write rides along with the attention in one launch
(pa_decode_append, or pa_decode_grouped_append with --grouped), then the merge when a sequence
spans several partitions; ``--separate`` times pa_write_kv, then the decode, instead. The
default workload is the OPT-13B-shaped MHA decode batch: 64 sequences, 40 heads x 128 dims, fp16
cache, block size 16, context lengths uniform in [128, 2048], blocks scattered through a pool
with 20% free blocks.

Inputs are uploaded before timing (``--replicas`` independent copies of the pools, rotated step by
step, so no step finds the previous step's data in the L2 or the MALL). The timed region is
bracketed by device synchronisation; the library records HIP events around its own launches on
the same stream, which gives the average duration of the attention kernel for the roofline.

Prints one JSON line. ``value`` is algorithmic bytes of the step / step time (GB/s).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: achieved HBM GB/s (% of peak), attended tokens/s"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # 200 untimed steps (about 50 ms of work): with 10, the first timed steps of the fp8 batch
    # still ran 9% slower than the steady state that the per-step percentiles show
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--config", type=int, default=2, help="workload 1..5 (2 = the headline batch)")
    p.add_argument("--dtype", default=None,
                   help="override the cache dtype of config 2, or of --measure prefill (f16|bf16)")
    p.add_argument("--first-step", action="store_true", help="config 4: every sample at its first step")
    p.add_argument("--replicas", type=int, default=4)
    p.add_argument("--partition", type=int, default=0, help="partition tokens (0 = library default)")
    p.add_argument("--variant", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-also", action="store_true",
                   help="skip the other decode workloads the headline run also measures")
    p.add_argument("--also-warmup", type=int, default=50,
                   help="untimed steps before each of the other workloads (at least --warmup): "
                        "those lines report the kernels at the steady state of a decode loop")
    p.add_argument("--no-ceiling", action="store_true", help="skip the read-ceiling measurement")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="time budget of each leg of the oracle timing (all cores, one thread)")
    p.add_argument("--calibrate-copy-mib", type=int, default=0,
                   help="also launch one plain device copy of this many MiB (counter calibration)")
    p.add_argument("--separate", action="store_true",
                   help="step through pa_write_kv, then the decode, instead of pa_decode_append / "
                        "pa_decode_grouped_append (the write riding along with the attention, the "
                        "default)")
    p.add_argument("--num-seqs", type=int, default=0,
                   help="configs 2, 3, 5: use only this many sequences (a smaller batch)")
    p.add_argument("--grouped", action="store_true",
                   help="decode through pa_decode_grouped: sequences sharing prefix blocks (found "
                        "in the tables) read each shared block once per group")
    p.add_argument("--block-size", type=int, default=0,
                   help="--measure prefill: block size of the cache (0 = 16)")
    p.add_argument("--measure", default="step", choices=("step", "swap", "paging", "prefill"),
                   help="step: the decode-step line (default); swap: block swap to and from pinned "
                        "host memory; paging: paged vs contiguous placement and block sizes; "
                        "prefill: chunked prefill over the cache")
    return p.parse_args()


def timing_batch(lens, num_heads, num_kv_heads, head_dim, block_size, dtype, placement, seed,
                 free_fraction=0.2):
    """Device inputs for timing only (no oracle check): tables from the block manager -- blocks
    handed out in a seeded random order, or in address order for ``placement="contiguous"`` --
    and K/V/q drawn on the GPU (seeded N(0,1)), which takes milliseconds instead of the host
    generator's seconds."""
    import numpy as np
    import torch

    from paged_kv_cache_318_amd.blocks import BlockPool

    B = block_size
    used = sum(-(-int(L) // B) for L in lens)
    NB = max(1, int(np.ceil((1.0 + free_fraction) * used)))
    rng = np.random.default_rng(seed)
    order = np.arange(NB) if placement == "contiguous" else rng.permutation(NB)
    pool = BlockPool(NB, B, free_order=order.tolist())
    for s, L in enumerate(lens):
        pool.add_sequence(s, int(L))
    tables = pool.block_table(list(range(len(lens))))
    g = torch.Generator(device="cuda").manual_seed(seed)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[dtype]
    dev = "cuda"
    return {
        "q": torch.randn(len(lens), num_heads, head_dim, generator=g, device=dev).to(tdt),
        "k": torch.randn(NB, num_kv_heads, B, head_dim, generator=g, device=dev).to(tdt),
        "v": torch.randn(NB, num_kv_heads, head_dim, B, generator=g, device=dev).to(tdt),
        "tables": torch.from_numpy(tables).to(dev),
        "lens": torch.tensor(np.asarray(lens, dtype=np.int32), device=dev),
        "num_blocks": NB, "used_blocks": used, "table_np": tables,
    }


def measure_swap(args, lib, torch):
    """Preemption by swapping: the blocks of the first half of the batch go out to a pinned host
    pool and come back (PA_SWAP_OUT, then PA_SWAP_IN), against the runtime's own copies of the
    same number of contiguous bytes in each direction (the host link's ceiling)."""
    import numpy as np

    from workloads.synth import config_lens
    spec = config_lens(args.config if args.config in (2, 3) else 2)
    b = timing_batch(spec["lens"], spec["num_heads"], spec["num_kv_heads"], spec["head_dim"], 16,
                     spec["dtype"], "scattered", seed=args.config)
    half = len(spec["lens"]) // 2
    blocks = np.concatenate([b["table_np"][s, : -(-int(L) // 16)]
                             for s, L in enumerate(spec["lens"][:half])]).astype(np.int32)
    n = blocks.size
    hk = torch.empty((n,) + tuple(b["k"].shape[1:]), dtype=b["k"].dtype, pin_memory=True)
    hv = torch.empty((n,) + tuple(b["v"].shape[1:]), dtype=b["v"].dtype, pin_memory=True)
    idx = np.arange(n, dtype=np.int32)
    out_pairs = torch.from_numpy(np.stack([blocks, idx], 1)).cuda()
    in_pairs = torch.from_numpy(np.stack([idx, blocks], 1)).cuda()
    nbytes = 2 * n * b["k"][0].numel() * b["k"].element_size()

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best

    t_out = timed(lambda: lib.pa_swap_blocks(b["k"], b["v"], hk, hv, out_pairs, lib.PA_SWAP_OUT))
    t_in = timed(lambda: lib.pa_swap_blocks(b["k"], b["v"], hk, hv, in_pairs, lib.PA_SWAP_IN))
    dev_buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    host_buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    t_d2h = timed(lambda: host_buf.copy_(dev_buf, non_blocking=True))
    t_h2d = timed(lambda: dev_buf.copy_(host_buf, non_blocking=True))
    gbs = lambda ms: round(nbytes / (ms * 1e-3) / 1e9, 2)
    line = {
        "metric": "block swap between HBM and pinned host memory: GB/s per direction",
        "value": gbs(max(t_out, t_in)), "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
        "dtype": spec["dtype"], "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": f"swap-{spec['name']}", "blocks": int(n), "bytes_per_direction": nbytes,
                   "block_bytes_kv": 2 * b["k"][0].numel() * b["k"].element_size()},
        "swap_out_gbs": gbs(t_out), "swap_in_gbs": gbs(t_in),
        "runtime_copy_d2h_gbs": gbs(t_d2h), "runtime_copy_h2d_gbs": gbs(t_h2d),
        "ms": {"swap_out": round(t_out, 3), "swap_in": round(t_in, 3), "copy_d2h": round(t_d2h, 3),
               "copy_h2d": round(t_h2d, 3)},
    }
    print(json.dumps(line), flush=True)


BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / fp16 matrix peak, published


def measure_prefill(args, lib, torch):
    """Chunked prefill: 16 sequences append 512-token chunks to contexts of 0..3584 tokens (32
    query / 8 kv heads x 128, bf16 unless --dtype f16, block size 16). A step writes the chunks'
    K/V (pa_write_kv) and runs causal attention of every new token over its sequence
    (pa_prefill)."""
    import numpy as np

    from workloads import make_prefill
    from workloads.device import upload
    rng = np.random.default_rng(15)
    ctx = rng.integers(0, 3584, endpoint=True, size=16)
    dt = args.dtype or "bf16"
    if dt not in ("bf16", "f16"):
        raise SystemExit("--measure prefill takes --dtype bf16 or f16")
    w = make_prefill(ctx, [512] * 16, num_heads=32, num_kv_heads=8, head_dim=128, dtype=dt,
                     block_size=args.block_size or 16, seed=15)
    reps = [upload(w) for _ in range(max(1, args.replicas))]
    qs = torch.from_numpy(np.ascontiguousarray(w.query_start, dtype=np.int32)).cuda()
    T = w.q.shape[0]
    out = torch.empty(T, w.num_heads, w.head_dim,
                      dtype=torch.bfloat16 if dt == "bf16" else torch.float16, device="cuda")

    def step(i):
        d = reps[i % len(reps)]
        lib.pa_write_kv(d.k_new, d.v_new, d.k_cache, d.v_cache, d.slots)
        lib.pa_prefill(out, d.q, d.k_cache, d.v_cache, d.tables, d.lens, qs, w.scale, 512)

    calibration_copy(args, torch)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    lib.pa_profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    p_ms, p_n = lib.pa_profile_read(lib.PA_KERNEL_PREFILL)
    w_ms, w_n = lib.pa_profile_read(lib.PA_KERNEL_WRITE_KV)
    lib.pa_profile_enable(False)
    k_ms = p_ms / max(p_n, 1)
    flops = w.prefill_flops()
    tflops = flops / (k_ms * 1e-3) / 1e12
    line = {
        "metric": "chunked prefill attention: TFLOP/s (causal pairs x 4 x head_dim x heads), new tokens/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "dtype": dt, "data": "synthetic (seeded N(0,1) K/V/q, scattered blocks; no dataset)",
        "new_tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "config": {"workload": f"prefill-16x512-gqa-{dt}", "num_seqs": 16, "chunk": 512,
                   "context": "U[0,3584]", "num_heads": 32, "num_kv_heads": 8, "head_dim": 128,
                   "block_size": w.block_size, "new_tokens": T, "causal_pairs": w.attended_pairs(),
                   "flops": flops, "bytes": w.prefill_bytes()},
        "kernels_us": {"prefill": round(1e3 * k_ms, 2),
                       "write_kv": round(1e3 * w_ms / max(w_n, 1), 2)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("prefill_mfma", f"prefill-16x512-gqa-{dt}",
                                                 "prefill_hbm_traffic.txt"),
                     "kernel": "prefill_mfma",
                     "bytes_gbs": round(w.prefill_bytes() / (k_ms * 1e-3) / 1e9, 1)},
    }
    print(json.dumps(line), flush=True)


def measure_paging(args, lib, torch):
    """The pages say the paged kernel pays for its indirection and that the block size trades
    table overhead against the unused tail. Same kernel, same lengths: blocks scattered through the
    pool vs handed out in address order (every sequence contiguous), for block sizes 8, 16 and 32,
    on the MHA batch (VALU kernel) and the GQA batch (MFMA kernel)."""
    from paged_kv_cache_318_amd.step import workspace_for
    from workloads.synth import config_lens
    rows = []
    for cfg in (2, 3):
        spec = config_lens(cfg)
        for B in (8, 16, 32):
            for placement in ("scattered", "contiguous"):
                b = timing_batch(spec["lens"], spec["num_heads"], spec["num_kv_heads"],
                                 spec["head_dim"], B, spec["dtype"], placement, seed=cfg)
                out = torch.empty_like(b["q"])
                ws = workspace_for(b["q"], b["k"], b["tables"], B)
                scale = spec["head_dim"] ** -0.5

                def call():
                    lib.pa_decode(out, b["q"], b["k"], b["v"], b["tables"], b["lens"], scale,
                                  workspace=ws)

                for _ in range(5):
                    call()
                torch.cuda.synchronize()
                lib.pa_profile_enable(True)
                for _ in range(args.steps):
                    call()
                torch.cuda.synchronize()
                k_ms, k_n = lib.pa_profile_read(lib.PA_KERNEL_DECODE_PARTITION)
                m_ms, m_n = lib.pa_profile_read(lib.PA_KERNEL_DECODE_MERGE)
                lib.pa_profile_enable(False)
                tokens = int(sum(spec["lens"]))
                kv = tokens * 2 * spec["num_kv_heads"] * spec["head_dim"] * b["k"].element_size()
                us = 1e3 * k_ms / max(k_n, 1)
                G = spec["num_heads"] // spec["num_kv_heads"]
                rows.append({
                    "workload": spec["name"], "block_size": B, "placement": placement,
                    "kernel": "decode_mfma" if G >= 2 else "decode_valu",
                    "attention_us": round(us, 2),
                    "merge_us": round(1e3 * m_ms / m_n, 2) if m_n else None,
                    "kv_gbs": round(kv / (us * 1e-6) / 1e9, 1),
                    "table_entries": int(sum(-(-int(L) // B) for L in spec["lens"])),
                    "unused_tail_slots": int(sum(-(-int(L) // B) * B - int(L) for L in spec["lens"])),
                })
                print(f"[bench] paging {rows[-1]}", file=sys.stderr, flush=True)
                del b, out, ws
    for r in rows:
        twin = [x for x in rows if x["workload"] == r["workload"] and x["block_size"] == r["block_size"]
                and x["placement"] == "contiguous"][0]
        r["vs_contiguous"] = round(r["attention_us"] / twin["attention_us"], 4)
    line = {"metric": "paged vs contiguous placement and block size: attention kernel time",
            "unit": "us", "n_gpus": 1, "higher_is_better": False, "steps": args.steps,
            "data": "synthetic (seeded, generated on the GPU)", "rows": rows}
    print(json.dumps(line), flush=True)


_CPU_STATE = {}  # the workload and its post-write pools, inherited by the forked workers


def host_cores() -> int:
    """Host cores the CPU baseline may use: the affinity set, capped by the cgroup's CPU quota when
    one is set and at 16 (the host share of one GPU on a shared node)."""
    n = len(os.sched_getaffinity(0))
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            n = min(n, max(1, int(float(quota) / float(period))))
    except (OSError, ValueError):
        pass
    return max(1, min(n, 16))


def _oracle_pass(seqs, budget_s: float):
    """Decode the given sequences with the oracle, again and again, until the budget is spent
    (at least one whole pass); BLAS limited to one thread. Returns (attended tokens, seconds)."""
    from threadpoolctl import threadpool_limits

    import oracle
    w, kp, vp, ks, vs = (_CPU_STATE[k] for k in ("w", "kp", "vp", "ks", "vs"))
    tokens = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            for s in seqs:
                oracle.decode(w.q, kp, vp, w.tables, w.lens, w.block_size, w.scale, w.dtype,
                              w.q_dtype, ks, vs, seqs=[s])
                tokens += int(w.lens[s])
                if time.perf_counter() - t0 >= budget_s:
                    return tokens, time.perf_counter() - t0
            if not seqs:
                return tokens, time.perf_counter() - t0


def cpu_baselines(w, budget_s: float):
    """The fp64 oracle as it stands, timed on the host over a bounded sample of the same workload:
    after the step's copies and writes (done once, timed in the 1-thread leg), whole sequences are
    decoded in turn until the time budget is spent. Two legs: one worker process per host core
    (forked before the GPU is touched; sequences dealt out longest first, each worker cycling
    through its own), and one thread. Returns (all-core result, 1-thread result)."""
    import multiprocessing as mp

    import oracle

    t0 = time.perf_counter()
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    ks = None if w.k_scale is None else w.k_scale.copy()
    vs = None if w.v_scale is None else w.v_scale.copy()
    oracle.copy_blocks(kp, vp, w.cow, ks, vs)
    oracle.write_kv(kp, vp, w.k_new, w.v_new, w.slots, w.block_size, w.dtype, ks, vs, w.new_dtype)
    t_write = time.perf_counter() - t0
    _CPU_STATE.update(w=w, kp=kp, vp=vp, ks=ks, vs=vs)
    per_tok = w.kv_bytes() / max(w.attended_tokens, 1)

    def result(tokens, dt, cores, sample):
        return {"value": round(tokens * per_tok / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
                "kind": "oracle", "attended_tokens_per_s": round(tokens / dt, 1), "sample": sample}

    n = host_cores()
    order = sorted(range(w.num_seqs), key=lambda s: -int(w.lens[s]))
    shares = [order[i::n] for i in range(n)]
    t1 = time.perf_counter()
    with mp.get_context("fork").Pool(n) as pool:
        res = pool.starmap(_oracle_pass, [(sh, budget_s) for sh in shares])
    wall = time.perf_counter() - t1
    tok_all = sum(r[0] for r in res)
    allcore = result(tok_all, wall, n,
                     f"{n} worker processes (one per host core, BLAS 1 thread each) decoding the "
                     f"{w.num_seqs} sequences ({w.num_heads} heads) round and round for "
                     f"{budget_s:.0f} s each: {tok_all} attended tokens in {wall:.1f} s wall, "
                     f"fp64 numpy, after the step's write")
    tok1, dt1 = _oracle_pass(list(range(w.num_seqs)), budget_s)
    one = result(tok1, dt1 + t_write, 1,
                 f"write of all {w.num_seqs} new tokens + decode of the {w.num_seqs} sequences in "
                 f"turn for {budget_s:.0f} s ({tok1} attended tokens x {w.num_heads} heads), "
                 f"fp64 numpy, 1 thread, {dt1 + t_write:.1f} s")
    _CPU_STATE.clear()
    return allcore, one


def read_ceiling(lib, tile_bytes: int, total_bytes: int = 4 << 30, reps: int = 5):
    """Read rate this GPU sustains for tiles of the attention kernel's size: whole 4 GiB buffer,
    tiles in address order and in a random order (the paged pattern), best of ``reps``."""
    import torch
    n = total_bytes // tile_bytes
    buf = torch.empty(n * tile_bytes, dtype=torch.uint8, device="cuda")
    order = torch.randperm(n, device="cuda", dtype=torch.int32)
    sink = torch.empty(64 * 1024, dtype=torch.int32, device="cuda")
    res = {}
    for name, o in (("linear", None), ("scattered", order)):
        lib.pa_diag_read_bandwidth(buf, tile_bytes, n, o, sink)
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            lib.pa_diag_read_bandwidth(buf, tile_bytes, n, o, sink)
            b.record()
            torch.cuda.synchronize()
            best = min(best, a.elapsed_time(b))
        res[name] = round(n * tile_bytes / (best * 1e-3) / 1e9, 1)
    res["tile_bytes"] = tile_bytes
    return res


def calibration_copy(args, torch):
    """A plain device-to-device copy of --calibrate-copy-mib MiB: what the HBM counters read for it
    scales their values for the kernels to bytes."""
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {n} bytes done", file=sys.stderr, flush=True)
        del src, dst


def kernel_source_hash(kernel: str) -> str:
    """First 16 hex digits of sha256 over the sources the attention kernel is built from."""
    import hashlib
    csrc = os.path.join(ROOT, "paged_kv_cache_318_amd", "csrc")
    h = hashlib.sha256()
    if kernel == "prefill_mfma":
        files = ["pa_device.h", "mfma_common.h", "prefill_mfma.hip"]
    else:
        files = ["pa_device.h", "pa_sched.h", "kv_write.h"]
        files += ["decode_valu.hip"] if kernel == "decode_valu" else ["mfma_common.h", "decode_mfma.hip"]
    for f in files:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, summary: str = "decode_hbm_traffic.txt"):
    """HBM bytes per launch (fetch + write) from a committed counter summary under profiles/, or
    None when it has no entry for this kernel and workload or the kernel sources changed since it
    was taken."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    src = kernel_source_hash(kernel)
    for line in open(path, encoding="utf-8"):
        if line.startswith("#") or "=" not in line:
            continue
        kv = dict(tok.split("=", 1) for tok in line.split())
        if kv.get("kernel") == kernel and kv.get("workload") == workload and kv.get("source") == src:
            return int(float(kv["fetch_bytes"]) + float(kv["write_bytes"]))
    return None


def blocks_shared_across_groups(w, group_start) -> bool:
    """Whether some physical block is attended by sequences of two different groups."""
    owner = {}
    for gi in range(len(group_start) - 1):
        for s in range(int(group_start[gi]), int(group_start[gi + 1])):
            for b in w.tables[s, : -(-int(w.lens[s]) // w.block_size)].tolist():
                if owner.setdefault(b, gi) != gi:
                    return True
    return False


def shared_blocks_flag(w, lib):
    """PA_DECODE_SHARED_BLOCKS when the host's tables show sequences sharing physical blocks."""
    import numpy as np
    used = np.concatenate([w.tables[s, : -(-int(L) // w.block_size)] for s, L in enumerate(w.lens)])
    shared = bool(used.size) and np.unique(used).size < used.size
    return (lib.PA_DECODE_SHARED_BLOCKS if shared else 0), shared


def prepare_steps(w, args, lib, torch, grouped=False, variant=0, partition=0, fused=False):
    """Uploads ``args.replicas`` copies of the workload and its workspace; returns the step
    function and what the timing needs (``time_steps``)."""
    from paged_kv_cache_318_amd.step import decode_step, decode_step_grouped, workspace_for
    from workloads.device import torch_dtype, upload

    flags, shared = shared_blocks_flag(w, lib)
    reps = [upload(w) for _ in range(max(1, args.replicas))]
    out = torch.empty(w.num_seqs, w.num_heads, w.head_dim, dtype=torch_dtype(w.q_dtype), device="cuda")
    ws = workspace_for(reps[0].q, reps[0].k_cache, reps[0].tables, w.block_size, partition)

    gr = None
    if grouped:
        # sequences sharing prefix blocks (the host's tables say which) decode through
        # pa_decode_grouped, each shared block read once per group
        from paged_kv_cache_318_amd.blocks import shared_prefix_groups
        G = w.num_heads // w.num_kv_heads
        mg = max(1, 16 // G)
        gs, pref = shared_prefix_groups(w.tables, w.lens, w.block_size, mg)
        # the grouped kernel reads each group's shared blocks once: K/V are streamed unless a
        # block is also shared between different groups
        flags = lib.PA_DECODE_SHARED_BLOCKS if blocks_shared_across_groups(w, gs) else 0
        shared = bool(flags)
        gws = torch.empty(lib.pa_decode_grouped_workspace_bytes(
            w.num_seqs, w.num_heads, w.head_dim, w.tables.shape[1], w.block_size, partition),
            dtype=torch.uint8, device="cuda")
        gr = {"gs": torch.from_numpy(gs).cuda(), "pref": torch.from_numpy(pref).cuda(), "mg": mg,
              "ws": gws, "groups": len(gs) - 1, "max_prefix_blocks": int(pref.max(initial=0))}

    def step(i):
        d = reps[i % len(reps)]
        if gr is not None:
            decode_step_grouped(out, d.q, d.k_cache, d.v_cache, d.tables, d.lens, d.k_new, d.v_new,
                                d.slots, d.cow, gr["gs"], gr["pref"], gr["mg"], w.scale,
                                d.k_scale, d.v_scale, partition_tokens=partition,
                                workspace=gr["ws"], flags=flags, fused=fused)
            return
        decode_step(out, d.q, d.k_cache, d.v_cache, d.tables, d.lens, d.k_new, d.v_new, d.slots,
                    d.cow, w.scale, d.k_scale, d.v_scale, partition_tokens=partition,
                    variant=variant, workspace=ws, flags=flags, fused=fused)

    G = w.num_heads // w.num_kv_heads
    mfma_ok = w.dtype != "f32" and G <= 16
    kernel = "decode_mfma" if (grouped or variant == 2 or (variant == 0 and mfma_ok and G >= 2)) \
        else "decode_valu"
    return {"w": w, "step": step, "buffers": [reps, out, ws, gr], "kernel": kernel, "shared": shared,
            "fused": fused,
            "grouped": None if gr is None else
            {"groups": gr["groups"], "max_prefix_blocks": gr["max_prefix_blocks"]}}


def time_steps(prep, args, lib, torch):
    """Runs ``args.warmup`` untimed steps of a prepared workload, then three passes of
    ``args.steps`` steps each: the timed pass (device-synchronised on both sides), a pass with the
    library's HIP events around every launch (per-kernel averages), and a pass with an event
    between steps (percentiles). Frees the workload's device buffers and returns the
    measurements."""
    w, step = prep["w"], prep["step"]
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: warmup of {args.warmup} steps done", file=sys.stderr, flush=True)

    # timed region: K steps, nothing else on the stream
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(args.warmup + i)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    # the same K steps again with the library's HIP events around every launch (kernel durations)
    lib.pa_profile_enable(True)
    start.record()
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
    end.record()
    torch.cuda.synchronize()
    ms_step_profiled = start.elapsed_time(end) / args.steps
    kern = {}
    for name, kind in (("decode_partition", lib.PA_KERNEL_DECODE_PARTITION),
                       ("decode_merge", lib.PA_KERNEL_DECODE_MERGE),
                       ("write_kv", lib.PA_KERNEL_WRITE_KV), ("copy_blocks", lib.PA_KERNEL_COPY_BLOCKS)):
        ms, n = lib.pa_profile_read(kind)
        kern[name] = (ms / n) if n else None
    lib.pa_profile_enable(False)
    # a third pass with an event before every step and after the last: the spread of step times
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for i in range(args.steps):
        evs[i].record()
        step(args.warmup + 2 * args.steps + i)
    evs[-1].record()
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps))

    def pct(q):
        return round(per_step[min(len(per_step) - 1, int(q * (len(per_step) - 1) + 0.5))], 2)

    print(f"[bench] {w.name}: timed {args.steps} steps, {ms_step * 1e3:.1f} us/step", file=sys.stderr,
          flush=True)
    prep["buffers"].clear()
    prep["step"] = None
    return {"ms_step": ms_step, "ms_step_profiled": ms_step_profiled, "kernels_ms": kern,
            "pcts": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)}, "kernel": prep["kernel"],
            "shared": prep["shared"], "grouped": prep["grouped"]}


def us(ms):
    return None if ms is None else round(1e3 * ms, 2)


def decode_roofline(w, m, unique, fused):
    """Achieved algorithmic GB/s of the attention kernel (average launch) and its fraction of the
    8 TB/s HBM peak. A fused launch (pa_decode_append) also moves the new tokens: their bytes are
    counted with it."""
    dec = w.decode_bytes(unique=unique) + (w.write_bytes() if fused else 0)
    achieved = dec / (m["kernels_ms"]["decode_partition"] * 1e-3) / 1e9
    return dec, achieved, achieved / HBM_PEAK_GBS


# The other workloads the decode kernels are held to, measured in the same run and the same way
# as the headline line: (label, config, overrides, grouped decode, bytes basis unique).
ALSO = (("cfg2-opt13b-mha-bf16", 2, {"dtype": "bf16"}, False, False),
        ("cfg3-gqa-long-bf16", 3, {}, False, False),
        ("cfg5-fp8-kv", 5, {}, False, False),
        ("cfg4-shared-prefix-bf16-grouped", 4, {}, True, True))


def generate_also(config):
    """The other workloads, generated on the host before any timing (so that no measurement
    follows seconds of an idle GPU)."""
    ws = []
    for label, n, over, grouped, unique in ALSO:
        t0 = time.perf_counter()
        ws.append(config(n, **over))
        print(f"[bench] generated {label} in {time.perf_counter() - t0:.1f}s", file=sys.stderr,
              flush=True)
    return ws


def measure_also(args, lib, torch, preps):
    """Times the prepared other workloads one after another (the GPU kept busy between them)."""
    res = {}
    also_args = argparse.Namespace(**vars(args))
    also_args.warmup = max(args.warmup, args.also_warmup)
    for (label, n, over, grouped, unique), prep in zip(ALSO, preps):
        w = prep["w"]
        m = time_steps(prep, also_args, lib, torch)
        dec, achieved, frac = decode_roofline(w, m, unique, prep["fused"])
        step_bytes = w.decode_bytes() + w.write_bytes() + w.copy_bytes()
        res[label] = {
            "kernel": m["kernel"],
            "decode": ("pa_decode_grouped" if grouped else "pa_decode") +
                      ("_append" if prep["fused"] else ""),
            "attention_kernel_us": us(m["kernels_ms"]["decode_partition"]),
            "merge_us": us(m["kernels_ms"]["decode_merge"]),
            "write_kv_us": us(m["kernels_ms"]["write_kv"]),
            "copy_blocks_us": us(m["kernels_ms"]["copy_blocks"]),
            "step_us": round(1e3 * m["ms_step"], 2), "step_us_percentiles": m["pcts"],
            "bytes_per_launch": dec, "bytes_basis": "unique" if unique else "logical",
            "achieved_gbs": round(achieved, 2), "frac": round(frac, 4),
            "step_gbs": round(step_bytes / (m["ms_step"] * 1e-3) / 1e9, 2),
            "attended_tokens_per_s": round(w.attended_tokens / (m["ms_step"] * 1e-3), 1),
            "cache_dtype": w.dtype, "num_seqs": w.num_seqs, "attended_tokens": w.attended_tokens,
        }
        print(f"[bench] also {label}: attention kernel {res[label]['attention_kernel_us']} us, "
              f"frac {res[label]['frac']}", file=sys.stderr, flush=True)
        prep["w"] = None
    return res


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the paged decode path here has no multi-GPU leg; see the design notes on sharding.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from paged_kv_cache_318_amd import lib
    from workloads import config

    # (counting devices does not initialise the GPU; the CPU baseline below forks before it is)
    assert torch.cuda.device_count() > 0, "bench.py needs the GPU"
    if args.measure != "step":
        assert torch.cuda.is_available(), "bench.py needs the GPU"
        lib.load()
        return {"swap": measure_swap, "paging": measure_paging,
                "prefill": measure_prefill}[args.measure](args, lib, torch)
    over = {}
    if args.dtype:
        over["dtype"] = args.dtype
    if args.first_step:
        over["first_step"] = True
    if args.num_seqs > 0:
        over["num_seqs"] = args.num_seqs
    t_gen = time.perf_counter()
    w = config(args.config, **over)
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] workload {w.name}: {w.num_seqs} seqs, {w.attended_tokens} attended tokens, "
          f"{w.kv_bytes() / 1e9:.3f} GB K/V per call, generated in {t_gen:.1f}s", file=sys.stderr,
          flush=True)

    do_also = not args.no_also and args.config == 2 and not over and not args.grouped
    also_ws = generate_also(config) if do_also else []

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        cpu = cpu_baselines(w, args.cpu_seconds)
        print(f"[bench] oracle: {cpu[0]['value']} GB/s on {cpu[0]['cores']} cores, "
              f"{cpu[1]['value']} GB/s on 1", file=sys.stderr, flush=True)

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    lib.load()
    calibration_copy(args, torch)
    # every workload is on the device before the first timed step; the others are timed right
    # after the headline one
    fused = not args.separate
    prep = prepare_steps(w, args, lib, torch, grouped=args.grouped, variant=args.variant,
                         partition=args.partition, fused=fused)
    also_preps = [prepare_steps(x, args, lib, torch, grouped=g, fused=fused)
                  for x, (_, _, _, g, _) in zip(also_ws, ALSO)]
    del also_ws
    m = time_steps(prep, args, lib, torch)
    ms_step = m["ms_step"]
    step_bytes = w.decode_bytes() + w.write_bytes() + w.copy_bytes()
    value = step_bytes / (ms_step * 1e-3) / 1e9
    unique = args.config == 4
    fused = prep["fused"]
    dec_bytes, achieved, frac = decode_roofline(w, m, unique, fused)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) K/V/q, scattered blocks; no dataset)",
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "attended_tokens_per_s": round(w.attended_tokens / (ms_step * 1e-3), 1),
        "config": {
            "workload": w.name, "num_seqs": w.num_seqs, "num_heads": w.num_heads,
            "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
            "cache_dtype": w.dtype, "q_dtype": w.q_dtype, "accumulate": "f32",
            "attended_tokens": w.attended_tokens, "num_blocks": w.num_blocks,
            "cow_pairs": int(w.cow.shape[0]), "step_bytes": step_bytes,
            "decode_bytes": w.decode_bytes(), "unique_decode_bytes": w.decode_bytes(unique=True),
            "replicas": args.replicas, "partition_tokens": args.partition, "variant": args.variant,
            "shared_blocks_flag": m["shared"],
            "write": ("fused into the attention (pa_decode_grouped_append)" if args.grouped
                      else "fused into the attention (pa_decode_append)") if fused
                     else "separate launch (pa_write_kv, then the decode)",
            "grouped": m["grouped"],
        },
        "kernels_us": {
            "step_with_events": round(1e3 * m["ms_step_profiled"], 2),
            "decode_partition": us(m["kernels_ms"]["decode_partition"]),
            "decode_merge": us(m["kernels_ms"]["decode_merge"]),
            "write_kv": us(m["kernels_ms"]["write_kv"]),
            "copy_blocks": us(m["kernels_ms"]["copy_blocks"]),
        },
        "step_us_percentiles": m["pcts"],
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(frac, 4),
            "traffic": measured_traffic(m["kernel"], w.name),
            "kernel": m["kernel"], "bytes_per_launch": dec_bytes,
            "bytes_basis": "unique" if unique else "logical",
        },
        "cpu_baseline": None if cpu is None else cpu[0],
        "cpu_baseline_1t": None if cpu is None else cpu[1],
    }
    del w, prep
    if also_preps:
        line["also"] = measure_also(args, lib, torch, also_preps)
        line["also_warmup"] = max(args.warmup, args.also_warmup)
    if not args.no_ceiling:
        ceil = read_ceiling(lib, line["config"]["block_size"] * line["config"]["head_dim"] *
                            (1 if line["dtype"] == "fp8" else 2) * (2 if line["dtype"] == "f32" else 1))
        line["read_ceiling_gbs"] = ceil
        line["roofline"]["frac_of_measured_ceiling"] = round(achieved / ceil["scattered"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
