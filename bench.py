"""Benchmark of the paged-decode hot path on one MI355X.

One step = the cache write of each sequence's newest token (t = len - 1) and
the decode over the whole batch, with every input already resident in HBM:
by default pa_decode_write_partials (the write fused into the attention
pass) + pa_decode_merge; with --separate-write, pa_cache_write +
pa_decode_partials + pa_decode_merge.  The KV pool is replicated R times
(at least 2 GiB in all) and successive steps rotate through the copies, so
each step reads its pool from HBM rather than from the 256 MB last-level
cache.

Steps run twice: eagerly, with HIP events around every launch (the per-kernel
breakdown), and as replays of HIP graphs holding the same launches (the step
time a decode loop sees once launch gaps are gone).  The pool copies stand
for a model's layers: one graph holds the step of every copy in turn, as a
model's decode graph holds every layer's attention, and the timed steps run
through it; one graph per step (a graph launch between steps) is timed
beside it.  Each graph's output is checked against the eager output before
timing.  A labelled warm figure (warm_ms_per_step) replays one graph on one
pool copy, so caches may hold part of the pool.

Prints one JSON line:
  value       KV-read GB/s of the whole step (algorithmic bytes / graph-replayed
              step time; the eager step time is reported beside it)
  roofline    the attention kernel's algorithmic bytes (the write's included
              when it is fused) / its mean duration from HIP events recorded
              around every launch in the timed region, against the 8 TB/s HBM
              peak; the whole call (attention + split-K merge, timed in a
              loop of its own with no event between its two launches) is
              reported beside it
  cpu_baseline  the float64 CPU oracle on the same batch (1 BLAS thread)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config llama7b]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

REPO = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, REPO)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode KV-read GB/s (% of HBM peak) + decode tokens/s/layer, 1 GPU"
ELEM = {"f16": 2, "bf16": 2, "fp8_e4m3": 1}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(b) -> dict:
    """Bytes the step must move at minimum (valid tokens only, one layer)."""
    lens = b.context_lens.astype(np.int64)
    B, Hq, Hkv, D, bs = b.num_seqs, b.num_heads, b.num_kv_heads, b.head_dim, b.block_size
    kv = int(lens.sum()) * 2 * Hkv * D * ELEM[b.kv_dtype]
    qo = B * Hq * D * (ELEM[b.q_dtype] * 2)
    tables = 4 * int(np.sum(-(-lens // bs))) + 4 * B
    decode = kv + qo + tables
    write = B * 2 * Hkv * D * (ELEM[b.src_dtype] + ELEM[b.kv_dtype]) + 4 * B + 4 * B
    out = {"kv": kv, "decode": decode, "write": write}
    if b.notes.get("prefix_blocks"):
        # a batch that shares prefix blocks: each stored token once (the HBM floor)
        unique_kv = b.unique_tokens_in_use() * 2 * Hkv * D * ELEM[b.kv_dtype]
        out["unique_kv"] = unique_kv
        out["unique_decode"] = unique_kv + qo + tables
    return out


# the sources the decode kernels and their launcher are built from, and the
# build script whose compiler flags shape the code too
DECODE_SOURCES = ("decode.hip", "decode_gqa_mfma.hip", "decode_gqa16_mfma.hip", "decode_common.h", "kv_encode.h",
                  "pa_internal.h", "pa_api.cpp", "../build.py")


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(REPO, "paged_kv_cache_132_amd", "csrc")
    for name in DECODE_SOURCES:
        with open(os.path.normpath(os.path.join(csrc, name)), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def counter_traffic(config: str, partition, fused: bool, run_size: int = 1):
    """HBM bytes per attention launch from committed rocprofv3 counter runs, if
    they were taken on the current decode sources, split (a fixed partition in
    tokens, or the token-chunk label the bench prints) and step form (cache
    write fused or separate, shared runs); otherwise None."""
    path = os.path.join(REPO, "profiles", f"decode_{config}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if (rec.get("source_hash") != source_hash() or rec.get("partition") != partition
            or rec.get("fused_write", False) != fused or rec.get("run_size", 1) != run_size):
        return None
    return rec.get("attention_hbm_bytes_per_launch")


def stream_read_gbs(torch, nbytes: int = 4 << 30, reps: int = 10) -> float:
    """HBM read bandwidth a plain streaming kernel reaches on this device."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(REPO, "paged_kv_cache_132_amd", "libpa_bench.so"))
    lib.pa_bench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    lib.pa_bench_read_grid.restype = ctypes.c_int
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(lib.pa_bench_read_grid(), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(2):
        lib.pa_bench_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        if lib.pa_bench_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream) != 0:
            raise RuntimeError("pa_bench_read launch failed")
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del buf
    return nbytes / (ms * 1e-3) / 1e9


def copy_calibration(torch, reps: int, nbytes: int = 1 << 30) -> int:
    """Run a plain 1 GiB device copy `reps` times: a kernel whose HBM traffic is
    known exactly (nbytes read + nbytes written), to scale byte counters."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(REPO, "paged_kv_cache_132_amd", "libpa_bench.so"))
    lib.pa_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(reps):
        if lib.pa_bench_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream) != 0:
            raise RuntimeError("pa_bench_copy launch failed")
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)
    return 0


def build_workload(name: str):
    from workloads import CONFIG_MAKERS

    return CONFIG_MAKERS[name]()


def upload(b, torch, pa, copies: int):
    """Device tensors for the batch; `copies` replicas of the KV pool."""
    dev = torch.device("cuda:0")

    def d16(raw, dt):
        t = torch.from_numpy(np.ascontiguousarray(raw).view(np.int16))
        return t.view(torch.float16 if dt == "f16" else torch.bfloat16).to(dev)

    bt = torch.from_numpy(b.block_table_array(pad=0)).to(dev)
    lens = torch.from_numpy(b.context_lens.astype(np.int32)).to(dev)
    q = d16(b.query, b.q_dtype)
    new_k = d16(b.new_key[0], b.src_dtype)
    new_v = d16(b.new_value[0], b.src_dtype)
    if b.kv_dtype == "fp8_e4m3":
        # Fill the fp8 pool through the cache write itself, in one launch:
        # every slot (block b, offset o) is presented as a one-token sequence
        # whose table is [b] and whose length is o + 1, so the write kernel
        # quantises each generated value into its own slot.
        nb, _, bs, hkv, hd = b.kv_source.shape
        src = d16(b.kv_source, b.src_dtype)
        keys = src[:, 0].reshape(nb * bs, hkv, hd).contiguous()
        vals = src[:, 1].reshape(nb * bs, hkv, hd).contiguous()
        del src
        slot_tables = torch.arange(nb, dtype=torch.int32, device=dev).repeat_interleave(bs).reshape(-1, 1)
        slot_lens = (torch.arange(nb * bs, dtype=torch.int32, device=dev) % bs + 1).contiguous()
        pool = torch.empty(b.kv_source.shape, dtype=torch.uint8, device=dev)
        pa.cache_write(pool, keys, vals, slot_tables, slot_lens, b.k_scale, b.v_scale)
        del keys, vals, slot_tables, slot_lens
    else:
        pool = d16(b.kv_pool, b.kv_dtype)
    pools = [pool] + [pool.clone() for _ in range(copies - 1)]
    torch.cuda.synchronize()
    return {"bt": bt, "lens": lens, "q": q, "k": new_k, "v": new_v, "pools": pools}


def cpu_baseline(b, budget_s: float = 20.0) -> dict:
    """The oracle, as it stands, on a bounded sample: whole sequences of the
    same batch, taken in order (and round again when the batch is done) until
    about `budget_s` seconds are spent."""
    import oracle

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:                      # pragma: no cover
        threadpool_limits = None
    bt = b.block_table_array()
    lens = b.context_lens
    if b.kv_dtype == "fp8_e4m3":
        pool = None                          # encode only the sample's blocks below
    else:
        pool = b.kv_pool
    ctx = threadpool_limits(limits=1) if threadpool_limits else None
    if ctx:
        ctx.__enter__()
    try:
        done, tokens, t_total = [], 0, 0.0
        order = [s for _ in range(1000) for s in range(b.num_seqs)]
        first = True                         # one untimed call first: one-off set-up is not the oracle's rate
        for s in order:
            if b.kv_dtype == "fp8_e4m3":
                blocks = sorted(set(b.tables[s]))
                sub = oracle.encode_pool(b.kv_source[blocks], b.src_dtype, "fp8_e4m3", b.k_scale, b.v_scale)
                remap = {blk: i for i, blk in enumerate(blocks)}
                bt_s = np.array([[remap[x] for x in b.tables[s]]], dtype=np.int32)
                t0 = time.perf_counter()
                oracle.paged_decode(b.query[s:s + 1], b.q_dtype, sub, "fp8_e4m3", bt_s, lens[s:s + 1],
                                    b.block_size, b.scale, b.k_scale, b.v_scale)
                dt = time.perf_counter() - t0
            else:
                t0 = time.perf_counter()
                oracle.paged_decode(b.query[s:s + 1], b.q_dtype, pool, b.kv_dtype, bt[s:s + 1], lens[s:s + 1],
                                    b.block_size, b.scale)
                dt = time.perf_counter() - t0
            if first:
                first = False
                continue
            t_total += dt
            done.append(s)
            tokens += int(lens[s])
            if t_total >= budget_s:
                break
    finally:
        if ctx:
            ctx.__exit__(None, None, None)
    kv_bytes = tokens * 2 * b.num_kv_heads * b.head_dim * ELEM[b.kv_dtype]
    return {
        "value": round(kv_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "host_cores_available": len(os.sched_getaffinity(0)),
        "kind": "oracle",
        "sample": f"{len(done)} sequence decodes ({len(done) / b.num_seqs:.2f} passes over the "
                  f"{b.num_seqs}-sequence batch, {tokens} context tokens), float64 numpy, {t_total:.1f} s",
        "tokens_per_s_per_layer": round(len(done) / t_total, 3),
    }


def bench_copy_blocks(args, torch, pa) -> int:
    """pa_copy_blocks (copy-on-write of shared blocks, [nano-vllm blog §4.3])
    at the 7B block geometry: 256 KiB blocks (16 tokens x 32 KV heads x 128
    x fp16, K and V), 2048 independent (source, destination) pairs per launch
    inside an 8192-block (2 GiB) pool; four different pair sets rotate so a
    launch does not find its blocks in the last-level cache.  Also timed: a
    swap out of 256 blocks to a pinned host pool (PCIe-bound)."""
    import oracle

    bs, hkv, d, nb, npairs, sets = 16, 32, 128, 8192, 2048, 4
    block_bytes = 2 * bs * hkv * d * 2
    rng = np.random.default_rng(7)
    pool = torch.empty((nb, 2, bs, hkv, d), dtype=torch.float16, device="cuda").normal_()
    maps = []
    for _ in range(sets):
        perm = rng.permutation(nb)[:2 * npairs]
        maps.append(torch.from_numpy(np.stack([perm[:npairs], perm[npairs:]], 1).astype(np.int32)).cuda())
    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        pa.copy_blocks(pool, pool, maps[i % sets])
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        pa.copy_blocks(pool, pool, maps[i % sets])
        e1.record(stream)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    kern_us = float(np.mean([a.elapsed_time(b) for a, b in ev]) * 1e3)
    moved = 2 * npairs * block_bytes
    achieved = moved / (kern_us * 1e-6) / 1e9

    host = torch.empty((256, 2, bs, hkv, d), dtype=torch.float16, pin_memory=True)
    m_out = torch.from_numpy(np.stack([rng.permutation(nb)[:256], np.arange(256)], 1).astype(np.int32)).cuda()
    pa.copy_blocks(pool, host, m_out)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(5):
        pa.copy_blocks(pool, host, m_out)
    torch.cuda.synchronize()
    swap_gbs = 5 * 256 * block_bytes / (time.perf_counter() - t1) / 1e9
    log(f"copy_blocks: {kern_us:.1f} us per launch ({achieved:.0f} GB/s read+write); swap out {swap_gbs:.1f} GB/s")

    res = {
        "metric": "KV block copy GB/s (bytes read + written), 1 GPU",
        "value": round(moved / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "copy_blocks_7b", "block_bytes": block_bytes, "pairs_per_launch": npairs,
                   "pool_blocks": nb},
        "copy_kernel_us": round(kern_us, 2),
        "swap_out_to_pinned_host_gbs": round(swap_gbs, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        hp = np.random.default_rng(8).integers(0, 1 << 16, size=(1024, 2, bs, hkv, d), dtype=np.uint16)
        perm = np.random.default_rng(9).permutation(1024)[:512]
        mp = np.stack([perm[:256], perm[256:]], 1)
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_budget, 10.0):
            oracle.copy_blocks(hp, hp, mp)
            reps += 1
        dt = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(reps * 2 * 256 * block_bytes / dt / 1e9, 3), "unit": "GB/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{reps} oracle copies of 256 pairs in a 1024-block host pool, {dt:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


def prefill_flops(b) -> int:
    """Causal attention multiply-adds x 2: each new query at position p scores
    and weights p + 1 keys (QK and PV: 2 x 2 x head_dim flops per key) for
    every query head."""
    lens = b.context_lens.astype(np.int64)
    new = b.new_lens.astype(np.int64)
    keys = sum(int(((L - n + 1) + L) * n // 2) for L, n in zip(lens, new))   # sum of (p + 1)
    return 4 * b.head_dim * b.num_heads * keys


def bench_prefill(args, torch, pa) -> int:
    """The prompt stage on the packed prompt batch of [CANN notes §1.2]:
    8 fresh prompts of 128..2048 tokens (5256 in all), 32/32 heads,
    head_dim 128, fp16, block size 16.  One step = the write of all 5256
    tokens and the causal attention: pa_prefill_write (one launch that does
    both) by default, pa_cache_write_tokens + pa_prefill with
    --separate-write."""
    import oracle
    from workloads import make_prefill_mixed

    b = make_prefill_mixed()
    flops = prefill_flops(b)
    dev = torch.device("cuda:0")
    d16 = lambda raw: torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.float16).to(dev)
    pool = d16(b.kv_pool)
    bt = torch.from_numpy(b.block_table_array()).to(dev)
    lens = torch.from_numpy(b.context_lens).to(dev)
    cu = torch.from_numpy(b.cu_seqlens).to(dev)
    q, k, v = d16(b.query), d16(b.new_key), d16(b.new_value)
    out = torch.empty_like(q)
    mx = int(b.new_lens.max())
    stream = torch.cuda.current_stream()

    fused = not args.separate_write

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if not fused:
            pa.cache_write_tokens(pool, k, v, bt, lens, cu)
        if ev is not None:
            ev[1].record(stream)
        if fused:
            pa.prefill(q, pool, bt, lens, cu, b.scale, out=out, max_new_tokens=mx, new_key=k, new_value=v)
        else:
            pa.prefill(q, pool, bt, lens, cu, b.scale, out=out, max_new_tokens=mx)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    write_us = float(np.mean([e[0].elapsed_time(e[1]) for e in events]) * 1e3)
    attn = np.array([e[1].elapsed_time(e[2]) for e in events]) * 1e3
    attn_us = float(attn.mean())
    achieved = flops / (attn_us * 1e-6) / 1e12
    log(f"prefill: attention {attn_us:.1f} us ({achieved:.0f} TFLOP/s), "
        f"{'write fused' if fused else f'write {write_us:.1f} us'}, step {ms_step * 1e3:.1f} us")
    res = {
        "metric": "paged prefill attention TFLOP/s (causal, packed prompts), 1 GPU",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": b.name, "num_seqs": b.num_seqs, "num_tokens": b.num_tokens,
                   "num_heads": b.num_heads, "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                   "block_size": b.block_size, "seed": b.seed},
        "step_kernels": "pa_prefill_write (write fused)" if fused else "pa_cache_write_tokens, pa_prefill",
        "prefill_kernel_us": round(attn_us, 2),
        "prefill_kernel_us_p10_p50_p90": [round(float(np.percentile(attn, x)), 2) for x in (10, 50, 90)],
        "write_tokens_kernel_us": None if fused else round(write_us, 2),
        "prefill_tokens_per_s_per_layer": round(b.num_tokens / (ms_step * 1e-3), 1),
        "flops": flops,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(achieved / 2500.0, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        try:
            from threadpoolctl import threadpool_limits
            ctx = threadpool_limits(limits=1)
        except ImportError:                  # pragma: no cover
            ctx = None
        done, f_done, t_total = 0, 0, 0.0
        try:
            for s in np.argsort(b.new_lens):  # shortest prompts first, until the budget is spent
                lo, hi = int(b.cu_seqlens[s]), int(b.cu_seqlens[s + 1])
                t1 = time.perf_counter()
                oracle.paged_prefill(b.query[lo:hi], "f16", b.kv_pool, "f16", b.block_table_array()[s:s + 1],
                                     b.context_lens[s:s + 1], np.array([0, hi - lo]), b.block_size, b.scale)
                t_total += time.perf_counter() - t1
                done += 1
                n = hi - lo
                f_done += 4 * b.head_dim * b.num_heads * n * (n + 1) // 2
                if t_total >= min(args.cpu_budget, 15.0):
                    break
        finally:
            if ctx is not None:
                ctx.__exit__(None, None, None)
        res["cpu_baseline"] = {"value": round(f_done / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{done} of {b.num_seqs} prompts (shortest first), float64 numpy, "
                                         f"{t_total:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


def run_decode(args, torch, pa, b) -> dict:
    """Time the decode step (write + attention + merge) on batch b; the
    result dict of the JSON line, without the CPU baseline."""
    nbytes = algorithmic_bytes(b)
    pool_bytes = b.num_blocks * 2 * b.block_size * b.num_kv_heads * b.head_dim * ELEM[b.kv_dtype]
    copies = max(2, math.ceil((2 << 30) / pool_bytes))
    log(f"uploading: pool {pool_bytes / 2**20:.0f} MiB x {copies} copies")
    dev = upload(b, torch, pa, copies)
    kvt = pa.pa_dtype(dev["pools"][0])
    mb = b.max_blocks_per_seq
    partition_size = args.partition_size
    run_size = args.run_size
    if b.notes.get("prefix_blocks") and args.run_size is None and args.partition_size is None:
        # the shared-prefix batch: shared runs as long as a share group, and a
        # partition that tiles the shared prefix exactly (4480 = 5 x 896) so
        # no shared block falls to the per-sequence kernel
        run_size = int(b.notes.get("share_group", 1))
        partition_size = int(b.notes["prefix_tokens"]) // 5
    partition_size = partition_size or 0
    run_size = run_size or 1
    partition = pa.decode_partition_size(b.num_seqs, b.num_heads, b.num_kv_heads, b.head_dim, b.block_size,
                                         mb, kvt, partition_size)
    if partition_size == 0:
        partition = f"token chunks (>= {partition})"
    ws = torch.zeros(pa.decode_workspace_size(b.num_seqs, b.num_heads, b.num_kv_heads, b.head_dim,
                                              b.block_size, mb, kvt, partition_size),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dev["q"])
    stream = torch.cuda.current_stream()

    fused = not args.separate_write and b.q_dtype == b.src_dtype
    if run_size != 1 and not fused:
        raise SystemExit("--run-size takes the fused step (pa_decode_write_partials_shared)")

    def step(i, ev=None, split=True):
        # one pass of the hot path: cache write, attention pass, split-K merge.
        # (split=False: no event between the two decode launches)
        # Fused (default): pa_decode_write_partials writes the newest token in
        # the attention pass; otherwise pa_cache_write runs first.
        pool = dev["pools"][i % copies]
        dargs = (dev["q"], pool, dev["bt"], dev["lens"], b.scale, b.k_scale, b.v_scale)
        dkw = dict(out=out, workspace=ws, partition_size=partition_size)
        if ev is not None:
            ev[0].record(stream)
        if not fused:
            pa.cache_write(pool, dev["k"], dev["v"], dev["bt"], dev["lens"], b.k_scale, b.v_scale)
        if ev is not None:
            ev[1].record(stream)
        if fused:
            pa.decode(*dargs, phase="partials", new_key=dev["k"], new_value=dev["v"], run_size=run_size, **dkw)
        else:
            pa.decode(*dargs, phase="partials", **dkw)
        if ev is not None and split:
            ev[2].record(stream)
        pa.decode(*dargs, phase="merge", **dkw)
        if ev is not None:
            ev[3].record(stream)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_ms_step = wall * 1e3 / args.steps
    # the whole pa_decode call (attention pass + merge) timed on its own,
    # without the event between its two launches
    call_events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + i, call_events[i], split=False)
    torch.cuda.synchronize()

    graph_ms_step = warm_ms_step = graph_ms_step_one = None
    if not args.eager:
        # one graph per pool copy, each holding write + attention + merge
        ref = out.clone()
        step(args.warmup + args.steps - 1)
        torch.cuda.synchronize()
        ref.copy_(out)
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    step(c)
                graphs.append(g)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        for c, g in enumerate(graphs):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(out, ref):
                raise RuntimeError(f"graph replay {c} differs from the eager step")
        # The pool copies stand for the layers of a model, whose decode graph
        # holds every layer's attention back to back: one graph with the step
        # of each copy in turn.  The timed steps run through it (and through
        # the per-copy graphs for a remainder), so consecutive steps meet no
        # graph-launch gap; one graph per step is timed beside it.
        layers = torch.cuda.CUDAGraph()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(layers, stream=side):
                for c in range(copies):
                    step(c)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        out.zero_()
        layers.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError("the graph of all pool copies differs from the eager step")
        log(f"graph replay: {copies} graphs and the graph of all {copies} copies checked against the eager step")

        def timed(run_steps):
            torch.cuda.synchronize()
            t = time.perf_counter()
            run_steps()
            torch.cuda.synchronize()
            return (time.perf_counter() - t) * 1e3 / args.steps

        def through_layers():
            for _ in range(args.steps // copies):
                layers.replay()
            for i in range(args.steps % copies):
                graphs[i].replay()

        def one_per_graph():
            for i in range(args.steps):
                graphs[(args.warmup + i) % copies].replay()

        for i in range(args.warmup):
            graphs[i % copies].replay()
        layers.replay()
        graph_ms_step = timed(through_layers)
        graph_ms_step_one = timed(one_per_graph)
        # labelled warm figure: every step on the same pool copy, so the L2s
        # and the MALL may still hold part of it from the step before
        t0 = time.perf_counter()
        for i in range(args.steps):
            graphs[0].replay()
        torch.cuda.synchronize()
        warm_ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
        del graphs, layers

    write_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    attn_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    merge_ms = np.array([e[2].elapsed_time(e[3]) for e in events])
    call_ms = np.array([e[1].elapsed_time(e[3]) for e in call_events])
    ms_step = graph_ms_step if graph_ms_step is not None else eager_ms_step
    attn_us = float(attn_ms.mean() * 1e3)
    call_us = float(call_ms.mean() * 1e3)
    # the attention kernel's algorithmic bytes: the decode's, plus the write's
    # when fused.  A batch that shares prefix blocks counts each stored token
    # once (its HBM floor); the logical bytes, every sequence's own tokens,
    # are reported beside.
    decode_bytes = nbytes.get("unique_decode", nbytes["decode"])
    attn_bytes = decode_bytes + (nbytes["write"] if fused else 0)
    achieved = attn_bytes / (attn_us * 1e-6) / 1e9
    step_bytes = decode_bytes + nbytes["write"]
    value = step_bytes / (ms_step * 1e-3) / 1e9
    log(f"attention pass mean {attn_us:.1f} us (p10 {np.percentile(attn_ms, 10) * 1e3:.1f}, "
        f"p90 {np.percentile(attn_ms, 90) * 1e3:.1f}); merge {merge_ms.mean() * 1e3:.1f} us; "
        f"pa_decode call {call_us:.1f} us; "
        f"{'write fused' if fused else f'write {write_ms.mean() * 1e3:.1f} us'}; eager step "
        f"{eager_ms_step * 1e3:.1f} us; graph step "
        f"{'-' if graph_ms_step is None else f'{graph_ms_step * 1e3:.1f}'} us "
        f"({'-' if graph_ms_step_one is None else f'{graph_ms_step_one * 1e3:.1f}'} us with one graph per step)")
    traffic = counter_traffic(b.name, partition, fused, run_size)
    achievable = stream_read_gbs(torch)
    log(f"streaming-read kernel reaches {achievable:.0f} GB/s on this device")

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.kv_dtype,
        "data": "synthetic",
        "config": {
            "workload": b.name, "num_seqs": b.num_seqs, "num_heads": b.num_heads,
            "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim, "block_size": b.block_size,
            "q_dtype": b.q_dtype, "kv_dtype": b.kv_dtype, "context_tokens": int(b.context_lens.sum()),
            "seed": b.seed, "partition_size": partition, "pool_copies": copies, "run_size": run_size,
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "step_launch": "hip_graph" if graph_ms_step is not None else "eager",
        "warm_ms_per_step": round(warm_ms_step, 4) if graph_ms_step is not None else None,
        "graph": (f"one graph holding the steps of all {copies} pool copies (the layers of a model) "
                  "in turn" if graph_ms_step is not None else None),
        "graph_ms_per_step_one_graph_per_step": (round(graph_ms_step_one, 4)
                                                  if graph_ms_step_one is not None else None),
        "step_kernels": (f"pa_decode_write_partials_shared (runs of {run_size}, cache write fused), "
                         "pa_decode_merge" if run_size != 1 else
                         "pa_decode_write_partials (cache write fused), pa_decode_merge" if fused else
                         "pa_cache_write, pa_decode_partials, pa_decode_merge"),
        "eager_ms_per_step": round(eager_ms_step, 4),
        "decode_tokens_per_s_per_layer": round(b.num_seqs / (ms_step * 1e-3), 1),
        "decode_only_tokens_per_s_per_layer": round(b.num_seqs / (call_us * 1e-6), 1),
        "decode_attention_kernel_us": round(attn_us, 2),
        "decode_attention_kernel_us_p10_p50_p90": [round(float(np.percentile(attn_ms, q)) * 1e3, 2)
                                                   for q in (10, 50, 90)],
        "decode_merge_kernel_us": round(float(merge_ms.mean() * 1e3), 2),
        "decode_call_us": round(call_us, 2),
        "decode_call_gbs": round(attn_bytes / (call_us * 1e-6) / 1e9, 1),
        "hbm_read_achievable_gbs": round(achievable, 1),
        "decode_frac_of_achievable": round(achieved / achievable, 4),
        "write_kernel_us": round(float(write_ms.mean() * 1e3), 2) if not fused else None,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "algorithmic_bytes": nbytes,
    }
    if "unique_decode" in nbytes:
        res["bytes_basis"] = "unique (each stored token once)"
        logical = nbytes["decode"] + (nbytes["write"] if fused else 0)
        res["logical_kv_gbs"] = round(logical / (attn_us * 1e-6) / 1e9, 1)
    return res


def bench_block_sizes(args, torch, pa) -> int:
    """The block-size sweep of [nano-vllm blog §5.1] / [CANN notes §5.1]: the
    7B decode batch (same lengths) at block sizes 8, 16 and 32, each with the
    allocator's usage counters ([CANN notes §5.4]) and its last-block waste."""
    from workloads import make_llama7b

    sweep = {}
    for bs in (8, 16, 32):
        b = make_llama7b(block_size=bs)
        r = run_decode(args, torch, pa, b)
        sweep[bs] = {
            "attention_kernel_us": r["decode_attention_kernel_us"],
            "decode_call_us": r["decode_call_us"],
            "ms_per_step": r["ms_per_step"],
            "kv_gbs": r["roofline"]["achieved"],
            "step_gbs": r["value"],
            "decode_tokens_per_s_per_layer": r["decode_tokens_per_s_per_layer"],
            "partition_size": r["config"]["partition_size"],
            "usage": b.manager.usage(b.tables, b.context_lens),
        }
        log(f"block size {bs}: attention {r['decode_attention_kernel_us']:.1f} us, "
            f"step {r['ms_per_step'] * 1e3:.1f} us, slot utilisation "
            f"{sweep[bs]['usage']['slot_utilisation']:.4f}")
        del b
        torch.cuda.empty_cache()
    base = sweep[16]
    for bs in sweep:
        sweep[bs]["step_throughput_vs_bs16"] = round(base["ms_per_step"] / sweep[bs]["ms_per_step"], 4)
    res = {
        "metric": "paged decode KV-read GB/s vs block size (8/16/32), 1 GPU",
        "value": base["step_gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": base["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "llama7b block-size sweep", "block_sizes": [8, 16, 32], "value_at": 16},
        "roofline": {"bound": "hbm", "achieved": base["kv_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(base["kv_gbs"] / HBM_PEAK_GBS, 4), "traffic": None},
        "sweep": sweep,
    }
    print(json.dumps(res), flush=True)
    return 0


def bench_block_manager(args) -> int:
    """The host block manager (libpa.so, pa_bm_*) on a serving-shaped trace:
    256 requests of 1024-token prompts sharing a 512-token system prompt
    (prefix-cache hits on 32 blocks each, [nano-vllm blog §3.1]), 128 decode
    appends per request, then release; block size 16, 40,000 blocks.  Host
    CPU only; the Python reference model is timed on the same trace."""
    import oracle
    from paged_kv_cache_132_amd.block_manager import BlockManager

    rng = np.random.default_rng(12)
    system = rng.integers(0, 32000, size=512).tolist()
    prompts = [system + rng.integers(0, 32000, size=512).tolist() for _ in range(256)]
    gen = rng.integers(0, 32000, size=(256, 128))

    def run(mgr, limit_s=None):
        t0 = time.perf_counter()
        ops = 0
        for r, p in enumerate(prompts):
            mgr.add_sequence(r, p)
            ops += 1
            if limit_s and time.perf_counter() - t0 > limit_s:
                return ops, time.perf_counter() - t0
        for j in range(gen.shape[1]):
            for r in range(len(prompts)):
                mgr.append_token(r, int(gen[r, j]))
                ops += 1
            if limit_s and time.perf_counter() - t0 > limit_s:
                return ops, time.perf_counter() - t0
        for r in range(len(prompts)):
            mgr.free_sequence(r)
            ops += 1
        return ops, time.perf_counter() - t0

    times = []
    for _ in range(max(1, args.steps // 10)):
        bm = BlockManager(40000, 16)
        ops, dt = run(bm)
        times.append(dt)
    st = bm.stats()
    ops_s = ops / min(times)
    res = {
        "metric": "host block manager operations/s (prefix-cached admit, append, free), CPU",
        "value": round(ops_s, 1), "unit": "ops/s", "n_gpus": 0, "steps": len(times), "warmup": 0,
        "ms_per_step": round(min(times) * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": "256 requests x (512 shared + 512 own) prompt tokens + 128 appends",
                   "block_size": 16, "pool_blocks": 40000},
        "trace_ops": ops, "prefix_hits": st["hits"], "prefix_lookups": st["lookups"],
        "roofline": None,
    }
    if not args.no_cpu_baseline:
        m = oracle.BlockManagerModel(40000, 16)
        m_ops, m_dt = run(m, limit_s=min(args.cpu_budget, 10.0))
        res["cpu_baseline"] = {"value": round(m_ops / m_dt, 1), "unit": "ops/s", "cores": 1, "kind": "oracle",
                               "sample": f"the reference model on the first {m_ops} operations of the trace, "
                                         f"{m_dt:.1f} s"}
    log(f"block manager: {ops} ops in {min(times) * 1e3:.1f} ms ({ops_s:.0f} ops/s); "
        f"hits {st['hits']}/{st['lookups']}")
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama7b")
    ap.add_argument("--op", default="decode",
                    choices=("decode", "copy_blocks", "prefill", "block_sizes", "block_manager"),
                    help="decode: the decode step (default); copy_blocks: the block-copy kernel; "
                         "prefill: the prompt stage (multi-token write + causal prefill); "
                         "block_sizes: the decode step at block sizes 8, 16, 32; "
                         "block_manager: the host block manager (CPU only)")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="tokens per split-K partition; 0: token chunks (the library's choice, the default "
                         "except for the shared-prefix batch, which takes 896 with runs of 8)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--run-size", type=int, default=None,
                    help="decode step: sequences share prefix blocks in aligned runs of this many "
                         "(pa_decode_write_partials_shared; 1, 2, 4 or 8)")
    ap.add_argument("--separate-write", action="store_true",
                    help="run pa_cache_write as its own launch instead of fusing it into the attention pass")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches only (no HIP graph replay)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the 1 GiB copy kernel --steps times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode path is "
              f"single-GPU and shards by sequence or KV head without communication.", file=sys.stderr)
        return 2

    if args.op == "block_manager":
        return bench_block_manager(args)

    import torch
    import paged_kv_cache_132_amd as pa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    pa.load()
    if args.copy_calibration:
        return copy_calibration(torch, args.steps)
    if args.op == "copy_blocks":
        return bench_copy_blocks(args, torch, pa)
    if args.op == "prefill":
        return bench_prefill(args, torch, pa)
    if args.op == "block_sizes":
        return bench_block_sizes(args, torch, pa)
    log(f"building workload {args.config}")
    b = build_workload(args.config)
    res = run_decode(args, torch, pa, b)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(b, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
