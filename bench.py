"""Benchmark of libpmattn on one MI355X.

Default workload: the mixed chunked batch the metric is quoted on (paged mixed
attention): 16 prefill chunks of 512 tokens at unaligned starts, 96 decode
rows and 32 sequences verifying 5 linear drafts, prefixes shared through a
branching radix tree; 32 query / 8 kv heads, head_dim 128, bf16, 16-token
blocks, random non-contiguous block tables. The same JSON line also carries
the decode (64 sequences), few-shot prefill (256 x 128 on one shared 2048
prefix) and long-context decode (8 x 32k) workloads, each timed the same way
(``configs``), so that both halves of the metric (decode GB/s, prefill
TFLOP/s) are measured by every run. ``--config N`` makes workload N the main
line instead (1 tiny fp32, 2 decode, 3 few-shot, 4 mixed, 5 long decode, 6
token-tree verify, 7 shared-prompt decode).

One step = one ``pmattn_forward`` of the whole batch (tile tasks + merge) with
inputs resident in HBM; the plan is built once per batch on the host (as a
serving loop reuses it for every layer) and its host time is reported apart.
Before each timed step a read sweep over a 1 GiB scratch buffer (four times
the 256 MiB Infinity Cache) evicts L2 and the MALL, so KV blocks come from HBM.
The sweep reads rather than writes: a write would leave dirty lines whose
write-back the next kernel would pay for. HIP events on the launch stream
bracket the tasks pass and the merge pass of every step.

Prints ONE JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode KV GB/s + prefill/verify TFLOP/s (% roofline), paged mixed attention"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, published (2.5 PFLOP/s)
FP32_PEAK_TFS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Workload -> (committed rocprofv3 counter summary, sources of the dominant
# kernel). The work the kernel is given is pinned by the plan's tables.
_WAVE_SRC = ("attn_bf16.hip", "task_wave.h", "task_common.h")
_WG_SRC = ("attn_prefill.hip", "task_wg.h", "task_common.h")
_MIXED_SRC = ("attn_mixed.hip", "task_wave.h", "task_wg.h", "task_common.h")
_TASK_KERNEL = {
    2: ("attn_bf16_decode_64seq.md", _WAVE_SRC),
    3: ("attn_prefill_fewshot_256x128.md", _WG_SRC),
    4: ("attn_mixed_chunk_144seq.md", _MIXED_SRC),
    5: ("attn_bf16_long_decode_8x32k.md", _WAVE_SRC),
    6: ("attn_prefill_tree_verify_64x32.md", _WG_SRC),
    7: ("cascade_shared_prompt_decode_128x8k.md", _MIXED_SRC),
}


def kernel_source_hash(files):
    """First 16 hex digits of the sha256 over the given sources (csrc/)."""
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "prefix_shared_paged_pmattn_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def plan_tables_hash(tabs):
    """First 16 hex digits of the sha256 over the tables that define a plan's
    kernel work: tasks, their streaming flags, merge rows, classes, the
    equal-work slots and the mixed-batch table."""
    import hashlib
    h = hashlib.sha256()
    for k in ("items", "item_stream", "merge_rows", "class_rows", "class_begin", "class_stream",
              "slot_begin", "mix_table", "mix_bundles"):
        v = tabs.get(k)
        h.update(k.encode())
        if v is not None:
            h.update(np.ascontiguousarray(v).tobytes())
    return h.hexdigest()[:16]


def measured_traffic(config_idx, tabs):
    """HBM bytes per launch of the tasks kernel from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE, calibrated by a 1 GiB copy),
    or None when there is none for this workload, or the kernel's sources or
    the plan's tables differ from those the counters were taken with."""
    prof = _TASK_KERNEL.get(config_idx)
    if prof is None:
        return None
    try:
        text = open(os.path.join(ROOT, "profiles", prof[0])).read()
        sha = kernel_source_hash(prof[1])
    except OSError:
        return None
    fields = dict(l.split(": ", 1) for l in text.splitlines()
                  if l.startswith(("traffic_bytes", "kernel_source", "plan_tables")))
    if (fields.get("kernel_source_sha256_16") != sha or fields.get("plan_tables_sha256_16") != plan_tables_hash(tabs)
            or "traffic_bytes_per_launch" not in fields):
        return None
    return int(fields["traffic_bytes_per_launch"])


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(batch, work, seconds=15.0):
    """The fp64 oracle on a bounded sample of the same batch: whole sequences
    in a fixed seeded order, each through ``oracle.attend`` on its rows, until
    ``seconds`` of CPU time; the rate is the sample's own algorithmic bytes
    (or FLOP) over that time, in the metric's unit."""
    import oracle
    import workloads as wl
    threads = _blas_threads()
    off = batch.row_offsets()
    seqs = [s for s in np.random.Generator(np.random.PCG64(7)).permutation(batch.num_seqs) if batch.q_len[s] > 0]
    done = np.zeros(batch.num_seqs, bool)
    t = 0.0
    for s in seqs:
        t0 = time.perf_counter()
        oracle.attend(batch, rows=np.arange(int(off[s]), int(off[s + 1])))
        t += time.perf_counter() - t0
        done[s] = True
        if t >= seconds:
            break
    sw = wl.algorithmic_work(wl.subset(batch, done, batch.name + "[sample]"))
    bound = "hbm" if work["flop"] / work["bytes"] < 315 else "mfma"
    if bound == "hbm":
        val, unit = sw["bytes"] / t / 1e9, "GB/s"
    else:
        val, unit = sw["flop"] / t / 1e12, "TFLOP/s"
    kinds = {}
    for s in np.nonzero(done)[0]:
        k = wl.seq_kind(int(batch.q_len[s]))
        kinds[k] = kinds.get(k, 0) + 1
    return dict(value=val, unit=unit, cores=int(threads), kind="oracle",
                sample=f"{int(done.sum())} of {batch.num_seqs} sequences ({', '.join(f'{v} {k}' for k, v in sorted(kinds.items()))}; "
                       f"{sw['bytes']} algorithmic bytes, {sw['flop']:.4g} FLOP) in {t:.1f} s, one oracle.attend "
                       f"call per sequence, numpy fp64 (BLAS threads={threads}; exp single-threaded); "
                       f"host os.cpu_count()={os.cpu_count()}")


def per_core_oracle():
    """The oracle on the whole tiny fp32 batch and the whole 64-sequence
    decode batch with BLAS limited to one thread (one core)."""
    import oracle
    import workloads as wl
    from threadpoolctl import threadpool_limits
    res = {}
    with threadpool_limits(1):
        for idx, key in ((1, "tiny"), (2, "decode")):
            b = wl.config(idx)
            w = wl.algorithmic_work(b)
            t0 = time.perf_counter()
            oracle.attend(b)
            t = time.perf_counter() - t0
            res[key] = dict(workload=b.name, seconds=t, gbs=w["bytes"] / t / 1e9, threads=1)
    return res


def timed_forward(pm, p, q, kp, vp, bt, out, lse, stream, args, flush):
    """W untimed then K timed ``pmattn_forward`` steps of plan ``p`` (a cache
    flush before each). HIP events on the launch stream bracket the tasks pass
    and the merge pass of every timed step. Returns the per-step tasks, merge
    and step times (ms) and the host wall time of the K steps (s)."""
    import ctypes

    import torch
    ws = torch.empty(max(p.workspace_bytes, 256), dtype=torch.uint8, device=q.device)
    p.upload(ws, stream)
    # Validate every tensor once through the binding, then call the two C-ABI
    # passes with pre-marshalled arguments so that host overhead stays far
    # below the GPU time of a step (the stream never waits for the host).
    pm.forward_tasks(p, q, kp, vp, bt, out, lse, ws, stream)
    pm.forward_merge(p, out, lse, ws, stream)
    lib = pm._lib.load()
    vptr = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    c_args = (p.handle, vptr(q), vptr(kp), vptr(vp), vptr(bt), vptr(out), vptr(lse), vptr(ws),
              ws.numel(), ctypes.c_void_p(int(stream.cuda_stream)))
    m_args = (p.handle, vptr(out), vptr(lse), vptr(ws), ws.numel(),
              ctypes.c_void_p(int(stream.cuda_stream)))

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        st = lib.pmattn_forward_tasks(*c_args)
        if ev is not None:
            ev[1].record(stream)
        st |= lib.pmattn_forward_merge(*m_args)
        if ev is not None:
            ev[2].record(stream)
        if st:
            raise RuntimeError(lib.pmattn_last_error().decode())

    for _ in range(args.warmup):
        if not args.no_flush:
            flush()
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for k in range(args.steps):
        if not args.no_flush:
            flush()
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    return ([e[0].elapsed_time(e[1]) for e in evs], [e[1].elapsed_time(e[2]) for e in evs],
            [e[0].elapsed_time(e[2]) for e in evs], wall)


def class_breakdown(pm, b, make_plan_for, kp, vp, conv, dev, stream, args, flush):
    """Each query class of a mixed batch (decode, verify, prefill) planned and
    timed alone on the same pool, with the same flush and events as the whole
    batch. Returns {kind: {...}} with the class's time and its rates against
    both peaks."""
    import torch
    import workloads as wl
    kinds = np.array([wl.seq_kind(int(n)) for n in b.q_len])
    res = {}
    for kind in ("prefill", "verify", "decode"):
        keep = (kinds == kind) & (b.q_len > 0)
        if not keep.any():
            continue
        sb = wl.subset(b, keep, f"{b.name}[{kind}]")
        w = wl.algorithmic_work(sb)
        p = make_plan_for(sb)
        q = conv(sb.q).to(dev)
        bt = torch.from_numpy(sb.block_table).to(dev)
        et = torch.bfloat16 if sb.dtype == "bf16" else torch.float32
        out = torch.empty((sb.num_rows, sb.num_q_heads, sb.head_dim), dtype=et, device=dev)
        lse = torch.empty((sb.num_rows, sb.num_q_heads), dtype=torch.float32, device=dev)
        t_task, t_merge, t_step, _ = timed_forward(pm, p, q, kp, vp, bt, out, lse, stream, args, flush)
        ms = statistics.mean(t_step)
        gbs = w["bytes"] / (ms * 1e-3) / 1e9
        tfs = w["flop"] / (ms * 1e-3) / 1e12
        res[kind] = dict(seqs=int(keep.sum()), rows=sb.num_rows, ms_per_step=ms,
                         tasks_ms=statistics.mean(t_task), merge_ms=statistics.mean(t_merge),
                         algorithmic_bytes=w["bytes"], flop=w["flop"], gbs=gbs, tflops=tfs,
                         hbm_frac=gbs / HBM_PEAK_GBS, mfma_frac=tfs / MFMA_BF16_PEAK_TFS)
        log(f"[bench] class {kind} alone: {int(keep.sum())} seqs, {sb.num_rows} rows, {ms:.4f} ms/step; "
            f"{gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% hbm), {tfs:.1f} TFLOP/s "
            f"({100 * tfs / MFMA_BF16_PEAK_TFS:.1f}% mfma)")
    return res


def bench_radix(args):
    """Host cost of the radix cache manager on a workload's requests. Token ids
    follow the block sharing of the batch: blocks shared between sequences get
    the same ids, so cached prefixes match exactly where the workload shares.
    Each timed round admits every request, publishes it, and releases it."""
    import workloads as wl
    from prefix_shared_paged_pmattn_amd.radix import RadixCache
    b = wl.config(args.config, values=False)
    reqs = []
    for s in range(b.num_seqs):
        n = int(b.seq_len[s])
        blocks = b.block_table[s, :(n + 15) // 16]
        toks = (np.repeat(blocks.astype(np.int64), 16)[:n] * 16 + np.arange(n) % 16) % (1 << 30)
        reqs.append(toks.astype(np.int32))
    need = sum((len(t) + 15) // 16 for t in reqs)
    times, cached = [], 0
    for rnd in range(args.warmup + args.steps):
        cache = RadixCache(need + 16)
        t0 = time.perf_counter()
        ids = []
        for t in reqs:
            sid, cl, _, _ = cache.admit(t)
            cache.publish(sid)
            ids.append(sid)
            if rnd == 0:
                cached += cl
        for sid in ids:
            cache.release(sid)
        if rnd >= args.warmup:
            times.append(time.perf_counter() - t0)
    us = statistics.median(times) / len(reqs) * 1e6
    tok = sum(len(t) for t in reqs)
    log(f"[bench] radix: {len(reqs)} requests, {tok} tokens, {cached} reused; {us:.1f} us per request "
        f"(admit + publish + release, binding overhead included)")
    print(json.dumps(dict(metric="radix cache us per request (host)", value=us, unit="us/request", n_gpus=0,
                          steps=args.steps, warmup=args.warmup, higher_is_better=False, dtype="int32",
                          data="synthetic", config=dict(workload=b.name + "+radix", requests=len(reqs),
                                                        tokens=tok, reused_tokens=cached),
                          host_cores=1)), flush=True)


def bench_append(args, b, pm, make_plan, dev, conv, kp, vp, bt):
    """Time pmattn_kv_append: this step's K/V rows written into their pool slots.
    Algorithmic bytes: the new rows read once and written once (2 x R x Hkv x d
    x 2 tensors x element size)."""
    import ctypes

    import torch
    rng = np.random.Generator(np.random.PCG64(1000 + args.config))
    shape = (b.num_rows, b.num_kv_heads, b.head_dim)
    kn_h = rng.standard_normal(shape).astype(np.float32)
    vn_h = rng.standard_normal(shape).astype(np.float32)
    if b.dtype == "bf16":
        import workloads as wl
        kn_h, vn_h = wl.f32_to_bf16_bits(kn_h), wl.f32_to_bf16_bits(vn_h)
    kn, vn = conv(kn_h).to(dev), conv(vn_h).to(dev)
    t = time.perf_counter()
    p = make_plan()
    plan_us = (time.perf_counter() - t) * 1e6
    stream = torch.cuda.current_stream(dev)
    ws = pm.kv_append(p, kn, vn, bt, kp, vp, None, stream)
    lib = pm._lib.load()
    vptr = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731
    c_args = (p.handle, vptr(kn), vptr(vn), vptr(bt), vptr(kp), vptr(vp), vptr(ws), ws.numel(),
              ctypes.c_void_p(int(stream.cuda_stream)))
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)
    for _ in range(args.warmup):
        torch.sum(scratch, dim=0, dtype=torch.int64, out=sink)
        if lib.pmattn_kv_append(*c_args):
            raise RuntimeError(lib.pmattn_last_error().decode())
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for k in range(args.steps):
        if not args.no_flush:
            torch.sum(scratch, dim=0, dtype=torch.int64, out=sink)
        evs[k][0].record(stream)
        st = lib.pmattn_kv_append(*c_args)
        evs[k][1].record(stream)
        if st:
            raise RuntimeError(lib.pmattn_last_error().decode())
    torch.cuda.synchronize()
    ms = statistics.mean(e[0].elapsed_time(e[1]) for e in evs)
    nbytes = 2 * 2 * b.num_rows * b.num_kv_heads * b.head_dim * b.elem_bytes
    value = nbytes / (ms * 1e-3) / 1e9
    units = p.tables()["append_units"].shape[0]
    log(f"[bench] append: {units} units, {nbytes} B; {ms * 1e3:.2f} us per append; {value:.1f} GB/s "
        f"= {100 * value / HBM_PEAK_GBS:.1f}% of hbm peak")
    res = dict(metric="KV append GB/s (% HBM roofline), paged pool", value=value, unit="GB/s", n_gpus=1,
               steps=args.steps, warmup=args.warmup, ms_per_step=ms, higher_is_better=True,
               scaling="weak", vs_baseline=None, dtype=b.dtype, data="synthetic",
               config=dict(workload=b.name + "+kv-append", query_rows=b.num_rows, kv_heads=b.num_kv_heads,
                           head_dim=b.head_dim, append_units=int(units), algorithmic_bytes=nbytes,
                           cache_flush_between_steps=not args.no_flush),
               roofline=dict(bound="hbm", achieved=value, peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=value / HBM_PEAK_GBS, traffic=None),
               plan_host_us=plan_us)
    if not args.no_cpu_baseline:
        import oracle
        n = min(b.num_rows, 256)
        sub = b.replace(q_len=np.minimum(b.q_len, np.maximum(0, n - np.concatenate(
            [[0], np.cumsum(b.q_len)[:-1]]))).astype(np.int32))
        r = int(sub.q_len.sum())
        t0 = time.perf_counter()
        oracle.append_kv(sub, kn_h[:r], vn_h[:r])
        dt = time.perf_counter() - t0
        sb = 2 * 2 * r * b.num_kv_heads * b.head_dim * b.elem_bytes
        res["cpu_baseline"] = dict(value=sb / dt / 1e9, unit="GB/s", cores=1, kind="oracle",
                                   sample=f"first {r} query rows of the batch, one run of {dt:.2f} s, "
                                          "pure-Python slot writes (single thread)")
        log(f"[bench] cpu baseline {res['cpu_baseline']['value']:.4f} GB/s")
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="do not evict caches between steps")
    ap.add_argument("--no-class-breakdown", action="store_true",
                    help="mixed batches: skip timing each query class alone")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the main workload (skip the other workloads' lines)")
    ap.add_argument("--num-kv-splits", type=int, default=None)
    ap.add_argument("--num-cus", type=int, default=0, help="compute units the plan balances for")
    ap.add_argument("--work-shuffle-seed", type=int, default=0,
                    help="launch the tasks of each class in a seeded random order (0: cost order)")
    ap.add_argument("--cascade", type=int, choices=(0, 1, 2), default=2,
                    help="shared-prefix cascade for decode/verify rows (plan option): 0 off, "
                         "1 every shared run, 2 automatic")
    ap.add_argument("--op", choices=("attention", "append", "radix"), default="attention",
                    help="attention: pmattn_forward (default); append: pmattn_kv_append of the "
                         "batch's query rows; radix: host radix-cache admit/publish/release of "
                         "the batch's requests (no GPU)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device-to-device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is a design note only)", file=sys.stderr)
        sys.exit(2)

    if args.op == "radix":
        return bench_radix(args)

    import torch
    import prefix_shared_paged_pmattn_amd as pm
    import workloads as wl

    if args.copy_calibration:
        # A copy of known size: FETCH_SIZE / WRITE_SIZE of this kernel calibrate
        # the counters against 1 GiB read + 1 GiB written per dispatch.
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(copy_bytes=1 << 30, dispatches=3)), flush=True)
        return

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    scratch = torch.ones(1 << 28, dtype=torch.int32, device=dev)       # 1 GiB, read to evict caches
    flush_sink = torch.empty((), dtype=torch.int64, device=dev)

    def flush():
        torch.sum(scratch, dim=0, dtype=torch.int64, out=flush_sink)

    def load(idx):
        t0 = time.perf_counter()
        b = wl.config(idx)
        if args.num_kv_splits is not None and idx == args.config:
            b = b.replace(num_kv_splits=args.num_kv_splits)
        work = wl.algorithmic_work(b)
        log(f"[bench] generated {b.name} in {time.perf_counter() - t0:.1f}s: rows={b.num_rows} "
            f"blocks={b.num_pool_blocks} unique_kv_tokens={work['unique_kv_tokens']} flop={work['flop']:.4g} "
            f"bytes={work['bytes']:.4g}")
        if b.dtype == "bf16":
            conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)  # noqa: E731
            et = torch.bfloat16
        else:
            conv = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
            et = torch.float32
        t = dict(q=conv(b.q).to(dev), kp=conv(b.k_pool).to(dev), vp=conv(b.v_pool).to(dev),
                 bt=torch.from_numpy(b.block_table).to(dev),
                 out=torch.empty((b.num_rows, b.num_q_heads, b.head_dim), dtype=et, device=dev),
                 lse=torch.empty((b.num_rows, b.num_q_heads), dtype=torch.float32, device=dev))
        return b, work, conv, t

    def make_plan_for(x):
        return pm.plan(x.q_len, x.seq_len, x.q_start, x.block_table,
                       num_pool_blocks=x.num_pool_blocks, num_q_heads=x.num_q_heads,
                       num_kv_heads=x.num_kv_heads, head_dim=x.head_dim, dtype=x.dtype,
                       scale=x.scale, num_kv_splits=x.num_kv_splits, num_cus=args.num_cus,
                       work_shuffle_seed=args.work_shuffle_seed, tree_parent=x.tree_parent,
                       cascade=args.cascade)

    if args.op == "append":
        b, work, conv, t = load(args.config)
        return bench_append(args, b, pm, lambda: make_plan_for(b), dev, conv, t["kp"], t["vp"], t["bt"])

    def run(idx, b, work, t):
        """Plan (host time: median of 20) and time K steps; the workload's
        summary with its rate against its own bound."""
        plan_times = []
        p = None
        for _ in range(20):
            p = None  # the previous plan is released outside the timed region
            t0 = time.perf_counter()
            p = make_plan_for(b)
            plan_times.append(time.perf_counter() - t0)
        tabs = p.tables()
        t_task, t_merge, t_step, wall = timed_forward(pm, p, t["q"], t["kp"], t["vp"], t["bt"], t["out"],
                                                      t["lse"], stream, args, flush)
        ms_step, ms_task = statistics.mean(t_step), statistics.mean(t_task)
        log(f"[bench] {b.name}: plan {statistics.median(plan_times) * 1e6:.1f} us host; items={tabs['items'].shape[0]} "
            f"classes={tabs['class_rows'].tolist()} one kernel={bool(tabs['mixed_kernel'])} "
            f"merge_rows={tabs['merge_rows'].shape[0]} ws={p.workspace_bytes} B")
        log(f"[bench] {b.name}: step ms mean {ms_step:.4f} median {statistics.median(t_step):.4f} "
            f"p10 {np.percentile(t_step, 10):.4f} p90 {np.percentile(t_step, 90):.4f}; "
            f"tasks {ms_task:.4f} merge {statistics.mean(t_merge):.4f}; wall incl. flush "
            f"{wall / args.steps * 1e3:.4f} ms/step")
        t_bytes = work["bytes"] / HBM_PEAK_GBS / 1e9 * 1e3        # ms at the HBM roofline
        peak_f = MFMA_BF16_PEAK_TFS if b.dtype == "bf16" else FP32_PEAK_TFS
        t_flop = work["flop"] / peak_f / 1e12 * 1e3               # ms at the MFMA (or fp32) roofline
        bound = "mfma" if t_flop > t_bytes else "hbm"
        if bound == "mfma":
            value, unit = work["flop"] / (ms_step * 1e-3) / 1e12, "TFLOP/s"
            achieved = work["flop"] / (ms_task * 1e-3) / 1e12
            peak = peak_f
        else:
            value, unit = work["bytes"] / (ms_step * 1e-3) / 1e9, "GB/s"
            achieved = work["bytes"] / (ms_task * 1e-3) / 1e9
            peak = HBM_PEAK_GBS
        plain = (args.num_kv_splits is None and not args.num_cus and not args.work_shuffle_seed
                 and args.cascade == 2)
        roof = dict(bound=bound, achieved=achieved, peak=peak, unit=unit, frac=achieved / peak,
                    traffic=measured_traffic(idx, tabs) if plain else None)
        res = dict(workload=b.name, ms_per_step=ms_step, tasks_ms=ms_task, merge_ms=statistics.mean(t_merge),
                   value=value, unit=unit, roofline=roof, frac_step=value / peak,
                   gbs=work["bytes"] / (ms_step * 1e-3) / 1e9, tflops=work["flop"] / (ms_step * 1e-3) / 1e12,
                   # both resources can be busy at once: the bound is the slower of the two
                   max_bound=dict(hbm_ms=t_bytes, mfma_ms=t_flop, frac_step=max(t_bytes, t_flop) / ms_step,
                                  frac_kernel=max(t_bytes, t_flop) / ms_task),
                   plan_host_us=statistics.median(plan_times) * 1e6, one_kernel=bool(tabs["mixed_kernel"]),
                   algorithmic_bytes=work["bytes"], flop=work["flop"])
        log(f"[bench] {b.name}: {value:.1f} {unit} per step; tasks pass {achieved:.1f} {unit} = "
            f"{100 * roof['frac']:.1f}% of {bound} peak; max-bound {100 * res['max_bound']['frac_step']:.1f}% of step")
        return p, res

    b, work, conv, t = load(args.config)
    p, main_res = run(args.config, b, work, t)
    res = dict(metric=METRIC, value=main_res["value"], unit=main_res["unit"], n_gpus=1, steps=args.steps,
               warmup=args.warmup, ms_per_step=main_res["ms_per_step"], higher_is_better=True, scaling="weak",
               vs_baseline=None, dtype=b.dtype, data="synthetic",
               config=dict(workload=b.name, num_seqs=b.num_seqs, query_rows=b.num_rows,
                           q_heads=b.num_q_heads, kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                           block_size=16, kv_splits=b.num_kv_splits or "auto", cascade=args.cascade,
                           unique_kv_bytes=work["kv_bytes_unique"],
                           logical_kv_bytes=work["kv_bytes_logical"], flop=work["flop"],
                           algorithmic_bytes=work["bytes"], cache_flush_between_steps=not args.no_flush),
               roofline=main_res["roofline"],
               **{k: main_res[k] for k in ("tasks_ms", "merge_ms", "plan_host_us", "one_kernel", "gbs", "tflops",
                                           "max_bound")})
    kinds = {wl.seq_kind(int(n)) for n in b.q_len if n > 0}
    if len(kinds) > 1 and not args.no_class_breakdown:
        res["class_breakdown"] = class_breakdown(pm, b, make_plan_for, t["kp"], t["vp"], conv, dev, stream, args,
                                                 flush)
        alone = sum(c["ms_per_step"] for c in res["class_breakdown"].values())
        log(f"[bench] classes alone sum to {alone:.4f} ms/step; together {main_res['ms_per_step']:.4f} ms/step")
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(b, work)
        log(f"[bench] cpu baseline {res['cpu_baseline']['value']:.3f} {res['cpu_baseline']['unit']} "
            f"({res['cpu_baseline']['sample']})")
        res["cpu_baseline"]["per_core"] = per_core_oracle()
        log(f"[bench] oracle at one thread: {res['cpu_baseline']['per_core']}")
        if res["cpu_baseline"]["unit"] == res["unit"]:
            # the GPU step's rate over the oracle's, in the same unit
            res["cpu_baseline"]["gpu_ratio"] = res["value"] / res["cpu_baseline"]["value"]
    del t, p
    torch.cuda.empty_cache()
    if not args.no_configs:
        res["configs"] = {}
        for idx in (2, 3, 5):
            if idx == args.config:
                continue
            bi, wi, _, ti = load(idx)
            _, ri = run(idx, bi, wi, ti)
            res["configs"][str(idx)] = ri
            del ti
            torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
