#!/usr/bin/env python3
"""Benchmark of one forward-pass step of the hot path on one MI355X.

A step = slot mapping + cache write + paged attention over one synthetic packed batch, inputs
resident in HBM, as one call of cb_paged_attention_write (the cache write, with its slots computed
in place, runs beside the planning workgroup; then the decode/split-KV and prefill kernels and the
log-sum-exp merge); --separate times the same step as the three entry points cb_slot_mapping,
cb_cache_write, cb_paged_attention.
Default workload: the Llama-3-8B-shaped decode batch (32 q-heads, 8 KV heads, head_dim 128,
block 16, 256 sequences with KV length uniform in [128, 4096], physical blocks shuffled). The
other full-size workloads of the metric follow it in the same run, each as a sub-object with its
own roofline and oracle sample: "mixed_batch" (the same model shape, 64 decode tokens + 1984
prefill-chunk tokens), "long_context_decode" (16 sequences of 32K-128K keys, split-KV partitions
and the log-sum-exp merge) and "mixed_batch_70b" (64 q-heads / 8 KV heads, block 32, 8192 tokens:
128 decodes + chunked prefills, a 2048-token prefix shared by a quarter of the sequences).
The mixed workloads also carry "decode_sub_batch": the decode KV rate of their decode rows
alone (same cache and tables), over the whole attention call and over the decode kernel.
"executor_step" is the --graphs measurement below (a 16-sequence decode step through the native
step executor, waited for and back to back, with direct launches and with graph replay).
"stream_read" is the measured streaming-read rate of this GPU (cb_stream_read over 2 GiB), which
the decode rooflines are also reported against. The headline step runs the given W warm-up and
K timed steps; the further workloads, and the prefill roofline's chunks-alone launches, are timed
after 0.15 s of untimed launches, in the steady state of the GPU's clocks under sustained load
(the first launches after idle run up to 18% slower), with the first launches reported beside.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N]

Prints ONE JSON line on stdout; progress goes to stderr.
value = algorithmic bytes of the step / step time (GB/s) for the decode workloads, tokens/s for
the mixed ones. The roofline object covers the dominant kernel (the decode kernel, HBM-bound, or
the prefill-chunk kernel, MFMA-bound), timed with HIP events that the library records around
that kernel on the stream it runs on (cb_time_next_kernel): average, median, p10 and p90 over K
further steps (the K timed steps run with no events enqueued), and the median after reading a
1 GiB scratch buffer (no input left in any cache).

Block manager data path (its own JSON line, not the default run):
    python bench.py --blocks [--steps K] [--warmup W]
        cb_copy_blocks on a Llama-3-8B-shaped pool (32 layers, block 16, 8 KV heads, head_dim 128)
        copying one shared partial block per sequence of a 256-sequence batch, against the HBM
        roofline; the swap tier moving the same 256 blocks to a pinned host pool and back, against
        PCIe 5.0 x16 (64 GB/s a direction); the host block manager's cost per decode step and per
        prompt admission.

Step graphs (its own JSON line, not the default run):
    python bench.py --graphs [--steps K] [--warmup W]
        a small Llama-3-8B-shaped decode batch (16 sequences, KV length uniform in [256, 2048]),
        one step = metadata upload + slot mapping + cache write + paged attention, run eagerly
        through the Python binding and through the step-graph executor (one upload + one graph
        launch); wall time per step of back-to-back steps, and the GPU time per step.

Async steps (its own JSON line, not the default run):
    python bench.py --async [--steps K] [--warmup W]
        64 decoding sequences of the Llama-3-8B shape (KV 512-2048): the CPU builds each step with
        the block manager and the GPU runs carry-over + a stand-in embedding lookup + the attention
        step + a stand-in greedy sampler; steps/s with each step waited for (synchronous) and with
        step N+1 prepared and begun before step N's tokens are read (async).

Measurement helpers (not part of the timed run):
    python bench.py --copy-calibration            # plain device copy of known size, for counters
    python bench.py --traffic-summary FETCH WRITE CFETCH CWRITE [--config N]
        reads rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of this bench (FETCH, WRITE)
        and of the copy calibration (CFETCH, CWRITE) and writes the per-launch HBM traffic of the
        dominant kernel to profiles/.
"""
import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ragged paged-attn decode KV GB/s (% HBM peak) + mixed-batch tokens/s"
HBM_PEAK_GBS = 8000.0
PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction
BF16_PEAK_TFLOPS = 2500.0
DECODE_CONFIGS = (1, 2, 4)
COPY_BYTES = 2 << 30  # copy calibration: bytes read and bytes written


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_of(b):
    """Algorithmic bytes and FLOPs of one step (what the method must move or compute)."""
    import numpy as np
    bs, Hq, Hkv, D = b.block_size, b.num_q_heads, b.num_kv_heads, b.head_dim
    G = Hq // Hkv
    q = (b.cu_seqlens_q[1:] - b.cu_seqlens_q[:-1]).astype(np.int64)
    L = b.kv_lens.astype(np.int64)
    decode = q * G <= 16
    kv_tok = 2 * Hkv * D * 2                       # K + V bytes per KV token
    blocks = -(-L // bs)
    T = int(q.sum())
    S = b.num_seqs
    kv_bytes = int((L * kv_tok).sum())
    attn = (kv_bytes + 2 * T * Hq * D * 2            # q in, out
            + int(4 * blocks.sum()) + 4 * (2 * S + 1))  # tables, cu, kv_lens
    write = 2 * (2 * T * Hkv * D * 2) + 4 * T      # K/V rows read + written, slots read
    slots = 4 * T + 4 * T + 4 * (2 * S + 1)        # table entries read, slots written
    pairs = q * (L - q) + q * (q + 1) // 2         # unmasked (query, key) pairs
    # decode kernel alone: the decode rows' K/V, q and output rows, block-table entries
    dec_bytes = int((L[decode] * kv_tok).sum() + 2 * q[decode].sum() * Hq * D * 2
                    + 4 * blocks[decode].sum())
    # prefill kernel alone: each prefill row's K/V once, its q and output rows, table entries
    pre_bytes = int((L[~decode] * kv_tok).sum() + 2 * q[~decode].sum() * Hq * D * 2
                    + 4 * blocks[~decode].sum())
    return {
        "T": T, "S": S,
        "kv_bytes": kv_bytes,
        "decode_kernel_bytes": dec_bytes,
        "prefill_kernel_bytes": pre_bytes,
        "attn_bytes": int(attn),
        "step_bytes": int(attn + write + slots),
        "attn_flops": int((4 * D * Hq * pairs).sum()),
        "prefill_flops": int((4 * D * Hq * pairs[~decode]).sum()),
    }


def traffic_record_path(workload, op="paged_attention"):
    return os.path.join(ROOT, "profiles", f"{op}_{workload}_hbm_traffic.json")


def strip_comments(text):
    """C/C++ source without its comments, trailing blanks and blank lines: the code itself."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c in "\"'":  # string or character literal, escapes included
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    lines = (l.rstrip() for l in "".join(out).split("\n"))
    return "\n".join(l for l in lines if l)


def code_sha256(name="attention.hip"):
    """Hash of a kernel source's code (comments and blank lines do not count): counter records
    taken on one code hash stay valid across comment edits, and only there."""
    src = open(os.path.join(ROOT, "ragged_paged_kv_amd", "csrc", name), encoding="utf-8").read()
    return hashlib.sha256(strip_comments(src).encode()).hexdigest()


def traffic_from_profile(workload, op="paged_attention", source="attention.hip"):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counter runs, if they
    were taken on the current kernel code; else None."""
    path = traffic_record_path(workload, op)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("code_sha256") != code_sha256(source):
        return None
    return rec.get("bytes_per_launch")


def host_info():
    """CPU model (from /proc/cpuinfo) and the BLAS build numpy's oracle runs on."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    blas, threads = "", 0
    try:
        from threadpoolctl import threadpool_info
        for d in threadpool_info():
            if d.get("user_api") == "blas":
                blas = f"{d.get('internal_api', '')} {d.get('version', '')} ({d.get('threading_layer', '')})"
                threads = max(threads, int(d.get("num_threads", 1)))
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "blas": blas.strip(),
            "cores": threads or len(os.sched_getaffinity(0))}


def clock_from_profile(workload):
    """The prefill kernel's clock (GHz) and MFMA-busy fraction under its own load on this
    workload, from the committed SQ / GRBM counter run, if it was taken on the current kernel
    code; else None."""
    path = os.path.join(ROOT, "profiles", "prefill_kernel_mfma_busy.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("code_sha256") != code_sha256(rec.get("source", "attention.hip")):
        return None
    return rec.get("workloads", {}).get(workload)


def cpu_baseline(batch, budget_s=20.0, mixed=False):
    """The oracle (numpy float64, test infrastructure) on this host's cores over a bounded sample
    of the same workload: slot mapping + cache write over the whole batch, attention over a
    sample that fits the time budget. Decode workloads: the first sequences (GB/s of their KV).
    Mixed workloads: every k-th packed token, k chosen from a probe so that the sample fits the
    budget (tokens/s = sampled tokens / time, an unbiased estimate of the whole batch's rate)."""
    import numpy as np
    import oracle
    info = host_info()
    t0 = time.perf_counter()
    sl = oracle.slot_mapping(batch.cu_seqlens_q, batch.kv_lens, batch.block_tables,
                             batch.block_size)
    kc, vc = oracle.cache_write(batch.k_cache, batch.v_cache, batch.k, batch.v, sl)
    t_write = time.perf_counter() - t0
    cu = batch.cu_seqlens_q
    Hkv, D = batch.num_kv_heads, batch.head_dim
    T = batch.num_tokens

    def attend(toks):
        t1 = time.perf_counter()
        oracle.paged_attention(batch.q, cu, batch.kv_lens, batch.block_tables, kc, vc,
                               batch.scale, tokens=list(toks))
        return time.perf_counter() - t1

    if mixed:
        probe_stride = max(1, T // 32)
        t_probe = attend(range(0, T, probe_stride))
        per_token = t_probe / len(range(0, T, probe_stride))
        stride = max(1, int(np.ceil(T * per_token / budget_s)))
        toks = range(stride // 2, T, stride)
        t_attn = attend(toks)
        n = len(toks)
        t_step = t_attn + t_write * n / T
        return {
            "value": round(n / t_step, 1), "unit": "tokens/s", "cores": info["cores"],
            "kind": "oracle",
            "sample": (f"numpy float64 oracle: slot mapping + cache write of all {T} tokens "
                       f"({t_write:.1f} s, counted pro rata) and attention of every {stride}-th "
                       f"packed token ({n} of {T}, {t_attn:.1f} s)"),
            "seconds": round(t_attn + t_write + t_probe, 2),
            "cpu_model": info["cpu_model"], "blas": info["blas"],
        }
    t_attn = 0.0
    kv_bytes = 0
    s = 0
    while s < batch.num_seqs and t_attn < budget_s:
        hi = min(batch.num_seqs, s + (16 if batch.num_seqs > 64 else 1))
        t_attn += attend(range(int(cu[s]), int(cu[hi])))
        kv_bytes += int(batch.kv_lens[s:hi].astype(np.int64).sum()) * 2 * Hkv * D * 2
        s = hi
    frac_seqs = s / batch.num_seqs
    # whole-step rate: attention over the sampled sequences, plus the write over the batch
    # scaled to the same fraction of sequences
    t_step = t_attn + t_write * frac_seqs
    return {
        "value": round(kv_bytes / t_step / 1e9, 4),
        "unit": "GB/s",
        "cores": info["cores"],
        "kind": "oracle",
        "sample": (f"numpy float64 oracle: slot mapping + cache write of all {T} "
                   f"tokens ({t_write:.1f} s, counted pro rata) and attention of the first {s} of "
                   f"{batch.num_seqs} sequences ({t_attn:.1f} s, {kv_bytes / 1e9:.3f} GB of KV)"),
        "seconds": round(t_attn + t_write, 2),
        "cpu_model": info["cpu_model"], "blas": info["blas"],
    }


def unique_kv_bytes(b):
    """KV bytes of the distinct cache slots the batch reads (a block shared by several tables
    counts once)."""
    import numpy as np
    bs = b.block_size
    slots = []
    for s in range(b.num_seqs):
        p = np.arange(int(b.kv_lens[s]), dtype=np.int64)
        slots.append(b.block_tables[s][p // bs].astype(np.int64) * bs + p % bs)
    return int(np.unique(np.concatenate(slots)).size) * 2 * b.num_kv_heads * b.head_dim * 2


STREAM_BYTES = 2 << 30


def stream_ceiling(reps=10):
    """Measured streaming-read rate: a plain non-temporal 16-byte read of 2 GiB (cb_stream_read),
    median of `reps` launches, GB/s."""
    import torch
    import ragged_paged_kv_amd as cb
    buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device="cuda")
    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")
    cb.cb_stream_read(buf, sink)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        cb.cb_stream_read(buf, sink)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    med = pct(ms, 0.5)
    return {"gbs": round(STREAM_BYTES / (med / 1e3) / 1e9, 1), "bytes": STREAM_BYTES,
            "ms_median": round(med, 5), "kernel": "cb_stream_read (non-temporal 16-byte loads)"}


def pct(xs, q):
    """The q-quantile (0..1) of xs, nearest rank."""
    ys = sorted(xs)
    return ys[min(len(ys) - 1, max(0, round(q * (len(ys) - 1))))]


FLUSH_BYTES = 1 << 30  # larger than the 256 MB Infinity Cache and the L2s together
FLUSH_LAUNCHES = 8
# Untimed launches of the prefill chunks alone before their timed ones (seconds of GPU time):
# on MI355X the 70B-shaped chunks take 1.23 ms over the first 10 launches after idle and settle
# at 1.045 ms after about 30 ms of back-to-back launches.
PREFILL_WARM_S = 0.15
# Untimed steps (seconds of wall time) before the timed steps of the further workloads of the
# default run: the 70B-shaped mixed step takes 1.76-1.82 ms over its first steps and 1.64 ms in
# steady state.
SUB_WARM_S = 0.15


def measure(args, config, steps, warmup, warm_s=0.0):
    """Generate workload `config`, run warmup + timed steps; returns the batch, its work and the
    timings (step wall time, dominant kernel times from the library's events). warm_s > 0: after
    the warmup steps, further untimed steps until that much wall time has passed, so that the
    timed steps run at the clocks of sustained load."""
    import numpy as np
    import torch

    import ragged_paged_kv_amd as cb
    import synth

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    b = synth.make_config(config)
    log(f"[bench] generated {b.name} in {time.perf_counter() - t0:.1f} s: S={b.num_seqs} "
        f"T={b.num_tokens} sumL={int(b.kv_lens.sum())} blocks={b.num_blocks}")
    cb.cb_validate_batch(b.cu_seqlens_q, b.kv_lens, b.block_tables, None, b.block_size,
                         b.num_blocks, b.max_q_len, b.max_kv_len)
    w = work_of(b)
    kernel = cb.CB_KERNEL_DECODE if config in DECODE_CONFIGS else cb.CB_KERNEL_PREFILL

    def up_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def up_i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    q, k, v = up_bf16(b.q), up_bf16(b.k), up_bf16(b.v)
    kc, vc = up_bf16(b.k_cache), up_bf16(b.v_cache)
    cu, kvl, bt = up_i32(b.cu_seqlens_q), up_i32(b.kv_lens), up_i32(b.block_tables)
    slots = torch.empty(b.num_tokens, dtype=torch.int32, device=dev)
    out = torch.empty((b.num_tokens, b.num_q_heads, b.head_dim), dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(b.num_seqs, b.num_tokens, b.num_q_heads, b.num_kv_heads, b.head_dim,
                            b.block_size, b.max_q_len, b.max_kv_len, args.split, device=dev)
    split = cb.cb_paged_attention_split_tokens(b.num_seqs, b.num_q_heads, b.num_kv_heads,
                                               b.max_q_len, b.max_kv_len, args.split)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if args.separate:  # the three entry points one after the other
            cb.cb_slot_mapping(cu, kvl, bt, slots, b.block_size, stream=stream)
            cb.cb_cache_write(k, v, slots, kc, vc, stream=stream)
        if ev is not None:
            ev[0].record(stream)
            cb.cb_time_next_kernel(kernel, ev[2], ev[3], stream=stream)
        if args.separate:
            cb.cb_paged_attention(q, cu, kvl, bt, kc, vc, out, b.scale, b.max_q_len, b.max_kv_len,
                                  ws, kv_split_tokens=args.split, stream=stream)
        else:  # one call: the cache write runs beside the planning workgroup
            cb.cb_paged_attention_write(q, k, v, cu, kvl, bt, kc, vc, out, b.scale, b.max_q_len,
                                        b.max_kv_len, ws, kv_split_tokens=args.split, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    warm_steps = 0
    if warm_s > 0:
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < warm_s:
            for _ in range(8):
                step()
            warm_steps += 8
            torch.cuda.synchronize()
    # the K timed steps, with nothing but the step enqueued
    t_start = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    # K more steps with HIP events around the attention call and the dominant kernel
    events = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(steps)]
    for ev in events:  # create the events before the measured steps
        for e in ev:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    attn_ms = [e[0].elapsed_time(e[1]) for e in events]
    kern_ms = [e[2].elapsed_time(e[3]) for e in events]
    r = {
        "batch": b, "work": w, "split": split, "kernel": kernel,
        "ms_per_step": elapsed / steps * 1e3, "warm_steps": warm_steps,
        "attn_ms": sum(attn_ms) / len(attn_ms),
        "kernel_ms": sum(kern_ms) / len(kern_ms),
        "kernel_ms_median": pct(kern_ms, 0.5),
        "kernel_ms_p10": pct(kern_ms, 0.1), "kernel_ms_p90": pct(kern_ms, 0.9),
    }
    # Cache check, outside the timed steps: the same launch after reading a scratch buffer larger
    # than every cache, so that none of its inputs can still be cached from the previous launch.
    # A read, not a write: written lines would be dirty, and the measured kernel would pay for
    # writing them back to HBM as its own reads evict them.
    scratch = torch.ones(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
    sink = torch.empty((), dtype=torch.int64, device=dev)

    def flushed(launch):
        ms = []
        for i in range(FLUSH_LAUNCHES):
            torch.sum(scratch, dim=0, dtype=torch.int64, out=sink)
            ev = tuple(torch.cuda.Event(enable_timing=True) for _ in range(4))
            launch(ev)
            torch.cuda.synchronize()
            ms.append(ev[2].elapsed_time(ev[3]))
        return pct(ms, 0.5)

    if kernel == cb.CB_KERNEL_DECODE:
        r["kernel_ms_flushed"] = flushed(step)
    log(f"[bench] {b.name}: {steps} steps, {r['ms_per_step']:.4f} ms/step; attention "
        f"{r['attn_ms']:.4f} ms; {'decode' if kernel == cb.CB_KERNEL_DECODE else 'prefill'} kernel "
        f"avg {r['kernel_ms']:.4f} ms (median {r['kernel_ms_median']:.4f}, min {min(kern_ms):.4f}, "
        f"max {max(kern_ms):.4f})")
    if kernel == cb.CB_KERNEL_PREFILL:
        # In the step the decode kernel runs beside the prefill kernel and shares the GPU; the
        # MFMA roofline is taken on the batch's prefill chunks alone (same cache and tables).
        pre = np.nonzero((b.cu_seqlens_q[1:] - b.cu_seqlens_q[:-1]) * (b.num_q_heads // b.num_kv_heads) > 16)[0]
        rows = np.concatenate([np.arange(b.cu_seqlens_q[s], b.cu_seqlens_q[s + 1]) for s in pre])
        ql = (b.cu_seqlens_q[1:] - b.cu_seqlens_q[:-1])[pre]
        qs = q[torch.from_numpy(rows).to(dev)].contiguous()
        cus = up_i32(np.concatenate([[0], np.cumsum(ql)]))
        kvs, bts = up_i32(b.kv_lens[pre]), up_i32(b.block_tables[pre])
        outs = torch.empty((len(rows), b.num_q_heads, b.head_dim), dtype=torch.bfloat16, device=dev)
        mq, mkv = int(ql.max()), int(b.kv_lens[pre].max())
        wss = cb.alloc_workspace(len(pre), len(rows), b.num_q_heads, b.num_kv_heads, b.head_dim,
                                 b.block_size, mq, mkv, 0, device=dev)
        def timed_alone():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            cb.cb_time_next_kernel(kernel, e0, e1, stream=stream)
            cb.cb_paged_attention(qs, cus, kvs, bts, kc, vc, outs, b.scale, mq, mkv, wss,
                                  stream=stream)
            return e0, e1

        # The GPU's clocks ramp up over the first tens of milliseconds of sustained load: the
        # first launches after the host-side set-up are timed on their own ("cold"), then the
        # same launches run untimed for PREFILL_WARM_S before the timed ones, so that the
        # roofline is taken in the steady state that back-to-back serving steps run in.
        cold = [timed_alone() for _ in range(max(1, warmup))]
        torch.cuda.synchronize()
        cold_ms = [e0.elapsed_time(e1) for e0, e1 in cold]
        n_warm = min(20000, int(PREFILL_WARM_S * 1e3 / max(min(cold_ms), 1e-3)))
        for _ in range(n_warm):
            cb.cb_paged_attention(qs, cus, kvs, bts, kc, vc, outs, b.scale, mq, mkv, wss,
                                  stream=stream)
        iso = [timed_alone() for _ in range(steps)]
        torch.cuda.synchronize()
        iso_ms = [e0.elapsed_time(e1) for e0, e1 in iso]
        r["kernel_ms_cold"] = pct(cold_ms, 0.5)
        r["warm_launches"] = n_warm
        r["step_kernel_ms"] = r["kernel_ms"]
        r["kernel_ms"] = sum(iso_ms) / len(iso_ms)
        r["kernel_ms_median"] = pct(iso_ms, 0.5)
        r["kernel_ms_p10"], r["kernel_ms_p90"] = pct(iso_ms, 0.1), pct(iso_ms, 0.9)

        def alone(ev):
            cb.cb_time_next_kernel(kernel, ev[2], ev[3], stream=stream)
            cb.cb_paged_attention(qs, cus, kvs, bts, kc, vc, outs, b.scale, mq, mkv, wss,
                                  stream=stream)

        r["kernel_ms_flushed"] = flushed(alone)
        log(f"[bench] {b.name} prefill chunks alone ({len(pre)} sequences, {len(rows)} tokens): "
            f"prefill kernel avg {r['kernel_ms']:.4f} ms (min {min(iso_ms):.4f}, max {max(iso_ms):.4f}) "
            f"after {n_warm} untimed launches; the first {len(cold_ms)} after set-up: median "
            f"{r['kernel_ms_cold']:.4f} ms")
        # The batch's decode rows alone (same cache and tables): the decode KV rate of a mixed
        # batch, timed over the whole attention call (the merge included) and on its kernel.
        dec = np.nonzero((b.cu_seqlens_q[1:] - b.cu_seqlens_q[:-1]) * (b.num_q_heads // b.num_kv_heads) <= 16)[0]
        if len(dec):
            drows = np.concatenate([np.arange(b.cu_seqlens_q[s], b.cu_seqlens_q[s + 1]) for s in dec])
            dql = (b.cu_seqlens_q[1:] - b.cu_seqlens_q[:-1])[dec]
            qd = q[torch.from_numpy(drows).to(dev)].contiguous()
            cud = up_i32(np.concatenate([[0], np.cumsum(dql)]))
            kvd, btd = up_i32(b.kv_lens[dec]), up_i32(b.block_tables[dec])
            outd = torch.empty((len(drows), b.num_q_heads, b.head_dim), dtype=torch.bfloat16, device=dev)
            mqd, mkvd = int(dql.max()), int(b.kv_lens[dec].max())
            wsd = cb.alloc_workspace(len(dec), len(drows), b.num_q_heads, b.num_kv_heads, b.head_dim,
                                     b.block_size, mqd, mkvd, 0, device=dev)

            def dec_call(ev=None):
                if ev is not None:
                    ev[0].record(stream)
                    cb.cb_time_next_kernel(cb.CB_KERNEL_DECODE, ev[2], ev[3], stream=stream)
                cb.cb_paged_attention(qd, cud, kvd, btd, kc, vc, outd, b.scale, mqd, mkvd, wsd,
                                      stream=stream)
                if ev is not None:
                    ev[1].record(stream)

            for _ in range(max(2, warmup)):
                dec_call()
            dev_ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(steps)]
            for ev in dev_ev:
                dec_call(ev)
            torch.cuda.synchronize()
            call_ms = [e[0].elapsed_time(e[1]) for e in dev_ev]
            dk_ms = [e[2].elapsed_time(e[3]) for e in dev_ev]
            r["decode_alone"] = {"sequences": int(len(dec)), "tokens": int(len(drows)),
                                 "call_ms_median": pct(call_ms, 0.5), "kernel_ms_median": pct(dk_ms, 0.5),
                                 "call_ms_p10": pct(call_ms, 0.1), "call_ms_p90": pct(call_ms, 0.9)}
            log(f"[bench] {b.name} decode rows alone ({len(dec)} sequences): attention call median "
                f"{r['decode_alone']['call_ms_median']:.4f} ms, decode kernel median "
                f"{r['decode_alone']['kernel_ms_median']:.4f} ms")
    log(f"[bench] {b.name} {'decode' if kernel == cb.CB_KERNEL_DECODE else 'prefill'} kernel "
        f"p10 / median / p90 {r['kernel_ms_p10']:.4f} / {r['kernel_ms_median']:.4f} / "
        f"{r['kernel_ms_p90']:.4f} ms; after reading {FLUSH_BYTES >> 20} MiB to flush the caches (median of "
        f"{FLUSH_LAUNCHES}) {r['kernel_ms_flushed']:.4f} ms")
    return r


def roofline_of(r, stream_gbs=None):
    import ragged_paged_kv_amd as cb
    w, b = r["work"], r["batch"]
    sec = r["kernel_ms"] / 1e3
    if r["kernel"] == cb.CB_KERNEL_DECODE:
        achieved = w["decode_kernel_bytes"] / sec / 1e9
        extra = {}
        if stream_gbs:  # against the measured streaming-read ceiling of this GPU
            extra = {"stream_ceiling_gbs": stream_gbs, "frac_of_stream_ceiling": round(achieved / stream_gbs, 4)}
        return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile(b.name), "kernel": "decode_kernel",
                "kernel_ms": round(r["kernel_ms"], 5), "bytes_per_launch": w["decode_kernel_bytes"],
                **extra, **timing_of(r)}
    achieved = w["prefill_flops"] / sec / 1e12
    in_step = w["prefill_flops"] / (r["step_kernel_ms"] / 1e3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_from_profile(b.name), "kernel": "prefill_kernel",
            "kernel_ms": round(r["kernel_ms"], 5), "flops_per_launch": w["prefill_flops"],
            "timed_on": "the batch's prefill chunks alone, in steady state after "
                        f"{r['warm_launches']} untimed launches",
            # the first launches after the set-up, before the clocks have ramped up
            "kernel_ms_cold": round(r["kernel_ms_cold"], 5),
            "frac_cold": round(w["prefill_flops"] / (r["kernel_ms_cold"] / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "kernel_ms_in_step": round(r["step_kernel_ms"], 5),
            # the same kernel inside the whole step, where the decode kernel shares the GPU
            "frac_in_step": round(in_step / BF16_PEAK_TFLOPS, 4),
            # measured clock and MFMA-busy fraction under this load (committed counter run)
            "counters": clock_from_profile(b.name), **timing_of(r)}


def sub_result(args, config, stream_gbs, cpu_budget_s):
    """One further workload of the default run, as a sub-object of the JSON line: step time, the
    workload's metric, its dominant kernel's roofline and the oracle's rate on a sample."""
    # the further workloads are timed in steady state (the headline step keeps the given W and K)
    m = measure(args, config, max(5, args.steps // 2), max(2, args.warmup // 2), warm_s=SUB_WARM_S)
    b, w = m["batch"], m["work"]
    step_s = m["ms_per_step"] / 1e3
    mixed = config not in DECODE_CONFIGS
    out = {
        "workload": b.name, "num_tokens": b.num_tokens, "num_seqs": b.num_seqs,
        "kv_tokens": int(b.kv_lens.sum()), "kv_split_tokens": int(m["split"]), "seed": b.seed,
        "ms_per_step": round(m["ms_per_step"], 5),
        "untimed_steps_before": int(m["warm_steps"]) + max(2, args.warmup // 2),
        "tokens_per_s": round(w["T"] / step_s, 1),
        "step_gbs": round(w["step_bytes"] / step_s / 1e9, 3),
        "hbm_frac": round(w["step_bytes"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": roofline_of(m, stream_gbs),
    }
    if mixed:
        out["prefill_flops"] = w["prefill_flops"]
        if m.get("decode_alone"):
            out["decode_sub_batch"] = decode_sub_batch_of(m, stream_gbs)
    uniq = unique_kv_bytes(b)
    if uniq < w["kv_bytes"]:  # blocks shared by several sequences: bytes of distinct slots
        out["kv_bytes_logical"] = w["kv_bytes"]
        out["kv_bytes_unique"] = uniq
    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on the host cores ({b.name}) ...")
        out["cpu_baseline"] = cpu_baseline(b, cpu_budget_s, mixed=mixed)
        log(f"[bench] cpu baseline: {out['cpu_baseline']}")
    return out


def decode_sub_batch_of(r, stream_gbs=None):
    """The decode KV rate of a mixed batch's decode rows alone (reported, no target): the decode
    kernel's algorithmic bytes over the median time of the whole attention call (merge
    included), and over the decode kernel's own median time."""
    d, by = r["decode_alone"], r["work"]["decode_kernel_bytes"]
    gbs = by / (d["call_ms_median"] / 1e3) / 1e9
    kgbs = by / (d["kernel_ms_median"] / 1e3) / 1e9
    out = {"metric": "decode KV GB/s of the batch's decode rows alone (same cache and tables)",
           "sequences": d["sequences"], "tokens": d["tokens"], "bytes": by,
           "call_ms_median": round(d["call_ms_median"], 5),
           "call_ms_p10": round(d["call_ms_p10"], 5), "call_ms_p90": round(d["call_ms_p90"], 5),
           "gbs": round(gbs, 2), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
           "kernel_ms_median": round(d["kernel_ms_median"], 5), "kernel_gbs": round(kgbs, 2),
           "kernel_hbm_frac": round(kgbs / HBM_PEAK_GBS, 4)}
    if stream_gbs:
        out["kernel_frac_of_stream_ceiling"] = round(kgbs / stream_gbs, 4)
    return out


def timing_of(r):
    """Spread of the dominant kernel's launch times, and its median time after a cache flush."""
    return {k: round(r[k], 5) for k in ("kernel_ms_median", "kernel_ms_p10", "kernel_ms_p90",
                                        "kernel_ms_flushed")}


def copy_calibration():
    """A plain elementwise copy kernel (negation) over COPY_BYTES, five times: it reads and writes
    COPY_BYTES each, so its counters give the scale between FETCH_SIZE / WRITE_SIZE and bytes
    actually moved. (A same-dtype copy_ would be a DMA transfer, invisible to the counters.)"""
    import torch
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] copied {COPY_BYTES} bytes 5 times")


def _pmc_means(d, counter, name_part, last_group=False):
    """Mean of a counter per dispatch of the kernel named like name_part. last_group: only the
    final run of dispatches with the grid size of the last one (the prefill chunks alone, which
    the bench launches after the full steps and times for the MFMA roofline)."""
    import csv
    import collections
    vals = collections.defaultdict(list)
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    for f in files:
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] == counter and name_part in row["Kernel_Name"]:
                vals[row["Kernel_Name"]].append(
                    (int(row["Dispatch_Id"]), row["Grid_Size"], float(row["Counter_Value"])))
    if not vals:
        raise SystemExit(f"no {counter} rows for a kernel named like {name_part!r} under {d}")
    name, rows = max(vals.items(), key=lambda kv: sum(r[2] for r in kv[1]) / len(kv[1]))
    rows.sort()
    if last_group:
        grid = rows[-1][1]
        i = len(rows)
        while i > 0 and rows[i - 1][1] == grid:
            i -= 1
        rows = rows[i:]
    v = [r[2] for r in rows]
    return name, sum(v) / len(v), len(v)


def traffic_summary(args):
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = args.traffic_summary
    if args.blocks:
        workload, op, source = BLOCKS_WORKLOAD, "copy_blocks", "block_copy.hip"
        kname, alone, alg = "copy_blocks_kernel", False, blocks_launch_bytes()
        bench_flags = "--blocks --steps 5 --warmup 1 --no-cpu-baseline"
        measured = "every launch of the copy kernel"
    else:
        import synth
        b = synth.make_config(args.config)
        workload, op, source = b.name, "paged_attention", "attention.hip"
        kname = "decode_kernel" if args.config in DECODE_CONFIGS else "prefill_kernel"
        alone = kname == "prefill_kernel"
        w = work_of(b)
        alg = w["decode_kernel_bytes"] if kname == "decode_kernel" else w["prefill_kernel_bytes"]
        bench_flags = f"--config {args.config} --steps 5 --warmup 2 --no-cpu-baseline --no-mixed"
        measured = ("the prefill chunks alone (the launches the MFMA roofline times)" if alone
                    else "every launch of the decode kernel")
    kn, fetch_kib, nf = _pmc_means(fetch_dir, "FETCH_SIZE", kname, last_group=alone)
    _, write_kib, nw = _pmc_means(write_dir, "WRITE_SIZE", kname, last_group=alone)
    cn, cfetch_kib, _ = _pmc_means(cfetch_dir, "FETCH_SIZE", "")
    _, cwrite_kib, _ = _pmc_means(cwrite_dir, "WRITE_SIZE", cn[:40])
    f_fetch = COPY_BYTES / 1024 / cfetch_kib
    f_write = COPY_BYTES / 1024 / cwrite_kib
    fetch_b = fetch_kib * 1024 * f_fetch
    write_b = write_kib * 1024 * f_write
    rec = {
        "workload": workload, "kernel": kn, "source": source, "code_sha256": code_sha256(source),
        "fetch_kib_per_launch": round(fetch_kib, 1), "write_kib_per_launch": round(write_kib, 1),
        "launches": [nf, nw], "launches_measured": measured,
        "copy_kernel": cn, "copy_bytes": COPY_BYTES,
        "copy_fetch_kib": round(cfetch_kib, 1), "copy_write_kib": round(cwrite_kib, 1),
        "fetch_scale": round(f_fetch, 5), "write_scale": round(f_write, 5),
        "bytes_per_launch": int(fetch_b + write_b),
        "algorithmic_bytes_per_launch": alg,
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o p --output-format csv -- python3 bench.py {bench_flags}",
            f"rocprofv3 --pmc WRITE_SIZE -d {write_dir} -o p --output-format csv -- python3 bench.py {bench_flags}",
            f"rocprofv3 --pmc FETCH_SIZE -d {cfetch_dir} -o p --output-format csv -- python3 bench.py --copy-calibration",
            f"rocprofv3 --pmc WRITE_SIZE -d {cwrite_dir} -o p --output-format csv -- python3 bench.py --copy-calibration",
            "python3 bench.py --traffic-summary " + " ".join(args.traffic_summary)
            + (" --blocks" if args.blocks else f" --config {args.config}"),
        ],
    }
    path = traffic_record_path(workload, op)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


BLOCKS_SHAPE = dict(layers=32, num_blocks=4096, block_size=16, kv_heads=8, head_dim=128, pairs=256)
BLOCKS_WORKLOAD = "cow-copy-llama3-8b-shape"


def blocks_launch_bytes():
    """Algorithmic bytes of one copy launch: every pair reads and writes one block of K and one of
    V in every layer."""
    sh = BLOCKS_SHAPE
    block_bytes = sh["block_size"] * sh["kv_heads"] * sh["head_dim"] * 2
    return 2 * sh["pairs"] * sh["layers"] * 2 * block_bytes


def bench_blocks(args):
    """cb_copy_blocks throughput and host manager cost; prints one JSON line."""
    import numpy as np
    import torch
    import ragged_paged_kv_amd as cb
    sh = BLOCKS_SHAPE
    L, NB, bs, hkv, d, n = (sh[k] for k in ("layers", "num_blocks", "block_size", "kv_heads",
                                            "head_dim", "pairs"))
    block_bytes = bs * hkv * d * 2
    shape = (L, NB, bs, hkv, d)
    kc = torch.randn(shape, dtype=torch.bfloat16, device="cuda")
    vc = torch.randn(shape, dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(5)
    ids = rng.permutation(NB)
    src = torch.from_numpy(ids[:n].astype(np.int32)).cuda()
    dst = torch.from_numpy(ids[n:2 * n].astype(np.int32)).cuda()
    launch_bytes = blocks_launch_bytes()
    for _ in range(args.warmup):
        cb.cb_copy_blocks(kc, vc, src, dst, num_layers=L)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        cb.cb_copy_blocks(kc, vc, src, dst, num_layers=L)
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    ok = torch.equal(kc[:, dst.long()], kc[:, src.long()]) and torch.equal(vc[:, dst.long()],
                                                                           vc[:, src.long()])
    gbs = launch_bytes / (ms / 1e3) / 1e9
    log(f"[bench] copy_blocks: {ms * 1e3:.1f} us per launch, {gbs:.0f} GB/s, copies intact: {ok}")

    # swap tier: the same 256 blocks (all layers, K and V: 512 MiB) to a pinned host pool and back
    pool = torch.empty((n, 2, L, bs, hkv, d), dtype=torch.bfloat16, pin_memory=True)
    slots = torch.arange(n, dtype=torch.int32, device="cuda")
    swap_bytes = n * L * 2 * block_bytes

    def time_launch(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out_ms = time_launch(lambda: cb.cb_swap_out_blocks(kc, vc, src, slots, pool, num_layers=L))
    in_ms = time_launch(lambda: cb.cb_swap_in_blocks(pool, slots, dst, kc, vc, num_layers=L))
    swap_ok = torch.equal(kc[:, dst.long()].cpu(), pool[:, 0].transpose(0, 1)) and \
        torch.equal(vc[:, dst.long()].cpu(), pool[:, 1].transpose(0, 1))
    flat = torch.empty(swap_bytes // 2, dtype=torch.bfloat16, device="cuda")
    flat_host = pool.view(-1)
    dma_d2h = time_launch(lambda: flat_host.copy_(flat, non_blocking=True))
    dma_h2d = time_launch(lambda: flat.copy_(flat_host, non_blocking=True))
    out_gbs, in_gbs = swap_bytes / out_ms / 1e6, swap_bytes / in_ms / 1e6
    log(f"[bench] swap: out {out_ms:.2f} ms {out_gbs:.1f} GB/s, in {in_ms:.2f} ms {in_gbs:.1f} GB/s "
        f"({swap_bytes} bytes each, blocks intact: {swap_ok}); a contiguous DMA copy of the same "
        f"size: to host {swap_bytes / dma_d2h / 1e6:.1f} GB/s, to device {swap_bytes / dma_h2d / 1e6:.1f} GB/s")

    # host manager: a 256-sequence decode step (append one token each, build the batch, take the
    # copies) and the admission of a 2048-token prompt whose first 1536 tokens are cached
    m = cb.BlockManager(1 << 16, bs)
    S = 256
    for s_ in range(S):
        m.add_sequence(s_, rng.integers(0, 32000, int(rng.integers(128, 4096))).tolist())
    pend = [m.sequence_info(s_)[0] for s_ in range(S)]
    m.build_batch(list(range(S)), pend, 512)
    m.take_copies()
    reps = 200
    t0 = time.perf_counter()
    ids, ones = np.arange(S, dtype=np.int64), np.ones(S, np.int32)
    bufs = (np.zeros(S + 1, np.int32), np.zeros(S, np.int32), np.full((S, 512), -1, np.int32),
            np.zeros(S, np.int32), np.zeros(S, np.int32))
    for r in range(reps):
        m.append_batch(ids, ones, np.full(S, r, np.int32))
        m.build_batch(ids, ones, 512, out=bufs)
        m.take_copies()
    step_us = (time.perf_counter() - t0) / reps * 1e6
    system = rng.integers(0, 32000, 1536).tolist()
    m.add_sequence(10_000, system + [1] * 512)
    m.build_batch([10_000], [2048], 512)
    m.take_copies()
    t0 = time.perf_counter()
    for r in range(reps):
        hit = m.add_sequence(20_000 + r, system + rng.integers(0, 32000, 512).tolist())
    admit_us = (time.perf_counter() - t0) / reps * 1e6
    log(f"[bench] manager: decode step of {S} sequences {step_us:.0f} us, admission {admit_us:.0f} us "
        f"(cached {hit} of 2048)")

    cpu = None
    if not args.no_cpu_baseline:   # the oracle's copy on the host cores, on a sample of the pairs
        import oracle.blocks as ob
        kh = kc[:, :64].view(torch.int16).cpu().numpy()
        vh = vc[:, :64].view(torch.int16).cpu().numpy()
        sp = np.arange(16, dtype=np.int32)
        dp = np.arange(16, 32, dtype=np.int32)
        t0 = time.perf_counter()
        it = 0
        while time.perf_counter() - t0 < 10.0:
            ob.copy_blocks(kh, vh, sp, dp)
            it += 1
        cpu_s = (time.perf_counter() - t0) / it
        cpu = {"value": round(2 * 16 * L * 2 * block_bytes / cpu_s / 1e9, 3), "unit": "GB/s",
               "cores": 1, "kind": "oracle",
               "sample": f"oracle copy_blocks, 16 pairs x {L} layers, {it} runs"}
    res = {
        "metric": "copy-on-write block copy GB/s (% HBM peak)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": BLOCKS_WORKLOAD, "layers": L, "num_blocks": NB,
                   "block_size": bs, "kv_heads": hkv, "head_dim": d, "pairs": n,
                   "block_bytes_per_layer_tensor": block_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_from_profile(BLOCKS_WORKLOAD, "copy_blocks", "block_copy.hip"),
                     "kernel": "copy_blocks_kernel", "kernel_ms": round(ms, 5),
                     "bytes_per_launch": launch_bytes},
        "wall_ms_per_launch": round(wall * 1e3, 5),
        "copies_verified": bool(ok),
        "swap": {
            "bytes_per_transfer": swap_bytes, "blocks_intact": bool(swap_ok),
            "out": {"bound": "pcie", "achieved": round(out_gbs, 2), "peak": PCIE_PEAK_GBS,
                    "unit": "GB/s", "frac": round(out_gbs / PCIE_PEAK_GBS, 4),
                    "kernel": "swap_blocks_kernel<true>", "kernel_ms": round(out_ms, 4)},
            "in": {"bound": "pcie", "achieved": round(in_gbs, 2), "peak": PCIE_PEAK_GBS,
                   "unit": "GB/s", "frac": round(in_gbs / PCIE_PEAK_GBS, 4),
                   "kernel": "swap_blocks_kernel<false>", "kernel_ms": round(in_ms, 4)},
            "dma_contiguous_gbs": {"to_host": round(swap_bytes / dma_d2h / 1e6, 2),
                                   "to_device": round(swap_bytes / dma_h2d / 1e6, 2)},
        },
        "host_manager": {"decode_step_us_256_seqs": round(step_us, 1),
                         "admission_us_2048_tokens_1536_cached": round(admit_us, 1)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


GRAPHS_SHAPE = dict(seqs=16, q_heads=32, kv_heads=8, head_dim=128, block_size=16, kv_lo=256,
                    kv_hi=2048)


def bench_graphs(args):
    """Eager vs recorded steps on a launch-bound decode batch; prints one JSON line."""
    print(json.dumps(graphs_result(args)), flush=True)


def graphs_result(args):
    """The step-graph measurement as a dict (its own JSON line, or the default run's
    "executor_step" sub-object)."""
    import numpy as np
    import torch
    import ragged_paged_kv_amd as cb
    sh = GRAPHS_SHAPE
    S, Hq, Hkv, D, bs = (sh[k] for k in ("seqs", "q_heads", "kv_heads", "head_dim", "block_size"))
    rng = np.random.default_rng(7)
    kv = rng.integers(sh["kv_lo"], sh["kv_hi"] + 1, S).astype(np.int32)
    MB = -(-sh["kv_hi"] // bs)
    nblk = -(-kv // bs)
    NB = int(nblk.sum()) + 64
    perm = rng.permutation(NB)
    tables = np.full((S, MB), -1, np.int32)
    o = 0
    for i in range(S):
        tables[i, :nblk[i]] = perm[o:o + nblk[i]]
        o += nblk[i]
    cu = np.arange(S + 1, dtype=np.int32)
    T, scale = S, 1.0 / np.sqrt(D)
    dev = "cuda"
    kc = torch.randn((NB, bs, Hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.randn_like(kc)
    maxT = 64
    q = torch.randn((maxT, Hq, D), dtype=torch.bfloat16, device=dev)
    k = torch.randn((maxT, Hkv, D), dtype=torch.bfloat16, device=dev)
    v = torch.randn_like(k)
    out = torch.empty_like(q)
    stream = torch.cuda.Stream()
    pin = [torch.from_numpy(a).pin_memory() for a in (cu, kv, tables)]
    dmeta = [torch.empty_like(t, device=dev) for t in pin]
    slots = torch.empty(T, dtype=torch.int32, device=dev)
    ws = cb.alloc_workspace(S, T, Hq, Hkv, D, bs, 1, int(kv.max()))

    def eager():
        for h, d in zip(pin, dmeta):
            d.copy_(h, non_blocking=True)
        cb.cb_slot_mapping(dmeta[0], dmeta[1], dmeta[2], slots, bs)
        cb.cb_cache_write(k[:T], v[:T], slots, kc, vc)
        cb.cb_paged_attention(q[:T], dmeta[0], dmeta[1], dmeta[2], kc, vc, out[:T], scale, 1,
                              int(kv.max()), ws)

    g = cb.StepGraphs(q, k, v, out, kc, vc, scale, max_seqs=S + 8, max_kv_len=MB * bs,
                      max_blocks_per_seq=MB, use_graphs=True)
    gd = cb.StepGraphs(q, k, v, out, kc, vc, scale, max_seqs=S + 8, max_kv_len=MB * bs,
                       max_blocks_per_seq=MB, use_graphs=False)

    def graph():
        g.run(cu, kv, tables, stream=stream)

    def direct():
        gd.run(cu, kv, tables, stream=stream)

    # the graph's padded shape, run eagerly: separates the cost of padding from that of replay
    shape = g.run(cu, kv, tables, stream=stream)
    stream.synchronize()
    Sb, Tb, mqb, mkvb = shape
    pcu = np.concatenate([cu, np.full(Sb - S, Tb)]).astype(np.int32)
    pkv = np.concatenate([kv, np.zeros(Sb - S)]).astype(np.int32)
    ptab = np.concatenate([tables, np.full((Sb - S, MB), -1)]).astype(np.int32)
    ppin = [torch.from_numpy(a).pin_memory() for a in (pcu, pkv, ptab)]
    pdev = [torch.empty_like(t, device=dev) for t in ppin]
    pslots = torch.empty(Tb, dtype=torch.int32, device=dev)
    pws = cb.alloc_workspace(Sb, Tb, Hq, Hkv, D, bs, mqb, mkvb)

    def eager_padded():
        for h, d in zip(ppin, pdev):
            d.copy_(h, non_blocking=True)
        cb.cb_slot_mapping(pdev[0], pdev[1], pdev[2], pslots, bs)
        cb.cb_cache_write(k[:Tb], v[:Tb], pslots, kc, vc)
        cb.cb_paged_attention(q[:Tb], pdev[0], pdev[1], pdev[2], kc, vc, out[:Tb], scale, mqb, mkvb,
                              pws)

    def timed(fn):
        """(synchronous: wall ms per step when every step is waited for, as an engine that needs
        the step's output before it can build the next; back-to-back: wall ms per step with no
        wait between steps, and the stream's span per step)"""
        for _ in range(max(args.warmup, 3)):
            fn()
        stream.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
            stream.synchronize()
        sync_ms = (time.perf_counter() - t0) / args.steps * 1e3
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        stream.synchronize()
        b2b_ms = (time.perf_counter() - t0) / args.steps * 1e3
        return {"sync_ms_per_step": round(sync_ms, 5), "back_to_back_ms_per_step": round(b2b_ms, 5),
                "stream_ms_per_step": round(a.elapsed_time(b) / args.steps, 5)}

    with torch.cuda.stream(stream):
        e = timed(eager)
        ref = out[:T].clone()
        ep = timed(eager_padded)
        gr = timed(graph)
        diff = float((out[:T].float() - ref.float()).abs().max())
        di = timed(direct)
        diff = max(diff, float((out[:T].float() - ref.float()).abs().max()))
    captures, replays, eager_runs, cached = g.stats()
    log(f"[bench] steps (synchronous / back to back, us): python calls {e['sync_ms_per_step'] * 1e3:.1f} / "
        f"{e['back_to_back_ms_per_step'] * 1e3:.1f}, python calls padded {ep['sync_ms_per_step'] * 1e3:.1f} / "
        f"{ep['back_to_back_ms_per_step'] * 1e3:.1f}, executor direct {di['sync_ms_per_step'] * 1e3:.1f} / "
        f"{di['back_to_back_ms_per_step'] * 1e3:.1f}, executor graphs {gr['sync_ms_per_step'] * 1e3:.1f} / "
        f"{gr['back_to_back_ms_per_step'] * 1e3:.1f}; max |executor - python| {diff:.3g}; "
        f"captures {captures} replays {replays}")
    g.close()
    gd.close()
    g_wall = min(gr["sync_ms_per_step"], di["sync_ms_per_step"])
    res = {
        "metric": "synchronous decode steps/s through the native step executor (small batch)",
        "value": round(1e3 / g_wall, 1), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(g_wall, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3-8b-decode-16seq-graphs", "num_seqs": S, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "block_size": bs,
                   "kv_tokens": int(kv.sum()),
                   "step": "metadata upload + slot_mapping + cache_write + paged_attention"},
        "timing": "synchronous steps (each waited for); value = the faster executor mode's steps/s",
        "python_calls": e, "python_calls_padded": ep, "executor_direct": di,
        "executor_graphs": dict(gr, captures=captures, replays=replays),
        "speedup_sync": round(e["sync_ms_per_step"] / g_wall, 3),
        "max_abs_diff_vs_eager": diff,
        "roofline": None,
        "cpu_baseline": None,
    }
    return res


ASYNC_SHAPE = dict(seqs=64, q_heads=32, kv_heads=8, head_dim=128, block_size=16, kv_lo=512,
                   kv_hi=2048, vocab=32000)


def bench_async(args):
    """Synchronous vs async steps through the async runtime; prints one JSON line."""
    import numpy as np
    import torch
    import ragged_paged_kv_amd as cb
    sh = ASYNC_SHAPE
    S, Hq, Hkv, D, bs, V = (sh[k] for k in ("seqs", "q_heads", "kv_heads", "head_dim",
                                            "block_size", "vocab"))
    steps = args.steps
    rng = np.random.default_rng(11)
    lens = rng.integers(sh["kv_lo"], sh["kv_hi"] + 1, S)
    MB = -(-(sh["kv_hi"] + 2 * (steps + args.warmup) + 8) // bs)
    NB = S * MB + 64
    dev = "cuda"
    kc = torch.randn((NB, bs, Hkv, D), dtype=torch.bfloat16, device=dev)
    vc = torch.randn_like(kc)
    T = 64
    q = torch.zeros((T, Hq, D), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((T, Hkv, D), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    out = torch.zeros_like(q)
    eq = torch.randn((V, Hq, D), dtype=torch.bfloat16, device=dev)
    ekv = torch.randn((V, Hkv, D), dtype=torch.bfloat16, device=dev)
    scale = 1.0 / np.sqrt(D)

    def run(async_mode):
        m = cb.BlockManager(NB, bs)
        for i in range(S):   # prompts whose KV is taken as computed (the cache holds random KV)
            m.add_sequence(i, rng.integers(0, V, int(lens[i])).tolist())
        ids = np.arange(S, dtype=np.int64)
        ones = np.ones(S, np.int32)
        m.build_batch(ids, lens.astype(np.int32), MB)
        m.take_copies()
        bufs = (np.zeros(S + 1, np.int32), np.zeros(S, np.int32), np.full((S, MB), -1, np.int32),
                np.zeros(S, np.int32), np.zeros(S, np.int32))
        a = cb.AsyncSteps(q, k, v, out, kc, vc, scale, max_seqs=S + 8, max_kv_len=MB * bs,
                          max_blocks_per_seq=MB)
        tokens = np.zeros(S, np.int32)
        dest = np.arange(S, dtype=np.int32)
        pending = None
        t_start = None
        for n in range(steps + args.warmup):
            if n == args.warmup:
                torch.cuda.synchronize()
                t_start = time.perf_counter()
            # CPU preparation of step n: the manager appends each sequence's next token (known in
            # the synchronous loop, a placeholder in the async one) and builds the batch
            m.append_batch(ids, ones, tokens if not async_mode else None)
            cu, kv, tables, _, _ = m.build_batch(ids, ones, MB, out=bufs)
            m.take_copies()
            slot = a.slot()
            a.in_ids_host[slot][:S].copy_(torch.from_numpy(tokens if not async_mode else np.zeros(S, np.int32)))
            carried = S if (async_mode and n > 0) else 0
            if carried:
                a.carry_dest_host[slot][:S].copy_(torch.from_numpy(dest))
            st = a.begin(cu, kv, tables, carried)
            with torch.cuda.stream(st):
                i = a.in_ids[slot][:S].long()
                q[:S].copy_(eq[i])
                k[:S].copy_(ekv[i])
                v[:S].copy_(ekv[i])
            a.attention()
            with torch.cuda.stream(st):
                a.out_ids[slot][:S].copy_((out[:S].float().sum(dim=1).argmax(dim=1) % V).to(torch.int32))
            a.end(S)
            if async_mode:
                if pending is not None:                 # the previous step's tokens
                    a.wait(pending)
                    tokens = a.out_ids_host[pending][:S].numpy().copy()
                    m.confirm_batch(ids, ones, tokens)  # the placeholders get their values
                pending = slot
            else:
                a.wait(slot)
                tokens = a.out_ids_host[slot][:S].numpy().copy()
        if pending is not None:
            a.wait(pending)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t_start) / steps * 1e3
        a.close()
        return ms

    sync_ms = run(False)
    async_ms = run(True)
    log(f"[bench] async steps: synchronous {sync_ms * 1e3:.1f} us/step, async {async_ms * 1e3:.1f} us/step "
        f"({sync_ms / async_ms:.2f}x)")
    res = {
        "metric": "decode steps/s with async steps (CPU prepares step N+1 during step N)",
        "value": round(1e3 / async_ms, 1), "unit": "steps/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": round(async_ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama3-8b-decode-64seq-async", "num_seqs": S, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "block_size": bs,
                   "step": "block manager prep + carry-over + stand-in embedding + attention step "
                           "+ stand-in sampler"},
        "synchronous_ms_per_step": round(sync_ms, 5), "async_ms_per_step": round(async_ms, 5),
        "speedup": round(sync_ms / async_ms, 3),
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--split", type=int, default=0, help="KV partition tokens (0 = library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mixed", action="store_true",
                    help="measure only --config (skip the other workloads of the default run)")
    ap.add_argument("--separate", action="store_true",
                    help="time the step as cb_slot_mapping + cb_cache_write + cb_paged_attention "
                         "(default: cb_paged_attention_write, the same work in one call)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--traffic-summary", nargs=4, metavar="DIR")
    ap.add_argument("--blocks", action="store_true", help="block copy and host manager measurement")
    ap.add_argument("--graphs", action="store_true", help="eager vs recorded steps, small decode batch")
    ap.add_argument("--async", dest="async_steps", action="store_true",
                    help="synchronous vs async steps with the block manager")
    args = ap.parse_args()

    if args.traffic_summary:
        traffic_summary(args)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
            "this hot path has no multi-GPU mode: run with --gpus 1.")
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.blocks:
        bench_blocks(args)
        return
    if args.graphs:
        bench_graphs(args)
        return
    if args.async_steps:
        bench_async(args)
        return

    stream = stream_ceiling()
    log(f"[bench] streaming-read ceiling: {stream['gbs']} GB/s ({stream['bytes']} bytes, median of 10)")
    r = measure(args, args.config, args.steps, args.warmup)
    b, w = r["batch"], r["work"]
    step_s = r["ms_per_step"] / 1e3
    if args.config in DECODE_CONFIGS:
        value, unit = w["step_bytes"] / step_s / 1e9, "GB/s"
    else:
        value, unit = w["T"] / step_s, "tokens/s"
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": b.name,
            "num_seqs": b.num_seqs, "num_tokens": b.num_tokens, "q_heads": b.num_q_heads,
            "kv_heads": b.num_kv_heads, "head_dim": b.head_dim, "block_size": b.block_size,
            "kv_tokens": int(b.kv_lens.sum()), "kv_split_tokens": int(r["split"]), "seed": b.seed,
            "step": ("slot_mapping + cache_write + paged_attention" if args.separate else
                     "paged_attention_write (slot mapping + cache write + paged attention)"),
        },
        "hbm_frac": round(w["step_bytes"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(w["T"] / step_s, 1),
        "attention_ms": round(r["attn_ms"], 5),
        "step_bytes": w["step_bytes"],
        "attention_bytes": w["attn_bytes"],
        "roofline": roofline_of(r, stream["gbs"]),
        "cpu_baseline": None,
        "stream_read": stream,
    }
    if w["prefill_flops"]:
        res["prefill_flops"] = w["prefill_flops"]
    if r.get("decode_alone"):
        res["decode_sub_batch"] = decode_sub_batch_of(r, stream["gbs"])
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores ...")
        res["cpu_baseline"] = cpu_baseline(b, mixed=args.config not in DECODE_CONFIGS)
        log(f"[bench] cpu baseline: {res['cpu_baseline']}")
    if args.config == 2 and not args.no_mixed:
        # the other full-size workloads of the metric, each as its own sub-object
        res["mixed_batch"] = sub_result(args, 3, stream["gbs"], 8.0)
        res["long_context_decode"] = sub_result(args, 4, stream["gbs"], 8.0)
        res["mixed_batch_70b"] = sub_result(args, 5, stream["gbs"], 8.0)
        # the small launch-bound decode step through the native step executor
        res["executor_step"] = graphs_result(args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
