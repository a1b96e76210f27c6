#!/usr/bin/env python3
"""Benchmark of one forward-pass step of the hot path on one MI355X.

A step = cb_slot_mapping + cb_cache_write + cb_paged_attention (planning prepass, decode/split-KV
and prefill kernels, log-sum-exp merge) over one synthetic packed batch, inputs resident in HBM.
Default workload: the Llama-3-8B-shaped decode batch (32 q-heads, 8 KV heads, head_dim 128,
block 16, 256 sequences with KV length uniform in [128, 4096], physical blocks shuffled).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N]

Prints ONE JSON line on stdout; progress goes to stderr.
value = algorithmic bytes of the step / step time (GB/s). The roofline object covers the
attention entry point's kernels, timed with HIP events on the stream they run on.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ragged paged-attn decode KV GB/s (% HBM peak) + mixed-batch tokens/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


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
    return {
        "T": T, "S": S,
        "kv_bytes": kv_bytes,
        "decode_kv_bytes": int((L[decode] * kv_tok).sum()),
        "attn_bytes": int(attn),
        "step_bytes": int(attn + write + slots),
        "attn_flops": int((4 * D * Hq * pairs).sum()),
        "prefill_flops": int((4 * D * Hq * pairs[~decode]).sum()),
    }


def traffic_from_profile(workload):
    """HBM bytes per attention call from committed rocprofv3 counter runs, if they were taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"paged_attention_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = open(os.path.join(ROOT, "ragged_paged_kv_amd", "csrc", "attention.hip"), "rb").read()
    if rec.get("attention_hip_sha256") != hashlib.sha256(src).hexdigest():
        return None
    return rec.get("bytes_per_call")


def cpu_baseline(batch, budget_s=20.0):
    """The oracle (numpy float64, test infrastructure) on this host's cores over a bounded sample
    of the same workload: slot mapping + cache write over the whole batch, attention over the
    first sequences that fit the time budget (estimated from a probe)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    sl = oracle.slot_mapping(batch.cu_seqlens_q, batch.kv_lens, batch.block_tables,
                             batch.block_size)
    kc, vc = oracle.cache_write(batch.k_cache, batch.v_cache, batch.k, batch.v, sl)
    t_write = time.perf_counter() - t0
    cu = batch.cu_seqlens_q
    Hkv, D = batch.num_kv_heads, batch.head_dim
    done_tokens = []
    t_attn = 0.0
    kv_bytes = 0
    s = 0
    while s < batch.num_seqs and t_attn < budget_s:
        hi = min(batch.num_seqs, s + 16)
        toks = list(range(int(cu[s]), int(cu[hi])))
        t1 = time.perf_counter()
        oracle.paged_attention(batch.q, cu, batch.kv_lens, batch.block_tables, kc, vc,
                               batch.scale, tokens=toks)
        t_attn += time.perf_counter() - t1
        kv_bytes += int(batch.kv_lens[s:hi].astype(np.int64).sum()) * 2 * Hkv * D * 2
        done_tokens += toks
        s = hi
    frac_seqs = s / batch.num_seqs
    # whole-step rate: attention over the sampled sequences, plus the write over the batch
    # scaled to the same fraction of sequences
    t_step = t_attn + t_write * frac_seqs
    return {
        "value": round(kv_bytes / t_step / 1e9, 4),
        "unit": "GB/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"numpy float64 oracle: slot mapping + cache write of all {batch.num_tokens} "
                   f"tokens ({t_write:.1f} s, counted pro rata) and attention of the first {s} of "
                   f"{batch.num_seqs} sequences ({t_attn:.1f} s, {kv_bytes / 1e9:.3f} GB of KV)"),
        "seconds": round(t_attn + t_write, 2),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--split", type=int, default=0, help="KV partition tokens (0 = library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        log(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
            "this hot path has no multi-GPU mode: run with --gpus 1.")
        sys.exit(2)

    import numpy as np
    import torch

    import ragged_paged_kv_amd as cb
    import synth

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    b = synth.make_config(args.config)
    log(f"[bench] generated {b.name} in {time.perf_counter() - t0:.1f} s: S={b.num_seqs} "
        f"T={b.num_tokens} sumL={int(b.kv_lens.sum())} blocks={b.num_blocks}")
    cb.cb_validate_batch(b.cu_seqlens_q, b.kv_lens, b.block_tables, None, b.block_size,
                         b.num_blocks, b.max_q_len, b.max_kv_len)
    w = work_of(b)

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
    split = cb.cb_paged_attention_split_tokens(b.num_seqs, b.num_kv_heads, b.max_kv_len, args.split)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        cb.cb_slot_mapping(cu, kvl, bt, slots, b.block_size, stream=stream)
        cb.cb_cache_write(k, v, slots, kc, vc, stream=stream)
        if ev is not None:
            ev[0].record(stream)
        cb.cb_paged_attention(q, cu, kvl, bt, kc, vc, out, b.scale, b.max_q_len, b.max_kv_len, ws,
                              kv_split_tokens=args.split, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed / args.steps * 1e3
    attn_ms = [e0.elapsed_time(e1) for e0, e1 in events]
    attn_avg_ms = sum(attn_ms) / len(attn_ms)
    attn_med_ms = sorted(attn_ms)[len(attn_ms) // 2]
    log(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step; attention avg {attn_avg_ms:.4f} ms "
        f"(median {attn_med_ms:.4f}, min {min(attn_ms):.4f}, max {max(attn_ms):.4f})")

    step_s = ms_per_step / 1e3
    if args.config in (2, 4):
        value = w["step_bytes"] / step_s / 1e9
        unit = "GB/s"
    else:
        value = w["T"] / step_s
        unit = "tokens/s"
    achieved = w["attn_bytes"] / (attn_avg_ms / 1e3) / 1e9
    traffic = traffic_from_profile(b.name)
    roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": b.name,
            "num_seqs": b.num_seqs, "num_tokens": b.num_tokens, "q_heads": b.num_q_heads,
            "kv_heads": b.num_kv_heads, "head_dim": b.head_dim, "block_size": b.block_size,
            "kv_tokens": int(b.kv_lens.sum()), "kv_split_tokens": int(split), "seed": b.seed,
            "step": "slot_mapping + cache_write + paged_attention",
        },
        "hbm_frac": round(w["step_bytes"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(w["T"] / step_s, 1),
        "attention_ms": round(attn_avg_ms, 5),
        "step_bytes": w["step_bytes"],
        "attention_bytes": w["attn_bytes"],
        "roofline": roof,
        "cpu_baseline": None,
    }
    if w["prefill_flops"]:
        res["prefill_flops"] = w["prefill_flops"]
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on the host cores ...")
        res["cpu_baseline"] = cpu_baseline(b)
        log(f"[bench] cpu baseline: {res['cpu_baseline']}")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
