"""GPU parity of the step-graph executor: every step (first eager run, recording, replay, replay
after eviction and after the workspace grows) must give outputs and caches bit-identical to the
same padded step run eagerly through the C ABI, with eager work and synchronisations between
replays; some steps are also checked against the oracle on the unpadded batch."""
import numpy as np
import pytest

import oracle
from gpu_helpers import dev_bf16, dev_i32, host_u16, say
from serving_helpers import rand_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
cb = pytest.importorskip("ragged_paged_kv_amd")

HQ, HKV, D, BS, NB, MB = 8, 2, 128, 16, 2048, 128
MAX_T, MAX_S, MAX_KV = 512, 24, MB * BS


def make_step(rng, qs, kv_range):
    """Host metadata for sequences with q lengths qs: KV lengths in kv_range (at least q), tables
    of distinct blocks drawn from the pool."""
    S = len(qs)
    kv = np.array([max(q, int(rng.integers(*kv_range))) for q in qs], np.int32)
    kv[-1] = max(qs[-1], kv_range[1] - 1)   # the longest KV fixes the padded KV bucket
    cu = np.concatenate([[0], np.cumsum(qs)]).astype(np.int32)
    tables = np.full((S, MB), -1, np.int32)
    perm = rng.permutation(NB)
    o = 0
    for s in range(S):
        n = -(-int(kv[s]) // BS)
        tables[s, :n] = perm[o:o + n]
        o += n
    return cu, kv, tables


def padded(cu, kv, tables, shape):
    Sb, Tb = shape[0], shape[1]
    S = kv.size
    cup = np.concatenate([cu, np.full(Sb - S, Tb)]).astype(np.int32)
    kvp = np.concatenate([kv, np.zeros(Sb - S)]).astype(np.int32)
    tp = np.concatenate([tables, np.full((Sb - S, MB), -1)]).astype(np.int32)
    return cup, kvp, tp


STEPS = [  # (name, q lengths, kv range, oracle check)
    ("decode-8", [1] * 8, (64, 700), True),
    ("decode-8", [1] * 8, (64, 700), False),      # recorded
    ("decode-8", [1] * 8, (64, 700), True),       # replayed
    ("mixed", [1] * 6 + [40, 70], (80, 900), True),
    ("mixed", [1] * 6 + [40, 70], (80, 900), False),
    ("decode-8", [1] * 8, (64, 700), False),
    ("decode-12-long", [1] * 12, (900, 1500), False),
    ("decode-12-long", [1] * 12, (900, 1500), False),   # evicts the least recent (max_graphs 2)
    ("mixed", [1] * 6 + [40, 70], (80, 900), True),     # recorded again
    ("prefill-big", [300, 150, 1], (300, 1200), True),  # more workspace: graphs dropped
    ("prefill-big", [300, 150, 1], (300, 1200), False),
    ("decode-8", [1] * 8, (64, 700), True),
    ("decode-8", [1] * 8, (64, 700), False),
    ("prefill-big", [300, 150, 1], (300, 1200), True),
]


@pytest.mark.parametrize("use_graphs", [True, False])
def test_step_graphs_match_eager_and_oracle(use_graphs):
    rng = np.random.default_rng(11)
    dev = "cuda"
    scale = 1.0 / np.sqrt(D)
    kc0, vc0 = rand_bf16(rng, (NB, BS, HKV, D)), rand_bf16(rng, (NB, BS, HKV, D))
    q = torch.zeros((MAX_T, HQ, D), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((MAX_T, HKV, D), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    out = torch.zeros_like(q)
    kc, vc = dev_bf16(kc0, dev), dev_bf16(vc0, dev)           # the executor's caches
    ekc, evc = dev_bf16(kc0, dev), dev_bf16(vc0, dev)         # the eager reference's caches
    eout = torch.zeros_like(q)
    eslots = torch.zeros(MAX_T, dtype=torch.int32, device=dev)
    g = cb.StepGraphs(q, k, v, out, kc, vc, scale, max_seqs=MAX_S, max_kv_len=MAX_KV,
                      max_blocks_per_seq=MB, token_interval=16, kv_interval=256, seq_interval=8,
                      max_graphs=2, use_graphs=use_graphs)
    stream = torch.cuda.Stream()
    shapes = set()
    with torch.cuda.stream(stream):
        for i, (name, qs, kvr, check) in enumerate(STEPS):
            cu, kv, tables = make_step(rng, qs, kvr)
            T = int(cu[-1])
            say(f"graph step {i} {name}: S={len(qs)} T={T} max_kv={int(kv.max())}")
            qh = rand_bf16(rng, (T, HQ, D))
            kh, vh = rand_bf16(rng, (T, HKV, D)), rand_bf16(rng, (T, HKV, D))
            q[:T].copy_(dev_bf16(qh, dev))
            k[:T].copy_(dev_bf16(kh, dev))
            v[:T].copy_(dev_bf16(vh, dev))
            shape = g.run(cu, kv, tables)
            shapes.add(shape)
            Sb, Tb, mq, mkv = shape
            assert Tb >= T and Tb % 16 == 0 or Tb == MAX_T
            # the same padded step, eagerly, on the reference caches
            cup, kvp, tp = padded(cu, kv, tables, shape)
            dcu, dkv, dt = dev_i32(cup, dev), dev_i32(kvp, dev), dev_i32(tp, dev)
            cb.cb_slot_mapping(dcu, dkv, dt, eslots[:Tb], BS)
            cb.cb_cache_write(k[:Tb], v[:Tb], eslots[:Tb], ekc, evc)
            ws = cb.alloc_workspace(Sb, Tb, HQ, HKV, D, BS, mq, mkv)
            cb.cb_paged_attention(q[:Tb], dcu, dkv, dt, ekc, evc, eout[:Tb], scale, mq, mkv, ws)
            stream.synchronize()
            got = host_u16(out[:T])
            assert np.array_equal(got, host_u16(eout[:T])), f"step {i}: graph output != eager"
            assert torch.equal(kc, ekc) and torch.equal(vc, evc), f"step {i}: caches differ"
            if check:
                ref, _ = oracle.paged_attention(qh, cu, kv, tables, host_u16(kc), host_u16(vc), scale)
                ok, rep = oracle.within_tolerance(oracle.bf16_to_f64(got), ref)
                assert ok, f"step {i}: {rep}"
    captures, replays, eager, cached = g.stats()
    say(f"graph stats: captures={captures} replays={replays} eager={eager} cached={cached}")
    if use_graphs:
        assert eager == len(shapes)
        assert captures >= 4 and replays >= 2 and cached <= 2
        assert eager + captures + replays == len(STEPS)
    else:
        assert (captures, replays, eager, cached) == (0, 0, len(STEPS), 0)
    g.close()


def test_step_graphs_refuse_null_stream_and_bad_sizes():
    q = torch.zeros((32, HQ, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((32, HKV, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((64, BS, HKV, D), dtype=torch.bfloat16, device="cuda")
    g = cb.StepGraphs(q, k, k.clone(), q.clone(), kc, kc.clone(), 0.1, max_seqs=4, max_kv_len=256,
                      max_blocks_per_seq=16, use_graphs=True)
    cu, kv = np.array([0, 1], np.int32), np.array([5], np.int32)
    tables = np.zeros((1, 16), np.int32)
    with pytest.raises(cb.CBError):           # the NULL stream cannot be recorded
        g.run(cu, kv, tables, stream=0)
    s = torch.cuda.Stream()
    with pytest.raises(cb.CBError):           # more tokens than the buffers hold
        g.run(np.array([0, 40], np.int32), np.array([40], np.int32), tables, stream=s)
    with pytest.raises(cb.CBError):           # a KV length past max_kv_len
        g.run(cu, np.array([300], np.int32), tables, stream=s)
    g.close()
