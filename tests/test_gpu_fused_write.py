"""cb_paged_attention_write (the cache write beside the planning workgroup, slots computed in
place) against cb_slot_mapping + cb_cache_write + cb_paged_attention: bit-identical caches and
outputs on every small workload, the edge cases and two full-size workloads; and against the
oracle on the decode workload."""
import zlib

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import Step, dev_bf16, dev_i32, host_u16, oracle_step, assert_close, say
from pins import tiny_batch
from test_gpu_parity import EDGE, _sample_tokens, check_full

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
cb = pytest.importorskip("ragged_paged_kv_amd")


def fused(step, b, split=0):
    kc, vc = dev_bf16(b.k_cache, "cuda"), dev_bf16(b.v_cache, "cuda")
    out = torch.full_like(step.out, float("nan"))
    cb.cb_paged_attention_write(step.q, step.k, step.v, step.cu, step.kv_lens, step.tables, kc, vc,
                                out, b.scale, step.max_q_len, step.max_kv_len, step.ws,
                                kv_split_tokens=split)
    torch.cuda.synchronize()
    return kc, vc, out


def same_as_separate(b, split=0):
    step = Step(b, kv_split_tokens=split).run()
    kc, vc, out = fused(step, b, split)
    # bit patterns: poisoned slots hold NaN, which torch.equal never counts as equal
    assert np.array_equal(host_u16(kc), host_u16(step.k_cache)), "k caches differ"
    assert np.array_equal(host_u16(vc), host_u16(step.v_cache)), "v caches differ"
    assert np.array_equal(host_u16(out), host_u16(step.out)), "outputs differ"
    return out


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("split", [0, 32])
def test_small_configs(n, split):
    b = synth.make_config(n, small=True)
    say(f"[fused] small config {n} split {split}")
    same_as_separate(b, split)


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_cases(name):
    specs, Hq, Hkv, D, bs = EDGE[name]
    b = tiny_batch(list(specs), Hq, Hkv, D, bs, seed=zlib.crc32(name.encode()) % 1000)
    say(f"[fused] edge {name}")
    same_as_separate(b)


def same_as_separate_on_gpu(b):
    """As same_as_separate, with the caches compared on the GPU (bit patterns as int16): the
    long-context and 70B-shaped caches are several GB each."""
    step = Step(b).run()
    kc, vc, out = fused(step, b)
    i16 = lambda t: t.view(torch.int16)  # noqa: E731
    assert torch.equal(i16(kc), i16(step.k_cache)), "k caches differ"
    assert torch.equal(i16(vc), i16(step.v_cache)), "v caches differ"
    assert torch.equal(i16(out), i16(step.out)), "outputs differ"
    return out


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_full_size(n):
    """The fused entry point (the step the benchmark times) bit-identical to the three separate
    ones at every full size, and against the oracle on every decode token and sampled prefill
    rows (every row of the mixed 2048-token batch: test_full_size_every_element)."""
    b = synth.make_config(n)
    say(f"[fused] full config {n} ({b.name})")
    out = same_as_separate(b) if n in (2, 3) else same_as_separate_on_gpu(b)
    if n != 3:
        toks = _sample_tokens(b)
        _, _, ref, _ = oracle_step(b, tokens=toks)
        got = out.float().cpu().numpy().astype(np.float64)
        rep = assert_close(got[toks], ref[toks], b.name)
        say(f"[fused] full config {n}: {len(toks)} tokens against the oracle: {rep}")


def test_full_size_every_element():
    """The mixed 2048-token batch at full size through the fused entry point: every output element
    of every token (decodes, the 1024-token chunk split along its keys, three prompts) against
    the oracle, and the caches bit-exact."""
    b = synth.make_config(3)
    step = Step(b)
    kc, vc = dev_bf16(b.k_cache, "cuda"), dev_bf16(b.v_cache, "cuda")
    out = torch.full_like(step.out, float("nan"))
    cb.cb_paged_attention_write(step.q, step.k, step.v, step.cu, step.kv_lens, step.tables, kc, vc,
                                out, b.scale, step.max_q_len, step.max_kv_len, step.ws)
    torch.cuda.synchronize()
    _, (kref, vref), ref, _ = oracle_step(b)
    assert np.array_equal(host_u16(kc), kref) and np.array_equal(host_u16(vc), vref)
    got = out.float().cpu().numpy().astype(np.float64)
    rep = assert_close(got, ref, b.name)
    say(f"[fused] {b.name}: all {b.num_tokens} tokens against the oracle: {rep}")


@pytest.mark.parametrize("split", [0, 64])
@pytest.mark.parametrize("nseq", [1102, 1024])
def test_more_sequences_than_one_planning_pass(nseq, split):
    """1102 sequences: the planning workgroup takes sequences 1024 at a time and reads each
    pass's inputs again, and the fused write searches the sequences in rounds of 64 evenly spaced
    entries. 1024 sequences: the most that one planning pass holds in registers, and the most
    the write's one-round search covers (16 entries per lane). Fused and separate paths agree bit
    for bit, every output row is written, and rows on both sides of the 1024 boundary and the
    prefill chunks' rows match the oracle (slot mapping and caches whole)."""
    rng = np.random.default_rng(77)
    specs = [synth.SeqSpec(1, int(L)) for L in rng.integers(1, 200, nseq - 2)]
    specs += [synth.SeqSpec(40, 300), synth.SeqSpec(70, 70)]
    b = tiny_batch(specs, 8, 2, 64, 16, seed=77)
    say(f"[fused] {nseq} sequences split {split}")
    out = same_as_separate(b, split)
    assert torch.isfinite(out.float()).all(), "an output row was not written"
    step = Step(b, kv_split_tokens=split).run()
    toks = np.concatenate([np.arange(0, 40), np.arange(nseq - 102, nseq - 2),
                           np.arange(b.num_tokens - 110, b.num_tokens)])
    check_full(b, step, tokens=toks)


def _decode_call(b, cu, kv_lens, tables, max_kv_len, split, write):
    """One attention call (with the cache write when ``write``) on fresh device copies of the
    batch's caches; returns (k cache, v cache, out) as host bit patterns."""
    kc, vc = dev_bf16(b.k_cache, "cuda"), dev_bf16(b.v_cache, "cuda")
    q, k, v = dev_bf16(b.q, "cuda"), dev_bf16(b.k, "cuda"), dev_bf16(b.v, "cuda")
    cu_d, kv_d = dev_i32(cu, "cuda"), dev_i32(kv_lens, "cuda")
    tb_d = dev_i32(tables, "cuda")
    out = torch.full((b.num_tokens, b.num_q_heads, b.head_dim), float("nan"),
                     dtype=torch.bfloat16, device="cuda")
    S = len(kv_lens)
    ws = cb.alloc_workspace(S, b.num_tokens, b.num_q_heads, b.num_kv_heads, b.head_dim,
                            b.block_size, 1, max_kv_len, split, device="cuda")
    if write:
        cb.cb_paged_attention_write(q, k, v, cu_d, kv_d, tb_d, kc, vc, out, b.scale, 1, max_kv_len,
                                    ws, kv_split_tokens=split)
    else:
        cb.cb_paged_attention(q, cu_d, kv_d, tb_d, kc, vc, out, b.scale, 1, max_kv_len, ws,
                              kv_split_tokens=split)
    torch.cuda.synchronize()
    return host_u16(kc), host_u16(vc), host_u16(out)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("write", [True, False])
def test_self_planned_decode_matches_planned(D, write):
    """A decode-only batch of 64 sequences plans inside the decode kernel (no planning launch);
    the same batch with a 65th sequence holding no tokens takes the planned path. Same partition
    size: caches and every output row must match bit for bit. One sequence is longer than the
    max_kv_len bound (by more than the partitions cover): no attention item in either path
    (its output row stays as it was), but its token is still written to the cache."""
    Hq, Hkv, bs, split, bound = 16, 4, 16, 128, 600
    rng = np.random.default_rng(4100 + D)
    lens = [int(x) for x in rng.integers(1, bound + 1, 64)]
    lens[5] = 690  # ceil(690 / 128) = 6 partitions > ceil(600 / 128) = 5: nothing merges it
    b = tiny_batch([synth.SeqSpec(1, n) for n in lens], Hq, Hkv, D, bs, seed=4100 + D)
    assert cb.cb_paged_attention_split_tokens(64, Hq, Hkv, 1, bound, split) == split
    say(f"[fused] self-planned vs planned D={D} write={write}")
    mine = _decode_call(b, b.cu_seqlens_q, b.kv_lens, b.block_tables, bound, split, write)
    cu65 = np.append(b.cu_seqlens_q, b.cu_seqlens_q[-1]).astype(np.int32)
    kv65 = np.append(b.kv_lens, 0).astype(np.int32)
    tb65 = np.concatenate([b.block_tables, np.full((1, b.block_tables.shape[1]), -1, np.int32)])
    ref = _decode_call(b, cu65, kv65, tb65, bound, split, write)
    for name, x, y in zip(("k cache", "v cache", "out"), mine, ref):
        assert np.array_equal(x, y), f"{name} differs between the self-planned and planned paths"
    # the long sequence's row was not written by attention; the other rows were, and (with the
    # write) agree with the oracle
    nan = host_u16(torch.full((1,), float("nan"), dtype=torch.bfloat16))[0]
    out = mine[2].reshape(b.num_tokens, Hq, D)
    assert np.all(out[5] == nan)
    rest = [t for t in range(b.num_tokens) if t != 5]
    assert not np.any(out[rest] == nan)
    if write:
        got = oracle.bf16_to_f64(out[rest])
        assert_close(got, oracle_step(b, tokens=rest)[2][rest], "self-planned decode")
        # the long sequence's token reached the cache at its slot
        kc0 = b.k_cache.reshape(-1, Hkv, D)
        slot = int(b.block_tables[5][(690 - 1) // bs]) * bs + (690 - 1) % bs
        got = mine[0].reshape(-1, Hkv, D)[slot]
        assert np.array_equal(got, b.k[5]) and not np.array_equal(got, kc0[slot])


@pytest.mark.parametrize("G,q", [(4, 4), (2, 8), (1, 16)])
def test_self_planned_write_across_partitions(G, q):
    """Decode-type chunks of q > 1 tokens (q * G = 16) whose new rows straddle a partition
    boundary (P = 32), 16 sequences: a self-planned batch, where the wave of each partition
    stores its own share of the new rows before reading them. Caches bit-exact and outputs within
    the tolerance, against the oracle."""
    Hkv, D, bs, P = 4, 128, 16, 32
    rng = np.random.default_rng(4300 + q)
    lens = [P * int(rng.integers(1, 20)) + int(rng.integers(1, q)) for _ in range(16)]
    b = tiny_batch([synth.SeqSpec(q, L) for L in lens], G * Hkv, Hkv, D, bs, seed=4300 + q)
    say(f"[fused] self-planned write across partitions G={G} q={q}")
    step = Step(b, kv_split_tokens=P)
    kc, vc, out = fused(step, b, P)
    _, (okc, ovc), oout, _ = oracle_step(b)
    assert np.array_equal(host_u16(kc), okc), "k cache differs from the oracle"
    assert np.array_equal(host_u16(vc), ovc), "v cache differs from the oracle"
    assert_close(oracle.bf16_to_f64(host_u16(out)), oout, f"spec decode G={G} q={q}")


def _random_small_decode_batch(seed):
    """A seeded decode-only batch within the self-planned bounds: 1-64 sequences, KV heads 1-8,
    query heads per KV head 1-16, head_dim 64 or 128, block sizes 16-80, 1 to 16 / G query
    tokens each, KV lengths up to 1500; a random partition request (0 = the library's choice),
    dropped to the library's choice when the items would reach the waves."""
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([g for g in (1, 2, 4, 8, 16) if g * Hkv <= 64]))
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 48, 64, 80]))
    S = int(rng.integers(1, 65))
    specs = []
    for _ in range(S):
        q = int(rng.integers(1, 16 // G + 1))
        specs.append(synth.SeqSpec(q, q + int(rng.integers(0, 1500))))
    split = int(rng.choice([0, 64, 160, 512]))
    max_kv = max(sp.L for sp in specs)
    if split and S * -(-max_kv // split) * Hkv >= 1024:
        split = 0
    return tiny_batch(specs, G * Hkv, Hkv, D, bs, seed=seed), split


@pytest.mark.parametrize("seed", range(12))
def test_self_planned_random_batches(seed):
    """Seeded small decode-only batches through the fused call against the oracle: caches bit
    exact, outputs within the tolerance on every element."""
    b, split = _random_small_decode_batch(6000 + seed)
    say(f"[fused] self-planned random batch {seed}: S={b.num_seqs} Hq={b.num_q_heads} "
        f"Hkv={b.num_kv_heads} D={b.head_dim} bs={b.block_size} split={split}")
    step = Step(b, kv_split_tokens=split)
    kc, vc, out = fused(step, b, split)
    _, (okc, ovc), oout, _ = oracle_step(b)
    assert np.array_equal(host_u16(kc), okc), "k cache differs from the oracle"
    assert np.array_equal(host_u16(vc), ovc), "v cache differs from the oracle"
    assert_close(oracle.bf16_to_f64(host_u16(out)), oout, f"random small decode batch {seed}")
