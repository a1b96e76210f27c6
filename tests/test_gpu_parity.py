"""HIP path against the oracle, through the C ABI, on an MI355X.

Slot mapping and the cache write must be bit-exact; attention outputs must satisfy
|gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise against the float64 oracle. Scaled-down copies of
the five workloads are compared on every output element; the full-size workloads (in the launch
configuration the benchmark times) on every decode token and a sample of prefill tokens.
"""
import copy
import zlib

import numpy as np
import pytest

import oracle
import synth
from gpu_helpers import (Step, assert_close, dev_bf16, dev_i32, host_u16, oracle_step,
                         readable_mask, say)
from pins import permute_blocks, table_slots, tiny_batch, widen

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ragged_paged_kv_amd  # noqa: F401  (raises if the library is not built)
    return torch


def check_full(batch, step, tokens=None):
    sl, (kc, vc), out, _ = oracle_step(batch, tokens=tokens)
    assert np.array_equal(step.slots_host(), sl), "slot mapping differs from the oracle"
    assert np.array_equal(host_u16(step.k_cache), kc), "K cache differs from the oracle"
    assert np.array_equal(host_u16(step.v_cache), vc), "V cache differs from the oracle"
    got = step.out_f64()
    if tokens is None:
        return assert_close(got, out, batch.name)
    return assert_close(got[tokens], out[tokens], batch.name)


SMALL = [1, 2, 3, 4, 5]


@pytest.mark.parametrize("n", SMALL)
@pytest.mark.parametrize("split", [0, 32, 64, 512])
def test_small_configs_every_element(torch_cuda, n, split):
    b = synth.make_config(n, small=True)
    say(f"[parity] small config {n} split {split}: S={b.num_seqs} T={b.num_tokens}")
    step = Step(b, kv_split_tokens=split).run()
    check_full(b, step)


def _sample_tokens(batch, per_chunk=24, seed=0):
    rng = np.random.default_rng(seed)
    cu = batch.cu_seqlens_q
    toks = []
    for s in range(batch.num_seqs):
        q = int(cu[s + 1] - cu[s])
        if q == 1:
            toks.append(int(cu[s]))
        else:
            pick = {0, 1, q - 2, q - 1} | set(rng.integers(0, q, size=per_chunk).tolist())
            toks += [int(cu[s]) + i for i in sorted(pick)]
    return np.array(sorted(set(toks)))


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_full_size_configs(torch_cuda, n):
    b = synth.make_config(n)
    say(f"[parity] full config {n} ({b.name}): S={b.num_seqs} T={b.num_tokens} "
        f"sumL={int(b.kv_lens.sum())} blocks={b.num_blocks}")
    step = Step(b).run()
    toks = _sample_tokens(b)
    rep = check_full(b, step, tokens=toks)
    say(f"[parity] full config {n}: {len(toks)} tokens checked, {rep}")


def test_split_matches_unsplit(torch_cuda):
    b = synth.make_config(4, small=True)
    outs = []
    for split in (32, 96, 1024, 4096):
        outs.append(Step(b, kv_split_tokens=split).run().out_f64())
    for o in outs[1:]:
        assert_close(o, outs[-1], "split vs unsplit")


def test_block_permutation_bit_identical(torch_cuda):
    for n in (1, 3, 5):
        b = synth.make_config(n, small=True)
        a = Step(b).run().out_u16()
        p = Step(permute_blocks(b, seed=n)).run().out_u16()
        assert np.array_equal(a, p), f"config {n}: output changed under a block permutation"


def test_deterministic_across_runs(torch_cuda):
    b = synth.make_config(3, small=True)
    st = Step(b, kv_split_tokens=64).run()
    first = st.out_u16()
    for _ in range(9):
        st.attention()
        torch_cuda.cuda.synchronize()
        assert np.array_equal(st.out_u16(), first)


@pytest.mark.parametrize("poison", [0x7F80, 0xFF80, 0xFFFF, 0x7F7F, None])
def test_unread_slots_do_not_matter(torch_cuda, poison):
    # Slots past each sequence's length, unassigned blocks: +inf, -inf, NaN, max finite, noise.
    b = synth.make_config(5, small=True)
    ref = Step(b).run().out_u16()
    m = readable_mask(b)
    b2 = copy.copy(b)
    rng = np.random.default_rng(1)
    for name in ("k_cache", "v_cache"):
        c = getattr(b, name).copy()
        fill = (rng.integers(0, 1 << 16, size=c.shape, dtype=np.uint32).astype(np.uint16)
                if poison is None else np.full(c.shape, poison, dtype=np.uint16))
        c[~m] = fill[~m]
        setattr(b2, name, c)
    # the new tokens' slots are unread before the write as well
    got = Step(b2).run().out_u16()
    assert np.array_equal(got, ref)


def _growing_keys(batch, rate):
    """The batch with every key row (cached and new) of every sequence scaled by 2^(p / rate) at
    position p: the scores grow along each sequence, so the online softmax's running reference
    maximum has to move again and again."""
    b = copy.copy(batch)
    Hkv, D, bs = b.num_kv_heads, b.head_dim, b.block_size
    kc = b.k_cache.copy().reshape(-1, Hkv, D)
    k = b.k.copy()
    cu = b.cu_seqlens_q
    for s in range(b.num_seqs):
        L, q0, q1 = int(b.kv_lens[s]), int(cu[s]), int(cu[s + 1])
        f = 2.0 ** (np.arange(L) / rate)
        slots = table_slots(b.block_tables[s], L, bs)
        for p in range(L - (q1 - q0)):
            kc[slots[p]] = synth.bf16_from_f32((widen(kc[slots[p]]) * f[p]).astype(np.float32))
        k[q0:q1] = synth.bf16_from_f32((widen(k[q0:q1]) * f[L - (q1 - q0):, None, None]).astype(np.float32))
    b.k_cache = kc.reshape(b.k_cache.shape)
    b.k = k
    return b


def _reference_moves(b):
    """Most moves of a lazily kept reference maximum over one query row and head of the batch
    (float64 scores in log2 units, 32-key tiles from key 0): the reference starts at the first
    tile's maximum and moves to a tile's maximum when that exceeds it by more than 8."""
    Hq, Hkv, D, bs = b.num_q_heads, b.num_kv_heads, b.head_dim, b.block_size
    G = Hq // Hkv
    kc = b.k_cache.reshape(-1, Hkv, D)
    c = b.scale / np.log(2.0)
    most = 0
    for s in range(b.num_seqs):
        L, q0, q1 = int(b.kv_lens[s]), int(b.cu_seqlens_q[s]), int(b.cu_seqlens_q[s + 1])
        qn = q1 - q0
        slots = table_slots(b.block_tables[s], L, bs)
        keys = np.concatenate([widen(kc[slots[: L - qn]]), widen(b.k[q0:q1])])  # [L, Hkv, D]
        q = widen(b.q[q0:q1])  # [qn, Hq, D]
        for hh in range(Hq):
            sc = c * (q[:, hh] @ keys[:, hh // G].T)  # [qn, L]
            for i in range(qn):
                row = sc[i, : L - qn + i + 1]
                m, moves = row[:32].max(), 0
                for t in range(32, len(row), 32):
                    if row[t:t + 32].max() > m + 8:
                        m, moves = row[t:t + 32].max(), moves + 1
                most = max(most, moves)
    return most


RESCALE = {
    # (specs, Hq, Hkv, D, bs, kv_split_tokens, positions per doubling of the key scale): the
    # scale ends near 2^3.5, so scaled scores reach a few tens of log2 units
    "decode": ([synth.SeqSpec(1, 700), synth.SeqSpec(1, 333), synth.SeqSpec(2, 520)], 32, 8, 128, 16, 0, 200.0),
    "decode-partitions": ([synth.SeqSpec(1, 700), synth.SeqSpec(1, 333), synth.SeqSpec(2, 520)], 32, 8, 128, 16, 64, 200.0),
    "prefill-split": ([synth.SeqSpec(64, 2000), synth.SeqSpec(130, 130)], 32, 8, 128, 16, 0, 570.0),
    "mixed-d64": ([synth.SeqSpec(1, 600), synth.SeqSpec(40, 700)], 16, 2, 64, 16, 0, 200.0),
}


@pytest.mark.parametrize("name", sorted(RESCALE))
def test_growing_scores_move_the_reference_max(torch_cuda, name):
    """Scores that keep growing along the sequence: the lazy rescale of both kernels (and the
    merge of partitions with different maxima) runs many times, and every output element still
    matches the oracle. The batch is checked first to make the path certain: a reference max kept
    the kernels' way (moved when a tile exceeds it by more than 8) moves several times in a row."""
    specs, Hq, Hkv, D, bs, split, rate = RESCALE[name]
    b = _growing_keys(tiny_batch(list(specs), Hq, Hkv, D, bs, seed=zlib.crc32(name.encode()) % 1000), rate)
    moves = _reference_moves(b)
    say(f"[rescale] {name}: a lazily kept reference max moves up to {moves} times in one row")
    assert moves >= 3
    step = Step(b, kv_split_tokens=split).run()
    rep = check_full(b, step)
    say(f"[rescale] {name}: {rep}")


def test_split_kv_reduce_entry(torch_cuda):
    import ragged_paged_kv_amd as cb
    torch = torch_cuda
    b = synth.make_config(3, small=True)
    sl, (kc, vc), ref, _ = oracle_step(b)
    rng = np.random.default_rng(4)
    bounds = []
    for L in b.kv_lens.tolist():
        cuts = sorted(set(rng.integers(1, L, size=min(L - 1, 5)).tolist())) if L > 1 else []
        bounds.append([0] + cuts + [L])
    o, lse, ns = oracle.split_partials(b.q, b.cu_seqlens_q, b.kv_lens, b.block_tables, kc, vc,
                                       b.scale, bounds)
    # an empty partition with garbage o must carry no weight
    o = np.concatenate([o, np.full(o.shape[:2] + (1,) + o.shape[3:], np.nan)], axis=2)
    lse = np.concatenate([lse, np.full(lse.shape[:2] + (1,), -np.inf)], axis=2)
    ns = ns + 1
    ns[5] = 0  # a token that must not be written
    want = oracle.merge_partials(o, lse, ns)
    out = torch.full(ref.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    cb.cb_split_kv_reduce(torch.from_numpy(o.astype(np.float32)).cuda(),
                          torch.from_numpy(lse.astype(np.float32)).cuda(),
                          dev_i32(ns, "cuda"), out)
    torch.cuda.synchronize()
    got = oracle.bf16_to_f64(host_u16(out))
    keep = ns > 0
    assert_close(got[keep], want[keep], "reduce vs oracle merge")
    assert_close(got[keep], ref[keep], "reduce vs unsplit oracle")
    assert np.all(got[~keep] == 7.0)


def _many_partition_batch(which):
    if which == "d128":
        return synth.make_config(3, small=True)
    return tiny_batch([synth.SeqSpec(1, 120), synth.SeqSpec(3, 90), synth.SeqSpec(20, 70)],
                      16, 2, 64, 16, seed=12)


@pytest.mark.parametrize("which", ["d64", "d128"])
def test_split_kv_reduce_many_partitions(torch_cuda, which):
    """Rows of more than four load batches of partitions (the merge then splits a row over a group
    of threads), head_dim 64 and 128, an empty partition first, a token left unwritten."""
    import ragged_paged_kv_amd as cb
    torch = torch_cuda
    b = _many_partition_batch(which)
    sl, (kc, vc), ref, _ = oracle_step(b)
    rng = np.random.default_rng(41)
    bounds = []
    for L in b.kv_lens.tolist():
        cuts = sorted(set(rng.integers(1, L, size=min(L - 1, 80)).tolist())) if L > 1 else []
        bounds.append([0] + cuts + [L])
    o, lse, ns = oracle.split_partials(b.q, b.cu_seqlens_q, b.kv_lens, b.block_tables, kc, vc,
                                       b.scale, bounds)
    assert ns.max() + 1 > 32, "the rows must span more than four load batches"
    o = np.concatenate([np.full(o.shape[:2] + (1,) + o.shape[3:], np.nan), o], axis=2)
    lse = np.concatenate([np.full(lse.shape[:2] + (1,), -np.inf), lse], axis=2)
    ns = ns + 1
    ns[1] = 0
    want = oracle.merge_partials(o, lse, ns)
    out = torch.full(ref.shape, 7.0, dtype=torch.bfloat16, device="cuda")
    cb.cb_split_kv_reduce(torch.from_numpy(o.astype(np.float32)).cuda(),
                          torch.from_numpy(lse.astype(np.float32)).cuda(),
                          dev_i32(ns, "cuda"), out)
    torch.cuda.synchronize()
    got = oracle.bf16_to_f64(host_u16(out))
    keep = ns > 0
    assert_close(got[keep], want[keep], "reduce vs oracle merge")
    assert_close(got[keep], ref[keep], "reduce vs unsplit oracle")
    assert np.all(got[~keep] == 7.0)


EDGE = {
    # (specs, Hq, Hkv, D, bs)
    "single-key": ([synth.SeqSpec(1, 1)] * 3, 8, 2, 128, 16),
    "prompt-of-one": ([synth.SeqSpec(1, 1), synth.SeqSpec(40, 40)], 8, 8, 128, 16),
    "block-edges": ([synth.SeqSpec(1, L) for L in (15, 16, 17, 31, 32, 33, 63, 64, 65)], 32, 8, 128, 16),
    "split-edges": ([synth.SeqSpec(1, L) for L in (255, 256, 257, 511, 512, 513)], 32, 8, 128, 16),
    "mha": ([synth.SeqSpec(1, 70), synth.SeqSpec(33, 90)], 4, 4, 128, 16),
    "gqa16": ([synth.SeqSpec(1, 70), synth.SeqSpec(2, 50), synth.SeqSpec(3, 90)], 32, 2, 128, 32),
    "d64-gqa8": ([synth.SeqSpec(1, 70), synth.SeqSpec(2, 40), synth.SeqSpec(19, 60)], 16, 2, 64, 16),
    "spec-decode": ([synth.SeqSpec(q, 100 + q) for q in (1, 2, 3, 4, 5, 8)], 32, 8, 128, 16),
    "prefill-only": ([synth.SeqSpec(130, 130), synth.SeqSpec(77, 300)], 32, 8, 128, 16),
    "bs64": ([synth.SeqSpec(1, 200), synth.SeqSpec(50, 150)], 32, 8, 128, 64),
    "bs256": ([synth.SeqSpec(1, 700), synth.SeqSpec(100, 600)], 32, 8, 128, 256),
    # block sizes that are not powers of two (keys divided by multiply and shift), with more
    # than 64 blocks per sequence so that the prefill block-id window moves
    "bs48-long": ([synth.SeqSpec(1, 3500), synth.SeqSpec(150, 4000)], 32, 8, 128, 48),
    "bs80-d64": ([synth.SeqSpec(1, 900), synth.SeqSpec(90, 5300)], 16, 2, 64, 80),
    "long-chunk-offset": ([synth.SeqSpec(200, 1500)], 32, 8, 128, 16),
    # prefill tiles split along the keys (few tiles, long contexts): 4 parts, uneven rounding,
    # head_dim 64, 256-row tiles of one head, and next to decodes and a short prompt
    "prefill-split-4": ([synth.SeqSpec(96, 6200)], 32, 8, 128, 16),
    "prefill-split-uneven": ([synth.SeqSpec(20, 2049), synth.SeqSpec(40, 3073)], 32, 8, 128, 32),
    "prefill-split-d64": ([synth.SeqSpec(70, 2500)], 16, 2, 64, 16),
    "prefill-split-mha": ([synth.SeqSpec(300, 2600)], 4, 4, 128, 16),
    "prefill-split-mixed": ([synth.SeqSpec(1, 3000), synth.SeqSpec(64, 2100), synth.SeqSpec(33, 33)],
                            32, 8, 128, 16),
}


@pytest.mark.parametrize("name", sorted(EDGE))
@pytest.mark.parametrize("split", [0, 32])
def test_edge_cases(torch_cuda, name, split):
    specs, Hq, Hkv, D, bs = EDGE[name]
    b = tiny_batch(list(specs), Hq, Hkv, D, bs, seed=zlib.crc32(name.encode()) % 1000)
    say(f"[parity] edge {name} split {split}")
    step = Step(b, kv_split_tokens=split).run()
    check_full(b, step)


def _random_batch(seed):
    """A seeded random batch within the contract: KV heads 1-8, query heads per KV head 1-16
    (at most 64 query heads), head_dim 64 or 128, block sizes 16, 32, 48 or 64, 1-20 sequences
    mixing decode-type (q * G <= 16) and prefill-type chunks at random offsets into their
    contexts; and a random KV partition request (0 = the library's choice)."""
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([g for g in (1, 2, 4, 8, 16) if g * Hkv <= 64]))
    D = int(rng.choice([64, 128]))
    bs = int(rng.choice([16, 32, 48, 64]))
    specs = []
    for _ in range(int(rng.integers(1, 21))):
        if rng.random() < 0.6:
            q = int(rng.integers(1, max(1, 16 // G) + 1))
            L = int(rng.integers(q, 2601))
        else:
            q = int(rng.integers(16 // G + 1, 161))
            L = q + int(rng.integers(0, 2401))
        specs.append(synth.SeqSpec(q, L))
    split = int(rng.choice([0, 32, 96, 256]))
    return tiny_batch(specs, G * Hkv, Hkv, D, bs, seed=seed), split


@pytest.mark.parametrize("seed", range(16))
def test_random_batches(torch_cuda, seed):
    b, split = _random_batch(5000 + seed)
    say(f"[parity] random batch {seed}: S={b.num_seqs} T={b.num_tokens} Hq={b.num_q_heads} "
        f"Hkv={b.num_kv_heads} D={b.head_dim} bs={b.block_size} split={split}")
    step = Step(b, kv_split_tokens=split).run()
    check_full(b, step)


# Decode-only batches whose automatic KV partition takes each branch of the size rule for small
# batches (the expected size is asserted first), compared with the oracle on every element:
# name -> (sequences, longest KV length, Hq, Hkv, head_dim, block size, expected partition).
AUTO_SPLIT = {
    "floor-128": (8, 583, 32, 8, 128, 16, 128),
    "keys-over-640": (16, 2048, 32, 8, 128, 32, 448),
    "cap-768": (40, 3867, 32, 8, 128, 48, 768),
    "long-sequence-cap": (8, 16310, 32, 8, 128, 64, 1664),
    "largest-2048": (1, 65536, 32, 8, 128, 16, 2048),
    "one-partition": (64, 699, 32, 8, 128, 16, 704),
    "one-partition-ends-mid-block": (96, 1500, 32, 8, 128, 64, 1504),
    "head-dim-64": (4, 900, 16, 8, 64, 16, 128),
}


@pytest.mark.parametrize("name", sorted(AUTO_SPLIT))
def test_automatic_split_of_small_decode_batches(torch_cuda, name):
    import ragged_paged_kv_amd as cb
    S, L, Hq, Hkv, D, bs, want = AUTO_SPLIT[name]
    assert cb.cb_paged_attention_split_tokens(S, Hq, Hkv, 1, L, 0) == want
    seed = zlib.crc32(name.encode()) % 100000
    rng = np.random.default_rng(seed)
    lens = [L] + [int(x) for x in rng.integers(max(1, L // 8), L + 1, S - 1)]
    b = tiny_batch([synth.SeqSpec(1, n) for n in lens], Hq, Hkv, D, bs, seed=seed)
    say(f"[parity] automatic split {name}: S={S} max_kv_len={b.max_kv_len} bs={bs} P={want}")
    step = Step(b).run()
    check_full(b, step)


def test_loose_upper_bounds(torch_cuda):
    # host bounds larger than the real maxima only size grids and the workspace
    b = synth.make_config(3, small=True)
    # the table must be able to address max_kv_len
    b2 = copy.copy(b)
    need = -(-(b.max_kv_len * 2 + 5) // b.block_size)
    b2.block_tables = np.concatenate(
        [b.block_tables, np.full((b.num_seqs, need - b.block_tables.shape[1]), -1, np.int32)], axis=1)
    step = Step(b2, max_q_len=b.max_q_len * 3, max_kv_len=b.max_kv_len * 2 + 5).run()
    check_full(b2, step)


def test_empty_batch_leaves_output(torch_cuda):
    import ragged_paged_kv_amd as cb
    torch = torch_cuda
    b = synth.make_config(1)
    st = Step(b)
    q0 = st.q[:0]
    out0 = torch.empty((0, b.num_q_heads, b.head_dim), dtype=torch.bfloat16, device="cuda")
    cu0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    kv0 = torch.zeros(0, dtype=torch.int32, device="cuda")
    bt0 = torch.zeros((0, 3), dtype=torch.int32, device="cuda")
    cb.cb_paged_attention(q0, cu0, kv0, bt0, st.k_cache, st.v_cache, out0, b.scale, 1, 1, st.ws)
    torch.cuda.synchronize()


def test_cache_write_skips_slots_outside_the_pool(torch_cuda):
    """Slot -1 and slots at or past num_blocks * block_size write nothing; the rest are written."""
    import ragged_paged_kv_amd as cb
    b = synth.make_config(1, small=True)
    st = Step(b)
    pool = b.k_cache.shape[0] * b.block_size
    slots = np.array([-1, pool, pool + 7, 3, pool - 1], np.int32)
    n = len(slots)
    assert st.k.shape[0] >= n
    kc, vc = dev_bf16(b.k_cache, "cuda"), dev_bf16(b.v_cache, "cuda")
    cb.cb_cache_write(st.k[:n], st.v[:n], dev_i32(slots, "cuda"), kc, vc)
    torch_cuda.cuda.synchronize()
    inside = np.where((slots >= 0) & (slots < pool), slots, -1)
    k_new, v_new = host_u16(st.k[:n]), host_u16(st.v[:n])
    ref_k, ref_v = oracle.cache_write(b.k_cache, b.v_cache, k_new, v_new, inside)
    assert np.array_equal(host_u16(kc), ref_k) and np.array_equal(host_u16(vc), ref_v)


def test_workspace_too_small_is_rejected(torch_cuda):
    import ragged_paged_kv_amd as cb
    b = synth.make_config(2, small=True)
    st = Step(b)
    st.ws = st.ws[:64]
    with pytest.raises(cb.CBError) as e:
        st.attention()
    assert e.value.status == -3


@pytest.mark.parametrize("which", [1, 2])
def test_kernel_timing_hook(torch_cuda, which):
    """The measurement hook records its events around the named kernel and leaves the results
    unchanged; it is one-shot."""
    import ragged_paged_kv_amd as cb
    torch = torch_cuda
    b = synth.make_config(1)  # decode rows and a prefill chunk: both kernels run
    ref = Step(b).run().out_u16()
    st = Step(b)
    st.slot_mapping()
    st.cache_write()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cb.cb_time_next_kernel(which, e0, e1)
    st.attention()
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) > 0.0
    assert np.array_equal(st.out_u16(), ref)
    # consumed: a second call records nothing new
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(); f1.record()
    torch.cuda.synchronize()
    st.attention()
    torch.cuda.synchronize()
    assert np.array_equal(st.out_u16(), ref)


def test_planned_decode_share_and_prefill_split(torch_cuda):
    """The planner's two measured rates (about 1.0 us per 32-key prefill step of a workgroup and
    5.5 GB/ms of decode streaming, both taken on MI355X) decide whether prefill tiles are split
    along their keys (only when the longest tile would outlast the decode work) and how many
    compute units the decode kernel takes beside the prefill kernel (its share of the estimated
    time, at least half). Their effect, read back from the caller's workspace (counts: decode
    items, prefill items, queue head, split flag, decode workgroups allowed):
      - the 8B mixed batch: 1.1 GB of decode (~200 us) outlasts its longest tile (96 steps): no
        split, decode takes most of the CUs;
      - its prefill chunks alone (no decode work): the tiles are split;
      - the 70B-shaped batch: prefill (~1 ms spread over the CUs) outweighs decode: no split
        (the partials would not fit the workspace budget either), decode at the floor of half."""
    torch = torch_cuda
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    b3 = synth.make_config(3)
    rng = np.random.default_rng(3)
    chunks = synth.build_batch("mixed-2048-chunks", 3, rng,
                               [synth.SeqSpec(1024, 3072)] + [synth.SeqSpec(320, 320)] * 3,
                               num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16)
    for name, b, split, lo, hi in (("8B mixed", b3, 0, cus // 2 + 1, cus),
                                   ("8B chunks alone", chunks, 1, cus + 1, 1 << 30),
                                   ("70B-shaped", synth.make_config(5), 0, cus // 2, cus // 2)):
        step = Step(b).run()
        counts = step.ws[:32].view(torch.int32).cpu().numpy()
        say(f"[plan] {name}: split {counts[3]}, decode workgroups allowed {counts[4]} ({cus} CUs)")
        assert counts[3] == split, (name, counts)
        assert lo <= counts[4] <= hi, (name, counts)
