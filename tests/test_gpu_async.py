"""GPU parity of the async step: cb_carry_over against the oracle (bit exact), and an async loop
(placeholders, carry-over, A/B slots, three streams) against a synchronous loop in which the CPU
feeds the real tokens: identical tokens at every step and identical outputs. The model around
attention is a stand-in written here (embedding lookups for q, k, v; a greedy argmax sampler),
only to make each step's tokens depend on the previous step's output."""
import numpy as np
import pytest

import oracle.carry as oc
from gpu_helpers import dev_bf16, host_u16, say
from serving_helpers import rand_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
cb = pytest.importorskip("ragged_paged_kv_amd")


def test_carry_over_bit_exact():
    rng = np.random.default_rng(3)
    for n_prev, n_next in [(1, 1), (300, 257), (5000, 4096)]:
        prev = rng.integers(0, 1 << 20, n_prev).astype(np.int32)
        dest = np.full(n_prev, -1, np.int32)
        k = min(n_prev, n_next) // 2
        dest[rng.choice(n_prev, k, replace=False)] = rng.choice(n_next, k, replace=False)
        dest[: min(3, n_prev)] = [-1, n_next, -5][: min(3, n_prev)]   # skipped entries
        nxt = rng.integers(0, 1 << 20, n_next).astype(np.int32)
        d_nxt = torch.from_numpy(nxt).cuda()
        cb.cb_carry_over(torch.from_numpy(prev).cuda(), torch.from_numpy(dest).cuda(), d_nxt)
        torch.cuda.synchronize()
        assert np.array_equal(d_nxt.cpu().numpy(), oc.carry_over(prev, dest, nxt).astype(np.int32))


HQ, HKV, D, BS, V = 8, 2, 128, 16, 61
S, STEPS = 12, 20


def schedule(rng):
    prompts = [rng.integers(0, V, int(rng.integers(5, 41))).astype(np.int32) for _ in range(S)]
    MB = -(-max(len(p) + STEPS + 1 for p in prompts) // BS)
    tables = np.full((S, MB), -1, np.int32)
    perm = rng.permutation(S * MB)
    for s in range(S):
        tables[s] = perm[s * MB:(s + 1) * MB]
    return prompts, tables, MB


def metadata(prompts, step):
    if step == 0:
        q = [len(p) for p in prompts]
        kv = q
    else:
        q = [1] * S
        kv = [len(p) + step for p in prompts]
    return np.concatenate([[0], np.cumsum(q)]).astype(np.int32), np.array(kv, np.int32)


class Model:
    """Stand-in for the layers around attention: embedding lookups and a greedy sampler."""

    def __init__(self, rng, T):
        self.eq = dev_bf16(rand_bf16(rng, (V, HQ, D)), "cuda")
        self.ek = dev_bf16(rand_bf16(rng, (V, HKV, D)), "cuda")
        self.ev = dev_bf16(rand_bf16(rng, (V, HKV, D)), "cuda")
        self.q = torch.zeros((T, HQ, D), dtype=torch.bfloat16, device="cuda")
        self.k = torch.zeros((T, HKV, D), dtype=torch.bfloat16, device="cuda")
        self.v = torch.zeros_like(self.k)
        self.out = torch.zeros_like(self.q)

    def pre(self, ids, T):
        i = ids[:T].long()
        self.q[:T].copy_(self.eq[i])
        self.k[:T].copy_(self.ek[i])
        self.v[:T].copy_(self.ev[i])

    def sample(self, out_ids, T):
        tok = self.out[:T].float().sum(dim=1).argmax(dim=1) % V
        out_ids[:T].copy_(tok.to(torch.int32))


@pytest.mark.parametrize("use_graphs", [False, True])
def test_async_loop_matches_sync_loop(use_graphs):
    rng = np.random.default_rng(5)
    prompts, tables, MB = schedule(rng)
    T0 = sum(len(p) for p in prompts)
    T = ((T0 + 15) // 16) * 16
    NB = S * MB
    kc0, vc0 = rand_bf16(rng, (NB, BS, HKV, D)), rand_bf16(rng, (NB, BS, HKV, D))
    models = [Model(np.random.default_rng(9), T) for _ in range(2)]   # identical weights
    scale = 1.0 / np.sqrt(D)
    kw = dict(max_seqs=S + 8, max_kv_len=MB * BS, max_blocks_per_seq=MB, use_graphs=use_graphs)

    # synchronous loop: the CPU reads each step's tokens and feeds them to the next
    m = models[0]
    kc, vc = dev_bf16(kc0, "cuda"), dev_bf16(vc0, "cuda")
    ex = cb.StepGraphs(m.q, m.k, m.v, m.out, kc, vc, scale, **kw)
    stream = torch.cuda.Stream()
    ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    out_ids = torch.zeros(T, dtype=torch.int32, device="cuda")
    sync_tokens = []
    last = None
    with torch.cuda.stream(stream):
        for step in range(STEPS):
            cu, kv = metadata(prompts, step)
            n = int(cu[-1])
            host = np.concatenate(prompts) if step == 0 else last[cu_prev[1:] - 1]
            ids[:n].copy_(torch.from_numpy(host.astype(np.int32)).cuda())
            m.pre(ids, n)
            ex.run(cu, kv, tables)
            m.sample(out_ids, n)
            stream.synchronize()
            last = out_ids[:n].cpu().numpy()
            sync_tokens.append(last.copy())
            cu_prev = cu
    sync_out = host_u16(m.out[:S])
    ex.close()

    # async loop: placeholders and carry-over; step N's tokens are read after step N+1 is begun
    m = models[1]
    kc, vc = dev_bf16(kc0, "cuda"), dev_bf16(vc0, "cuda")
    a = cb.AsyncSteps(m.q, m.k, m.v, m.out, kc, vc, scale, **kw)
    async_tokens = [None] * STEPS
    prev = None   # (slot, rows) of the previous step
    for step in range(STEPS):
        cu, kv = metadata(prompts, step)
        n = int(cu[-1])
        slot = a.slot()
        if step == 0:
            a.in_ids_host[slot][:n].copy_(torch.from_numpy(np.concatenate(prompts)))
            carried = 0
        else:
            a.in_ids_host[slot][:n].zero_()                       # placeholders
            pcu = prev_cu
            dest = np.full(int(pcu[-1]), -1, np.int32)
            dest[pcu[1:] - 1] = np.arange(S)                      # last row of each sequence
            a.carry_dest_host[slot][:dest.size].copy_(torch.from_numpy(dest))
            carried = dest.size
        st = a.begin(cu, kv, tables, carried)
        with torch.cuda.stream(st):
            m.pre(a.in_ids[slot], n)
        a.attention()
        with torch.cuda.stream(st):
            m.sample(a.out_ids[slot], n)
        a.end(n)
        if prev is not None:                                      # the previous step's tokens
            pslot, pn, pstep = prev
            a.wait(pslot)
            async_tokens[pstep] = a.out_ids_host[pslot][:pn].numpy().copy()
        prev = (slot, n, step)
        prev_cu = cu
    pslot, pn, pstep = prev
    a.wait(pslot)
    async_tokens[pstep] = a.out_ids_host[pslot][:pn].numpy().copy()
    torch.cuda.synchronize()
    async_out = host_u16(m.out[:S])
    a.close()

    for step in range(STEPS):
        assert np.array_equal(sync_tokens[step], async_tokens[step]), f"step {step} tokens differ"
    assert np.array_equal(sync_out, async_out)
    say(f"async == sync over {STEPS} steps; last tokens {async_tokens[-1][:6]}")
    assert len({t.tobytes() for t in sync_tokens[1:]}) > 1   # the tokens do change step to step


class ScriptedModel(Model):
    """The stand-in model with a scripted sampler: the token that step n samples for packed row r
    is fixed in advance (a host table), so every step's inputs are known on the host and the
    oracle can replay the loop. Each step's attention output is kept for the comparison."""

    def __init__(self, rng, T, script):
        super().__init__(rng, T)
        self.script = torch.from_numpy(script).cuda()   # [STEPS, T] int32
        self.kept = []
        self.step = 0

    def sample(self, out_ids, T):
        self.kept.append(self.out[:T].clone())
        out_ids[:T].copy_(self.script[self.step, :T])
        self.step += 1


@pytest.mark.parametrize("use_graphs", [False, True])
def test_async_loop_against_oracle(use_graphs):
    """Every step of an async loop (placeholders, carry-over, A/B slots, three streams) against
    the oracle replaying the same steps on the host: slot mapping, cache write and attention of
    each step from host-known inputs. The tokens each step samples are scripted, so the inputs of
    step n + 1 (carried into its placeholders on the GPU) are known without reading the GPU."""
    import oracle
    rng = np.random.default_rng(15)
    prompts, tables, MB = schedule(rng)
    T0 = sum(len(p) for p in prompts)
    T = ((T0 + 15) // 16) * 16
    NB = S * MB
    kc0, vc0 = rand_bf16(rng, (NB, BS, HKV, D)), rand_bf16(rng, (NB, BS, HKV, D))
    script = rng.integers(0, V, (STEPS, T)).astype(np.int32)
    m = ScriptedModel(np.random.default_rng(9), T, script)
    eq, ek, ev = (host_u16(x) for x in (m.eq, m.ek, m.ev))
    scale = 1.0 / np.sqrt(D)
    kc, vc = dev_bf16(kc0, "cuda"), dev_bf16(vc0, "cuda")
    a = cb.AsyncSteps(m.q, m.k, m.v, m.out, kc, vc, scale, max_seqs=S + 8, max_kv_len=MB * BS,
                      max_blocks_per_seq=MB, use_graphs=use_graphs)
    prev_cu = None
    for step in range(STEPS):
        cu, kv = metadata(prompts, step)
        n = int(cu[-1])
        slot = a.slot()
        if step == 0:
            a.in_ids_host[slot][:n].copy_(torch.from_numpy(np.concatenate(prompts)))
            carried = 0
        else:
            a.in_ids_host[slot][:n].zero_()
            dest = np.full(int(prev_cu[-1]), -1, np.int32)
            dest[prev_cu[1:] - 1] = np.arange(S)
            a.carry_dest_host[slot][:dest.size].copy_(torch.from_numpy(dest))
            carried = dest.size
        st = a.begin(cu, kv, tables, carried)
        with torch.cuda.stream(st):
            m.pre(a.in_ids[slot], n)
        a.attention()
        with torch.cuda.stream(st):
            m.sample(a.out_ids[slot], n)
        a.end(n)
        if step > 0:
            a.wait(1 - slot)
        prev_cu = cu
    a.wait(a.slot() ^ 1)
    torch.cuda.synchronize()
    got = [host_u16(o) for o in m.kept]
    a.close()

    # the oracle replays the loop: step 0 reads the prompts, step n > 0 the token that step n - 1
    # sampled for each sequence's last row
    kch, vch = kc0.copy(), vc0.copy()
    prev_cu = None
    worst = 0.0
    for step in range(STEPS):
        cu, kv = metadata(prompts, step)
        ids = (np.concatenate(prompts) if step == 0 else script[step - 1][prev_cu[1:] - 1])
        sl = oracle.slot_mapping(cu, kv, tables, BS)
        kch, vch = oracle.cache_write(kch, vch, ek[ids], ev[ids], sl)
        ref, _ = oracle.paged_attention(eq[ids], cu, kv, tables, kch, vch, np.float32(scale))
        ok, rep = oracle.within_tolerance(oracle.bf16_to_f64(got[step]), ref)
        assert ok and rep["max_abs"] <= oracle.ATOL, f"step {step}: {rep}"
        worst = max(worst, rep["max_abs"])
        prev_cu = cu
    say(f"async loop == oracle at all {STEPS} steps (graphs {use_graphs}), max_abs {worst:.3g}")
