"""cb_paged_attention_write_noalloc (the library's own scratch, no allocation in the call) against
cb_paged_attention_write (caller workspace): two calls in a row, the second on a smaller batch,
so the second runs on scratch the first left behind. Caches bit-exact against the workspace
entry point; outputs bit-identical where both plan the same work (decode-only batches), within
the attention tolerance of the workspace entry point's output and of the oracle otherwise."""
import numpy as np
import pytest

import synth
from gpu_helpers import Step, dev_bf16, host_u16, oracle_step, assert_close, say
from test_gpu_parity import _sample_tokens

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
cb = pytest.importorskip("ragged_paged_kv_amd")


def run_both(b, tokens=None):
    """(workspace entry point's out, no-alloc out) on fresh copies of the batch's caches; the
    caches written by both are compared bit for bit."""
    step = Step(b)
    kc1, vc1 = dev_bf16(b.k_cache, "cuda"), dev_bf16(b.v_cache, "cuda")
    out1 = torch.full_like(step.out, float("nan"))
    cb.cb_paged_attention_write(step.q, step.k, step.v, step.cu, step.kv_lens, step.tables, kc1, vc1,
                                out1, b.scale, step.max_q_len, step.max_kv_len, step.ws)
    kc2, vc2 = dev_bf16(b.k_cache, "cuda"), dev_bf16(b.v_cache, "cuda")
    out2 = torch.full_like(step.out, float("nan"))
    cb.cb_paged_attention_write_noalloc(step.q, step.k, step.v, step.cu, step.kv_lens, step.tables,
                                        kc2, vc2, out2, b.scale, step.max_q_len, step.max_kv_len)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(kc1), host_u16(kc2)), "k caches differ"
    assert np.array_equal(host_u16(vc1), host_u16(vc2)), "v caches differ"
    assert torch.isfinite(out2.float()).all(), "an output row was not written"
    return out1, out2


def check(b, decode_only):
    say(f"[noalloc] {b.name} S={b.num_seqs} T={b.num_tokens}")
    out1, out2 = run_both(b)
    if decode_only:
        assert np.array_equal(host_u16(out1), host_u16(out2)), "outputs differ"
    a1 = out1.float().cpu().numpy().astype(np.float64)
    a2 = out2.float().cpu().numpy().astype(np.float64)
    assert_close(a2, a1, f"{b.name}: no-alloc vs workspace entry point")
    toks = _sample_tokens(b) if b.num_tokens > 64 else None
    _, _, ref, _ = oracle_step(b, tokens=toks)
    sel = slice(None) if toks is None else toks
    assert_close(a2[sel], ref[sel], f"{b.name}: no-alloc vs oracle")


@pytest.mark.parametrize("first,second", [
    ((2, False), (2, True)),   # decode 256 sequences, then its scaled-down copy
    ((5, True), (1, False)),   # 70B-shaped mixed (scaled down), then the tiny batch
    ((3, False), (4, True)),   # 8B mixed 2048 tokens, then the long-context decode scaled down
])
def test_two_calls_second_smaller(first, second):
    b1 = synth.make_config(first[0], small=first[1])
    b2 = synth.make_config(second[0], small=second[1])
    assert b2.num_tokens < b1.num_tokens
    check(b1, first[0] in (2, 4))
    check(b2, second[0] in (2, 4))


def test_refuses_a_batch_larger_than_the_scratch():
    """512 decode sequences of up to 128K keys need more split-KV partials than the scratch
    holds: CB_ERR_WORKSPACE, nothing launched, and the next call still works."""
    dev = "cuda"
    S, Hq, Hkv, D, bs = 512, 32, 8, 128, 16
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((S, Hkv, D), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((8, bs, Hkv, D), dtype=torch.bfloat16, device=dev)
    cu = torch.arange(S + 1, dtype=torch.int32, device=dev)
    kvl = torch.ones(S, dtype=torch.int32, device=dev)
    bt = torch.zeros((S, 8192), dtype=torch.int32, device=dev)
    out = torch.zeros_like(q)
    with pytest.raises(cb.CBError) as ei:
        cb.cb_paged_attention_write_noalloc(q, k, k.clone(), cu, kvl, bt, kc, kc.clone(), out,
                                            0.1, 1, 131072)
    assert ei.value.status == -3
    check(synth.make_config(1), False)
