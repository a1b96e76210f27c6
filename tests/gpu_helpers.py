"""Shared GPU-side helpers for the parity tests: upload a synthetic batch, run the step through
the C ABI (slot mapping -> cache write -> paged attention), read results back."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth


def dev_bf16(a: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def dev_i32(a: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def host_u16(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class Step:
    """One forward pass of the hot path for ``batch`` on ``device``."""

    def __init__(self, batch: synth.Batch, device="cuda", kv_split_tokens: int = 0,
                 max_q_len=None, max_kv_len=None):
        import torch
        import ragged_paged_kv_amd as cb
        self.cb = cb
        self.b = batch
        self.max_q_len = batch.max_q_len if max_q_len is None else int(max_q_len)
        self.max_kv_len = batch.max_kv_len if max_kv_len is None else int(max_kv_len)
        # host-side precondition check before anything reaches the GPU
        cb.cb_validate_batch(batch.cu_seqlens_q, batch.kv_lens, batch.block_tables, None,
                             batch.block_size, batch.num_blocks, self.max_q_len, self.max_kv_len)
        self.device = device
        self.split = int(kv_split_tokens)
        self.q = dev_bf16(batch.q, device)
        self.k = dev_bf16(batch.k, device)
        self.v = dev_bf16(batch.v, device)
        self.k_cache = dev_bf16(batch.k_cache, device)
        self.v_cache = dev_bf16(batch.v_cache, device)
        self.cu = dev_i32(batch.cu_seqlens_q, device)
        self.kv_lens = dev_i32(batch.kv_lens, device)
        self.tables = dev_i32(batch.block_tables, device)
        T = batch.num_tokens
        self.slots = torch.full((T,), -7, dtype=torch.int32, device=device)
        self.out = torch.full((T, batch.num_q_heads, batch.head_dim), float("nan"),
                              dtype=torch.bfloat16, device=device)
        self.ws = cb.alloc_workspace(batch.num_seqs, T, batch.num_q_heads, batch.num_kv_heads,
                                     batch.head_dim, batch.block_size, self.max_q_len,
                                     self.max_kv_len, self.split, device=device)

    def slot_mapping(self):
        self.cb.cb_slot_mapping(self.cu, self.kv_lens, self.tables, self.slots, self.b.block_size)

    def cache_write(self):
        self.cb.cb_cache_write(self.k, self.v, self.slots, self.k_cache, self.v_cache)

    def attention(self):
        self.cb.cb_paged_attention(self.q, self.cu, self.kv_lens, self.tables, self.k_cache,
                                   self.v_cache, self.out, self.b.scale, self.max_q_len,
                                   self.max_kv_len, self.ws, kv_split_tokens=self.split)

    def run(self):
        import torch
        self.slot_mapping()
        self.cache_write()
        self.attention()
        torch.cuda.synchronize()
        return self

    def out_u16(self):
        return host_u16(self.out)

    def out_f64(self):
        return oracle.bf16_to_f64(self.out_u16())

    def slots_host(self):
        return self.slots.cpu().numpy()


def oracle_step(batch: synth.Batch, tokens=None):
    """(slots, (k_cache, v_cache), out, lse) from the oracle for ``batch``."""
    sl = oracle.slot_mapping(batch.cu_seqlens_q, batch.kv_lens, batch.block_tables,
                             batch.block_size)
    kc, vc = oracle.cache_write(batch.k_cache, batch.v_cache, batch.k, batch.v, sl)
    out, lse = oracle.paged_attention(batch.q, batch.cu_seqlens_q, batch.kv_lens,
                                      batch.block_tables, kc, vc, batch.scale, tokens=tokens)
    return sl, (kc, vc), out, lse


def assert_close(got, ref, where=""):
    """The attention bound: |d| <= 2e-2 + 1e-2 |ref| elementwise, and max |d| <= 2e-2 on its own
    (the max-abs half of the bound, without the relative allowance)."""
    ok, rep = oracle.within_tolerance(got, ref)
    assert ok, f"{where}: outside |d| <= 2e-2 + 1e-2|ref|: {rep}"
    assert rep["max_abs"] <= oracle.ATOL, f"{where}: max |d| above 2e-2: {rep}"
    return rep


def readable_mask(batch: synth.Batch) -> np.ndarray:
    """bool [num_blocks, block_size]: slots at positions < L of some sequence (after the write)."""
    m = np.zeros((batch.num_blocks, batch.block_size), dtype=bool)
    bs = batch.block_size
    for s in range(batch.num_seqs):
        L = int(batch.kv_lens[s])
        nfull, rem = divmod(L, bs)
        row = batch.block_tables[s]
        m[row[:nfull]] = True
        if rem:
            m[row[nfull], :rem] = True
    return m
