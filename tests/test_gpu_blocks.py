"""GPU parity of the block manager's data path: cb_copy_blocks against the oracle's copy (bit
exact), and serving steps driven by the library's block manager (prefix reuse, forks with
copy-on-write, chunked prefill, decode, eviction) whose attention output, read through shared
block tables, must match the oracle's attention over each sequence's own contiguous KV."""
import ctypes

import numpy as np
import pytest

import oracle
import oracle.blocks as ob
from gpu_helpers import dev_bf16, dev_i32, host_u16, say
from serving_helpers import rand_bf16, serving_run

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
cb = pytest.importorskip("ragged_paged_kv_amd")


def copy_pairs(rng, nb, n):
    ids = rng.permutation(nb)
    return ids[:n].astype(np.int32), ids[n:2 * n].astype(np.int32)   # disjoint src and dst


@pytest.mark.parametrize("layers,nb,bs,hkv,d,n", [
    (1, 64, 16, 8, 128, 17),      # 32 KiB blocks: two workgroups per block and tensor
    (3, 40, 16, 2, 64, 9),        # 4 KiB blocks, layer stride
    (1, 32, 48, 1, 64, 5),        # 6 KiB blocks: a partial workgroup chunk
    (2, 1024, 16, 8, 128, 500),   # many pairs
])
def test_copy_blocks_bit_exact(layers, nb, bs, hkv, d, n):
    rng = np.random.default_rng(layers * 1000 + nb + n)
    shape = ((layers,) if layers > 1 else ()) + (nb, bs, hkv, d)
    say(f"copy_blocks layers={layers} nb={nb} bs={bs} hkv={hkv} d={d} n={n}")
    k, v = rand_bf16(rng, shape), rand_bf16(rng, shape)
    src, dst = copy_pairs(rng, nb, n)
    # pairs with an id out of range, and a block onto itself, are skipped
    spare = int(rng.permutation(nb)[0])
    src = np.concatenate([src, [nb, -1, spare]]).astype(np.int32)
    dst = np.concatenate([dst, [spare, spare, spare]]).astype(np.int32)
    ek, ev = ob.copy_blocks(k, v, src, dst)
    kd, vd = dev_bf16(k, "cuda"), dev_bf16(v, "cuda")
    cb.cb_copy_blocks(kd, vd, dev_i32(src, "cuda"), dev_i32(dst, "cuda"), num_layers=layers)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(kd), ek)
    assert np.array_equal(host_u16(vd), ev)


# ---------------------------------------------------------------------------------------------
# serving steps through the block manager


class GpuBackend:
    def __init__(self, kc, vc, num_slots):
        self.kc, self.vc = dev_bf16(kc, "cuda"), dev_bf16(vc, "cuda")
        self.pool = torch.zeros((num_slots, 2, 1) + tuple(self.kc.shape[1:]), dtype=torch.bfloat16,
                                pin_memory=True)

    def step(self, src, dst, outs, ins, knew, vnew, slots, q, cu, kv_lens, tables, scale, max_q,
             max_kv):
        if src.size:
            cb.cb_copy_blocks(self.kc, self.vc, dev_i32(src, "cuda"), dev_i32(dst, "cuda"))
        if len(outs[0]):
            cb.cb_swap_out_blocks(self.kc, self.vc, dev_i32(np.array(outs[0]), "cuda"),
                                  dev_i32(np.array(outs[1]), "cuda"), self.pool)
        if len(ins[0]):
            cb.cb_swap_in_blocks(self.pool, dev_i32(np.array(ins[0]), "cuda"),
                                 dev_i32(np.array(ins[1]), "cuda"), self.kc, self.vc)
        if q is None:
            torch.cuda.synchronize()
            return None
        cb.cb_cache_write(dev_bf16(knew, "cuda"), dev_bf16(vnew, "cuda"), dev_i32(slots, "cuda"),
                          self.kc, self.vc)
        T, hq, d = q.shape
        out = torch.full((T, hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
        ws = cb.alloc_workspace(len(kv_lens), T, hq, self.kc.shape[2], d, self.kc.shape[1], max_q,
                                max_kv)
        cb.cb_paged_attention(dev_bf16(q, "cuda"), dev_i32(cu, "cuda"), dev_i32(kv_lens, "cuda"),
                              dev_i32(tables, "cuda"), self.kc, self.vc, out, scale, max_q, max_kv,
                              ws)
        torch.cuda.synchronize()
        return oracle.bf16_to_f64(host_u16(out))


@pytest.mark.parametrize("hq,hkv,d,bs,nb", [(8, 2, 128, 16, 96), (4, 4, 64, 32, 40)])
def test_serving_steps_through_block_manager(hq, hkv, d, bs, nb):
    stats = serving_run(cb, GpuBackend, hq, hkv, d, bs, nb, seed=hq * 100 + d + bs, log=say)
    assert stats["hits"] > 0 and stats["copies"] > 0 and stats["steps"] >= 20
    assert stats["swap_outs"] > 0 and stats["swap_ins"] > 0


@pytest.mark.parametrize("layers,nb,bs,hkv,d,n,num_slots", [
    (1, 64, 16, 8, 128, 9, 20),       # 32 KiB blocks
    (3, 40, 16, 2, 64, 5, 8),         # layer stride, 4 KiB blocks
    (2, 512, 16, 8, 128, 200, 256),   # many pairs
])
def test_swap_blocks_bit_exact(layers, nb, bs, hkv, d, n, num_slots):
    rng = np.random.default_rng(layers * 7 + nb + n)
    shape = ((layers,) if layers > 1 else ()) + (nb, bs, hkv, d)
    say(f"swap layers={layers} nb={nb} n={n} slots={num_slots}")
    k, v = rand_bf16(rng, shape), rand_bf16(rng, shape)
    pool0 = rand_bf16(rng, (num_slots, 2, layers, bs, hkv, d))
    blocks = rng.permutation(nb)[:n].astype(np.int32)
    slots = rng.permutation(num_slots)[:n].astype(np.int32)
    # pairs with an id out of range are skipped (a block past the pool; a slot past the pool)
    blocks_x = np.concatenate([blocks, [nb, 0]]).astype(np.int32)
    slots_x = np.concatenate([slots, [int(slots[0]), num_slots]]).astype(np.int32)
    pool = torch.from_numpy(pool0.view(np.int16)).view(torch.bfloat16).pin_memory()
    kd, vd = dev_bf16(k, "cuda"), dev_bf16(v, "cuda")
    cb.cb_swap_out_blocks(kd, vd, dev_i32(blocks_x, "cuda"), dev_i32(slots_x, "cuda"), pool,
                          num_layers=layers)
    torch.cuda.synchronize()
    want_pool = ob.swap_out_blocks(k, v, blocks_x, slots_x, pool0)
    assert np.array_equal(pool.view(torch.int16).numpy().view(np.uint16), want_pool)
    # scatter back into other blocks
    dst = rng.permutation(nb)[:n].astype(np.int32)
    dst_x = np.concatenate([dst, [-1, nb]]).astype(np.int32)
    cb.cb_swap_in_blocks(pool, dev_i32(slots_x, "cuda"), dev_i32(dst_x, "cuda"), kd, vd,
                         num_layers=layers)
    torch.cuda.synchronize()
    ek, ev = ob.swap_in_blocks(want_pool, slots_x, dst_x, k, v)
    assert np.array_equal(host_u16(kd), ek) and np.array_equal(host_u16(vd), ev)


def test_swap_refuses_pageable_pool():
    kd = torch.zeros((8, 16, 2, 64), dtype=torch.bfloat16, device="cuda")
    idx = dev_i32(np.array([0], np.int32), "cuda")
    pageable = np.zeros((2, 2, 1, 16, 2, 64), np.uint16)
    st = cb.lib.cb_swap_out_blocks(ctypes.c_void_p(kd.data_ptr()), ctypes.c_void_p(kd.data_ptr()),
                                   ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(idx.data_ptr()), 1,
                                   ctypes.c_void_p(pageable.ctypes.data), 2, 16 * 2 * 64 * 2, 8, 1, 0,
                                   None)
    assert st == -1
