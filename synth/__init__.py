"""Seeded synthetic inputs for one ragged paged-attention step.

This module builds the *inputs* of a forward pass the way a continuous-batching
engine would hand them to its attention layer: a packed query batch with no
batch axis delimited by ``cu_seqlens_q`` (ragged batching, "Continuous batching
from first principles", Takeaways), per-sequence KV lengths, per-sequence block
tables into a pool of fixed-size physical blocks ("3.3 Batching & Memory
Management", section "PagedAttention: block tables"), the paged K/V cache
holding every sequence's earlier tokens, and the new K/V rows of this step.

It holds none of the attention arithmetic and none of the slot arithmetic that
the method computes; both the oracle and the HIP path consume what it returns.
The cache is filled block by block from the block-table definition (logical
block j of a sequence covers its token positions [j*bs, (j+1)*bs)), which is
how the input is laid out, not a step of the method.

Every value is bf16, carried as uint16 bit patterns. Slots nobody may read
(block tails past a sequence's length, unassigned blocks, the positions this
step is about to write) hold the bf16 quiet NaN 0x7FC0, and unused block-table
entries hold -1, so a kernel that touches them shows it.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

POISON_BF16 = np.uint16(0x7FC0)  # bf16 quiet NaN

__all__ = [
    "Batch",
    "SeqSpec",
    "POISON_BF16",
    "bf16_from_f32",
    "f32_from_bf16",
    "build_batch",
    "make_config",
    "CONFIG_NAMES",
]


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16(u: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_CHUNK = 1 << 20  # values per independent random stream
_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                      else (os.cpu_count() or 1)))


def _scale_bf16(b: np.ndarray, mul: float) -> np.ndarray:
    """bf16 values times a power of two (exact), as new uint16 bits."""
    return bf16_from_f32(f32_from_bf16(b) * np.float32(mul))


def _normal_bf16(key: tuple, shape, k_mul: float = 1.0) -> np.ndarray:
    """N(0,1) draws rounded to bf16, as uint16 bits.

    The array is cut into fixed chunks of ``_CHUNK`` values; chunk c is drawn from its own
    stream ``default_rng([*key, c])``, so the result depends only on ``key`` and ``shape``
    (not on thread count or scheduling). ``k_mul`` (a power of two) scales after rounding,
    which is exact in bf16.
    """
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=np.uint16)

    def fill(c):
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        x = np.random.default_rng([*key, c]).standard_normal(hi - lo, dtype=np.float32)
        if k_mul != 1.0:
            x = f32_from_bf16(bf16_from_f32(x)) * np.float32(k_mul)
        out[lo:hi] = bf16_from_f32(x)

    nchunks = -(-n // _CHUNK)
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(min(_THREADS, nchunks)) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


@dataclasses.dataclass
class SeqSpec:
    """One sequence of the step: ``q`` new query tokens, ``L`` KV tokens after the write.

    ``shared`` names a prefix group: every sequence with the same group maps its first
    ``shared_tokens // block_size`` logical blocks to the same physical blocks.
    ``k_mul`` multiplies this sequence's K values (cached and new) by a power of two.
    """

    q: int
    L: int
    shared: int | None = None
    k_mul: float = 1.0


@dataclasses.dataclass
class Batch:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float                 # fp32 value of the softmax scale
    q_lens: np.ndarray           # int32 [S]
    kv_lens: np.ndarray          # int32 [S]
    cu_seqlens_q: np.ndarray     # int32 [S+1]
    block_tables: np.ndarray     # int32 [S, max_blocks_per_seq], -1 where unused
    k_cache: np.ndarray          # uint16 [num_blocks, block_size, Hkv, D] before this step's write
    v_cache: np.ndarray          # uint16 same
    q: np.ndarray                # uint16 [T, Hq, D]
    k: np.ndarray                # uint16 [T, Hkv, D] new keys of this step
    v: np.ndarray                # uint16 [T, Hkv, D]
    specs: list                  # list[SeqSpec]
    shared_prefix_tokens: int = 0

    @property
    def num_seqs(self) -> int:
        return int(self.q_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_lens.max()) if self.num_seqs else 0

    def describe(self) -> dict:
        return {
            "name": self.name, "seed": self.seed, "S": self.num_seqs, "T": self.num_tokens,
            "Hq": self.num_q_heads, "Hkv": self.num_kv_heads, "D": self.head_dim,
            "block_size": self.block_size, "num_blocks": self.num_blocks,
            "q_lens": self.q_lens.tolist(), "kv_lens": self.kv_lens.tolist(),
        }


def build_batch(name: str, seed: int, rng: np.random.Generator, specs: list, *,
                num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                num_blocks: int | None = None, shared_prefix_tokens: int = 0,
                scale: float | None = None, max_blocks_per_seq: int | None = None) -> Batch:
    """Allocate blocks, fill the cache with each sequence's earlier tokens, draw new K/V and Q.

    ``rng`` (already used for lengths and composition) draws the block permutation; the
    values come from keyed streams (seed, what): 1 = cached K, 2 = cached V (history of all
    sequences, concatenated in sequence order), 3 = new K, 4 = new V, 5 = Q.
    """
    bs = int(block_size)
    S = len(specs)
    Hkv, D, Hq = int(num_kv_heads), int(head_dim), int(num_q_heads)
    nblk = [(-(-s.L // bs)) for s in specs]  # ceil-div: blocks a sequence occupies
    n_shared = shared_prefix_tokens // bs if shared_prefix_tokens else 0
    groups = sorted({s.shared for s in specs if s.shared is not None})
    private = sum(nb - (n_shared if s.shared is not None else 0) for s, nb in zip(specs, nblk))
    needed = private + n_shared * len(groups)
    if num_blocks is None:
        num_blocks = needed + max(8, needed // 4)
    if needed > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks cannot hold {needed}")
    width = max_blocks_per_seq if max_blocks_per_seq is not None else max(nblk + [1])

    perm = rng.permutation(num_blocks).astype(np.int32)
    cursor = 0
    group_blocks = {}
    for gid in groups:
        group_blocks[gid] = perm[cursor:cursor + n_shared]
        cursor += n_shared
    tables = np.full((S, width), -1, dtype=np.int32)
    for i, (s, nb) in enumerate(zip(specs, nblk)):
        if s.shared is not None:
            if s.L <= shared_prefix_tokens:
                raise ValueError("a sharer must own tokens past the shared prefix")
            tables[i, :n_shared] = group_blocks[s.shared]
            k0 = n_shared
        else:
            k0 = 0
        tables[i, k0:nb] = perm[cursor:cursor + (nb - k0)]
        cursor += nb - k0

    k_cache = np.full((num_blocks, bs, Hkv, D), POISON_BF16, dtype=np.uint16)
    v_cache = np.full((num_blocks, bs, Hkv, D), POISON_BF16, dtype=np.uint16)
    # which positions each sequence must fill: [start, L - q); a shared prefix is filled once
    fills = []
    group_filled = set()
    for i, s in enumerate(specs):
        hist = s.L - s.q  # tokens already in the cache before this step
        start = 0
        if s.shared is not None and hist > 0:
            if s.shared in group_filled:
                start = shared_prefix_tokens  # prefix blocks already hold the shared history
            group_filled.add(s.shared)
        fills.append((start, max(0, hist - start)))
    total = sum(n for _, n in fills)
    k_hist = _normal_bf16((seed, 1), (total, Hkv, D))
    v_hist = _normal_bf16((seed, 2), (total, Hkv, D))
    off = 0
    for i, (s, (start, n)) in enumerate(zip(specs, fills)):
        if n == 0:
            continue
        kh = k_hist[off:off + n]
        vh = v_hist[off:off + n]
        off += n
        if s.k_mul != 1.0:
            kh = _scale_bf16(kh, s.k_mul)
        # logical block j covers positions [j*bs, (j+1)*bs); start is a block boundary
        j0 = start // bs
        nfull = n // bs
        if nfull:
            ids = tables[i, j0:j0 + nfull]
            k_cache[ids] = kh[:nfull * bs].reshape(nfull, bs, Hkv, D)
            v_cache[ids] = vh[:nfull * bs].reshape(nfull, bs, Hkv, D)
        rem = n - nfull * bs
        if rem:
            b = tables[i, j0 + nfull]
            k_cache[b, :rem] = kh[nfull * bs:]
            v_cache[b, :rem] = vh[nfull * bs:]
    del k_hist, v_hist

    q_lens = np.array([s.q for s in specs], dtype=np.int32)
    kv_lens = np.array([s.L for s in specs], dtype=np.int32)
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    T = int(cu[-1])
    k = _normal_bf16((seed, 3), (T, Hkv, D))
    v = _normal_bf16((seed, 4), (T, Hkv, D))
    for i, s in enumerate(specs):
        if s.k_mul != 1.0:
            k[cu[i]:cu[i + 1]] = _scale_bf16(k[cu[i]:cu[i + 1]], s.k_mul)
    q = _normal_bf16((seed, 5), (T, Hq, D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Batch(name=name, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                 block_size=bs, num_blocks=int(num_blocks), scale=float(np.float32(scale)),
                 q_lens=q_lens, kv_lens=kv_lens, cu_seqlens_q=cu, block_tables=tables,
                 k_cache=k_cache, v_cache=v_cache, q=q, k=k, v=v, specs=list(specs),
                 shared_prefix_tokens=int(shared_prefix_tokens))


CONFIG_NAMES = {
    1: "tiny-ragged-4q2kv-d64-bs16",
    2: "llama3-8b-decode-256seq-bs16",
    3: "llama3-8b-mixed-2048tok-bs16",
    4: "llama3-8b-longctx-decode-16seq-bs16",
    5: "llama-70b-mixed-8192tok-shared-prefix-bs32",
}


def _uniform(rng, a, b, n):
    return [int(x) for x in rng.integers(a, b + 1, size=n)]


def make_config(n: int, small: bool = False, seed: int | None = None) -> Batch:
    """The five workload shapes; ``small=True`` gives a scaled-down copy of the same mix.

    Full sizes:
      1  4 q-heads / 2 kv-heads, D 64, bs 16, 32-block pool: decodes at L 17, 40, 5, then
         one 24-token prompt (q = L = 24).
      2  32/8, D 128, bs 16: 256 decodes, L ~ U[128, 4096].
      3  32/8, D 128, bs 16, 2048 tokens: 64 decodes L ~ U[256, 8192], a 1024-token chunk
         at offset 2048 (L = 3072), and three new 320-token prompts.
      4  32/8, D 128, bs 16: 16 decodes, L ~ U[32768, 131072]; sequence 0 has K x 8.
      5  64/8, D 128, bs 32, 8192 tokens: 128 decodes L ~ U[512, 16384], a 4096-token chunk
         at offset 4096, a new 2048-token prompt, and a 1920-token chunk at offset 2048 whose
         first 2048 tokens are a shared prefix; 32 decodes with L >= 2049 share it too.
    Packed order: decodes first, then prefill chunks.
    """
    if n == 1:
        small = False  # already tiny
    if seed is None:
        seed = 1000 + n + (100 if small else 0)
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[n] + ("-small" if small else "")
    if n == 1:
        specs = [SeqSpec(1, 17), SeqSpec(1, 40), SeqSpec(1, 5), SeqSpec(24, 24)]
        return build_batch(name, seed, rng, specs, num_q_heads=4, num_kv_heads=2, head_dim=64,
                           block_size=16, num_blocks=32, scale=1.0 / 8.0)
    if n == 2:
        cnt, lo, hi = (24, 2, 300) if small else (256, 128, 4096)
        specs = [SeqSpec(1, L) for L in _uniform(rng, lo, hi, cnt)]
        return build_batch(name, seed, rng, specs, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=16)
    if n == 3:
        if small:
            dec = [SeqSpec(1, L) for L in _uniform(rng, 16, 512, 8)]
            pre = [SeqSpec(64, 192)] + [SeqSpec(40, 40) for _ in range(3)]
        else:
            dec = [SeqSpec(1, L) for L in _uniform(rng, 256, 8192, 64)]
            pre = [SeqSpec(1024, 3072)] + [SeqSpec(320, 320) for _ in range(3)]
        return build_batch(name, seed, rng, dec + pre, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=16)
    if n == 4:
        cnt, lo, hi = (4, 1024, 4096) if small else (16, 32768, 131072)
        Ls = _uniform(rng, lo, hi, cnt)
        specs = [SeqSpec(1, L, k_mul=(8.0 if i == 0 else 1.0)) for i, L in enumerate(Ls)]
        return build_batch(name, seed, rng, specs, num_q_heads=32, num_kv_heads=8,
                           head_dim=128, block_size=16)
    if n == 5:
        if small:
            ndec, lo, hi, pref, nshare = 12, 32, 1024, 128, 3
            chunks = [(256, 512), (128, 128), (120, 248)]
        else:
            ndec, lo, hi, pref, nshare = 128, 512, 16384, 2048, 32
            chunks = [(4096, 8192), (2048, 2048), (1920, 3968)]
        Ls = _uniform(rng, lo, hi, ndec)
        eligible = [i for i, L in enumerate(Ls) if L >= pref + 1]
        sharers = set(int(i) for i in rng.choice(eligible, size=min(nshare, len(eligible)),
                                                 replace=False))
        specs = [SeqSpec(1, L, shared=(0 if i in sharers else None)) for i, L in enumerate(Ls)]
        specs += [SeqSpec(chunks[0][0], chunks[0][1]), SeqSpec(chunks[1][0], chunks[1][1]),
                  SeqSpec(chunks[2][0], chunks[2][1], shared=0)]
        return build_batch(name, seed, rng, specs, num_q_heads=64, num_kv_heads=8,
                           head_dim=128, block_size=32, shared_prefix_tokens=pref)
    raise ValueError(f"unknown config {n}")
