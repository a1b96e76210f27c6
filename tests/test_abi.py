"""The C-ABI library on the CPU: it loads, exports every entry point include/cbattn.h declares,
rejects host-checkable bad arguments with the documented status codes before touching a GPU,
and its host-only validator enforces the documented preconditions."""
import ctypes
import glob
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import synth
from conftest import ROOT

cb = pytest.importorskip("ragged_paged_kv_amd")

HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cb_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_binding_names():
    assert declared_functions() == sorted(cb.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", cb.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(cb_[a-z0-9_]+)$", out, flags=re.M))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    for f in declared_functions():
        assert hasattr(cb.lib, f)


def test_library_carries_gfx950_code_object():
    # the offload bundle inside the library names its target
    data = open(cb.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in data


def test_status_strings():
    assert cb.cb_status_string(0) == "CB_OK"
    assert cb.cb_status_string(-1) == "CB_ERR_INVALID_ARG"
    assert cb.cb_status_string(-2) == "CB_ERR_UNSUPPORTED"
    assert cb.cb_status_string(-3) == "CB_ERR_WORKSPACE"
    assert cb.cb_status_string(-4) == "CB_ERR_HIP"
    assert cb.cb_status_string(-5) == "CB_ERR_OUT_OF_BLOCKS"
    assert cb.cb_status_string(7) == "CB_ERR_UNKNOWN"


N = None
FAKE = ctypes.c_void_p(0x10000)  # aligned, never dereferenced: every call below fails its checks


def attn(**kw):
    a = dict(q=FAKE, cu=FAKE, kv=FAKE, bt=FAKE, kc=FAKE, vc=FAKE, out=FAKE, scale=0.125, S=4, T=27,
             Hq=4, Hkv=2, D=64, bs=16, mb=3, nb=32, mq=24, mkv=40, split=0, ws=FAKE,
             wsb=1 << 30, stream=N)
    a.update(kw)
    return cb.lib.cb_paged_attention(a["q"], a["cu"], a["kv"], a["bt"], a["kc"], a["vc"], a["out"],
                                     a["scale"], a["S"], a["T"], a["Hq"], a["Hkv"], a["D"], a["bs"],
                                     a["mb"], a["nb"], a["mq"], a["mkv"], a["split"], a["ws"],
                                     a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(bs=3), -1), (dict(bs=0), -1), (dict(Hq=6, Hkv=4), -1), (dict(scale=0.0), -1),
    (dict(scale=float("nan")), -1), (dict(scale=float("inf")), -1), (dict(D=96), -2),
    (dict(Hq=12, Hkv=4), -2), (dict(Hq=64, Hkv=2), -2), (dict(bs=8), -2), (dict(bs=24), -2),
    (dict(q=N), -1), (dict(out=N), -1), (dict(kc=ctypes.c_void_p(0x10008)), -1),
    (dict(ws=N), -3), (dict(wsb=16), -3), (dict(mkv=49), -1), (dict(split=-32), -1),
    (dict(mq=0), -1), (dict(S=-1), -1),
])
def test_paged_attention_host_checks(kw, status):
    st = attn(**kw)
    assert st == status, (st, cb.cb_last_error())
    assert cb.cb_last_error() != ""


def test_empty_batch_is_a_noop():
    assert attn(T=0, q=N, cu=N, kv=N, bt=N, kc=N, vc=N, out=N, ws=N) == 0
    assert attn(S=0, T=0, q=N, cu=N, kv=N, bt=N, kc=N, vc=N, out=N, ws=N) == 0
    assert cb.lib.cb_cache_write(N, N, N, N, N, 0, 2, 64, 16, 32, N) == 0
    assert cb.lib.cb_slot_mapping(N, N, N, 0, 0, 3, 16, N, N) == 0


def test_cache_write_host_checks():
    f = cb.lib.cb_cache_write
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 64, 3, 32, N) == -1       # block_size < 4
    assert f(FAKE, N, FAKE, FAKE, FAKE, 4, 2, 64, 16, 32, N) == -1         # NULL
    assert f(FAKE, FAKE, FAKE, ctypes.c_void_p(0x10002), FAKE, 4, 2, 64, 16, 32, N) == -1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1, 4, 16, 32, N) == -2        # Hkv*D % 8
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, -1, 2, 64, 16, 32, N) == -1


def test_slot_mapping_and_reduce_host_checks():
    assert cb.lib.cb_slot_mapping(FAKE, FAKE, FAKE, 4, 27, 3, 2, FAKE, N) == -1
    assert cb.lib.cb_slot_mapping(FAKE, N, FAKE, 4, 27, 3, 16, FAKE, N) == -1
    assert cb.lib.cb_split_kv_reduce(FAKE, FAKE, FAKE, FAKE, 4, 8, 96, 2, N) == -2
    assert cb.lib.cb_split_kv_reduce(FAKE, N, FAKE, FAKE, 4, 8, 128, 2, N) == -1
    assert cb.lib.cb_split_kv_reduce(FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 0, N) == -1


def test_kernel_timing_hook_host_checks():
    assert cb.lib.cb_time_next_kernel(3, FAKE, FAKE) == -1       # unknown kernel
    assert cb.lib.cb_time_next_kernel(1, N, FAKE) == -1          # NULL event
    assert cb.lib.cb_time_next_kernel(2, FAKE, N) == -1
    assert cb.lib.cb_time_next_kernel(0, N, N) == 0              # clear
    assert cb.lib.cb_time_next_kernel(1, FAKE, FAKE) == 0        # armed ...
    assert cb.lib.cb_time_next_kernel(0, N, N) == 0              # ... and cleared, nothing recorded


def test_workspace_size_and_split_choice():
    # decode-only batch: only partials and the work list
    p = cb.cb_paged_attention_split_tokens(256, 32, 8, 1, 4096)
    assert p % 32 == 0 and 256 <= p <= 4096
    assert cb.cb_paged_attention_split_tokens(4, 4, 2, 1, 40, 100) == 128   # rounded up to 32
    # automatic: ~5461 (partition, KV head) items over the upper-bound keys, steps of 256 keys
    assert cb.cb_paged_attention_split_tokens(256, 32, 8, 1, 4096) == 1536
    assert cb.cb_paged_attention_split_tokens(64, 32, 8, 1, 8192) == 768
    assert cb.cb_paged_attention_split_tokens(16, 32, 8, 1, 131072) == 2048     # the cap
    assert cb.cb_paged_attention_split_tokens(4, 4, 2, 24, 40) == 256         # the floor
    for S, L in ((1, 100000), (300, 3000), (2048, 512), (7, 65536), (1, 40), (16, 2048)):
        p = cb.cb_paged_attention_split_tokens(S, 32, 8, 64, L)
        assert p % 256 == 0 and 256 <= p <= 2048
        p = cb.cb_paged_attention_split_tokens(S, 32, 8, 1, L)
        assert p % 32 == 0 and 32 <= p <= 2048
    # decode-only batches where that gives its floor: about upper-bound keys / 640, at least
    # max_kv_len / 24, at most max(768, max_kv_len / 8), in steps of 64 within [128, 2048]; the
    # longest sequence rounded up to 32 when twice that covers it (one partition each)
    assert cb.cb_paged_attention_split_tokens(8, 32, 8, 1, 583) == 128       # the floor
    assert cb.cb_paged_attention_split_tokens(3, 32, 8, 1, 1816) == 128      # L / 24 = 76
    assert cb.cb_paged_attention_split_tokens(16, 32, 8, 1, 2048) == 448     # 262144 keys / 640
    assert cb.cb_paged_attention_split_tokens(40, 32, 8, 1, 3867) == 768     # capped at 768
    assert cb.cb_paged_attention_split_tokens(8, 32, 8, 1, 16310) == 1664    # cap L / 8 = 2038
    assert cb.cb_paged_attention_split_tokens(1, 32, 8, 1, 116544) == 2048   # L / 24, at most 2048
    assert cb.cb_paged_attention_split_tokens(64, 32, 8, 1, 699) == 704      # one partition each
    assert cb.cb_paged_attention_split_tokens(96, 32, 8, 1, 1500) == 1504    # 2 x 768 >= 1500
    assert cb.cb_paged_attention_split_tokens(4, 4, 2, 1, 40) == 64          # one partition each
    assert cb.cb_paged_attention_split_tokens(1, 32, 8, 1, 0) == 32
    assert cb.cb_paged_attention_split_tokens(64, 32, 8, 1, 4095) == 768     # 2096640 keys
    assert cb.cb_paged_attention_split_tokens(64, 32, 8, 1, 4096) == 512     # the rule above
    assert cb.cb_paged_attention_split_tokens(32, 32, 8, 64, 4096) == 256    # prefill possible
    assert cb.cb_paged_attention_split_tokens(64, 32, 8, 1, 8192) == 768     # above the floor
    # the same rule with prefill-type sequences possible (q > 16 / G)
    assert cb.cb_paged_attention_split_tokens(68, 32, 8, 1024, 8192) == 768
    assert cb.cb_paged_attention_split_tokens(68, 32, 8, 4, 8192) == 768      # q = 4: decode-type
    assert cb.cb_paged_attention_split_tokens(131, 64, 8, 4096, 16384) == 2048
    assert cb.cb_paged_attention_split_tokens(4, 4, 2, 1, 40, 100000) == 2048
    one = cb.cb_paged_attention_workspace_size(4, 27, 4, 2, 64, 16, 24, 40, 64)
    assert one > 0
    assert cb.cb_paged_attention_workspace_size(0, 0, 4, 2, 64, 16, 1, 1) == 0
    # more partitions need more workspace
    assert cb.cb_paged_attention_workspace_size(4, 27, 4, 2, 64, 16, 24, 40, 32) > one


def _valid(batch):
    return oracle.slot_mapping(batch.cu_seqlens_q, batch.kv_lens, batch.block_tables,
                               batch.block_size)


def _v(b, cu=None, kv=None, bt=None, sl=None, bs=None, mq=None, mkv=None):
    return cb.cb_validate_batch(b.cu_seqlens_q if cu is None else cu,
                                b.kv_lens if kv is None else kv,
                                b.block_tables if bt is None else bt,
                                _valid(b) if sl is None else sl,
                                b.block_size if bs is None else bs, b.num_blocks,
                                b.max_q_len if mq is None else mq,
                                b.max_kv_len if mkv is None else mkv, raise_on_error=False)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_validator_accepts_workloads(n):
    b = synth.make_config(n, small=True)
    assert _v(b) == 0, cb.cb_last_error()


def test_validator_rejections():
    b = synth.make_config(5, small=True)
    sl = _valid(b)
    cu = b.cu_seqlens_q.copy()
    # zero-length row: two equal consecutive offsets
    cu0 = np.concatenate([cu[:2], cu[1:]])
    kv0 = np.concatenate([b.kv_lens[:1], [5], b.kv_lens[1:]]).astype(np.int32)
    bt0 = np.concatenate([b.block_tables[:1], b.block_tables[:1], b.block_tables[1:]])
    assert _v(b, cu=cu0, kv=kv0, bt=bt0) == -1 and "zero-length" in cb.cb_last_error()
    # kv_len shorter than the chunk
    kv = b.kv_lens.copy(); kv[-1] = 1
    assert _v(b, kv=kv) == -1
    # block id out of range, and -1 inside the used part of a table
    bt = b.block_tables.copy(); bt[0, 0] = b.num_blocks
    assert _v(b, bt=bt) == -1
    bt = b.block_tables.copy(); bt[0, 0] = -1
    assert _v(b, bt=bt) == -1
    # kv_len beyond the table's capacity
    kv = b.kv_lens.copy(); kv[0] = b.block_tables.shape[1] * b.block_size + 1
    assert _v(b, kv=kv, mkv=int(kv.max())) == -1
    # duplicate slot, slot out of range
    s2 = sl.copy(); s2[1] = s2[0]
    assert _v(b, sl=s2) == -1 and "same slot" in cb.cb_last_error()
    s2 = sl.copy(); s2[0] = b.num_blocks * b.block_size
    assert _v(b, sl=s2) == -1
    # a write into a block that two tables share (needs a copy first)
    shared_blk = int(b.block_tables[b.num_seqs - 1, 0])
    s2 = sl.copy(); s2[0] = shared_blk * b.block_size
    assert _v(b, sl=s2) == -1 and "more than one" in cb.cb_last_error()
    # -1 slots are allowed (skip)
    s2 = sl.copy(); s2[3] = -1
    assert _v(b, sl=s2) == 0
    # bounds
    assert _v(b, mq=b.max_q_len - 1) == -1
    assert _v(b, mkv=b.max_kv_len - 1) == -1
    assert _v(b, bs=3) == -1
    cu2 = cu.copy(); cu2[0] = 1
    assert _v(b, cu=cu2) == -1


def test_graphs_host_checks():
    fake = ctypes.c_void_p(0x10000)
    cfg = cb.GraphsConfig(8, 2, 128, 16, 64, 16, 32, 4, 256, 16, 256, 8, 4, 1, 0.1,
                          fake, fake, fake, fake, fake, fake)
    h = ctypes.c_void_p()
    for field, bad in [("max_seqs", 1), ("block_size", 3), ("token_interval", 0),
                       ("max_kv_len", 257), ("max_graphs", 0), ("scale", float("nan")), ("q", None)]:
        c = cb.GraphsConfig.from_buffer_copy(cfg)
        setattr(c, field, bad)
        assert cb.lib.cb_graphs_create(ctypes.byref(c), ctypes.byref(h)) == -1, field
        assert not h.value
    assert cb.lib.cb_graphs_create(None, ctypes.byref(h)) == -1
    assert cb.lib.cb_graphs_run(None, None, None, None, 0, None, None) == -1
    assert cb.lib.cb_graphs_stats(None, None, None, None, None) == -1
    cb.lib.cb_graphs_destroy(None)


def noalloc(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, kv=FAKE, bt=FAKE, kc=FAKE, vc=FAKE, out=FAKE,
             scale=0.125, S=4, T=27, Hq=4, Hkv=2, D=64, bs=16, mb=3, nb=32, mq=24, mkv=40, split=0,
             stream=N)
    a.update(kw)
    return cb.lib.cb_paged_attention_write_noalloc(
        a["q"], a["k"], a["v"], a["cu"], a["kv"], a["bt"], a["kc"], a["vc"], a["out"], a["scale"],
        a["S"], a["T"], a["Hq"], a["Hkv"], a["D"], a["bs"], a["mb"], a["nb"], a["mq"], a["mkv"],
        a["split"], a["stream"])


def test_noalloc_host_checks():
    """The no-allocation entry point takes the fused entry point's host checks, and a batch whose
    work needs more than the library's scratch is refused with both sizes in the message, before
    anything touches a GPU."""
    for kw, status in ((dict(bs=3), -1), (dict(D=96), -2), (dict(k=N), -1),
                       (dict(v=ctypes.c_void_p(0x10008)), -1), (dict(scale=0.0), -1),
                       (dict(mkv=49), -1)):
        assert noalloc(**kw) == status, (kw, cb.cb_last_error())
    assert noalloc(T=0, q=N, k=N, v=N, cu=N, kv=N, bt=N, kc=N, vc=N, out=N) == 0
    # 512 decode sequences of up to 128K keys, 32 query heads: the split-KV partials alone are
    # 512 x 64 partitions x 32 heads x 129 floats = 541 MB
    big = dict(S=512, T=512, Hq=32, Hkv=8, D=128, mb=8192, nb=1 << 17, mq=1, mkv=131072)
    need = cb.cb_paged_attention_workspace_size(512, 512, 32, 8, 128, 16, 1, 131072, 0)
    assert need > cb.CB_NOALLOC_SCRATCH_BYTES
    assert noalloc(**big) == -3
    msg = cb.cb_last_error()
    assert str(need) in msg and str(cb.CB_NOALLOC_SCRATCH_BYTES) in msg, msg


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "cbattn.h")).read()
    m = re.search(r"#define CB_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == cb.CB_NOALLOC_SCRATCH_BYTES


def test_stream_read_host_checks():
    f = cb.lib.cb_stream_read
    sink = ctypes.c_void_p(0x20000)
    assert f(FAKE, 0, N, 0, N) == 0                                 # nothing to read: no launch
    assert f(N, 1024, sink, 256, N) == -1                           # NULL buffer
    assert f(FAKE, 1024, N, 256, N) == -1                           # NULL sink
    assert f(ctypes.c_void_p(0x10008), 1024, sink, 256, N) == -1    # misaligned
    assert f(FAKE, 1000, sink, 256, N) == -1                        # not a multiple of 16 bytes
    assert f(FAKE, 1024, sink, 255, N) == -1                        # sink below 256 words
