"""Plant plausible mistakes in copies of the oracle (on the CPU) and require that some pin
catches each one. This shows the pins would notice a dropped term, a wrong index or sign, or
a transposed operand, rather than agreeing with whatever the oracle computes."""
import os
import types

import pytest

import oracle
import synth
from conftest import ROOT, read_golden
from pins import (pin_bruteforce, pin_cache_write, pin_gqa_mapping, pin_hand_cases,
                  pin_permutation_invariance, pin_sdpa, pin_single_key,
                  pin_slot_mapping_bruteforce, pin_slot_mapping_p3, pin_split_merge,
                  pin_uniform_prefix_means)

SRC = open(os.path.join(ROOT, "oracle", "attention.py")).read()

MUTANTS = {
    # causal alignment from the top-left instead of L - q + i
    "causal-top-left": ("last = np.repeat(L - qn + ii, G)", "last = np.repeat(ii, G)", 2),
    # off-by-one in the causal limit
    "causal-off-by-one": ("visible = j <= last_key[:, None]", "visible = j < last_key[:, None]", 1),
    # query head h reads the wrong KV head
    "gqa-wrong-head": ("Q = bf16_to_f64(q[t, g * G:(g + 1) * G]).reshape(-1, D)  # [len(ii) * G, D]",
                       "Q = bf16_to_f64(q[t, g::Hkv][:, :G]).reshape(-1, D)", 1),
    # the softmax scale is dropped
    "no-scale": ("z = scale * (qrows @ K.T)", "z = qrows @ K.T", 1),
    # the softmax is not normalised
    "no-normalise": ("out = (w @ V) / np.where(empty, 1.0, ssum)[:, None]", "out = (w @ V)", 1),
    # K used in place of V
    "k-for-v": ("V = unpage(v_cache, block_tables[s], L, g)\n            for c0",
                "V = unpage(k_cache, block_tables[s], L, g)\n            for c0", 1),
    # offsets within a block reversed when reading
    "unpage-reversed-offset": ("rows = cache[table_row[p // bs], p % bs, kv_head]",
                               "rows = cache[table_row[p // bs], bs - 1 - p % bs, kv_head]", 1),
    # slot arithmetic: offset taken from the wrong position
    "slot-offset": ("out[cu[s] + i] = blk * bs + p % bs", "out[cu[s] + i] = blk * bs + i % bs", 1),
    # slot arithmetic: the block id is not multiplied by the block size
    "slot-no-stride": ("out[cu[s] + i] = blk * bs + p % bs", "out[cu[s] + i] = blk + p % bs", 1),
    # cache write puts V rows into the K cache
    "write-swap": ("kflat[slot] = k[t]", "kflat[slot] = v[t]", 1),
    # merge forgets the max shift's weight for each range
    "merge-unweighted": ("num = (w[:, :, None] * o).sum(axis=1)", "num = o.sum(axis=1)", 1),
    # merge lets an empty range's undefined o through
    "merge-empty-range": ("o = np.where(nonempty[:, :, None], o_part[t, :, :n], 0.0)",
                          "o = o_part[t, :, :n]", 1),
    # lse misses the max term
    "lse-no-max": ("lse = np.where(empty, -np.inf, m[:, 0] + np.log(np.where(empty, 1.0, ssum)))",
                   "lse = np.where(empty, -np.inf, np.log(np.where(empty, 1.0, ssum)))", 1),
}


def mutant(name):
    old, new, count = MUTANTS[name]
    assert SRC.count(old) == count, f"mutation site for {name} not found exactly {count} time(s)"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SRC.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in dir(oracle) if not k.startswith("_")})
    for k in ("slot_mapping", "cache_write", "unpage", "paged_attention", "split_partials",
              "merge_partials", "within_tolerance"):
        setattr(ns, k, getattr(mod, k))
    return ns


def _tiny():
    from test_oracle_pins import _tiny_mixed
    return _tiny_mixed(21)


PINS = [
    ("slot-p3", lambda o: pin_slot_mapping_p3(o, read_golden("p3_block_table_example.txt"))),
    ("slot-brute", lambda o: pin_slot_mapping_bruteforce(o)),
    ("cache-write", lambda o: pin_cache_write(o)),
    ("single-key", lambda o: pin_single_key(o)),
    ("prefix-means", lambda o: pin_uniform_prefix_means(o)),
    ("hand", lambda o: pin_hand_cases(o)),
    ("gqa", lambda o: pin_gqa_mapping(o)),
    ("sdpa", lambda o: pin_sdpa(o)),
    ("brute-config1", lambda o: pin_bruteforce(o, synth.make_config(1))),
    ("brute-tiny", lambda o: pin_bruteforce(o, _tiny())),
    ("permutation", lambda o: pin_permutation_invariance(o, _tiny())),
    ("split-merge", lambda o: pin_split_merge(o, _tiny())),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    orc = mutant(name)
    caught = []
    for pname, pin in PINS:
        try:
            pin(orc)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught.append(pname)
    assert caught, f"no pin catches the planted mistake {name}"


def test_unmutated_copy_passes_every_pin():
    mod = types.ModuleType("oracle_copy")
    exec(compile(SRC, "<copy>", "exec"), mod.__dict__)
    ns = types.SimpleNamespace(**{k: getattr(oracle, k) for k in dir(oracle) if not k.startswith("_")})
    for k in ("slot_mapping", "cache_write", "unpage", "paged_attention", "split_partials",
              "merge_partials"):
        setattr(ns, k, getattr(mod, k))
    for _, pin in PINS:
        pin(ns)
