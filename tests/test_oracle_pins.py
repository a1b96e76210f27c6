"""The oracle against the pages' printed values, closed forms, a library routine, an
independent brute-force formulation and invariants (CPU only)."""
import numpy as np
import pytest

import oracle
import synth
from pins import (pin_block_arithmetic, pin_bruteforce, pin_cache_write, pin_gqa_mapping,
                  pin_hand_cases, pin_padding_closed_form, pin_padding_waste,
                  pin_permutation_invariance, pin_sdpa, pin_single_key, pin_slot_mapping_bruteforce,
                  pin_slot_mapping_p3, pin_split_merge, pin_tolerance, pin_uniform_prefix_means,
                  tiny_batch)


def test_padding_waste_printed_values(golden):
    pin_padding_waste(oracle, golden("padding_waste.txt"))


def test_padding_waste_closed_form():
    pin_padding_closed_form(oracle)


def test_zero_length_row_raises():
    with pytest.raises(ValueError):
        oracle.rectangle_count([100, 0, 1])
    with pytest.raises(ValueError):
        oracle.pack_ragged([np.zeros((3, 2)), np.zeros((0, 2))])


def test_block_arithmetic_printed_values(golden):
    pin_block_arithmetic(oracle, golden("block_arithmetic.txt"))


def test_block_size_below_four_raises():
    for bad in (0, 1, 2, 3):
        with pytest.raises(ValueError):
            oracle.block_layout(10, bad)
    assert oracle.block_layout(10, 4) == {"blocks": 3, "unused_tail": 2}


def test_page_bytes_per_token(golden):
    # bytes of K + V for one token in one layer at the 8-KV-head, D-128, bf16 shape
    rows = {r[0]: r[1:] for r in golden("block_arithmetic.txt")}
    assert 2 * 8 * 128 * 2 == int(rows["page_bytes"][0])


def test_slot_mapping_worked_example(golden):
    pin_slot_mapping_p3(oracle, golden("p3_block_table_example.txt"))


def test_slot_mapping_bruteforce():
    pin_slot_mapping_bruteforce(oracle)


def test_cache_write():
    pin_cache_write(oracle)


def test_single_key_returns_value():
    pin_single_key(oracle)


def test_uniform_scores_give_prefix_means():
    pin_uniform_prefix_means(oracle)


def test_hand_cases():
    pin_hand_cases(oracle)


def test_gqa_head_mapping():
    pin_gqa_mapping(oracle)


def test_sdpa_library_case():
    pin_sdpa(oracle)


def _tiny_mixed(seed):
    specs = [synth.SeqSpec(1, 9), synth.SeqSpec(1, 13, shared=0), synth.SeqSpec(2, 7),
             synth.SeqSpec(6, 6), synth.SeqSpec(5, 14, shared=0), synth.SeqSpec(1, 1),
             synth.SeqSpec(3, 11, k_mul=8.0)]
    return tiny_batch(specs, 8, 2, 16, 4, seed, shared_prefix_tokens=8)


BRUTE = {
    "config1": lambda: synth.make_config(1),
    "config2-small": lambda: synth.make_config(2, small=True),
    "config3-small": lambda: synth.make_config(3, small=True),
    "tiny-mixed-shared": lambda: _tiny_mixed(21),
}


@pytest.mark.parametrize("name", sorted(BRUTE))
def test_bruteforce_block_diagonal_mask(name):
    pin_bruteforce(oracle, BRUTE[name]())


@pytest.mark.parametrize("name", ["config1", "tiny-mixed-shared", "config5-small"])
def test_block_permutation_invariance(name):
    b = synth.make_config(5, small=True) if name == "config5-small" else BRUTE[name]()
    pin_permutation_invariance(oracle, b)


@pytest.mark.parametrize("name", ["config1", "tiny-mixed-shared"])
def test_split_merge(name):
    pin_split_merge(oracle, BRUTE[name]())


def test_tolerance_rule():
    pin_tolerance(oracle)


def test_sampled_tokens_match_full():
    b = synth.make_config(3, small=True)
    from pins import run_oracle
    full, lse = run_oracle(oracle, b)
    toks = [0, 5, 9, 100, b.num_tokens - 1]
    part, lse_p = run_oracle(oracle, b, tokens=toks)
    assert np.array_equal(part[toks], full[toks]) and np.array_equal(lse_p[toks], lse[toks])
    others = np.setdiff1d(np.arange(b.num_tokens), toks)
    assert np.isnan(part[others]).all()
