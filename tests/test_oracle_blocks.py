"""The block-manager oracle against the pages' worked examples, eviction-order checks and a
brute force over random operation streams (CPU only)."""
import oracle.blocks as ob
from pins_blocks import (pin_block_table_example, pin_eviction_order, pin_fork_cow_example,
                         pin_last_token_block_not_reused, pin_prefix_worked_example, pin_placeholders, pin_protocol_rules, pin_swap,
                         pin_random_bruteforce)


def test_fork_cow_example(golden):
    pin_fork_cow_example(ob, golden("p3_fork_cow_example.txt"))


def test_block_table_example(golden):
    pin_block_table_example(ob, golden("p3_block_table_example.txt"))


def test_prefix_examples(golden):
    pin_prefix_worked_example(ob, golden("p3_prefix_examples.txt"))


def test_last_token_block_not_reused():
    pin_last_token_block_not_reused(ob)


def test_eviction_order():
    pin_eviction_order(ob)


def test_random_bruteforce():
    pin_random_bruteforce(ob)


def test_protocol_rules():
    pin_protocol_rules(ob)


def test_swap():
    pin_swap(ob)


def test_placeholders():
    pin_placeholders(ob)
