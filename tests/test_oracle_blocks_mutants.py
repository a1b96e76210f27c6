"""Plant plausible mistakes in copies of the block-manager oracle (on the CPU) and require that
some pin catches each one."""
import os
import types

import pytest

from conftest import ROOT, read_golden
from pins_blocks import (pin_block_table_example, pin_eviction_order, pin_fork_cow_example,
                         pin_last_token_block_not_reused, pin_prefix_worked_example,
                         pin_placeholders, pin_protocol_rules, pin_random_bruteforce, pin_swap)

SRC = open(os.path.join(ROOT, "oracle", "blocks.py")).read()

MUTANTS = {
    # a write into a shared partial block goes in place
    "no-cow": [("cow = n % bs != 0 and self.ref[last] > 1", "cow = False", 1)],
    # the original's count is not decremented on a copy
    "cow-keeps-ref": [("            self.ref[last] -= 1\n", "", 1)],
    # the block holding the last prompt token is reused too
    "hit-last-block": [("for j in range((n - 1) // bs):", "for j in range(n // bs):", 1)],
    # most recently freed cached block evicted first
    "mru-eviction": [("b = self.cached.pop(0)", "b = self.cached.pop()", 1)],
    # a sequence's blocks freed first block first
    "free-forward": [('raise BlockError(INVALID, "sequence in the open step\'s batch")\n        for b in reversed(s["table"]):',
                      'raise BlockError(INVALID, "sequence in the open step\'s batch")\n        for b in s["table"]:', 1)],
    # an evicted block keeps its key
    "evict-keeps-key": [("            self.key[b] = None\n            self.visible[b] = False\n",
                         "", 1)],
    # a copy's source goes straight back to the pool
    "no-hold": [("        if self.pending[b] > 0:\n            self.state[b] = HELD\n        elif",
                 "        if", 1)],
    # blocks computed in the open step are found at once
    "visible-at-once": [("                self.visible[b] = False\n                self.step_blocks.append(b)",
                         "                self.visible[b] = True\n                self.step_blocks.append(b)", 1)],
    # a copy of a block written in the open step is allowed
    "cow-of-dirty": [("if cow and self.dirty[last]:", "if False:", 1)],
    # a block keyed by its own tokens only, not by the whole prefix
    "key-own-tokens": [('self.key[b] = tuple(s["tokens"][:(j + 1) * bs])',
                        'self.key[b] = tuple(s["tokens"][j * bs:(j + 1) * bs])', 1),
                       ("b = self._lookup(tuple(tokens[:(j + 1) * bs]))",
                        "b = self._lookup(tuple(tokens[j * bs:(j + 1) * bs]))", 1)],
    # the slot offset taken from the batch row instead of the position
    "slot-offset": [("slots.append(b * bs + p % bs)", "slots.append(b * bs + (p - p0) % bs)", 1)],
    # fork does not take references
    "fork-no-ref": [('        for b in c["table"]:\n            self._add_ref(b)\n', "", 1)],
    # a swapped-out block goes back to the pool before the step's gather has read it
    "swap-no-hold": [("            self.slot_state[slot] = 1\n            self.pending[b] += 1\n            self.swap_src.append(b)\n",
                      "            self.slot_state[slot] = 1\n", 1)],
    # a swap-in's destination blocks are not held until the step closes
    "scatter-no-hold": [("        for b in table:                  # the scatter's destinations are held like the gathers'\n            self.pending[b] += 1\n            self.swap_src.append(b)\n", "", 1)],
    # a copy's destination is not held until the step closes
    "copy-dst-no-hold": [("            self.pending[dst] += 1      # a copy's destination is held until the step closes too\n", "", 1),
                         ("for src in [b for pair in out for b in pair] + self.swap_src:",
                          "for src in [s_ for s_, _ in out] + self.swap_src:", 1)],
    # swapped-in blocks are not counted as written in the open step
    "swap-in-not-dirty": [("        for b in table:\n            self.dirty[b] = True\n", "        for b in table:\n", 1)],
    # slots released by a swap-in are free at once
    "swap-slot-free-at-once": [("            self.slot_state[slot] = 2\n        for b in table:",
                                "            self.slot_state[slot] = 0\n        for b in table:", 1)],
    # a sequence with blocks written in the open step may be swapped out
    "swap-out-dirty": [('if s["in_batch"] or any(self.dirty[b] for b in s["table"]):', 'if s["in_batch"]:', 1)],
    # blocks are keyed whatever their tokens' confirmation
    "key-unconfirmed": [('min(s["computed"], s["confirmed"]) // bs', 's["computed"] // bs', 2)],
    # placeholders count as confirmed
    "placeholders-confirmed": [('elif s["confirmed"] == len(s["tokens"]):', 'if s["confirmed"] == len(s["tokens"]):', 1)],
    # a fork of a parent with unconfirmed tokens
    "fork-unconfirmed": [(' or p["confirmed"] != len(p["tokens"]):', ':', 1)],
    # a swap-in reuses the sequence's old block ids instead of taking blocks
    "swap-in-nothing-taken": [("table = [self._take() for _ in s[\"slots\"]]", "table = list(s[\"slots\"])", 1)],
}


def mutant(name):
    src = SRC
    for old, new, count in MUTANTS[name]:
        assert src.count(old) == count, f"mutation site for {name} not found exactly {count} time(s)"
        src = src.replace(old, new)
    mod = types.ModuleType(f"blocks_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def caught(mod):
    pins = [
        lambda: pin_fork_cow_example(mod, read_golden("p3_fork_cow_example.txt")),
        lambda: pin_block_table_example(mod, read_golden("p3_block_table_example.txt")),
        lambda: pin_prefix_worked_example(mod, read_golden("p3_prefix_examples.txt")),
        lambda: pin_last_token_block_not_reused(mod),
        lambda: pin_eviction_order(mod),
        lambda: pin_protocol_rules(mod),
        lambda: pin_swap(mod),
        lambda: pin_placeholders(mod),
        lambda: pin_random_bruteforce(mod, seeds=range(6), n_ops=120),
    ]
    for pin in pins:
        try:
            pin()
        except Exception:  # noqa: BLE001 -- any failure of a pin counts as caught
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert caught(mutant(name)), f"no pin notices the planted mistake {name}"


def test_unmutated_oracle_passes_every_pin():
    mod = types.ModuleType("blocks_unmutated")
    exec(compile(SRC, "<unmutated>", "exec"), mod.__dict__)
    assert not caught(mod)
