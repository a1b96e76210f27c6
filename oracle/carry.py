"""Oracle of the async step's carry-over (test infrastructure only).

"Continuous batching in transformers", section "Async batching": batch N+1's inputs are built
before batch N has produced its tokens, so each token batch N will produce is entered in batch
N+1 as a placeholder 0, and a carry-over mask holding, for each output of batch N, the index of
its destination in batch N+1's inputs (or -1: not carried) adds the real token in before batch
N+1's forward pass. Plain Python over lists.
"""
from __future__ import annotations

import numpy as np


def carry_over(prev_outputs, dest, next_inputs):
    """next_inputs after the carry-over: entry dest[i] gains prev_outputs[i] for every i with
    dest[i] in [0, len(next_inputs)); other entries are unchanged."""
    out = [int(x) for x in next_inputs]
    for i, d in enumerate(np.asarray(dest).tolist()):
        if 0 <= d < len(out):
            out[d] += int(prev_outputs[i])
    return np.array(out, dtype=np.int64)
