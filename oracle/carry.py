"""Oracle of the async step's carry-over (test infrastructure only).

Source: "Continuous batching in transformers", section "Async batching". When the next step's
inputs are assembled while the current step is still running, the tokens the current step will
emit are not known yet; their input positions hold 0 for now. The carry-over fills them in on
the device just before the next step runs: dest[i] names the input position of the next step
that output i of the current step belongs to, and that position gains output i. An entry of
dest outside the next step's inputs (-1 by convention) moves nothing. Plain Python over lists.
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
