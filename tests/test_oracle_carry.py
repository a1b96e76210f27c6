"""The carry-over oracle against the page's description of async batching (CPU only)."""
import numpy as np

import oracle.carry as oc


def test_placeholders_receive_the_previous_steps_tokens():
    # step N: three decoding sequences produce tokens 41, 42, 43 (one output row each) and a
    # prompt chunk produces 4 rows nobody carries. Step N+1: a new 3-token prompt first, then the
    # decodes of sequences 0 and 2 (sequence 1 finished): placeholders 0 at indices 3 and 4.
    prev_out = [7, 8, 9, 10, 41, 42, 43]
    dest = [-1, -1, -1, -1, 3, -1, 4]
    next_in = [101, 102, 103, 0, 0]
    assert oc.carry_over(prev_out, dest, next_in).tolist() == [101, 102, 103, 41, 43]


def test_minus_one_and_out_of_range_leave_inputs_unchanged():
    rng = np.random.default_rng(0)
    nxt = rng.integers(0, 1000, 50)
    prev = rng.integers(0, 1000, 30)
    dest = np.full(30, -1)
    assert np.array_equal(oc.carry_over(prev, dest, nxt), nxt)
    dest[:3] = [50, 51, -7]
    assert np.array_equal(oc.carry_over(prev, dest, nxt), nxt)


def test_matches_a_direct_construction():
    """Random mappings: placeholders at the destinations, the carried tokens appear exactly there."""
    rng = np.random.default_rng(1)
    for _ in range(50):
        n_prev, n_next = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        prev = rng.integers(1, 32000, n_prev)
        k = int(rng.integers(0, min(n_prev, n_next) + 1))
        src = rng.choice(n_prev, k, replace=False)
        dst = rng.choice(n_next, k, replace=False)
        dest = np.full(n_prev, -1)
        dest[src] = dst
        nxt = rng.integers(1, 32000, n_next)
        nxt[dst] = 0
        want = nxt.copy()
        want[dst] = prev[src]
        assert np.array_equal(oc.carry_over(prev, dest, nxt), want)


def test_planted_mistakes_are_caught():
    import inspect
    import types
    src = inspect.getsource(oc)
    for old, new in [("out[d] += int(prev_outputs[i])", "out[i] += int(prev_outputs[d])"),
                     ("if 0 <= d < len(out):", "if d < len(out):"),
                     ("out[d] += int(prev_outputs[i])", "out[d] = int(prev_outputs[d])")]:
        assert src.count(old) == 1
        mod = types.ModuleType("carry_mutant")
        exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
        caught = False
        for test in (test_placeholders_receive_the_previous_steps_tokens,
                     test_minus_one_and_out_of_range_leave_inputs_unchanged,
                     test_matches_a_direct_construction):
            g = dict(test.__globals__, oc=mod)
            try:
                types.FunctionType(test.__code__, g)()
            except (AssertionError, IndexError):
                caught = True
        assert caught, new
