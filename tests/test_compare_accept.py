"""The acceptance comparison used by the GPU parity tests (gpu_util.
compare_accept), checked on the CPU against hand-made outcomes: what it
excuses after a near tie, and what it still fails."""
import numpy as np
import pytest

from gpu_util import compare_accept

# root 0 -> {1, 2}, 1 -> {3, 4}; tokens per node
PARENTS = np.array([[-1, 0, 0, 1, 1]])
TOKENS = np.array([[9, 4, 5, 6, 7]])
V = 16


def _res(path, final, near=0, flags=0, depth=-1, slot=-1):
    T = PARENTS.shape[1]
    nodes = np.full((1, T), -1, dtype=np.int32)
    toks = np.full((1, T), -1, dtype=np.int32)
    nodes[0, :len(path)] = path
    toks[0, :len(path)] = [TOKENS[0, n] for n in path]
    toks[0, len(path)] = final
    return {"accept_len": np.array([len(path)], dtype=np.int32), "accepted_nodes": nodes, "out_tokens": toks,
            "flags": np.array([flags], dtype=np.uint32), "near_ties": np.array([near], dtype=np.int32),
            "first_near_depth": np.array([depth], dtype=np.int32),
            "first_near_slot": np.array([slot], dtype=np.int32)}


def _cmp(got, ref):
    return compare_accept(got, ref, "case", PARENTS, TOKENS, V)


def test_identical_results_pass():
    assert _cmp(_res([1, 3], 2), _res([1, 3], 2)) == 0


def test_any_difference_without_a_near_tie_fails():
    with pytest.raises(AssertionError):
        _cmp(_res([1, 3], 2), _res([1, 3], 3))
    with pytest.raises(AssertionError):
        _cmp(_res([1, 3], 2, flags=8), _res([1, 3], 2))
    with pytest.raises(AssertionError):          # near-tie counts must be equal too
        _cmp(_res([1, 3], 2, near=1), _res([1, 3], 2))


def test_terminal_near_tie_excuses_only_the_final_token():
    ref = _res([1, 3], 2, near=1, depth=2, slot=-1)
    assert _cmp(_res([1, 3], 3, near=1), ref) == 1
    with pytest.raises(AssertionError):          # the path may not change
        _cmp(_res([1, 4], 3, near=1), ref)
    with pytest.raises(AssertionError):          # and the GPU must flag the tie too
        _cmp(_res([1, 3], 3, near=0), ref)


def test_test_near_tie_excuses_what_follows_it_only():
    # the oracle's first near tie: sibling 1 (node 4) of node 1, at depth 1
    ref = _res([1, 4], 2, near=1, depth=1, slot=1)
    assert _cmp(_res([1], 7, near=1), ref) == 1             # rejected there instead
    with pytest.raises(AssertionError):                     # diverged at depth 0
        _cmp(_res([2], 7, near=1), ref)
    with pytest.raises(AssertionError):                     # took sibling 0, decided before the tie
        _cmp(_res([1, 3], 7, near=1), ref)
    with pytest.raises(AssertionError):                     # not a walk: token of node 4 wrong
        bad = _res([1], 7, near=1)
        bad["accepted_nodes"][0, 1] = 4
        bad["accept_len"][0] = 2
        bad["out_tokens"][0, 1] = 0
        bad["out_tokens"][0, 2] = 7
        _cmp(bad, ref)
    with pytest.raises(AssertionError):                     # final token outside the vocabulary
        _cmp(_res([1], V, near=1), ref)
