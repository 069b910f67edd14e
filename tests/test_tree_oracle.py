"""Pins of the greedy tree-acceptance oracle (CPU only).

What fixes the oracle here, other than itself:

* the pages' worked example (tests/golden/tokens_per_pass.txt): five drafted
  tokens, the target agrees with the first four, the pass advances five;
* a chain of drafts reduces to the longest common prefix of the drafted tokens
  and the target's choices, a closed form written as a plain loop;
* trees built so that exactly one root path is valid, known by construction;
* the special cases: nothing accepted, equal depths, ties in the logits,
  malformed trees;
* plausible slips planted in the oracle fail at least one of the pins above
  (test_planted_mistakes_are_caught).

Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
(blog.dailydoseofds.com), sections "Producing several tokens from one model
pass" and "Issue with parallel draft generation".
"""
import os

import numpy as np
import pytest

from oracle import tree_oracle as TO

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tokens_per_pass.txt")


def _golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    return vals


def _onehot_logits(choices, V, rng):
    """Logits whose row r has its unique maximum at choices[r]."""
    logits = rng.standard_normal((len(choices), V)).astype(np.float32)
    for r, c in enumerate(choices):
        logits[r, c] = np.float32(5.0)
    return logits


def test_worked_example_five_drafted_four_agree():
    g = _golden()
    proposed, agreed, advance = int(g["draft_proposed"]), int(g["draft_agreed_prefix"]), int(g["draft_advance"])
    V = 100
    rng = np.random.default_rng(0)
    drafts = [11, 22, 33, 44, 55]                       # the drafter's five tokens
    assert len(drafts) == proposed
    parent = [-1] + list(range(proposed))               # root, then a chain of five
    draft = [7] + drafts                                # node 0 is the last committed token
    # the target agrees with the first four drafted tokens, not with the fifth
    choices = drafts[:agreed] + [66, 77]
    logits = _onehot_logits(choices, V, rng)
    target, path, emit = TO.verify_tree(logits, parent, draft)
    assert list(target) == choices
    assert len(emit) == advance
    assert path == [1, 2, 3, 4]
    assert emit == drafts[:agreed] + [66]               # four drafts, then the target's own token
    assert float(g["plain_decoding_tokens_per_pass"]) == 1.0
    # plain decoding: no drafts, one token per pass
    _t, path1, emit1 = TO.verify_tree(_onehot_logits([9], V, rng), [-1], [7])
    assert path1 == [] and emit1 == [9]


@pytest.mark.parametrize("seed", range(20))
def test_chain_is_longest_common_prefix(seed):
    rng = np.random.default_rng(seed)
    T = int(rng.integers(1, 34))
    V = int(rng.integers(2, 4))                          # small vocabularies: long agreements happen
    draft = rng.integers(0, V, size=T)
    target = rng.integers(0, V, size=T)
    parent = [-1] + list(range(T - 1))
    n = 1                                                # tokens emitted
    while n < T and draft[n] == target[n - 1]:
        n += 1
    path, emit = TO.accept_greedy(parent, draft, target)
    assert len(emit) == n
    assert path == list(range(1, n))
    assert emit == [int(t) for t in draft[1:n]] + [int(target[n - 1])]


@pytest.mark.parametrize("seed", range(20))
def test_planted_unique_valid_path(seed):
    """Distinct drafted tokens; the targets agree along one chosen root path and
    name an unused token everywhere else: that path, and only it, is valid."""
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(2, 33))
    V = T + 1
    unused = T                                           # no node carries this token
    parent = [-1] + [int(rng.integers(max(0, i - 3), i)) for i in range(1, T)]
    draft = rng.permutation(T)                           # distinct tokens 0..T-1
    x = int(rng.integers(0, T))
    chosen = [x]
    while chosen[-1] != 0:
        chosen.append(parent[chosen[-1]])
    chosen = chosen[::-1]
    target = np.full(T, unused)
    for a, b in zip(chosen, chosen[1:]):
        target[a] = draft[b]
    target[x] = int(rng.integers(0, V))                  # the bonus token: anything
    path, emit = TO.accept_greedy(parent, draft, target)
    # a child of x may still agree with target[x] by chance: then it is deeper
    kids = [i for i in range(T) if parent[i] == x and draft[i] == target[x]]
    if kids:
        c = min(kids)
        assert path == chosen[1:] + [c]
        assert emit == [int(draft[n]) for n in chosen[1:]] + [int(draft[c]), int(target[c])]
    else:
        assert path == chosen[1:]
        assert emit == [int(draft[n]) for n in chosen[1:]] + [int(target[x])]


def test_nothing_accepted_emits_the_targets_token():
    parent = [-1, 0, 0, 0, 1, 2]
    draft = [9, 1, 2, 3, 4, 5]
    target = [8, 4, 5, 0, 0, 0]                          # root wants 8: no child drafted it
    path, emit = TO.accept_greedy(parent, draft, target)
    assert path == [] and emit == [8]


def test_equal_depth_takes_the_smaller_index_and_depth_wins():
    # two root children drafted the token the root wants; the later one has a
    # valid child, so it is deeper and wins despite its larger index
    parent = [-1, 0, 0, 2]
    draft = [0, 5, 5, 6]
    target = [5, 1, 6, 2]
    path, emit = TO.accept_greedy(parent, draft, target)
    assert path == [2, 3] and emit == [5, 6, 2]
    # without the grandchild's agreement both are depth 1: the smaller index wins
    target2 = [5, 1, 7, 2]
    path2, emit2 = TO.accept_greedy(parent, draft, target2)
    assert path2 == [1] and emit2 == [5, 1]


def test_target_choice_is_the_first_maximum():
    logits = np.array([[0, 3, 1, 3, 2],
                       [4, 4, 4, 4, 4],
                       [-np.inf, -np.inf, -1, -np.inf, -1],
                       [1, 2, 3, 4, 5],
                       [-1, -0.0, -2, 0.0, -3],     # -0 and +0 are one value
                       [-1, 0.0, -2, -0.0, -3]], dtype=np.float32)
    assert list(TO.target_choices(logits)) == [1, 0, 2, 4, 1, 1]
    with pytest.raises(ValueError):
        TO.target_choices(np.zeros((2, 0), np.float32))


@pytest.mark.parametrize("parent", [[0], [-1, 1], [-1, 0, 2], [-1, 0, -1], [-1, 5], [-1, 0, 1, 3]])
def test_malformed_trees_are_rejected(parent):
    T = len(parent)
    with pytest.raises(TO.MalformedTree):
        TO.accept_greedy(parent, [0] * T, [0] * T)


def test_generated_trees_are_well_formed():
    import synth
    for shape in ("chain", "star", "bushy"):
        logits, parent, draft = synth.draft_tree(32, 1000, 3, shape=shape, accept=6, ties=True)
        TO.check_tree(parent)
        assert logits.shape == (32, 1000) and logits.dtype == np.float32
        assert draft.min() >= 0 and draft.max() < 1000


# ------------------------------------------------- planted-mistake check
def _fails(fn):
    try:
        fn()
    except (AssertionError, TO.MalformedTree, pytest.fail.Exception):
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    def accept_compares_own_target(parent, draft, target):
        TO.check_tree(parent)
        best, best_depth = 0, 0
        for i in range(len(parent)):
            nodes = TO.root_path(parent, i)
            ok = all(int(draft[b]) == int(target[b]) for b in nodes[1:])   # slip: child's own choice
            if ok and len(nodes) - 1 > best_depth:
                best, best_depth = i, len(nodes) - 1
        path = TO.root_path(parent, best)[1:]
        return path, [int(draft[n]) for n in path] + [int(target[best])]

    def accept_no_bonus(parent, draft, target):
        path, emit = _orig_accept(parent, draft, target)
        return path, emit[:-1]                                             # slip: drops the target's token

    def accept_ties_last(parent, draft, target):
        TO.check_tree(parent)
        best, best_depth = 0, 0
        for i in range(len(parent)):
            nodes = TO.root_path(parent, i)
            ok = all(int(draft[b]) == int(target[a]) for a, b in zip(nodes, nodes[1:]))
            if ok and len(nodes) - 1 >= best_depth:                        # slip: later index wins ties
                best, best_depth = i, len(nodes) - 1
        path = TO.root_path(parent, best)[1:]
        return path, [int(draft[n]) for n in path] + [int(target[best])]

    def accept_bonus_from_parent(parent, draft, target):
        path, emit = _orig_accept(parent, draft, target)
        last = path[-1] if path else 0
        return path, emit[:-1] + [int(target[max(parent[last], 0)])]      # slip: wrong row for the bonus

    def choices_last_max(logits):
        logits = np.asarray(logits)
        return (logits.shape[1] - 1 - np.argmax(logits[:, ::-1], axis=1)).astype(np.int64)  # slip

    def check_tree_lenient(parent):
        return None                                                        # slip: no validation

    _orig_accept = TO.accept_greedy
    caught = []
    for name, fake, test in [
        ("accept_greedy", accept_compares_own_target, test_worked_example_five_drafted_four_agree),
        ("accept_greedy", accept_no_bonus, test_worked_example_five_drafted_four_agree),
        ("accept_greedy", accept_ties_last, test_equal_depth_takes_the_smaller_index_and_depth_wins),
        ("accept_greedy", accept_bonus_from_parent, test_worked_example_five_drafted_four_agree),
        ("target_choices", choices_last_max, test_target_choice_is_the_first_maximum),
        ("check_tree", check_tree_lenient, lambda: test_malformed_trees_are_rejected([0])),
    ]:
        with monkeypatch.context() as mp:
            mp.setattr(TO, name, fake)
            caught.append(_fails(test))
    assert all(caught), caught
