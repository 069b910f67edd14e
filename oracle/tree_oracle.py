"""Greedy acceptance of a verified draft tree: the plain CPU oracle.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline may import this module; the HIP library never does, and it shares
no code with it.

Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
(blog.dailydoseofds.com).  Section "Producing several tokens from one model
pass": the main model checks all drafted positions in one pass, keeps the
valid prefix and goes on from the first rejected position with its own token;
five drafted tokens of which it agrees with the first four advance the
sequence by five.  Section "Issue with parallel draft generation": with a
tree of alternative drafted continuations, what is kept is the deepest root
path whose every edge the target agrees with.

The pages give no procedure beyond that.  Readings taken here:

  T1. A tree of T nodes in the order of the verify batch.  Node 0 is the root:
      the last token already in the sequence, whose logits row predicts the
      first drafted position.  Node i >= 1 is a drafted token whose parent
      parent[i] is an earlier node (0 <= parent[i] < i); parent[0] = -1.
      Row i of the logits is the target's prediction for the position after
      node i.
  T2. Greedy verification (temperature 0; the pages name a distribution-
      preserving acceptance but do not give it): the target's choice at node i
      is the index of the largest logit of row i, the smallest such index when
      several are equal.
  T3. Node i >= 1 is valid when its parent is valid and draft[i] equals the
      target's choice at the parent.  The root is valid.
  T4. The accepted path is the root path of the deepest valid node; among
      equally deep valid nodes, the one with the smallest index.
  T5. The pass emits the drafted tokens along the accepted path, then the
      target's choice at the path's last node: depth + 1 tokens.
  T6. A tree that breaks T1 (parent[0] != -1, or parent[i] outside [0, i)) is
      rejected as a whole.

This is written as brute force over root paths: every node's path to the root
is taken explicitly and checked edge by edge (obviously correct, quadratic in T).
"""
from __future__ import annotations

import numpy as np


class MalformedTree(ValueError):
    """parent[] does not describe a tree in verify-batch order (reading T6)."""


def target_choices(logits) -> np.ndarray:
    """Reading T2: per row, the index of the largest logit, smallest on ties
    (numpy's argmax returns the first maximum)."""
    logits = np.asarray(logits)
    if logits.ndim != 2 or logits.shape[1] < 1:
        raise ValueError("logits must be [T, V] with V >= 1")
    return np.argmax(logits, axis=1).astype(np.int64)


def check_tree(parent) -> None:
    """Reading T1/T6."""
    parent = [int(p) for p in parent]
    if not parent or parent[0] != -1:
        raise MalformedTree("parent[0] must be -1 (the root)")
    for i, p in enumerate(parent[1:], start=1):
        if not 0 <= p < i:
            raise MalformedTree(f"parent[{i}] = {p} is not an earlier node")


def root_path(parent, i: int) -> list:
    """Nodes from the root to node i, both included."""
    path = [i]
    while path[-1] != 0:
        if len(path) > len(parent) or not 0 <= int(parent[path[-1]]) < len(parent):
            raise MalformedTree(f"node {i} has no path to the root")
        path.append(int(parent[path[-1]]))
    return path[::-1]


def accept_greedy(parent, draft, target):
    """Readings T3-T5 by brute force over the root paths of all nodes.

    Returns (path, emit): the accepted nodes below the root, root side first,
    and the emitted tokens (their drafted tokens, then the target's choice at
    the last accepted node)."""
    check_tree(parent)
    T = len(parent)
    best = 0
    best_depth = 0
    for i in range(T):
        nodes = root_path(parent, i)
        valid = all(int(draft[b]) == int(target[a]) for a, b in zip(nodes, nodes[1:]))
        depth = len(nodes) - 1
        if valid and depth > best_depth:          # equal depth keeps the smaller index
            best, best_depth = i, depth
    path = root_path(parent, best)[1:]
    emit = [int(draft[n]) for n in path] + [int(target[best])]
    return path, emit


def verify_tree(logits, parent, draft):
    """The whole step: the target's choices from the logits, then acceptance.
    Returns (target, path, emit)."""
    target = target_choices(logits)
    path, emit = accept_greedy(parent, draft, target)
    return target, path, emit
