"""Rollback-free verification of a draft tree through a fixed-state recurrent
layer (gated delta rule): the plain CPU oracle, fp64.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline may import this module; the HIP library shares no code with it.

Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
(blog.dailydoseofds.com), section "Verifying a draft tree without restoring
model state": the checkpoint's Gated DeltaNet layers squeeze the whole past
into a fixed-size state that every accepted token changes; each branch of a
draft tree would change it differently, so the runtime computes what every
branch needs without touching the live state, and applies the updates of the
accepted tokens only, once the path is chosen.

The pages give no equations.  The recurrence taken here is the gated delta
rule of the Gated DeltaNet publication (Yang, Kautz and Hatamizadeh, "Gated
Delta Networks: Improving Mamba2 with Delta Rule"), in the plainest form:

  D1. Per head a state S of d_v x d_k values.  A token brings a query q and
      a key k (d_k values, the key of unit length), a value v (d_v), a decay
      gate alpha in (0, 1] and a write strength beta in [0, 1]:
          S' = alpha * S (I - beta k k^T) + beta v k^T,      o = S' q
      (the output reads the state after the token's own update).
  D2. The tree is that of the acceptance step: node 0 is the root, the last
      token already in the sequence but not yet through the layer, and node
      i >= 1 hangs under parent[i] < i.  Node i's state is its parent's state
      advanced by node i (the root's parent state is the live state).
  D3. Verification returns o for every node and leaves the live state as it
      was.  Commit replaces the live state by the state of the last accepted
      node: the root, then the accepted path (the acceptance step's `path`).
  D4. Heads are independent.

Written as sequential replay per branch: each node's root path is replayed
from the live state, token by token (obviously correct; quadratic in T).
"""
from __future__ import annotations

import numpy as np

from oracle.tree_oracle import check_tree, root_path


def gdn_step(S, q, k, v, alpha, beta):
    """D1 for one head: returns (S', o), fp64."""
    S = np.asarray(S, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    q = np.asarray(q, np.float64)
    d_k = k.shape[0]
    S2 = alpha * S @ (np.eye(d_k) - beta * np.outer(k, k)) + beta * np.outer(v, k)
    return S2, S2 @ q


def replay(S0, q, k, v, alpha, beta, nodes, h):
    """Head h's state after the tokens `nodes` in order, from S0[h]; also the
    last output."""
    S = np.asarray(S0[h], np.float64)
    o = None
    for n in nodes:
        S, o = gdn_step(S, q[n, h], k[n, h], v[n, h], float(alpha[n, h]), float(beta[n, h]))
    return S, o


def tree_verify(S0, q, k, v, alpha, beta, parent):
    """D2/D3: outputs o[T, H, d_v] of every node; S0 [H, d_v, d_k] untouched."""
    check_tree(parent)
    T, H = alpha.shape
    d_v = v.shape[-1]
    out = np.zeros((T, H, d_v))
    for i in range(T):
        nodes = root_path(parent, i)
        for h in range(H):
            out[i, h] = replay(S0, q, k, v, alpha, beta, nodes, h)[1]
    return out


def tree_commit(S0, q, k, v, alpha, beta, parent, path):
    """D3: the new live state after the root and the accepted path."""
    check_tree(parent)
    nodes = [0] + [int(n) for n in path]
    return np.stack([replay(S0, q, k, v, alpha, beta, nodes, h)[0] for h in range(S0.shape[0])])
