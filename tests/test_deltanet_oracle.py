"""Pins of the rollback-free tree-verification oracle for the gated delta
rule (CPU only): closed forms of the recurrence and of the tree, the pages'
five-drafted / four-accepted example for commit, and planted slips.

Source: "Karpathy's Trick for Faster Local LLMs Finally Has Proper Tooling"
(blog.dailydoseofds.com), section "Verifying a draft tree without restoring
model state"; the recurrence is the gated delta rule of the Gated DeltaNet
publication (the pages give no equations).
"""
import numpy as np
import pytest

import synth
from oracle import deltanet_oracle as DN
from oracle import tree_oracle as TO


def _case(T=9, H=2, dk=8, dv=6, seed=1, shape="bushy"):
    return synth.deltanet_case(T, H, dk, dv, seed, shape)


def test_no_writes_only_decay():
    # beta = 0: every update is S <- alpha S, so o_i = (prod of alpha on the
    # root path of i) * S0 q_i
    S0, q, k, v, a, b, parent = _case()
    b[:] = 0
    out = DN.tree_verify(S0, q, k, v, a, b, parent)
    for i in range(len(parent)):
        nodes = TO.root_path(parent, i)
        for h in range(S0.shape[0]):
            g = np.prod([float(a[n, h]) for n in nodes])
            assert np.allclose(out[i, h], g * (S0[h].astype(np.float64) @ q[i, h]), rtol=1e-12, atol=1e-12)


def test_full_write_returns_the_value_at_its_key():
    # beta = 1: S' k = alpha (S k - S k (k.k)) + v (k.k) = v for a unit key,
    # whatever the decay and the state: querying a node at its own key gives
    # its own value
    S0, q, k, v, a, b, parent = _case(seed=2)
    b[:] = 1
    k = k.astype(np.float64)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)   # unit length in fp64
    q = k.copy()
    out = DN.tree_verify(S0, q, k, v, a, b, parent)
    assert np.allclose(out, v.astype(np.float64), rtol=1e-12, atol=1e-12)


def test_orthogonal_writes_do_not_interfere():
    # chain, alpha = beta = 1, keys the unit vectors e_0, e_1, ...: after the
    # chain the state holds v_j at e_j (j on the path) and S0 elsewhere
    T, H, dk, dv = 6, 1, 8, 5
    S0, q, k, v, a, b, parent = _case(T, H, dk, dv, seed=3, shape="chain")
    a[:] = 1
    b[:] = 1
    k[:] = 0
    for t in range(T):
        k[t, 0, t] = 1.0
    q[:] = 0
    q[T - 1, 0, 2] = 1.0               # the last node asks for the key of node 2
    out = DN.tree_verify(S0, q, k, v, a, b, parent)
    assert np.allclose(out[T - 1, 0], v[2, 0], rtol=0, atol=1e-12)
    q[T - 1, 0, :] = 0
    q[T - 1, 0, dk - 1] = 1.0          # a direction no node wrote
    out = DN.tree_verify(S0, q, k, v, a, b, parent)
    assert np.allclose(out[T - 1, 0], S0[0, :, dk - 1], rtol=0, atol=1e-12)


def test_a_node_only_sees_its_root_path():
    # the same tokens laid out as a plain chain give the same output
    S0, q, k, v, a, b, parent = _case(T=12, seed=4)
    out = DN.tree_verify(S0, q, k, v, a, b, parent)
    for i in (5, 11):
        nodes = TO.root_path(parent, i)
        sel = np.array(nodes)
        chain = [-1] + list(range(len(nodes) - 1))
        out_c = DN.tree_verify(S0, q[sel], k[sel], v[sel], a[sel], b[sel], chain)
        assert np.allclose(out_c[-1], out[i], rtol=1e-12, atol=1e-12)


def test_commit_of_the_five_drafted_example_and_no_rollback():
    # five drafted tokens in a chain under the root, the first four accepted:
    # the live state advances by the root and those four, not the fifth
    S0, q, k, v, a, b, parent = _case(T=6, H=2, seed=5, shape="chain")
    S0_before = S0.copy()
    DN.tree_verify(S0, q, k, v, a, b, parent)
    assert np.array_equal(S0, S0_before)                  # verification leaves the live state
    S_new = DN.tree_commit(S0, q, k, v, a, b, parent, [1, 2, 3, 4])
    k64, v64 = k.astype(np.float64), v.astype(np.float64)
    for h in range(2):
        S = S0[h].astype(np.float64)
        for t in range(5):                                # root + four accepted
            S = a[t, h] * (S - b[t, h] * np.outer(S @ k64[t, h], k64[t, h])) + b[t, h] * np.outer(v64[t, h], k64[t, h])
        assert np.allclose(S_new[h], S, rtol=1e-12, atol=1e-12)
    # nothing accepted: only the root goes through
    S_root = DN.tree_commit(S0, q, k, v, a, b, parent, [])
    assert np.allclose(S_root[0], DN.gdn_step(S0[0], q[0, 0], k[0, 0], v[0, 0], a[0, 0], b[0, 0])[0])


# ------------------------------------------------- planted-mistake check
def _fails(fn):
    try:
        fn()
    except (AssertionError, TO.MalformedTree):
        return True
    return False


def test_planted_mistakes_are_caught(monkeypatch):
    def step_output_before_update(S, q, k, v, alpha, beta):
        S2, _o = _orig(S, q, k, v, alpha, beta)
        return S2, np.asarray(S, np.float64) @ np.asarray(q, np.float64)   # slip: reads the old state

    def step_wrong_sign(S, q, k, v, alpha, beta):
        S = np.asarray(S, np.float64)
        S2 = alpha * S @ (np.eye(len(k)) + beta * np.outer(k, k)) + beta * np.outer(v, k)  # slip: + instead of -
        return S2, S2 @ q

    def step_decays_the_write(S, q, k, v, alpha, beta):
        S = np.asarray(S, np.float64)
        S2 = alpha * (S @ (np.eye(len(k)) - beta * np.outer(k, k)) + beta * np.outer(v, k))  # slip: alpha on v
        return S2, S2 @ q

    def commit_with_rejected(S0, q, k, v, alpha, beta, parent, path):
        return _orig_commit(S0, q, k, v, alpha, beta, parent, list(path) + [len(parent) - 1])  # slip

    _orig, _orig_commit = DN.gdn_step, DN.tree_commit
    caught = []
    for name, fake, test in [
        ("gdn_step", step_output_before_update, test_full_write_returns_the_value_at_its_key),
        ("gdn_step", step_wrong_sign, test_full_write_returns_the_value_at_its_key),
        ("gdn_step", step_decays_the_write, test_full_write_returns_the_value_at_its_key),
        ("tree_commit", commit_with_rejected, test_commit_of_the_five_drafted_example_and_no_rollback),
    ]:
        with monkeypatch.context() as mp:
            mp.setattr(DN, name, fake)
            caught.append(_fails(test))
    assert all(caught), caught
