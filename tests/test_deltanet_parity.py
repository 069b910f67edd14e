"""GPU parity of rollback-free tree verification through a gated delta-rule
layer: tree_deltanet_verify / tree_deltanet_commit against the fp64 oracle
(oracle/deltanet_oracle.py), through the C ABI.

The kernels compute in fp32 with fused multiply-adds, so outputs and states
are compared within a tolerance: max |gpu - ref| <= 1e-4 * (max |ref| + 1),
per node and head (the rule is contractive -- alpha <= 1 and I - beta k k^T
has norm <= 1 -- so fp32 rounding does not grow along a path of <= 32
tokens; observed errors are ~1e-6).  What must be exact is exact: the live
state after verification is bit-identical to before, and a rejected commit
leaves it bit-identical.

Source of the step: "Karpathy's Trick for Faster Local LLMs Finally Has Proper
Tooling" (blog.dailydoseofds.com), section "Verifying a draft tree without
restoring model state".
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import deltanet_oracle as DN
from oracle import tree_oracle as TO

pytestmark = pytest.mark.gpu

TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global C, svg
    import svg_cases as C  # noqa: F401  (imports the binding, which loads libsvgemm)
    import speculative_verify_gemm_amd as svg


def close(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.max(np.abs(got - ref), axis=-1)
    bound = TOL * (np.max(np.abs(ref), axis=-1) + 1.0)
    assert np.all(err <= bound), float(np.max(err / bound))


def dev(case):
    S0, q, k, v, a, b, parent = case
    return [C.to_dev(t) for t in (S0, q, k, v, a, b)] + [C.to_dev(parent.astype(np.int32))]


CASES = [  # T, H, dk, dv, tree shape
    (1, 1, 128, 128, "chain"), (16, 16, 128, 128, "bushy"), (32, 4, 128, 128, "chain"),
    (9, 3, 64, 64, "star"), (12, 2, 64, 128, "bushy"), (7, 5, 128, 64, "bushy"), (5, 2, 64, 256, "chain"),
    (32, 2, 64, 64, "bushy"), (10, 3, 128, 256, "bushy"),
]


@pytest.mark.parametrize("T,H,dk,dv,shape", CASES)
def test_verify_matches_oracle_and_keeps_the_state(T, H, dk, dv, shape):
    C.say(f"tree_deltanet_verify T={T} H={H} dk={dk} dv={dv} {shape}")
    case = synth.deltanet_case(T, H, dk, dv, seed=T * 13 + H + dk + dv, shape=shape)
    S0, q, k, v, a, b, parent = case
    Sd, qd, kd, vd, ad, bd, pd = dev(case)
    out = torch.empty((T, H, dv), dtype=torch.float32, device=C.DEV)
    svg.tree_deltanet_verify(Sd, qd, kd, vd, ad, bd, pd, out)
    ref = DN.tree_verify(S0, q, k, v, a, b, parent)
    close(C.host(out), ref)
    assert np.array_equal(C.host(Sd), S0)                  # the live state is only read


@pytest.mark.parametrize("T,H,dk,dv", [(16, 8, 128, 128), (6, 2, 64, 256), (32, 3, 128, 64)])
def test_accept_then_commit(T, H, dk, dv):
    """The whole step: greedy acceptance on the verify pass's logits, then the
    commit of the accepted path, both on the device."""
    C.say(f"accept + tree_deltanet_commit T={T} H={H} dk={dk} dv={dv}")
    case = synth.deltanet_case(T, H, dk, dv, seed=7 * T + H, shape="bushy")
    S0, q, k, v, a, b, parent = case
    logits, _p, draft = synth.draft_tree(T, 1000, seed=T + 3, accept=T // 2)
    _t, path_ref, emit_ref = TO.verify_tree(logits, parent, draft)
    Sd, qd, kd, vd, ad, bd, pd = dev(case)
    i32 = lambda t: torch.empty(t, dtype=torch.int32, device=C.DEV)  # noqa: E731
    target, path, emit, n = i32(T), i32(T), i32(T), i32(1)
    svg.tree_accept_greedy(C.to_dev(logits), pd, C.to_dev(draft.astype(np.int32)), target, path, emit, n,
                           svg.tree_workspace())
    svg.tree_deltanet_commit(Sd, kd, vd, ad, bd, path, n)
    assert int(C.host(n)[0]) == len(emit_ref)
    ref = DN.tree_commit(S0, q, k, v, a, b, parent, path_ref)
    close(C.host(Sd), ref)


@pytest.mark.parametrize("T,H,dk,dv", [(16, 4, 128, 128), (9, 3, 64, 256)])
def test_gates_at_their_bounds(T, H, dk, dv):
    """Decay and write strength at the ends of their ranges, mixed over the
    tree: alpha = 1 (no decay), beta = 0 (no write: only the decay acts),
    beta = 1 (the key's old value replaced), and alpha near 0."""
    S0, q, k, v, a, b, parent = synth.deltanet_case(T, H, dk, dv, seed=31 + T, shape="bushy")
    a = a.copy()
    b = b.copy()
    a[::3] = 1.0
    a[1::5] = 1e-3
    b[::4] = 0.0
    b[2::4] = 1.0
    case = (S0, q, k, v, a, b, parent)
    Sd, qd, kd, vd, ad, bd, pd = dev(case)
    out = torch.empty((T, H, dv), dtype=torch.float32, device=C.DEV)
    svg.tree_deltanet_verify(Sd, qd, kd, vd, ad, bd, pd, out)
    close(C.host(out), DN.tree_verify(*case))
    path = TO.root_path(parent, T - 1)[1:]
    n = torch.tensor([len(path) + 1], dtype=torch.int32, device=C.DEV)
    pathd = torch.full((T,), -1, dtype=torch.int32, device=C.DEV)
    if path:
        pathd[:len(path)] = C.to_dev(np.array(path, np.int32))
    svg.tree_deltanet_commit(Sd, kd, vd, ad, bd, pathd, n)
    close(C.host(Sd), DN.tree_commit(*case, path))


def test_commit_of_a_rejected_tree_leaves_the_state():
    T, H, dk, dv = 6, 2, 128, 128
    case = synth.deltanet_case(T, H, dk, dv, seed=11)
    S0 = case[0]
    Sd, _q, kd, vd, ad, bd, _pd = dev(case)
    path = torch.full((T,), -1, dtype=torch.int32, device=C.DEV)
    svg.tree_deltanet_commit(Sd, kd, vd, ad, bd, path, torch.tensor([-1], dtype=torch.int32, device=C.DEV))
    assert np.array_equal(C.host(Sd), S0)
    # a path naming a node outside the tree is refused the same way
    bad = torch.tensor([1, 9, -1, -1, -1, -1], dtype=torch.int32, device=C.DEV)
    svg.tree_deltanet_commit(Sd, kd, vd, ad, bd, bad, torch.tensor([3], dtype=torch.int32, device=C.DEV))
    assert np.array_equal(C.host(Sd), S0)


def test_malformed_links_give_nan_only_below_them():
    T, H, dk, dv = 8, 2, 64, 64
    S0, q, k, v, a, b, parent = synth.deltanet_case(T, H, dk, dv, seed=12, shape="chain")
    bad = parent.copy()
    bad[4] = 6                                               # not an earlier node
    Sd, qd, kd, vd, ad, bd, _pd = dev((S0, q, k, v, a, b, parent))
    out = torch.empty((T, H, dv), dtype=torch.float32, device=C.DEV)
    svg.tree_deltanet_verify(Sd, qd, kd, vd, ad, bd, C.to_dev(bad.astype(np.int32)), out)
    got = C.host(out)
    ref = DN.tree_verify(S0, q, k, v, a, b, parent)
    assert np.isnan(got[4:]).all()                           # nodes 4..7 of the chain hang below node 4
    close(got[:4], ref[:4])
