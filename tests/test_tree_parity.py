"""GPU parity of greedy tree acceptance: tree_accept_greedy against the CPU
oracle (oracle/tree_oracle.py), through the C ABI.  Everything compared is
integer, so everything must match exactly: the target's choice per node, the
accepted path, the emitted tokens and their count.

Source of the step: "Karpathy's Trick for Faster Local LLMs Finally Has Proper
Tooling" (blog.dailydoseofds.com), sections "Producing several tokens from one
model pass" and "Issue with parallel draft generation".
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import tree_oracle as TO

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global C, svg
    import svg_cases as C  # noqa: F401  (imports the binding, which loads libsvgemm)
    import speculative_verify_gemm_amd as svg


def _outputs(T):
    z = lambda: torch.full((T,), -7, dtype=torch.int32, device=C.DEV)  # noqa: E731
    return z(), z(), z(), torch.full((1,), -7, dtype=torch.int32, device=C.DEV)


def gpu_tree(logits_dev, parent, draft, ws):
    T = logits_dev.shape[0]
    target, path, emit, n = _outputs(T)
    svg.tree_accept_greedy(logits_dev, C.to_dev(parent.astype(np.int32)), C.to_dev(draft.astype(np.int32)),
                           target, path, emit, n, ws)
    torch.cuda.synchronize()
    return (target.cpu().numpy(), path.cpu().numpy(), emit.cpu().numpy(), int(n.cpu().numpy()[0]))


def check(got, logits, parent, draft):
    target, path, emit, n = got
    t_ref, p_ref, e_ref = TO.verify_tree(logits, parent, draft)
    T = len(parent)
    assert np.array_equal(target, t_ref.astype(np.int32))
    assert n == len(e_ref)
    assert list(path) == p_ref + [-1] * (T - len(p_ref))
    assert list(emit) == e_ref + [-1] * (T - len(e_ref))
    return n


CASES = [  # T, V, tree shape, planted agreement depth, exact ties
    (1, 1, "chain", None, False), (1, 7, "chain", None, False), (2, 5, "chain", 1, False),
    (5, 3, "bushy", 2, True), (9, 2, "star", None, True), (12, 4, "chain", 6, False),
    (16, 131072, "bushy", 6, True), (32, 131072, "bushy", 10, True), (32, 131072, "chain", 31, False),
    (32, 50257, "chain", 20, True),        # V % 4 != 0: element-wise loads
    (17, 8193, "bushy", 5, True),          # two slices per row, ragged
    (32, 262144, "star", 1, True), (24, 1000003, "bushy", 8, False), (31, 12, "bushy", 4, True),
]


@pytest.mark.parametrize("T,V,shape,accept,ties", CASES)
def test_tree_accept_matches_oracle(T, V, shape, accept, ties):
    C.say(f"tree_accept_greedy T={T} V={V} shape={shape} accept={accept} ties={ties}")
    logits, parent, draft = synth.draft_tree(T, V, seed=T * 7 + V, shape=shape, accept=accept, ties=ties)
    ws = svg.tree_workspace()
    check(gpu_tree(C.to_dev(logits), parent, draft, ws), logits, parent, draft)
    assert int(ws.count_nonzero()) == 0, "the workspace must be left zero-filled"


def test_worked_example_on_the_gpu():
    """Five drafted tokens, the target agrees with the first four: five tokens."""
    V = 100
    drafts = [11, 22, 33, 44, 55]
    parent = np.array([-1, 0, 1, 2, 3, 4])
    draft = np.array([7] + drafts)
    logits = np.zeros((6, V), np.float32)
    for r, c in enumerate(drafts[:4] + [66, 77]):
        logits[r, c] = 1.0
    got = gpu_tree(C.to_dev(logits), parent, draft, svg.tree_workspace())
    assert check(got, logits, parent, draft) == 5
    assert list(got[2][:5]) == drafts[:4] + [66]


def test_unaligned_rows_take_the_elementwise_loads():
    T, V = 8, 4096
    logits, parent, draft = synth.draft_tree(T, V, seed=3, accept=4, ties=True)
    flat = torch.zeros(T * V + 1, dtype=torch.float32, device=C.DEV)
    flat[1:] = C.to_dev(logits.reshape(-1))
    view = flat[1:].view(T, V)                      # 4-byte but not 16-byte aligned
    assert view.data_ptr() % 16 != 0
    check(gpu_tree(view, parent, draft, svg.tree_workspace()), logits, parent, draft)


def test_infinite_logits():
    """Rows holding +inf (the first +inf wins), rows entirely -inf (index 0
    wins), -0.0 against +0.0 (equal values: the first wins, whichever sign it
    has) and the largest finite values: the order on the keys is the order of
    the floats."""
    T, V = 12, 3000
    logits, parent, draft = synth.draft_tree(T, V, seed=21, accept=5, ties=True)
    logits = logits.copy()
    logits[1, [7, 2900]] = np.inf
    logits[2, :] = -np.inf
    logits[3, :] = 0.0
    logits[3, 5] = -0.0
    logits[3, 4] = -0.0
    logits[4, [10, 11]] = np.finfo(np.float32).max
    logits[5, 0] = -np.inf
    logits[6, :] = -1.0
    logits[6, [3, 9]] = [-0.0, 0.0]  # equal maxima: -0.0 comes first and wins
    check(gpu_tree(C.to_dev(logits), parent, draft, svg.tree_workspace()), logits, parent, draft)


def test_malformed_tree_is_flagged():
    T, V = 6, 50
    logits, parent, draft = synth.draft_tree(T, V, seed=4, accept=3)
    parent = parent.copy()
    parent[3] = 5                                   # not an earlier node
    target, path, emit, n = gpu_tree(C.to_dev(logits), parent, draft, svg.tree_workspace())
    assert n == -1 and (path == -1).all() and (emit == -1).all()
    assert np.array_equal(target, TO.target_choices(logits).astype(np.int32))


def test_workspace_reuse_across_calls():
    """One workspace, calls of different sizes back to back: each is right."""
    ws = svg.tree_workspace()
    for i, (T, V) in enumerate([(32, 70000), (3, 9), (16, 131072), (32, 5), (1, 1000)]):
        logits, parent, draft = synth.draft_tree(T, V, seed=50 + i, accept=T // 2, ties=True)
        check(gpu_tree(C.to_dev(logits), parent, draft, ws), logits, parent, draft)
    assert int(ws.count_nonzero()) == 0


def test_tree_accept_in_captured_graph():
    """Captured once, replayed on new inputs copied into the same buffers."""
    T, V = 16, 131072
    ws = svg.tree_workspace()
    logits_d = torch.empty((T, V), dtype=torch.float32, device=C.DEV)
    parent_d = torch.empty((T,), dtype=torch.int32, device=C.DEV)
    draft_d = torch.empty((T,), dtype=torch.int32, device=C.DEV)
    target, path, emit, n = _outputs(T)
    inputs = [synth.draft_tree(T, V, seed=90 + i, accept=3 + 2 * i, ties=True) for i in range(4)]

    def load(i):
        lg, pa, dr = inputs[i]
        logits_d.copy_(C.to_dev(lg))
        parent_d.copy_(C.to_dev(pa.astype(np.int32)))
        draft_d.copy_(C.to_dev(dr.astype(np.int32)))

    load(0)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        svg.tree_accept_greedy(logits_d, parent_d, draft_d, target, path, emit, n, ws)  # warm-up, eager
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        svg.tree_accept_greedy(logits_d, parent_d, draft_d, target, path, emit, n, ws)
    for i in range(4):
        load(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        lg, pa, dr = inputs[i]
        got = (target.cpu().numpy(), path.cpu().numpy(), emit.cpu().numpy(), int(n.cpu().numpy()[0]))
        check(got, lg, pa, dr)
    assert int(ws.count_nonzero()) == 0
