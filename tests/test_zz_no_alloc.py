"""tree_accept_greedy_static (the entry point that allocates nothing: its
workspace is the library's static device array) against tree_accept_greedy
with a caller workspace, through the C ABI: bit-identical outputs on two calls
in a row, the second on a smaller tree and vocabulary, then once more on the
first inputs (the array must have been left zero-filled by every call).

Source of the rule: "Karpathy's Trick for Faster Local LLMs Finally Has Proper
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


def _run(svg, fn, logits, parent, draft, ws=None):
    dev = torch.device("cuda:0")
    T = logits.shape[0]
    lg = torch.from_numpy(logits).to(dev)
    pa = torch.from_numpy(parent.astype(np.int32)).to(dev)
    dr = torch.from_numpy(draft.astype(np.int32)).to(dev)
    outs = [torch.full((T,), -7, dtype=torch.int32, device=dev) for _ in range(3)]
    n = torch.full((1,), -7, dtype=torch.int32, device=dev)
    if ws is None:
        fn(lg, pa, dr, outs[0], outs[1], outs[2], n)
    else:
        fn(lg, pa, dr, outs[0], outs[1], outs[2], n, ws)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs] + [n.cpu().numpy()]


def test_static_workspace_matches_caller_workspace():
    import speculative_verify_gemm_amd as svg
    cases = [(32, 131072, 11, "bushy"), (7, 3001, 12, "chain"), (32, 131072, 11, "bushy")]
    ws = svg.tree_workspace()
    for T, V, seed, shape in cases:
        print(f"[no-alloc] tree_accept_greedy_static T={T} V={V} seed={seed} {shape}", flush=True)
        logits, parent, draft = synth.draft_tree(T, V, seed=seed, shape=shape, accept=T // 2, ties=True)
        got = _run(svg, svg.tree_accept_greedy_static, logits, parent, draft)
        ref = _run(svg, svg.tree_accept_greedy, logits, parent, draft, ws)
        for g, r in zip(got, ref):
            assert np.array_equal(g, r), (T, V)
        # and both are the oracle's
        t_ref, p_ref, e_ref = TO.verify_tree(logits, parent, draft)
        assert np.array_equal(got[0], t_ref.astype(np.int32))
        assert int(got[3][0]) == len(e_ref)
        assert list(got[1]) == p_ref + [-1] * (T - len(p_ref))
        assert list(got[2]) == e_ref + [-1] * (T - len(e_ref))
