"""GPU parity of the fused calls with a workspace (act_quant_w4a8_linear_ws /
act_quant_w8a8_linear_ws), whose verify-batch rows are rotated and quantized
inside the linear's own launch by workgroups 0 .. M-1 (each publishing its
rows to the others), through the C ABI, against the CPU oracle:

 * activation codes and scales bit-exact, per-group partials bit-exact, y
   within 2e-3 of the fp64 reference;
 * y bit-identical to the same call without a workspace (the rows quantized
   in a launch of their own, then the same linear kernel);
 * the workspace's counters back to zero after every call, the give-up flag
   clear;
 * repeated calls on new inputs (a stale row would show), and replays of a
   captured graph.

Cases span M = 1 (rows longer than the single-row fused kernel holds) to 32,
both W4 zero formats, groups of 64 and 128, W8, ragged N, K up to 16384.

Source of the method: "Karpathy's Trick for Faster Local LLMs Finally Has
Proper Tooling" (blog.dailydoseofds.com), sections "Producing several tokens
from one model pass" and "How Uzu optimizes bytes and tokens per pass".
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import svg_oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global C, svg
    import svg_cases as C  # noqa: F401  (imports the binding, which loads libsvgemm)
    import speculative_verify_gemm_amd as svg


def _call(x, signs, w, ws, debug=True):
    xd, sd = C.to_dev(x), C.to_dev(signs)
    M, K = x.shape
    N = w["N"]
    xq = torch.full((M, K), 99, dtype=torch.int8, device=C.DEV)
    xs = torch.full((M,), -1.0, device=C.DEV)
    y = torch.full((M, N), 12345.0, device=C.DEV)
    if w["fmt"] == "w8":
        dbg = torch.empty((M, N), dtype=torch.int32, device=C.DEV) if debug else None
        svg.act_quant_w8a8_linear(xd, sd, xq, xs, w["wq"], w["ws"], N, y, dbg, workspace=ws)
    else:
        dbg = torch.empty((M, N, K // w["group"]), dtype=torch.int32, device=C.DEV) if debug else None
        svg.act_quant_w4a8_linear(xd, sd, xq, xs, w["wq"], w["ws"], w["wz"], w["fmt"], w["group"], N, y, dbg,
                                  workspace=ws)
    return xq, xs, y, dbg


def _clean(ws):
    return not C.host(ws)[:4].any()


CASES = [("w4_z16", 64, 16, 300, 4096), ("w4_z16", 64, 2, 37, 1024), ("w4_z4", 64, 5, 130, 2048),
         ("w4_z16", 128, 8, 64, 12288), ("w4_z4", 128, 32, 200, 4096), ("w4_z16", 64, 17, 45, 640),
         ("w4_z16", 64, 1, 96, 16384), ("w8", 0, 32, 300, 4096), ("w8", 0, 3, 37, 1024),
         ("w8", 0, 16, 64, 12288)]


@pytest.mark.parametrize("fmt,group,M,N,K", CASES)
def test_shared_matches_oracle_and_the_separate_launch(fmt, group, M, N, K):
    C.say(f"shared quantization {fmt} g{group} M={M} N={N} K={K}")
    x, W, signs = synth.random_case(M, N, K, seed=M * 101 + N + K + group, x_kind="student_t3")
    if fmt == "w8":
        ow = O.prepare_w8(W, signs)
        y_ref, S_ref, qx, sx = O.linear_w8(x, signs, ow)
    else:
        ow = O.prepare_w4(W, signs, group)
        y_ref, S_ref, qx, sx = O.linear_w4(x, signs, ow)
    w = C.oracle_weights_to_dev(ow, fmt)
    ws = svg.linear_workspace(C.DEV)
    xq, xs, y, dbg = _call(x, signs, w, ws)
    rows = torch.empty((M, K), dtype=torch.int8, device=C.DEV)
    svg.export_act_codes(xq, rows)
    assert np.array_equal(C.host(rows), qx)
    assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32))
    assert np.array_equal(C.host(dbg).astype(np.int64), S_ref)
    e, r, ex = O.output_error(C.host(y), y_ref)
    assert e <= TOL and r <= TOL, (e, r, ex)
    assert _clean(ws), "the workspace's counters must be left zero-filled"
    # the same call without a workspace: bit-identical outputs
    _xq2, _xs2, y2, _d2 = _call(x, signs, w, None, debug=False)
    assert np.array_equal(C.host(y2).view(np.uint32), C.host(y).view(np.uint32))


@pytest.mark.parametrize("fmt,group,M", [("w4_z16", 64, 16), ("w8", 0, 32)])
def test_shared_repeats_and_replays(fmt, group, M):
    """Several calls on one workspace with new inputs each time, then replays
    of a captured graph of the call: every output against the eager call of
    the same inputs, bit for bit."""
    N, K = 256, 4096
    C.say(f"shared quantization repeats {fmt} M={M}")
    _x, W, signs = synth.random_case(M, N, K, seed=7 + M)
    ow = O.prepare_w8(W, signs) if fmt == "w8" else O.prepare_w4(W, signs, group)
    w = C.oracle_weights_to_dev(ow, fmt)
    ws = svg.linear_workspace(C.DEV)
    for rep in range(3):
        x = synth.random_case(M, 1, K, seed=100 + rep, x_kind="normal")[0]
        _xq, _xs, y, _d = _call(x, signs, w, ws, debug=False)
        y_ref = (O.linear_w8(x, signs, ow) if fmt == "w8" else O.linear_w4(x, signs, ow))[0]
        e, r, ex = O.output_error(C.host(y), y_ref)
        assert e <= TOL and r <= TOL, (rep, e, r, ex)
        assert _clean(ws)
    # graph replay
    x = synth.random_case(M, 1, K, seed=300, x_kind="student_t3")[0]
    xd, sd = C.to_dev(x), C.to_dev(signs)
    xq = torch.empty((M, K), dtype=torch.int8, device=C.DEV)
    xs = torch.empty((M,), device=C.DEV)
    y = torch.empty((M, N), device=C.DEV)

    def call():
        if fmt == "w8":
            svg.act_quant_w8a8_linear(xd, sd, xq, xs, w["wq"], w["ws"], N, y, workspace=ws)
        else:
            svg.act_quant_w4a8_linear(xd, sd, xq, xs, w["wq"], w["ws"], w["wz"], fmt, group, N, y, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = C.host(y).copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        y.fill_(0.0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.host(y).view(np.uint32), ref.view(np.uint32)), rep
        assert _clean(ws)
