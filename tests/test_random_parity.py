"""GPU parity over seeded random shapes, through the C ABI, against the CPU
oracle: every weight format, group, transform block, row count from 1 to 32,
ragged N and K (any multiple of 32 the format admits, below one 128-k chunk
too), each through the fused call, the workspace call and the separate
quantization + linear calls.  Codes, scales and per-group partials compare
bit for bit; y within 2e-3 of the fp64 reference; the three calls' y agree
bit for bit (one set of codes, one fixed summation order per output).

The shapes are drawn once from a fixed seed (the list is printed with each
case), so every run checks the same cases.

Source of the method: "Karpathy's Trick for Faster Local LLMs Finally Has
Proper Tooling" (blog.dailydoseofds.com), section "How Uzu optimizes bytes
and tokens per pass".
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
import storage_layout as SL
from oracle import svg_oracle as O

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _draw_cases(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        fmt = ("w4_z4", "w4_z16", "w8")[i % 3]
        group = 0 if fmt == "w8" else int(rng.choice([32, 64, 128]))
        block = int(rng.choice([32, 64]))
        step = max(32, group, block)
        K = step * int(rng.integers(1, max(2, 6144 // step) + 1))
        M = int(rng.choice([1, 1, 2, 3, 5, 8, 13, 16, 17, 24, 32]))
        N = int(rng.integers(1, 400))
        cases.append((fmt, group, block, M, N, K, 1000 + i))
    return cases


# plus rows shorter than one 128-k chunk
CASES = _draw_cases() + [("w4_z16", 32, 32, 1, 50, 96, 2000), ("w8", 0, 32, 3, 20, 64, 2001),
                         ("w4_z4", 64, 64, 2, 7, 64, 2002), ("w4_z16", 128, 64, 17, 33, 128, 2003)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global C, svg
    import svg_cases as C  # noqa: F401  (imports the binding, which loads libsvgemm)
    import speculative_verify_gemm_amd as svg


def _call(fmt, group, block, X, signs, w, N, workspace):
    M, K = X.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=C.DEV)
    xs = torch.empty((M,), dtype=torch.float32, device=C.DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=C.DEV)
    if fmt == "w8":
        dbg = torch.empty((M, N), dtype=torch.int32, device=C.DEV)
        svg.act_quant_w8a8_linear(X, signs, xq, xs, w["wq"], w["ws"], N, y, dbg, block=block, workspace=workspace)
    else:
        dbg = torch.empty((M, N, K // group), dtype=torch.int32, device=C.DEV)
        svg.act_quant_w4a8_linear(X, signs, xq, xs, w["wq"], w["ws"], w["wz"], fmt, group, N, y, dbg,
                                  block=block, workspace=workspace)
    return xq, xs, y, dbg


@pytest.mark.parametrize("fmt,group,block,M,N,K,seed", CASES)
def test_random_shape(fmt, group, block, M, N, K, seed):
    C.say(f"random case fmt={fmt} g={group} block={block} M={M} N={N} K={K} seed={seed}")
    x, W, signs = synth.random_case(M, N, K, seed=seed, x_kind="student_t3" if seed % 2 else "normal_outlier")
    if fmt == "w8":
        ow = O.prepare_w8(W, signs, block=block)
        y_ref, S_ref, qx, sx = O.linear_w8(x, signs, ow)
    else:
        ow = O.prepare_w4(W, signs, group, block=block)
        y_ref, S_ref, qx, sx = O.linear_w4(x, signs, ow)
    w = C.gpu_prepare(W, signs, fmt, group, block=block)
    X, sd = C.to_dev(x), C.to_dev(signs)
    ws = svg.linear_workspace(C.DEV)
    outs = {"fused": _call(fmt, group, block, X, sd, w, N, None),
            "workspace": _call(fmt, group, block, X, sd, w, N, ws)}
    xq_s, xs_s = C.gpu_quant_acts(x, signs, block=block)
    y_s, dbg_s = C.gpu_linear(xq_s, xs_s, w)
    outs["separate"] = (xq_s, xs_s, y_s, dbg_s)
    assert not svg.linear_workspace_gave_up(ws)
    assert int(C.host(ws)[:3].sum()) == 0  # counters back to zero
    ref_bits = None
    for name, (xq, xs, y, dbg) in outs.items():
        assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx)), name
        assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32)), name
        assert np.array_equal(C.host(dbg).astype(np.int64), S_ref), name
        yh = C.host(y)
        e, r, ex = O.output_error(yh, y_ref)
        assert e <= TOL and r <= TOL, (name, e, r, ex)
        if ref_bits is None:
            ref_bits = yh.view(np.uint32)
        assert np.array_equal(yh.view(np.uint32), ref_bits), name
