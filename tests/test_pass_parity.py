"""GPU parity of the one-launch pass (svg_pass_plan / svg_pass_run) against
the CPU oracle, through the C ABI.

Every step of a pass is act_quant_w4a8_linear on its own input rows, so every
step is checked as that call is: activation codes and scales and the per-group
int32 partial sums bit for bit (xq in the library's slab layout), y within
2e-3 of the fp64 reference.  Passes mix the launch shapes the kernel has:
M = 1 (dot products, the row quantized by every workgroup) and M = 2..16
(matrix cores, the rows quantized once per XCC), K up to 12288 (rows cut along
K into two halves where M x K does not fit LDS), ragged N, both zero formats,
groups of 64 and 128, both transform blocks, steps with and without a
dependency, and chains whose input IS the previous step's output.

Source of the method: "Karpathy's Trick for Faster Local LLMs Finally Has
Proper Tooling" (blog.dailydoseofds.com), sections "How Uzu optimizes bytes and
tokens per pass" and "Why batch-one decoding is memory-bound".
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import svg_oracle as O
import storage_layout as SL

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global C, svg
    import svg_cases as C  # noqa: F401  (imports the binding, which loads libsvgemm)
    import speculative_verify_gemm_amd as svg


def check_y(y, y_ref, tol=TOL):
    e, r, ex = O.output_error(y, y_ref)
    assert e <= tol and r <= tol, (e, r, ex)


def _step(M, N, K, fmt, group, seed, block=32, after=1, debug=True, x=None):
    """A step's inputs (host) and device buffers; the oracle's encoded weights
    go to the device in the library's storage."""
    xh, W, signs = synth.random_case(M, N, K, seed=seed, x_kind="student_t3")
    if x is not None:
        xh = x
    ow = O.prepare_w4(W, signs, group, block)
    w = C.oracle_weights_to_dev(ow, fmt)
    st = dict(X=C.to_dev(xh), signs=C.to_dev(signs), xq=torch.full((M, K), 99, dtype=torch.int8, device=C.DEV),
              x_scale=torch.full((M,), -1.0, device=C.DEV), wq=w["wq"], w_scale=w["ws"], w_zero=w["wz"], N=N,
              y=torch.full((M, N), 12345.0, device=C.DEV), after=after)
    if debug:
        st["partials_debug"] = torch.full((M, N, K // group), -7, dtype=torch.int32, device=C.DEV)
    return st, dict(x=xh, signs=signs, ow=ow, block=block)


def _check_step(st, ref, M):
    y_ref, S_ref, qx, sx = O.linear_w4(ref["x"], ref["signs"], ref["ow"])
    assert np.array_equal(C.host(st["xq"]).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(st["x_scale"]).view(np.uint32), sx.view(np.uint32))
    if "partials_debug" in st:
        assert np.array_equal(C.host(st["partials_debug"]).astype(np.int64), S_ref)
    check_y(C.host(st["y"]), y_ref)


def _counters_clean(p):
    """Every counter word of the workspace is back to zero after a run (word 0
    is the give-up flag; the staging rows and split partials after the
    counters are data and keep the last run's values)."""
    hdr = C.host(p.plan[:64]).view(np.uint32)
    xbase = int(hdr[8])                      # first word after the counters
    ws = C.host(p.workspace).view(np.uint32)
    return not ws[1:xbase].any()


def _run(steps, fmt, group, block=32, reps=1):
    p = svg.LinearPass(steps, fmt, group, block=block)
    for _ in range(reps):
        p.run()
    torch.cuda.synchronize()
    assert not p.gave_up()
    assert _counters_clean(p), "the workspace's counters must be left zero-filled"
    return p


# (M, fmt, group, block, [(N, K, after), ...])
PASSES = [
    (1, "w4_z16", 64, 32, [(300, 4096, 1), (37, 1024, 1), (96, 12288, 0), (16, 4096, 1)]),
    (1, "w4_z4", 128, 32, [(130, 8192, 1), (1, 384, 1), (48, 12288, 1)]),
    (1, "w4_z4", 64, 64, [(64, 2048, 1), (33, 4096, 1)]),
    (16, "w4_z16", 64, 32, [(300, 4096, 1), (37, 1024, 1), (64, 12288, 1), (16, 4096, 1)]),
    (16, "w4_z16", 128, 32, [(130, 8192, 1), (50, 12288, 1)]),
    (2, "w4_z4", 64, 32, [(70, 4096, 1), (40, 12288, 1), (33, 640, 0)]),
    (5, "w4_z16", 128, 64, [(100, 2048, 1), (20, 12288, 1)]),
    (16, "w4_z4", 128, 32, [(17, 128, 1), (300, 6144, 1)]),
    (9, "w4_z16", 64, 32, [(512, 10240, 1)]),
]


@pytest.mark.parametrize("M,fmt,group,block,shape", PASSES)
def test_pass_matches_oracle(M, fmt, group, block, shape):
    C.say(f"pass M={M} {fmt} g{group} block {block}: steps {shape}")
    steps, refs = [], []
    for i, (N, K, after) in enumerate(shape):
        st, ref = _step(M, N, K, fmt, group, seed=1000 * M + 10 * i + group, block=block, after=after)
        steps.append(st)
        refs.append(ref)
    _run(steps, fmt, group, block)
    for st, ref in zip(steps, refs):
        _check_step(st, ref, M)


@pytest.mark.parametrize("M,group", [(1, 64), (16, 64), (4, 128)])
def test_pass_chain_reads_the_previous_output(M, group):
    """Step 2's input is step 1's y (and step 3's is step 2's): the codes of
    the later steps must be the oracle's codes of the values the earlier step
    wrote, so the later step read them only after they were complete.  Run
    twice on different first inputs (stale values from the first run would
    show in the second)."""
    fmt, N1, K1, N2, N3 = "w4_z16", 1024, 4096, 2048, 64
    C.say(f"pass chain M={M} g{group}")
    s1, r1 = _step(M, N1, K1, fmt, group, seed=71 + M, after=1)
    s2, r2 = _step(M, N2, N1, fmt, group, seed=72 + M, after=1)
    s3, r3 = _step(M, N3, N2, fmt, group, seed=73 + M, after=1)
    s2["X"] = s1["y"]
    s3["X"] = s2["y"]
    p = svg.LinearPass([s1, s2, s3], fmt, group)
    for rep in range(2):
        if rep:
            x1 = synth.random_case(M, 1, K1, seed=500 + M, x_kind="normal")[0]
            s1["X"].copy_(C.to_dev(x1))
            r1["x"] = x1
        p.run()
        torch.cuda.synchronize()
        assert not p.gave_up()
        _check_step(s1, r1, M)
        r2["x"] = C.host(s1["y"]).copy()
        _check_step(s2, r2, M)
        r3["x"] = C.host(s2["y"]).copy()
        _check_step(s3, r3, M)


@pytest.mark.parametrize("M", [1, 16])
def test_pass_repeats_and_replays_in_a_graph(M):
    """The same pass run eagerly three times and replayed from a captured HIP
    graph three times: every run bit-identical, the workspace clean after
    each."""
    fmt, group = "w4_z16", 64
    C.say(f"pass graph M={M}")
    steps = [_step(M, N, K, fmt, group, seed=90 + i, debug=False)[0]
             for i, (N, K) in enumerate([(256, 4096), (64, 12288), (512, 4096)])]
    p = _run(steps, fmt, group, reps=3)
    ref = [C.host(s["y"]).copy() for s in steps]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        p.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        p.run()
    for rep in range(3):
        for s in steps:
            s["y"].fill_(0.0)
        g.replay()
        torch.cuda.synchronize()
        assert not p.gave_up()
        for s, r in zip(steps, ref):
            assert np.array_equal(C.host(s["y"]).view(np.uint32), r.view(np.uint32)), rep
        assert _counters_clean(p)


@pytest.mark.parametrize("M", [1, 16])
def test_pass_on_a_stack_layer(M):
    """One layer of the 7B stack (q/k/v stacked, o, gate/up stacked, down) at
    full size, as the benchmark runs it: sampled output rows of every launch
    against the oracle (partials bit-exact, y within tolerance), the
    activation codes whole."""
    fmt, group = "w4_z16", 64
    C.say(f"pass stack layer M={M}")
    steps, meta = [], []
    for launch in ("qkv", "o", "gateup", "down"):
        w, Ws, signs, space = C.stack_launch(0, launch, fmt, group)
        K, N = w["K"], w["N"]
        x = synth.stack_acts("stack_w4g64", 0, space, M)
        steps.append(dict(X=C.to_dev(x), signs=C.to_dev(signs), xq=torch.empty((M, K), dtype=torch.int8, device=C.DEV),
                          x_scale=torch.empty((M,), device=C.DEV), wq=w["wq"], w_scale=w["ws"], w_zero=w["wz"], N=N,
                          y=torch.empty((M, N), device=C.DEV),
                          partials_debug=torch.empty((M, N, K // group), dtype=torch.int32, device=C.DEV), after=1))
        meta.append((Ws, signs, x, N, K))
    _run(steps, fmt, group)
    rng = np.random.default_rng(5)
    for st, (Ws, signs, x, N, K) in zip(steps, meta):
        rows = sorted(set(rng.choice(N, size=24, replace=False).tolist()) | {0, N - 1})
        W = C.stacked_rows(Ws, rows)
        ow = O.prepare_w4(W, signs, group)
        y_ref, S_ref, qx, sx = O.linear_w4(x, signs, ow)
        assert np.array_equal(C.host(st["xq"]).reshape(-1), SL.pack_act_codes(qx))
        assert np.array_equal(C.host(st["x_scale"]).view(np.uint32), sx.view(np.uint32))
        assert np.array_equal(C.host(st["partials_debug"])[:, rows].astype(np.int64), S_ref)
        check_y(C.host(st["y"])[:, rows], y_ref)
