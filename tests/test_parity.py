"""GPU parity: the HIP library against the CPU oracle, through the C ABI.

Integer stages (activation codes, weight codes, scales and zeros, per-group
int32 partial sums) must match bit for bit, in the library's storage orders
(the oracle's packers give them); fp32 outputs must match the fp64
reference within 2e-3 (oracle.output_error: elementwise over |y_ref| >= 1e-3
of the row maximum, and row-normwise over all elements).

Source of the method: "Karpathy's Trick for Faster Local LLMs Finally Has
Proper Tooling" (blog.dailydoseofds.com), section "How Uzu optimizes bytes and
tokens per pass".
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synth
from oracle import svg_oracle as O
import storage_layout as SL
from oracle import tree_oracle as TO

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
    return e, r


# ------------------------------------------------------------ activations
ACT_CASES = [(1, 1024, "single_1k"), (1, 4096, "decode_12k"), (16, 4096, None), (32, 12288, None),
             (3, 96, None), (5, 1120, None), (2, 32, None), (7, 2080, None),
             # one row length per launch shape of the stand-alone kernel (rows of
             # 3, 6 and 8 chunks per thread, and a row read twice)
             (2, 8224, None), (2, 16416, None), (3, 32736, None), (1, 32800, None)]


@pytest.mark.parametrize("M,K,src", ACT_CASES)
def test_act_codes_bit_exact(M, K, src):
    C.say(f"act_rht_quant_i8 M={M} K={K}")
    if src:
        x, W, signs, spec = synth.single_inputs(src)
    else:
        x, _W, signs = synth.random_case(M, 1, K, seed=M * 1000 + K, x_kind="student_t3")
        if M >= 2:
            x[1] = 0.0  # an all-zero token
    qx, sx = O.quant_acts(x, signs)
    xq, xs = C.gpu_quant_acts(x, signs)
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32))


# ---------------------------------------------------------------- weights
W_CASES = [("w4_z4", 32, 64, 1024), ("w4_z16", 64, 48, 4096), ("w4_z16", 128, 37, 384),
           ("w4_z4", 64, 33, 192), ("w4_z4", 128, 20, 384), ("w4_z16", 32, 17, 96),
           ("w8", 0, 45, 1120), ("w8", 0, 16, 32)]


@pytest.mark.parametrize("fmt,group,N,K", W_CASES)
def test_weight_codes_bit_exact(fmt, group, N, K):
    C.say(f"rht_rotate_weights fmt={fmt} g={group} N={N} K={K}")
    _x, W, signs = synth.random_case(1, N, K, seed=N + K + group)
    W[0, :] = 0.0        # a zero row (every group constant)
    W[1, : min(K, 64)] = 0.013
    w = C.gpu_prepare(W, signs, fmt, group, debug=True)
    u = O.rht(W, signs)
    assert np.array_equal(C.host(w["rot"]).view(np.uint32), u.view(np.uint32))
    if fmt == "w8":
        q, s = O.quant_w8(u)
        ow = dict(q=q, s=s)
    else:
        q, s, z = O.quant_w4(u, group)
        ow = dict(q=q, s=s, z=z, group=group)
    wq, ws, wz = C.oracle_storage(ow, fmt, K)
    assert np.array_equal(C.host(w["wq"]).view(np.uint8), wq.view(np.uint8).reshape(-1))
    assert np.array_equal(C.host(w["ws"]).view(np.uint16), ws.view(np.uint16).reshape(-1))
    if wz is not None:
        assert np.array_equal(C.host(w["wz"]).view(np.uint8), wz.view(np.uint8).reshape(-1))


# ----------------------------------------------------------------- linear
LIN_CASES = []
for fmt in ("w4_z4", "w4_z16"):
    for g in (32, 64, 128):
        for M in (1, 2, 3, 8, 16, 17, 32):
            LIN_CASES.append((fmt, g, M, 37, 384))
LIN_CASES += [("w4_z16", 64, M, 64, 320) for M in (1, 2, 5, 16, 32)]      # K % 128 == 64
LIN_CASES += [("w4_z4", 32, M, 50, 96) for M in (1, 4, 32)]               # K < 128
LIN_CASES += [("w4_z16", 64, 16, 300, 4096), ("w4_z16", 128, 32, 130, 12288)]
LIN_CASES += [("w8", 0, M, 37, 384) for M in (1, 2, 3, 16, 17, 32)]
LIN_CASES += [("w8", 0, M, 29, 96) for M in (1, 32)] + [("w8", 0, 32, 70, 12288)]
# more than 16 rows with long K: 8-wave workgroups of 256 registers, also
# with K short of the shape's chunks (the last waves read zeros)
LIN_CASES += [("w4_z16", 64, 24, 48, 12288), ("w4_z4", 64, 20, 33, 10240), ("w4_z16", 128, 31, 16, 8320),
              ("w8", 0, 17, 40, 11264), ("w8", 0, 25, 24, 12288)]


@pytest.mark.parametrize("fmt,group,M,N,K", LIN_CASES)
def test_linear_matches_oracle(fmt, group, M, N, K):
    C.say(f"linear fmt={fmt} g={group} M={M} N={N} K={K}")
    x, W, signs = synth.random_case(M, N, K, seed=7 * M + N + K + group)
    if fmt == "w8":
        ow = O.prepare_w8(W, signs)
        y_ref, S_ref, qx, sx = O.linear_w8(x, signs, ow)
    else:
        ow = O.prepare_w4(W, signs, group)
        y_ref, S_ref, qx, sx = O.linear_w4(x, signs, ow)
    w = C.oracle_weights_to_dev(ow, fmt)
    y, dbg = C.gpu_linear(C.to_dev(SL.pack_act_codes(qx).reshape(qx.shape)), C.to_dev(sx), w)
    assert np.array_equal(C.host(dbg).astype(np.int64), S_ref)
    check_y(C.host(y), y_ref)


@pytest.mark.parametrize("fmt,group,M", [("w4_z4", 32, 1), ("w4_z16", 64, 16), ("w4_z16", 128, 32),
                                         ("w4_z16", 64, 2), ("w8", 0, 32), ("w8", 0, 1)])
def test_end_to_end_and_deterministic(fmt, group, M):
    """All three entry points chained on the device; two runs bit-identical;
    guard bands around the output untouched; the hot path without the debug
    pointer gives the same y."""
    N, K = 96, 1024
    C.say(f"end-to-end fmt={fmt} g={group} M={M}")
    x, W, signs = synth.random_case(M, N, K, seed=99 + M)
    if fmt == "w8":
        y_ref, *_ = O.linear_w8(x, signs, O.prepare_w8(W, signs))
    else:
        y_ref, *_ = O.linear_w4(x, signs, O.prepare_w4(W, signs, group))
    w = C.gpu_prepare(W, signs, fmt, group)
    xq, xs = C.gpu_quant_acts(x, signs)
    y1, _ = C.gpu_linear(xq, xs, w, debug=True)
    y2, _ = C.gpu_linear(xq, xs, w, debug=False)
    check_y(C.host(y1), y_ref)
    assert np.array_equal(C.host(y1).view(np.uint32), C.host(y2).view(np.uint32))
    # guard bands
    import speculative_verify_gemm_amd as svg
    pad = 4096
    buf = torch.full((pad + M * N + pad,), 12345.0, dtype=torch.float32, device=C.DEV)
    yv = buf[pad:pad + M * N].view(M, N)
    if fmt == "w8":
        svg.w8a8_linear(xq, xs, w["wq"], w["ws"], N, yv)
    else:
        svg.w4a8_linear(xq, xs, w["wq"], w["ws"], w["wz"], fmt, group, N, yv)
    b = C.host(buf)
    assert np.all(b[:pad] == 12345.0) and np.all(b[pad + M * N:] == 12345.0)
    assert np.array_equal(b[pad:pad + M * N].view(np.uint32), C.host(y1).reshape(-1).view(np.uint32))


@pytest.mark.parametrize("src", ["single_1k", "decode_12k"])
def test_full_size_single_matrix(src):
    """The two single-matrix workloads at their full sizes, every output."""
    x, W, signs, spec = synth.single_inputs(src)
    fmt, g = spec["fmt"], spec["group"]
    C.say(f"full-size {src}: M={x.shape[0]} K={x.shape[1]} N={W.shape[0]} {fmt} g{g}")
    ow = O.prepare_w4(W, signs, g)
    y_ref, S_ref, qx, sx = O.linear_w4(x, signs, ow)
    w = C.gpu_prepare(W, signs, fmt, g)
    xq, xs = C.gpu_quant_acts(x, signs)
    y, dbg = C.gpu_linear(xq, xs, w)
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(w["wq"]), SL.pack_w4_codes(ow["q"]))
    assert np.array_equal(C.host(w["ws"]).view(np.uint16),
                          SL.tile_group_params(ow["s"], x.shape[1], g).view(np.uint16))
    assert np.array_equal(C.host(dbg).astype(np.int64), S_ref)
    check_y(C.host(y), y_ref)


# ------------------------------------------------------------ maximum sizes
def test_w8_partials_reach_the_int32_bound():
    """W8 at its largest K (131072) and M (32), on inputs with one non-zero
    value per 32-block (the first): the rotated block is that value times its
    sign in all 32 places (the first Hadamard column is all ones), so every
    activation and weight code is +-127 with the same sign on both sides and
    S = 127^2 * K = 2,114,060,288 in every output -- just under 2^31, which
    the int32 accumulation must reach without wrapping."""
    M, N, K = 32, 16, 131072
    _x, _W, signs = synth.random_case(1, 1, K, seed=131072)
    x = np.zeros((M, K), np.float32)
    x[:, ::32] = (1.0 + np.arange(M, dtype=np.float32) / 64.0)[:, None]
    W = np.zeros((N, K), np.float32)
    W[:, ::32] = (0.02 * (1.0 + np.arange(N, dtype=np.float32) / 8.0))[:, None]
    C.say(f"w8 int32 bound M={M} N={N} K={K}")
    ow = O.prepare_w8(W, signs)
    y_ref, S_ref, qx, sx = O.linear_w8(x, signs, ow)
    assert (np.abs(qx) == 127).all() and (np.abs(ow["q"]) == 127).all()
    assert (S_ref == 127 * 127 * K).all()
    w = C.gpu_prepare(W, signs, "w8", 0)
    xq, xs, y, dbg = C.gpu_fused(x, signs, w)
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert (C.host(dbg).astype(np.int64) == 127 * 127 * K).all()
    check_y(C.host(y), y_ref)


@pytest.mark.parametrize("M", [1, 16])
def test_w4_long_k(M):
    """K = 2^20: the linear's plain loop (no resident launch shape holds that
    many chunks per wave) and the stand-alone activation kernel reading each
    row twice, at a length far beyond the workloads'."""
    N, K, g = 16, 1 << 20, 64
    x, W, signs = synth.random_case(M, N, K, seed=M + 20)
    C.say(f"w4 long K M={M} N={N} K={K}")
    ow = O.prepare_w4(W, signs, g)
    y_ref, S_ref, qx, sx = O.linear_w4(x, signs, ow)
    w = C.gpu_prepare(W, signs, "w4_z16", g)
    xq, xs, y, dbg = C.gpu_fused(x, signs, w)
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32))
    assert np.array_equal(C.host(dbg).astype(np.int64), S_ref)
    check_y(C.host(y), y_ref)


# ------------------------------------------------------- extreme magnitudes
def _scaled_rows(a, scales):
    """Rows of `a` rescaled to the given maximum magnitudes (0 gives zeros)."""
    peak = np.abs(a).max(axis=1, keepdims=True)
    return (a / peak * np.asarray(scales, np.float32)[:, None]).astype(np.float32)


def test_act_codes_extreme_rows():
    """Rows whose maxima span fp32: a denormal row (its scale sigma * 2^-5
    underflows to 0 and 1 / sigma overflows, so every code takes the exact
    division), the edge of the normal range, and rows up to 1e36 (the
    transform's sums of 32 stay finite).  Codes and scales bit-exact."""
    M, K = 6, 1024
    x, _W, signs = synth.random_case(M, 1, K, seed=77, x_kind="student_t3")
    x = _scaled_rows(x, [1e-42, 1e-39, 1e-30, 1.0, 1e30, 1e36])
    qx, sx = O.quant_acts(x, signs)
    xq, xs = C.gpu_quant_acts(x, signs)
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32))


@pytest.mark.parametrize("fmt,group", [("w4_z4", 32), ("w4_z16", 64), ("w4_z16", 128), ("w8", 0)])
def test_weight_codes_extreme_rows(fmt, group):
    """Weight rows from zero through scales below fp16's range (the scale
    falls back to 1.0) and in its subnormal range, up to 1e3.  Codes,
    scales and zeros bit-exact."""
    N, K = 21, 384
    _x, W, signs = synth.random_case(1, N, K, seed=78)
    W = np.nan_to_num(_scaled_rows(W, np.repeat([0.0, 1e-30, 1e-7, 3e-5, 1e-3, 1.0, 1e3], 3)))
    w = C.gpu_prepare(W, signs, fmt, group)
    u = O.rht(W, signs)
    if fmt == "w8":
        q, s = O.quant_w8(u)
        ow = dict(q=q, s=s)
    else:
        q, s, z = O.quant_w4(u, group)
        ow = dict(q=q, s=s, z=z, group=group)
    wq, ws, wz = C.oracle_storage(ow, fmt, K)
    assert np.array_equal(C.host(w["wq"]).view(np.uint8), wq.view(np.uint8).reshape(-1))
    assert np.array_equal(C.host(w["ws"]).view(np.uint16), ws.view(np.uint16).reshape(-1))
    if wz is not None:
        assert np.array_equal(C.host(w["wz"]).view(np.uint8), wz.view(np.uint8).reshape(-1))


@pytest.mark.parametrize("fmt,group,M", [("w4_z16", 64, 1), ("w4_z16", 64, 16), ("w8", 0, 32),
                                         ("w4_z4", 32, 3), ("w4_z4", 64, 16)])
def test_linear_extreme_rows(fmt, group, M):
    """The whole call on rows of very different magnitudes (activations from
    1e-20 to 1e20, weights from fp16-subnormal scales to 1e3), with every
    output inside fp32's normal range: partial sums bit-exact, y within
    tolerance row by row."""
    N, K = 35, 512
    x, W, signs = synth.random_case(M, N, K, seed=79 + M)
    x = _scaled_rows(x, np.resize([1e-20, 1e-5, 1.0, 1e10, 1e20], M))
    W = _scaled_rows(W, np.resize([3e-5, 1e-3, 1.0, 1e3, 0.02], N))
    if fmt == "w8":
        y_ref, S_ref, qx, sx = O.linear_w8(x, signs, O.prepare_w8(W, signs))
    else:
        y_ref, S_ref, qx, sx = O.linear_w4(x, signs, O.prepare_w4(W, signs, group))
    w = C.gpu_prepare(W, signs, fmt, group)
    xq, xs, y, dbg = C.gpu_fused(x, signs, w)
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(dbg).astype(np.int64), S_ref)
    check_y(C.host(y), y_ref)


@pytest.mark.parametrize("fmt,group,M", [("w4_z4", 32, 1), ("w4_z4", 64, 16), ("w4_z16", 128, 2),
                                         ("w4_z16", 64, 16)])
def test_zero_point_clamp(fmt, group, M):
    """One-sided weight groups (every value <= 0) of ranges 1e-7 .. 1e-5,
    where the fp16 scale is subnormal and -lo / s passes 15: the 4-bit zero
    point is clamped to 15 (no carry into the neighbouring group's nibble in
    the 4-bit zero format).  Codes, scales and zeros bit-exact; partial sums
    bit-exact; y within tolerance."""
    N, K = 48, 512
    C.say(f"zero-point clamp fmt={fmt} g={group} M={M}")
    x, W, signs = synth.random_case(M, N, K, seed=90 + M + group)
    ranges = np.resize([1e-7, 3e-7, 1e-6, 3e-6, 1e-5, 1.0], N).astype(np.float32)
    W = -np.abs(_scaled_rows(W, ranges))
    u = O.rht(W, signs)
    # fold the signs back so the rotated rows themselves are one-sided: W = D H^T u / 32
    target = -np.abs(u)
    W = (O.fwht32(target.astype(np.float64)) * signs.astype(np.float64) / 32.0).astype(np.float32)
    ow = O.prepare_w4(W, signs, group)
    assert ow["z"].max() == 15
    y_ref, S_ref, qx, sx = O.linear_w4(x, signs, ow)
    w = C.gpu_prepare(W, signs, fmt, group)
    wq, ws, wz = C.oracle_storage(ow, fmt, K)
    assert np.array_equal(C.host(w["wq"]).view(np.uint8), wq.view(np.uint8).reshape(-1))
    assert np.array_equal(C.host(w["ws"]).view(np.uint16), ws.view(np.uint16).reshape(-1))
    assert np.array_equal(C.host(w["wz"]).view(np.uint8), wz.view(np.uint8).reshape(-1))
    xq, xs, y, dbg = C.gpu_fused(x, signs, w)
    assert np.array_equal(C.host(dbg).astype(np.int64), S_ref)
    check_y(C.host(y), y_ref)


def _banded(shape, dtype, fill, pad=4096):
    """A device buffer with `pad` elements of `fill` on both sides of a view
    of `shape` (the pad keeps 16-byte alignment for every dtype used)."""
    n = int(np.prod(shape))
    buf = torch.full((pad + n + pad,), fill, dtype=dtype, device=C.DEV)
    return buf, buf[pad:pad + n].view(*shape), pad


def _bands_intact(buf, pad, n, fill):
    b = C.host(buf)
    return bool(np.all(b[:pad] == fill) and np.all(b[pad + n:] == fill))


@pytest.mark.parametrize("fmt,group,M,N,K", [("w4_z16", 64, 1, 100, 4096), ("w4_z16", 64, 16, 100, 4096),
                                             ("w8", 0, 32, 70, 1024), ("w4_z4", 32, 3, 50, 96),
                                             ("w4_z16", 128, 1, 33, 12288)])
def test_guard_bands_of_the_fused_call(fmt, group, M, N, K):
    """Canary bytes around xq, x_scale and y stay untouched by the fused call
    (one launch at M = 1, where workgroup 0 writes xq and x_scale; two
    otherwise), and the outputs between them equal a plain call's."""
    import speculative_verify_gemm_amd as svg
    x, W, signs = synth.random_case(M, N, K, seed=600 + M + N)
    w = C.gpu_prepare(W, signs, fmt, group)
    ref = [C.host(t).copy() for t in C.gpu_fused(x, signs, w, debug=False)[:3]]
    bq, xq, pq = _banded((M, K), torch.int8, 77)
    bs, xs, ps = _banded((M,), torch.float32, 12345.0)
    by, y, py = _banded((M, N), torch.float32, 12345.0)
    xd, sd = C.to_dev(x), C.to_dev(signs)
    if fmt == "w8":
        svg.act_quant_w8a8_linear(xd, sd, xq, xs, w["wq"], w["ws"], N, y)
    else:
        svg.act_quant_w4a8_linear(xd, sd, xq, xs, w["wq"], w["ws"], w["wz"], fmt, group, N, y)
    assert _bands_intact(bq, pq, M * K, 77)
    assert _bands_intact(bs, ps, M, 12345.0)
    assert _bands_intact(by, py, M * N, 12345.0)
    for got, r in zip((xq, xs, y), ref):
        assert np.array_equal(C.host(got).view(np.uint8), r.view(np.uint8))


def test_guard_bands_of_the_tree_calls():
    """Canary words around the outputs of tree_accept_greedy (target, path,
    emit, n_emit) and tree_deltanet_verify (out), and around the state that
    tree_deltanet_commit rewrites in place."""
    import speculative_verify_gemm_amd as svg
    from oracle import deltanet_oracle as DN
    T, V = 12, 5000
    logits, parent, draft = synth.draft_tree(T, V, seed=61, accept=5, ties=True)
    outs = [_banded((T,), torch.int32, -12345) for _ in range(3)] + [_banded((1,), torch.int32, -12345)]
    svg.tree_accept_greedy(C.to_dev(logits), C.to_dev(parent.astype(np.int32)), C.to_dev(draft.astype(np.int32)),
                           outs[0][1], outs[1][1], outs[2][1], outs[3][1], svg.tree_workspace())
    for (buf, _v, pad), n in zip(outs, (T, T, T, 1)):
        assert _bands_intact(buf, pad, n, -12345)
    H, dk, dv = 3, 64, 128
    S0, q, k, v, a, b, par = synth.deltanet_case(T, H, dk, dv, seed=62)
    ob, out, po = _banded((T, H, dv), torch.float32, 12345.0)
    sb, state, ps = _banded((H, dv, dk), torch.float32, 12345.0)
    state.copy_(C.to_dev(S0))
    devs = [C.to_dev(t) for t in (q, k, v, a, b)]
    svg.tree_deltanet_verify(state, *devs, C.to_dev(par.astype(np.int32)), out)
    assert _bands_intact(ob, po, T * H * dv, 12345.0)
    path = [int(n) for n in TO.root_path(par, T - 1)[1:]]
    pd = torch.full((T,), -1, dtype=torch.int32, device=C.DEV)
    if path:
        pd[:len(path)] = C.to_dev(np.array(path, np.int32))
    svg.tree_deltanet_commit(state, devs[1], devs[2], devs[3], devs[4], pd,
                             torch.tensor([len(path) + 1], dtype=torch.int32, device=C.DEV))
    assert _bands_intact(sb, ps, H * dv * dk, 12345.0)
    ref = DN.tree_commit(S0, q, k, v, a, b, par, path)
    got = C.host(state)
    assert np.max(np.abs(got - ref)) <= 1e-4 * (np.max(np.abs(ref)) + 1.0)


def test_calls_on_two_streams_at_once():
    """The library keeps no device state between calls: two sequences of
    fused calls (different formats, M and shapes, each call with its own
    buffers), enqueued alternately on two streams of default priority, give
    bit for bit what the same calls give one after the other."""
    cases = [("w4_z16", 64, 16, 4096, 4096), ("w8", 0, 32, 1024, 4096), ("w4_z4", 32, 1, 2048, 1024),
             ("w4_z16", 128, 1, 4096, 4096)]
    prepared = []
    for i, (fmt, g, M, N, K) in enumerate(cases):
        x, W, signs = synth.random_case(M, N, K, seed=500 + i)
        prepared.append((C.to_dev(x), C.to_dev(signs), C.gpu_prepare(W, signs, fmt, g)))

    def call(i):
        xd, sd, w = prepared[i]
        return C.gpu_fused(xd, sd, w, debug=False)[:3]

    serial = [[C.host(t).copy() for t in call(i)] for i in range(len(cases))]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        torch.cuda.synchronize()
        for st in streams:
            st.wait_stream(torch.cuda.current_stream())
        outs = []
        for k in range(4):  # A: cases 0, 2, 0, 2; B: cases 1, 3, 1, 3 -- enqueued in turn
            for j, st in enumerate(streams):
                i = 2 * (k % 2) + j
                with torch.cuda.stream(st):
                    outs.append((i, call(i)))
        torch.cuda.synchronize()
        for i, out in outs:
            for got, ref in zip(out, serial[i]):
                assert np.array_equal(C.host(got).view(np.uint8), ref.view(np.uint8)), (rep, i)


def test_rejects_bad_arguments_without_writing():
    import speculative_verify_gemm_amd as svg
    xq = torch.zeros((2, 64), dtype=torch.int8, device=C.DEV)
    xs = torch.ones(2, dtype=torch.float32, device=C.DEV)
    wq = torch.zeros((16 * 64,), dtype=torch.uint8, device=C.DEV)
    ws = torch.ones((32,), dtype=torch.float16, device=C.DEV)
    wz = torch.zeros((32,), dtype=torch.float16, device=C.DEV)
    y = torch.full((2, 8), 7.0, device=C.DEV)
    with pytest.raises(svg.SvgError) as ei:
        svg.w4a8_linear(xq, xs, wq, ws, wz, "w4_z16", 48, 8, y)
    assert ei.value.status == svg.SVG_EUNSUPPORTED
    assert torch.all(y == 7.0)


# ------------------------------------------------------------- rounding ties
@pytest.mark.parametrize("nudge", [False, True])
def test_act_codes_at_rounding_ties(nudge):
    """Rotated values exactly on (or one ulp off) half-integer multiples of the
    row scale: the int8 rounding must follow the IEEE quotient and
    round-half-to-even bit for bit, in the stand-alone and the fused kernels."""
    M, K, N = 4, 2048, 48
    C.say(f"act codes at ties nudge={nudge}")
    x, signs = C.tie_rows(M, K, seed=5 + int(nudge), nudge=nudge)
    qx, sx = O.quant_acts(x, signs)
    xq, xs = C.gpu_quant_acts(x, signs)
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32))
    _x, W, _s = synth.random_case(1, N, K, seed=77)
    w = C.oracle_weights_to_dev(O.prepare_w4(W, signs, 64), "w4_z16")
    fq, fs, _y, _d = C.gpu_fused(x, signs, w)
    assert np.array_equal(C.host(fq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(fs).view(np.uint32), sx.view(np.uint32))


# ------------------------------------------------------------- fused calls
FUSED_CASES = [("w4_z16", 64, M, 37, 384) for M in (1, 2, 3, 16, 17, 32)]
FUSED_CASES += [("w4_z4", 32, 1, 50, 96), ("w4_z4", 32, 5, 50, 96), ("w4_z16", 128, 32, 130, 12288),
                ("w4_z16", 64, 16, 300, 4096), ("w4_z16", 64, 1, 64, 12288), ("w4_z16", 64, 32, 40, 320),
                ("w4_z4", 128, 2, 20, 384)]
FUSED_CASES += [("w8", 0, M, 37, 384) for M in (1, 2, 16, 32)]
FUSED_CASES += [("w8", 0, 32, 70, 12288), ("w8", 0, 1, 33, 12288), ("w8", 0, 3, 24, 12288), ("w8", 0, 4, 50, 4096)]
FUSED_CASES += [("w4_z16", 128, 4, 40, 12288), ("w4_z16", 64, 2, 300, 4096), ("w4_z4", 64, 4, 20, 1024),
                ("w4_z16", 64, 5, 33, 512)]


@pytest.mark.parametrize("fmt,group,M,N,K", FUSED_CASES)
def test_fused_matches_oracle(fmt, group, M, N, K):
    """act_quant_w4a8_linear / act_quant_w8a8_linear (one launch for M <= 2,
    two otherwise): activation codes and scales bit-exact, partial sums
    bit-exact, y within tolerance."""
    C.say(f"fused fmt={fmt} g={group} M={M} N={N} K={K}")
    x, W, signs = synth.random_case(M, N, K, seed=11 * M + N + K + group, x_kind="student_t3")
    if fmt == "w8":
        ow = O.prepare_w8(W, signs)
        y_ref, S_ref, qx, sx = O.linear_w8(x, signs, ow)
    else:
        ow = O.prepare_w4(W, signs, group)
        y_ref, S_ref, qx, sx = O.linear_w4(x, signs, ow)
    w = C.oracle_weights_to_dev(ow, fmt)
    xq, xs, y, dbg = C.gpu_fused(x, signs, w)
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32))
    assert np.array_equal(C.host(dbg).astype(np.int64), S_ref)
    check_y(C.host(y), y_ref)


@pytest.mark.parametrize("M", [1, 2, 16])
def test_fused_repeats_on_new_inputs(M):
    """Consecutive fused calls, each on new activations written to the same xq
    buffer: every call matches the two-launch path bit for bit."""
    C.say(f"fused repeats M={M}")
    N, K = 96, 1024
    _x, W, signs = synth.random_case(M, N, K, seed=123)
    xs_in = [synth.random_case(M, N, K, seed=500 + i, x_kind="student_t3")[0] for i in range(4)]
    w4 = C.gpu_prepare(W, signs, "w4_z16", 64)
    w8 = C.gpu_prepare(W, signs, "w8", 0)
    sd = C.to_dev(signs)
    xq = torch.empty((M, K), dtype=torch.int8, device=C.DEV)
    xsc = torch.empty((M,), dtype=torch.float32, device=C.DEV)
    ys = []
    for i, x in enumerate(xs_in):
        y = torch.empty((M, N), dtype=torch.float32, device=C.DEV)
        if i % 2 == 0:
            svg.act_quant_w4a8_linear(C.to_dev(x), sd, xq, xsc, w4["wq"], w4["ws"], w4["wz"], "w4_z16", 64, N, y)
        else:
            svg.act_quant_w8a8_linear(C.to_dev(x), sd, xq, xsc, w8["wq"], w8["ws"], N, y)
        ys.append(y)
    for i, x in enumerate(xs_in):
        q, sc = C.gpu_quant_acts(x, signs)
        ref, _ = C.gpu_linear(q, sc, w4 if i % 2 == 0 else w8, debug=False)
        assert np.array_equal(C.host(ys[i]).view(np.uint32), C.host(ref).view(np.uint32)), i


def test_fused_in_captured_graph():
    """Two fused calls (M = 16: two launches; M = 1: one) captured in a HIP
    graph and replayed several times, with eager fused calls in between:
    every replay matches the eager results bit for bit."""
    C.say("fused calls in a captured graph")
    M, K = 16, 1024
    x1, W1, s1 = synth.random_case(M, 80, K, seed=301)
    x2, W2, s2 = synth.random_case(1, 48, K, seed=302)
    wa = C.gpu_prepare(W1, s1, "w4_z16", 64)
    wb = C.gpu_prepare(W2, s2, "w8", 0)
    X1, S1, X2, S2 = C.to_dev(x1), C.to_dev(s1), C.to_dev(x2), C.to_dev(s2)
    ref1 = C.host(C.gpu_fused(X1, S1, wa, debug=False)[2])
    ref2 = C.host(C.gpu_fused(X2, S2, wb, debug=False)[2])
    xq1 = torch.empty((M, K), dtype=torch.int8, device=C.DEV)
    xs1 = torch.empty((M,), dtype=torch.float32, device=C.DEV)
    y1 = torch.empty((M, 80), dtype=torch.float32, device=C.DEV)
    xq2 = torch.empty((1, K), dtype=torch.int8, device=C.DEV)
    xs2 = torch.empty((1,), dtype=torch.float32, device=C.DEV)
    y2 = torch.empty((1, 48), dtype=torch.float32, device=C.DEV)

    def run():
        svg.act_quant_w4a8_linear(X1, S1, xq1, xs1, wa["wq"], wa["ws"], wa["wz"], "w4_z16", 64, 80, y1)
        svg.act_quant_w8a8_linear(X2, S2, xq2, xs2, wb["wq"], wb["ws"], 48, y2)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        y1.fill_(-1.0)
        y2.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(C.host(y1).view(np.uint32), ref1.view(np.uint32)), rep
        assert np.array_equal(C.host(y2).view(np.uint32), ref2.view(np.uint32)), rep
        C.gpu_fused(X1, S1, wa, debug=False)  # eager work in between


# ------------------------------------------------- full-size stack launches
# every launch kind of the timed passes (W4 g64 at M = 16 and 1, W8 at M = 32),
# the g128 sweep's M values, and more two-row launches
STACK_CASES = [("stack_w4g64", 16, "qkv"), ("stack_w4g64", 16, "o"), ("stack_w4g64", 16, "gateup"),
               ("stack_w4g64", 16, "down"), ("stack_w4g64", 1, "qkv"), ("stack_w4g64", 1, "o"),
               ("stack_w4g64", 1, "gateup"), ("stack_w4g64", 1, "down"), ("stack_w8", 32, "qkv"),
               ("stack_w8", 32, "o"), ("stack_w8", 32, "gateup"), ("stack_w8", 32, "down"),
               ("stack_w8", 1, "o"), ("stack_w4g128", 32, "down"), ("stack_w4g128", 32, "gateup"),
               ("stack_w4g128", 1, "qkv"), ("stack_w4g128", 2, "gateup"), ("stack_w4g128", 4, "down"),
               ("stack_w4g128", 8, "o"), ("stack_w4g128", 16, "qkv"), ("stack_w4g128", 2, "down"),
               ("stack_w4g64", 2, "qkv")]


@pytest.mark.parametrize("workload,M,launch", STACK_CASES)
def test_stack_launch_sampled_rows(workload, M, launch):
    """One launch of the benchmark's stack at full size, issued as bench.py
    issues it (stacked members, the fused call), checked on sampled output
    rows: activation codes and scales bit-exact over the whole row, per-group
    partial sums bit-exact and y within tolerance for 48 random rows plus the
    first and last row of every member, against the oracle encoding those
    rows itself.  A second call without the debug output (the timed kernel
    instance) gives the same y bit for bit."""
    spec = synth.WORKLOADS[workload]
    fmt, group = spec["fmt"], spec["group"]
    w, Ws, signs, space = C.stack_launch(0, launch, fmt, group)
    N, K = w["N"], w["K"]
    C.say(f"stack launch {workload} {launch} M={M} N={N} K={K}")
    x = synth.stack_acts(workload, 0, space, M)
    xq, xs, y, dbg = C.gpu_fused(x, signs, w)
    y2 = C.gpu_fused(x, signs, w, debug=False)[2]
    rng = np.random.default_rng(N + K + M)
    edges, r0 = [], 0
    for W in Ws:
        edges += [r0, r0 + W.shape[0] - 1]
        r0 += W.shape[0]
    rows = sorted(set(rng.choice(N, 48, replace=False).tolist()) | set(edges))
    Wr = C.stacked_rows(Ws, rows)
    if fmt == "w8":
        y_ref, S_ref, qx, sx = O.linear_w8(x, signs, O.prepare_w8(Wr, signs))
    else:
        y_ref, S_ref, qx, sx = O.linear_w4(x, signs, O.prepare_w4(Wr, signs, group))
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32))
    assert np.array_equal(C.host(dbg)[:, rows].astype(np.int64), S_ref)
    yh = C.host(y)
    check_y(yh[:, rows], y_ref)
    assert np.array_equal(C.host(y2).view(np.uint32), yh.view(np.uint32))


@pytest.mark.parametrize("workload,M,launch", [("stack_w4g64", 16, "o"), ("stack_w8", 32, "o"),
                                               ("stack_w4g128", 2, "o"), ("stack_w4g64", 16, "down"),
                                               ("stack_w4g64", 1, "down")])
def test_stack_launch_every_output(workload, M, launch):
    """A projection of the stack -- o (4096 x 4096) at the verify batch of
    each format, down (4096 x 12288, the 16-wave x 6-chunk shape) at 16 rows
    and at one row (quantized inside the launch) -- issued as bench.py issues
    it, against the oracle on EVERY output: the per-group partial sums of all
    M x 4096 outputs bit-exact and all of y within tolerance (one full-size
    launch of each matrix-core policy; the two-row launch pads a 16-row MFMA
    tile)."""
    spec = synth.WORKLOADS[workload]
    fmt, group = spec["fmt"], spec["group"]
    w, Ws, signs, space = C.stack_launch(0, launch, fmt, group)
    N, K = w["N"], w["K"]
    C.say(f"stack {launch} launch, every output: {workload} M={M} N={N} K={K}")
    x = synth.stack_acts(workload, 0, space, M)
    xq, xs, y, dbg = C.gpu_fused(x, signs, w)
    W = C.stacked_rows(Ws, list(range(N)))
    if fmt == "w8":
        y_ref, S_ref, qx, sx = O.linear_w8(x, signs, O.prepare_w8(W, signs))
    else:
        y_ref, S_ref, qx, sx = O.linear_w4(x, signs, O.prepare_w4(W, signs, group))
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32))
    assert np.array_equal(C.host(dbg).astype(np.int64), S_ref)
    check_y(C.host(y), y_ref)


# ------------------------------------------- the wave-wide transform block
# Block 64 (a variant sized to the 64-lane wave): the same checks as for the
# pages' 32, against the oracle run with block 64.
ACT64_CASES = [(1, 64), (3, 192), (16, 4096), (5, 12288), (2, 40960)]


@pytest.mark.parametrize("M,K", ACT64_CASES)
def test_act_codes_block64(M, K):
    C.say(f"act_rht_quant_i8 block=64 M={M} K={K}")
    x, _W, signs = synth.random_case(M, 1, K, seed=M * 31 + K, x_kind="student_t3")
    qx, sx = O.quant_acts(x, signs, 64)
    xq, xs = C.gpu_quant_acts(x, signs, block=64)
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32))


W64_CASES = [("w4_z4", 32, 64, 1024), ("w4_z16", 64, 48, 4096), ("w4_z16", 128, 37, 384),
             ("w4_z4", 64, 33, 192), ("w8", 0, 45, 1152), ("w8", 0, 16, 64)]


@pytest.mark.parametrize("fmt,group,N,K", W64_CASES)
def test_weight_codes_block64(fmt, group, N, K):
    C.say(f"rht_rotate_weights block=64 fmt={fmt} g={group} N={N} K={K}")
    _x, W, signs = synth.random_case(1, N, K, seed=N + K + group + 64)
    w = C.gpu_prepare(W, signs, fmt, group, debug=True, block=64)
    u = O.rht(W, signs, np.float32, 64)
    assert np.array_equal(C.host(w["rot"]).view(np.uint32), u.view(np.uint32))
    if fmt == "w8":
        q, s = O.quant_w8(u)
        ow = dict(q=q, s=s)
    else:
        q, s, z = O.quant_w4(u, group)
        ow = dict(q=q, s=s, z=z, group=group)
    wq, ws, wz = C.oracle_storage(ow, fmt, K)
    assert np.array_equal(C.host(w["wq"]).view(np.uint8), wq.view(np.uint8).reshape(-1))
    assert np.array_equal(C.host(w["ws"]).view(np.uint16), ws.view(np.uint16).reshape(-1))
    if wz is not None:
        assert np.array_equal(C.host(w["wz"]).view(np.uint8), wz.view(np.uint8).reshape(-1))


@pytest.mark.parametrize("fmt,group,M,N,K", [("w4_z16", 64, 1, 300, 4096), ("w4_z4", 32, 2, 64, 1024),
                                             ("w4_z16", 128, 16, 130, 12288), ("w8", 0, 1, 70, 4096),
                                             ("w8", 0, 32, 40, 12288)])
def test_linear_block64_end_to_end(fmt, group, M, N, K):
    """Weights and activations both rotated with 64-blocks, through the
    fp32-input entry points (one launch at M = 1, two above): codes, partial
    sums and outputs against the oracle."""
    C.say(f"block=64 linear fmt={fmt} g={group} M={M} N={N} K={K}")
    x, W, signs = synth.random_case(M, N, K, seed=3 * M + N + K)
    w = C.gpu_prepare(W, signs, fmt, group, block=64)
    ow = O.prepare_w8(W, signs, 64) if fmt == "w8" else O.prepare_w4(W, signs, group, 64)
    y_ref, S, qx, sx = (O.linear_w8 if fmt == "w8" else O.linear_w4)(x, signs, ow)
    xq, xs, y, dbg = C.gpu_fused(x, signs, w)
    assert np.array_equal(C.host(xq).reshape(-1), SL.pack_act_codes(qx))
    assert np.array_equal(C.host(xs).view(np.uint32), sx.view(np.uint32))
    assert np.array_equal(C.host(dbg).astype(np.int64), S)
    check_y(C.host(y), y_ref)
