"""GPU tests of the layout conversions (svg_import_weights / svg_export_weights,
svg_import_act_codes / svg_export_act_codes) through the C ABI: the oracle's
canonical row-major arrays go straight in.

 * import of the oracle's canonical codes, scales and zeros gives, byte for
   byte, what rht_rotate_weights writes for the same matrix and what the
   host-side layout definition places (tests/storage_layout.py), padding
   included;
 * export gives back the canonical arrays bit for bit;
 * the linear run on imported weights and imported activation codes matches
   the oracle (partials bit-exact, y within 2e-3);
 * act_rht_quant_i8's codes exported to rows are the oracle's codes.

Shapes span several tiles and 512-k parameter blocks with ragged N, K not a
multiple of 128, odd group counts (4-bit zeros with a half-used last byte),
every format and group.

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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    global C, svg
    import svg_cases as C  # noqa: F401  (imports the binding, which loads libsvgemm)
    import speculative_verify_gemm_amd as svg


def _canonical(ow, fmt, K):
    """The oracle's encoding as canonical device arrays (codes, scale, zero)."""
    if fmt == "w8":
        return C.to_dev(ow["q"]), C.to_dev(ow["s"]), None
    zero = SL.canonical_z4(ow["z"]) if fmt == "w4_z4" else ow["z"].astype(np.float16)
    return C.to_dev(SL.canonical_w4_codes(ow["q"])), C.to_dev(ow["s"]), C.to_dev(zero)


def _empty_canonical(fmt, N, K, g):
    dev = C.DEV
    if fmt == "w8":
        return (torch.empty((N, K), dtype=torch.int8, device=dev), torch.empty((N,), dtype=torch.float16, device=dev),
                None)
    ng = K // g
    zero = (torch.empty((N, (ng + 1) // 2), dtype=torch.uint8, device=dev) if fmt == "w4_z4"
            else torch.empty((N, ng), dtype=torch.float16, device=dev))
    return (torch.empty((N, K // 2), dtype=torch.uint8, device=dev),
            torch.empty((N, ng), dtype=torch.float16, device=dev), zero)


def _bits(t):
    a = C.host(t)
    return a.view(np.uint16) if a.dtype == np.float16 else a


# (fmt, group, N, K): ragged N and K, several 128-k tiles and 512-k blocks,
# odd group counts
CASES = [("w4_z4", 32, 37, 384), ("w4_z4", 64, 300, 4096), ("w4_z4", 128, 16, 384), ("w4_z4", 128, 50, 1152),
         ("w4_z16", 32, 21, 1120), ("w4_z16", 64, 130, 2112), ("w4_z16", 128, 1, 640),
         ("w8", 0, 37, 320), ("w8", 0, 300, 4096), ("w8", 0, 16, 64)]


@pytest.mark.parametrize("fmt,group,N,K", CASES)
def test_import_export_weights(fmt, group, N, K):
    C.say(f"layout weights {fmt} g{group} N={N} K={K}")
    _x, W, signs = synth.random_case(1, N, K, seed=N * 7 + K + group)
    ow = O.prepare_w8(W, signs) if fmt == "w8" else O.prepare_w4(W, signs, group)
    codes, scale, zero = _canonical(ow, fmt, K)
    # import into storage pre-filled with a marker: every byte must be written
    wq, ws, wz = svg.empty_weights(N, K, fmt, group, device=C.DEV)
    for t in (wq, ws, wz):
        if t is not None:
            t.view(torch.uint8).fill_(0xA5)
    svg.import_weights(codes, scale, zero, fmt, group, K, wq, ws, wz)
    # what the library's own encoder writes for the same matrix
    rq, rs, rz = svg.empty_weights(N, K, fmt, group, device=C.DEV)
    svg.rht_rotate_weights(C.to_dev(W), C.to_dev(signs), fmt, group, rq, rs, rz)
    assert np.array_equal(_bits(wq), _bits(rq))
    assert np.array_equal(_bits(ws), _bits(rs))
    if wz is not None:
        assert np.array_equal(_bits(wz), _bits(rz))
    # and what the host-side layout definition places
    hq, hs, hz = C.oracle_storage(ow, fmt, K)
    assert np.array_equal(C.host(wq).view(np.uint8), np.asarray(hq).view(np.uint8))
    assert np.array_equal(_bits(ws), np.asarray(hs).view(np.uint16))
    if wz is not None:
        assert np.array_equal(C.host(wz).view(np.uint8), np.asarray(hz).view(np.uint8))
    # export gives the canonical arrays back
    ec, es, ez = _empty_canonical(fmt, N, K, group)
    svg.export_weights(wq, ws, wz, fmt, group, N, K, ec, es, ez)
    assert np.array_equal(_bits(ec), _bits(codes))
    assert np.array_equal(_bits(es), _bits(scale))
    if ez is not None:
        assert np.array_equal(_bits(ez), _bits(zero))


@pytest.mark.parametrize("fmt,group,M,N,K", [("w4_z4", 64, 16, 300, 4096), ("w4_z16", 128, 5, 130, 2048),
                                             ("w4_z16", 32, 1, 37, 384), ("w8", 0, 32, 300, 4096),
                                             ("w8", 0, 3, 37, 320)])
def test_linear_on_imported_canonical_arrays(fmt, group, M, N, K):
    """The oracle's canonical weight and activation arrays, imported, run
    through the unfused linear call: partials bit-exact, y within 2e-3."""
    C.say(f"layout linear {fmt} g{group} M={M} N={N} K={K}")
    x, W, signs = synth.random_case(M, N, K, seed=M * 31 + N + K, x_kind="student_t3")
    if fmt == "w8":
        ow = O.prepare_w8(W, signs)
        y_ref, S_ref, qx, sx = O.linear_w8(x, signs, ow)
    else:
        ow = O.prepare_w4(W, signs, group)
        y_ref, S_ref, qx, sx = O.linear_w4(x, signs, ow)
    codes, scale, zero = _canonical(ow, fmt, K)
    wq, ws, wz = svg.empty_weights(N, K, fmt, group, device=C.DEV)
    svg.import_weights(codes, scale, zero, fmt, group, K, wq, ws, wz)
    xq = torch.empty((M, K), dtype=torch.int8, device=C.DEV)
    svg.import_act_codes(C.to_dev(qx), xq)
    xs = C.to_dev(sx)
    y = torch.full((M, N), 12345.0, device=C.DEV)
    if fmt == "w8":
        dbg = torch.empty((M, N), dtype=torch.int32, device=C.DEV)
        svg.w8a8_linear(xq, xs, wq, ws, N, y, dbg)
    else:
        dbg = torch.empty((M, N, K // group), dtype=torch.int32, device=C.DEV)
        svg.w4a8_linear(xq, xs, wq, ws, wz, fmt, group, N, y, dbg)
    assert np.array_equal(C.host(dbg).astype(np.int64), S_ref)
    e, r, ex = O.output_error(C.host(y), y_ref)
    assert e <= TOL and r <= TOL, (e, r, ex)


@pytest.mark.parametrize("M,K", [(1, 32), (3, 384), (16, 4096), (32, 12288), (7, 1120)])
def test_act_codes_round_trip(M, K):
    """act_rht_quant_i8's slab codes exported to rows are the oracle's [M][K]
    codes; importing those rows gives the slab bytes back."""
    C.say(f"layout act codes M={M} K={K}")
    x, _W, signs = synth.random_case(M, 1, K, seed=M + K, x_kind="student_t3")
    qx, sx = O.quant_acts(x, signs)
    xq = torch.empty((M, K), dtype=torch.int8, device=C.DEV)
    xs = torch.empty((M,), dtype=torch.float32, device=C.DEV)
    svg.act_rht_quant_i8(C.to_dev(x), C.to_dev(signs), xq, xs)
    rows = torch.full((M, K), 99, dtype=torch.int8, device=C.DEV)
    svg.export_act_codes(xq, rows)
    assert np.array_equal(C.host(rows), qx)
    back = torch.full((M, K), 99, dtype=torch.int8, device=C.DEV)
    svg.import_act_codes(rows, back)
    assert np.array_equal(C.host(back), C.host(xq))
    assert np.array_equal(C.host(back).reshape(-1), SL.pack_act_codes(qx))
