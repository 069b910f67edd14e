"""The C ABI library loads, exports every entry point the header declares, and
rejects bad arguments on the host with the documented status codes.

No GPU: every call here fails validation (or is an empty call) before
anything could be enqueued, so no pointer passed is ever dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svgemm.h")


def _header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(\w+)\s*\(", text, flags=re.M))
                  - {"if", "defined"})


@pytest.fixture(scope="module")
def svg():
    import speculative_verify_gemm_amd as svg
    return svg


def test_header_declares_the_entry_points():
    assert _header_functions() == sorted(
        ["act_quant_w4a8_linear", "act_quant_w4a8_linear_ws", "act_quant_w8a8_linear", "act_quant_w8a8_linear_ws",
         "act_rht_quant_i8", "rht_rotate_weights",
         "svg_export_act_codes", "svg_export_weights", "svg_import_act_codes", "svg_import_weights",
         "svg_last_error", "svg_pass_plan", "svg_pass_run", "svg_weight_sizes", "tree_accept_greedy", "tree_accept_greedy_static",
         "tree_deltanet_commit",
         "tree_deltanet_verify", "w4a8_linear", "w8a8_linear"])


def test_library_exports_every_declared_symbol(svg):
    for name in _header_functions():
        assert hasattr(svg.lib, name), name
        assert ctypes.cast(getattr(svg.lib, name), ctypes.c_void_p).value


A = ctypes.c_void_p(0x10000)      # aligned, never dereferenced
MIS = ctypes.c_void_p(0x10001)    # misaligned
NULL = None


def _w4(svg, **kw):
    args = dict(xq=A, xs=A, M=1, K=128, wq=A, ws=A, wz=A, fmt=1, g=64, N=16, y=A, dbg=NULL)
    args.update(kw)
    return svg.lib.w4a8_linear(args["xq"], args["xs"], args["M"], args["K"], args["wq"], args["ws"],
                               args["wz"], args["fmt"], args["g"], args["N"], args["y"], args["dbg"],
                               NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(xq=NULL), 1), (dict(y=NULL), 1), (dict(wz=NULL), 1), (dict(M=-1), 1), (dict(K=0), 1),
    (dict(N=-3), 1),
    (dict(g=16), 2), (dict(g=96), 2), (dict(K=96, g=64), 2), (dict(K=48, g=32), 2),
    (dict(M=33), 2), (dict(fmt=2), 2), (dict(fmt=7), 2),
    (dict(xq=MIS), 3), (dict(wq=MIS), 3), (dict(y=MIS), 3), (dict(ws=MIS), 3),
])
def test_w4a8_validation(svg, kw, code):
    assert _w4(svg, **kw) == code
    assert svg.last_error().startswith("w4a8_linear:")


def test_transform_block_64_is_accepted_and_checked(svg):
    # block 64 (K a multiple of 64) passes validation: empty calls return OK
    assert svg.lib.act_rht_quant_i8(A, 0, 128, A, 64, A, A, NULL) == 0
    assert svg.lib.rht_rotate_weights(A, 0, 128, A, 64, 1, 32, A, A, A, NULL, NULL) == 0
    # K not a multiple of the block, and blocks other than 32 / 64
    assert svg.lib.act_rht_quant_i8(A, 1, 96, A, 64, A, A, NULL) == 2
    assert svg.lib.rht_rotate_weights(A, 4, 96, A, 64, 1, 32, A, A, A, NULL, NULL) == 2
    assert svg.lib.rht_rotate_weights(A, 4, 128, A, 128, 1, 32, A, A, A, NULL, NULL) == 2
    assert svg.lib.act_quant_w8a8_linear(A, 1, 96, A, 64, A, A, A, A, 16, A, NULL, NULL) == 2


def test_empty_calls_are_ok(svg):
    assert _w4(svg, M=0) == 0 and svg.last_error() == ""
    assert _w4(svg, N=0) == 0
    assert svg.lib.act_rht_quant_i8(A, 0, 64, A, 32, A, A, NULL) == 0
    assert svg.lib.rht_rotate_weights(A, 0, 64, A, 32, 1, 32, A, A, A, NULL, NULL) == 0
    assert svg.lib.w8a8_linear(A, A, 0, 64, A, A, 8, A, NULL, NULL) == 0


@pytest.mark.parametrize("args,code", [
    ((NULL, 1, 64, A, 32, A, A), 1), ((A, -1, 64, A, 32, A, A), 1), ((A, 1, 0, A, 32, A, A), 1),
    ((A, 1, 64, A, 16, A, A), 2), ((A, 1, 48, A, 32, A, A), 2), ((A, 33, 64, A, 32, A, A), 2),
    ((MIS, 1, 64, A, 32, A, A), 3), ((A, 1, 64, MIS, 32, A, A), 3), ((A, 1, 64, A, 32, MIS, A), 3),
])
def test_act_quant_validation(svg, args, code):
    assert svg.lib.act_rht_quant_i8(*args, NULL) == code
    assert svg.last_error().startswith("act_rht_quant_i8:")


@pytest.mark.parametrize("args,code", [
    ((NULL, 4, 64, A, 32, 1, 32, A, A, A, NULL), 1),
    ((A, 4, 64, A, 32, 0, 32, A, A, NULL, NULL), 1),     # W4 needs w_zero
    ((A, 4, 64, A, 32, 3, 32, A, A, A, NULL), 2),        # unknown fmt
    ((A, 4, 64, A, 16, 1, 32, A, A, A, NULL), 2),        # block not 32 or 64
    ((A, 4, 96, A, 32, 1, 64, A, A, A, NULL), 2),        # K % group
    ((A, 4, 64, A, 32, 1, 48, A, A, A, NULL), 2),        # group
    ((A, 4, 64, MIS, 32, 1, 32, A, A, A, NULL), 3),      # signs alignment
    ((A, 4, 64, A, 32, 2, 0, MIS, A, NULL, NULL), 3),    # wq alignment
])
def test_rotate_validation(svg, args, code):
    assert svg.lib.rht_rotate_weights(*args, NULL) == code


@pytest.mark.parametrize("args,code", [
    ((A, A, 1, 64, A, A, 8, NULL, NULL), 1),
    ((A, A, 1, 131104, A, A, 8, A, NULL), 2),
    ((A, A, 1, 48, A, A, 8, A, NULL), 2),
    ((A, A, 40, 64, A, A, 8, A, NULL), 2),
    ((A, A, 1, 64, MIS, A, 8, A, NULL), 3),
])
def test_w8a8_validation(svg, args, code):
    assert svg.lib.w8a8_linear(*args, NULL) == code


def _fused4(svg, **kw):
    args = dict(X=A, M=1, K=128, signs=A, block=32, xq=A, xs=A, wq=A, ws=A, wz=A, fmt=1, g=64, N=16, y=A,
                dbg=NULL)
    args.update(kw)
    return svg.lib.act_quant_w4a8_linear(args["X"], args["M"], args["K"], args["signs"], args["block"],
                                         args["xq"], args["xs"], args["wq"], args["ws"], args["wz"],
                                         args["fmt"], args["g"], args["N"], args["y"], args["dbg"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(X=NULL), 1), (dict(signs=NULL), 1), (dict(xq=NULL), 1), (dict(wz=NULL), 1),
    (dict(block=16), 2), (dict(block=64, K=96), 2), (dict(M=33), 2), (dict(g=96), 2), (dict(fmt=2), 2),
    (dict(X=MIS), 3), (dict(xq=MIS), 3), (dict(signs=MIS), 3), (dict(wq=MIS), 3),
])
def test_fused_w4_validation(svg, kw, code):
    assert _fused4(svg, **kw) == code
    assert svg.last_error().startswith("act_quant_w4a8_linear:")


@pytest.mark.parametrize("args,code", [
    ((NULL, 1, 64, A, 32, A, A, A, A, 8, A, NULL), 1),         # X
    ((A, 1, 64, A, 16, A, A, A, A, 8, A, NULL), 2),            # block
    ((A, 1, 131104, A, 32, A, A, A, A, 8, A, NULL), 2),        # K too large for int32 sums
    ((A, 1, 64, MIS, 32, A, A, A, A, 8, A, NULL), 3),          # signs alignment
])
def test_fused_w8_validation(svg, args, code):
    assert svg.lib.act_quant_w8a8_linear(*args, NULL) == code
    assert svg.last_error().startswith("act_quant_w8a8_linear:")


def test_fused_empty_calls_are_ok(svg):
    assert _fused4(svg, M=0) == 0 and svg.last_error() == ""
    assert svg.lib.act_quant_w8a8_linear(A, 0, 64, A, 32, A, A, A, A, 8, A, NULL, NULL) == 0


def test_weight_sizes_match_the_oracle_layout(svg):
    import numpy as np
    import storage_layout as SL
    for N, K, fmt, g in [(37, 384, "w4_z4", 32), (12288, 4096, "w4_z16", 64), (20, 384, "w4_z16", 128), (20, 320, "w4_z16", 64),
                         (5, 96, "w4_z4", 32), (45, 1120, "w8", 0), (16, 64, "w8", 0)]:
        wb, sb, zb = svg.weight_sizes(N, K, fmt, g)
        if fmt == "w8":
            assert wb == SL.pack_w8_codes(np.zeros((N, K), np.int8)).nbytes and sb == 2 * N and zb == 0
        else:
            q = np.zeros((N, K), np.uint8)
            z = np.zeros((N, K // g), np.uint8)
            assert wb == SL.pack_w4_codes(q).nbytes
            assert sb == SL.tile_group_params(z.astype(np.float16), K, g).nbytes
            zref = SL.pack_z4(z, K, g) if fmt == "w4_z4" else SL.zeros_as_f16(z, K, g)
            assert zb == zref.nbytes
    with pytest.raises(svg.SvgError):
        svg.weight_sizes(16, 48, "w4_z16", 64)


def test_binding_has_no_cpu_path(svg):
    import torch
    x = torch.zeros((1, 64), dtype=torch.float32)
    with pytest.raises(ValueError):
        svg.act_rht_quant_i8(x, torch.ones(64, dtype=torch.int8), torch.zeros((1, 64), dtype=torch.int8),
                             torch.zeros(1))


def _tree(svg, **kw):
    args = dict(logits=A, T=4, V=100, parent=A, draft=A, target=A, path=A, emit=A, n=A, ws=A)
    args.update(kw)
    return svg.lib.tree_accept_greedy(args["logits"], args["T"], args["V"], args["parent"], args["draft"],
                                      args["target"], args["path"], args["emit"], args["n"], args["ws"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(logits=NULL), 1), (dict(parent=NULL), 1), (dict(draft=NULL), 1), (dict(target=NULL), 1),
    (dict(path=NULL), 1), (dict(emit=NULL), 1), (dict(n=NULL), 1), (dict(ws=NULL), 1),
    (dict(T=0), 1), (dict(V=0), 1), (dict(T=-2), 1),
    (dict(T=33), 2),
    (dict(logits=MIS), 3), (dict(ws=ctypes.c_void_p(0x10004)), 3), (dict(parent=MIS), 3),
    (dict(draft=MIS), 3), (dict(target=MIS), 3), (dict(path=MIS), 3), (dict(emit=MIS), 3), (dict(n=MIS), 3),
])
def test_tree_accept_validation(svg, kw, code):
    assert _tree(svg, **kw) == code
    assert svg.last_error().startswith("tree_accept_greedy:")


@pytest.mark.parametrize("kw,code", [
    (dict(logits=NULL), 1), (dict(parent=NULL), 1), (dict(n=NULL), 1), (dict(T=0), 1), (dict(V=0), 1),
    (dict(T=33), 2), (dict(V=(1 << 30) + 1), 2),
    (dict(logits=MIS), 3), (dict(emit=MIS), 3),
])
def test_tree_accept_static_validation(svg, kw, code):
    # checked on the host before the library's workspace is looked up
    args = dict(logits=A, T=4, V=100, parent=A, draft=A, target=A, path=A, emit=A, n=A)
    args.update(kw)
    assert svg.lib.tree_accept_greedy_static(args["logits"], args["T"], args["V"], args["parent"], args["draft"],
                                             args["target"], args["path"], args["emit"], args["n"], NULL) == code
    assert svg.last_error().startswith("tree_accept_greedy_static:")


def _gdn_verify(svg, **kw):
    a = dict(state=A, q=A, k=A, v=A, alpha=A, beta=A, parent=A, T=4, H=2, dk=128, dv=128, out=A)
    a.update(kw)
    return svg.lib.tree_deltanet_verify(a["state"], a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["parent"],
                                        a["T"], a["H"], a["dk"], a["dv"], a["out"], NULL)


def _gdn_commit(svg, **kw):
    a = dict(state=A, k=A, v=A, alpha=A, beta=A, path=A, n=A, T=4, H=2, dk=128, dv=128)
    a.update(kw)
    return svg.lib.tree_deltanet_commit(a["state"], a["k"], a["v"], a["alpha"], a["beta"], a["path"], a["n"],
                                        a["T"], a["H"], a["dk"], a["dv"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(state=NULL), 1), (dict(q=NULL), 1), (dict(parent=NULL), 1), (dict(out=NULL), 1),
    (dict(T=0), 1), (dict(H=0), 1),
    (dict(T=33), 2), (dict(dk=96), 2), (dict(dk=128, dv=512), 2), (dict(dv=32), 2),
    (dict(state=MIS), 3), (dict(k=ctypes.c_void_p(0x10004)), 3), (dict(out=MIS), 3),
])
def test_tree_deltanet_verify_validation(svg, kw, code):
    assert _gdn_verify(svg, **kw) == code
    assert svg.last_error().startswith("tree_deltanet_verify:")


@pytest.mark.parametrize("kw,code", [
    (dict(state=NULL), 1), (dict(path=NULL), 1), (dict(n=NULL), 1), (dict(T=0), 1),
    (dict(T=40), 2), (dict(dk=32), 2), (dict(state=ctypes.c_void_p(0x10008)), 3), (dict(path=MIS), 3),
])
def test_tree_deltanet_commit_validation(svg, kw, code):
    assert _gdn_commit(svg, **kw) == code
    assert svg.last_error().startswith("tree_deltanet_commit:")


def test_size_limits_are_refused(svg):
    # K beyond 2^24, and weight storage of 4 GiB or more (one buffer range)
    assert _w4(svg, K=(1 << 24) + 128, g=64) == 2
    assert svg.lib.w8a8_linear(A, A, 1, 131072, A, A, 1 << 19, A, NULL, NULL) == 2   # 64 GiB of codes
    assert _w4(svg, N=1 << 21, K=8192, g=64) == 2                                     # 8 GiB of codes
    assert svg.lib.rht_rotate_weights(A, 1 << 21, 8192, A, 32, 1, 64, A, A, A, NULL, NULL) == 2
    assert _tree(svg, V=(1 << 30) + 1) == 2


# ------------------------------------------------------------ one-launch pass
def _pass_steps(svg, n=2, **kw):
    arr = (svg.PassStepC * n)()
    for i in range(n):
        d = dict(X=0x10000, signs=0x10000, xq=0x10000, x_scale=0x10000, wq=0x10000, w_scale=0x10000,
                 w_zero=0x10000, y=0x10000, partials_debug=None, N=64, K=4096, after=1)
        d.update(kw if i == n - 1 else {})
        arr[i] = svg.PassStepC(**d)
    return arr


def _plan(svg, steps, n=2, M=16, fmt=1, g=64, block=32):
    info = svg.PassInfoC()
    st = svg.lib.svg_pass_plan(steps, n, M, fmt, g, block, None, 0, ctypes.byref(info))
    return st, info


def test_pass_plan_sizes_the_plan_and_workspace(svg):
    st, info = _plan(svg, _pass_steps(svg))
    assert st == 0 and info.nsteps == 2 and info.M == 16
    assert info.plan_bytes == 64 + 2 * 136
    # counters, the per-XCC staging rows (M >= 2) and the two halves' partials of
    # each K = 4096 step (none: 16 x 4096 fits LDS)
    assert info.workspace_bytes % 256 == 0 and info.workspace_bytes > 8 * 16 * 12288
    st1, info1 = _plan(svg, _pass_steps(svg), M=1)
    assert st1 == 0 and info1.workspace_bytes < 64 * 1024       # no staging at M = 1
    # a K = 12288 step at M = 16 is cut in two halves: 4 tiles x 2 x 256 fp32 partials more
    st2, info2 = _plan(svg, _pass_steps(svg, K=12288))
    assert st2 == 0 and info2.workspace_bytes >= info.workspace_bytes + 4 * 2 * 256 * 4


def test_pass_plan_writes_the_image(svg):
    steps = _pass_steps(svg)
    st, info = _plan(svg, steps)
    buf = ctypes.create_string_buffer(info.plan_bytes)
    assert svg.lib.svg_pass_plan(steps, 2, 16, 1, 64, 32, buf, info.plan_bytes, ctypes.byref(info)) == 0
    raw = bytes(buf.raw)
    assert int.from_bytes(raw[:4], "little") == 0x53564750 and int.from_bytes(raw[4:8], "little") == 2
    small = ctypes.create_string_buffer(info.plan_bytes - 8)
    assert svg.lib.svg_pass_plan(steps, 2, 16, 1, 64, 32, small, info.plan_bytes - 8, ctypes.byref(info)) == 1


@pytest.mark.parametrize("kw,args,code", [
    (dict(X=None), {}, 1), (dict(y=None), {}, 1), (dict(w_zero=None), {}, 1), (dict(N=0), {}, 1),
    (dict(after=2), {}, 1),
    ({}, dict(M=17), 2), ({}, dict(g=32), 2), ({}, dict(fmt=2), 2), ({}, dict(block=16), 2),
    (dict(K=12416), {}, 2), (dict(K=4000), {}, 2), (dict(K=4160), dict(g=128), 2),
    (dict(X=0x10004), {}, 3), (dict(wq=0x10008), {}, 3), (dict(y=0x10002), {}, 3),
])
def test_pass_plan_validation(svg, kw, args, code):
    st, _info = _plan(svg, _pass_steps(svg, **kw), **args)
    assert st == code
    assert svg.last_error().startswith("svg_pass_plan:")


def test_pass_plan_needs_steps(svg):
    info = svg.PassInfoC()
    assert svg.lib.svg_pass_plan(None, 1, 1, 1, 64, 32, None, 0, ctypes.byref(info)) == 1
    assert svg.lib.svg_pass_plan(_pass_steps(svg), 0, 1, 1, 64, 32, None, 0, ctypes.byref(info)) == 2


def test_pass_run_validation(svg):
    st, info = _plan(svg, _pass_steps(svg))
    assert st == 0
    assert svg.lib.svg_pass_run(None, ctypes.byref(info), A, NULL) == 1
    assert svg.lib.svg_pass_run(A, ctypes.byref(info), None, NULL) == 1
    assert svg.lib.svg_pass_run(A, ctypes.byref(info), ctypes.c_void_p(0x10080), NULL) == 3   # not 256-aligned
    bad = svg.PassInfoC(2, 17, 1, 64, 32, info.plan_bytes, info.workspace_bytes)
    assert svg.lib.svg_pass_run(A, ctypes.byref(bad), A, NULL) == 2


# ------------------------------------------------------ layout conversions
def _imp(svg, export=False, **kw):
    args = dict(fmt=1, g=64, N=16, K=128, codes=A, scale=A, zero=A, wq=A, ws=A, wz=A)
    args.update(kw)
    fn = svg.lib.svg_export_weights if export else svg.lib.svg_import_weights
    if export:
        return fn(args["fmt"], args["g"], args["N"], args["K"], args["wq"], args["ws"], args["wz"],
                  args["codes"], args["scale"], args["zero"], NULL)
    return fn(args["fmt"], args["g"], args["N"], args["K"], args["codes"], args["scale"], args["zero"],
              args["wq"], args["ws"], args["wz"], NULL)


@pytest.mark.parametrize("export", [False, True])
@pytest.mark.parametrize("kw,code", [
    (dict(codes=NULL), 1), (dict(scale=NULL), 1), (dict(zero=NULL), 1), (dict(wq=NULL), 1), (dict(ws=NULL), 1),
    (dict(wz=NULL), 1), (dict(N=-1), 1), (dict(K=0), 1),
    (dict(fmt=7), 2), (dict(K=48), 2), (dict(g=16), 2), (dict(K=96, g=64), 2), (dict(K=1 << 25), 2),
    (dict(wq=MIS), 3), (dict(ws=ctypes.c_void_p(0x10002)), 3), (dict(wz=ctypes.c_void_p(0x10002)), 3),
    (dict(scale=MIS), 3), (dict(zero=MIS), 3),
])
def test_weight_layout_calls_validate_before_any_launch(svg, export, kw, code):
    """Every invalid call is refused on the host with its status code (the
    pointers are never dereferenced: no device work is enqueued)."""
    assert _imp(svg, export, **kw) == code, (kw, svg.last_error())


def test_weight_layout_calls_accept_w8_without_zeros(svg):
    # W8 needs no zero arrays; N = 0 is a no-op that touches nothing
    assert _imp(svg, fmt=2, g=0, N=0, zero=NULL, wz=NULL) == 0
    assert _imp(svg, True, fmt=2, g=0, N=0, zero=NULL, wz=NULL) == 0
    # a 4-bit zero array is bytes: any alignment
    assert _imp(svg, fmt=0, N=0, zero=MIS, wz=MIS) == 0
    assert _imp(svg, fmt=1, N=0) == 0


@pytest.mark.parametrize("name", ["svg_import_act_codes", "svg_export_act_codes"])
def test_act_layout_calls_validate_before_any_launch(svg, name):
    fn = getattr(svg.lib, name)
    assert fn(NULL, 1, 64, A, NULL) == 1
    assert fn(A, 1, 64, NULL, NULL) == 1
    assert fn(A, -1, 64, A, NULL) == 1
    assert fn(A, 1, 0, A, NULL) == 1
    assert fn(A, 1, 48, A, NULL) == 2
    slab_mis = (MIS, A) if name == "svg_export_act_codes" else (A, MIS)
    assert fn(slab_mis[0], 2, 64, slab_mis[1], NULL) == 3
    rows_mis = ctypes.c_void_p(0x10002)
    args = (A, 2, 64, rows_mis) if name == "svg_export_act_codes" else (rows_mis, 2, 64, A)
    assert fn(*args, NULL) == 3
    assert fn(A, 0, 64, A, NULL) == 0  # M = 0: nothing to do


def test_workspace_calls_validate_the_workspace(svg):
    """The _ws variants refuse a null or misaligned workspace before anything
    else (pointers never dereferenced)."""
    w4 = lambda ws: svg.lib.act_quant_w4a8_linear_ws(A, 2, 128, A, 32, A, A, A, A, A, 1, 64, 16, A, NULL,  # noqa: E731
                                                      ws, NULL)
    w8 = lambda ws: svg.lib.act_quant_w8a8_linear_ws(A, 2, 128, A, 32, A, A, A, A, 16, A, NULL, ws, NULL)  # noqa: E731
    for fn in (w4, w8):
        assert fn(NULL) == 1
        assert fn(ctypes.c_void_p(0x10040)) == 3
    # with a valid workspace the usual checks apply (here: M = 0 is a no-op)
    assert svg.lib.act_quant_w4a8_linear_ws(A, 0, 128, A, 32, A, A, A, A, A, 1, 64, 16, A, NULL, A, NULL) == 0
    assert svg.lib.act_quant_w4a8_linear_ws(A, 2, 128, A, 32, NULL, A, A, A, A, 1, 64, 16, A, NULL, A, NULL) == 1
