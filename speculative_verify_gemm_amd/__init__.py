"""Python binding of libsvgemm (the MI355X RHT + W4A8 / W8A8 quantized linear).

Argument marshalling only: every function checks tensor devices, dtypes and
shapes, derives the sizes, and calls the C entry point of the same name in
libsvgemm.so on the current HIP stream (or the one given).  All computation
runs in the library's HIP kernels; there is no Python or CPU fallback, and
importing this module fails if the library has not been built
(``python speculative_verify_gemm_amd/build.py``).

The operations follow the page "Karpathy's Trick for Faster Local LLMs Finally
Has Proper Tooling" (blog.dailydoseofds.com), section "How Uzu optimizes bytes
and tokens per pass": rotate the weights (random sign flips, then a 32-wide
+/-1 Hadamard per block) and quantize them as 4-bit asymmetric or 8-bit
symmetric integers; rotate and quantize the activations to int8 on the fly;
multiply integer by integer.  Layouts and numerics are those of
include/svgemm.h.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvgemm.so")

SVG_OK, SVG_EINVAL, SVG_EUNSUPPORTED, SVG_EALIGN, SVG_EHIP = 0, 1, 2, 3, 4
W4_Z4, W4_Z16, W8 = 0, 1, 2
FORMATS = {"w4_z4": W4_Z4, "w4_z16": W4_Z16, "w8": W8}
BLOCK = 32


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python speculative_verify_gemm_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.rht_rotate_weights.argtypes = [vp, i, i, vp, i, i, i, vp, vp, vp, vp, vp]
    lib.act_rht_quant_i8.argtypes = [vp, i, i, vp, i, vp, vp, vp]
    lib.w4a8_linear.argtypes = [vp, vp, i, i, vp, vp, vp, i, i, i, vp, vp, vp]
    lib.w8a8_linear.argtypes = [vp, vp, i, i, vp, vp, i, vp, vp, vp]
    lib.act_quant_w4a8_linear.argtypes = [vp, i, i, vp, i, vp, vp, vp, vp, vp, i, i, i, vp, vp, vp]
    lib.act_quant_w8a8_linear.argtypes = [vp, i, i, vp, i, vp, vp, vp, vp, i, vp, vp, vp]
    lib.act_quant_w4a8_linear_ws.argtypes = [vp, i, i, vp, i, vp, vp, vp, vp, vp, i, i, i, vp, vp, vp, vp]
    lib.act_quant_w8a8_linear_ws.argtypes = [vp, i, i, vp, i, vp, vp, vp, vp, i, vp, vp, vp, vp]
    lib.tree_accept_greedy.argtypes = [vp, i, i, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.tree_accept_greedy_static.argtypes = [vp, i, i, vp, vp, vp, vp, vp, vp, vp]
    lib.tree_deltanet_verify.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp, vp]
    lib.tree_deltanet_commit.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
    for fn in (lib.rht_rotate_weights, lib.act_rht_quant_i8, lib.w4a8_linear, lib.w8a8_linear,
               lib.act_quant_w4a8_linear, lib.act_quant_w8a8_linear, lib.tree_accept_greedy,
               lib.tree_accept_greedy_static,
               lib.tree_deltanet_verify, lib.tree_deltanet_commit):
        fn.restype = ctypes.c_int
    lib.svg_pass_plan.argtypes = [vp, i, i, i, i, i, vp, ctypes.c_uint64, vp]
    lib.svg_pass_run.argtypes = [vp, vp, vp, vp]
    lib.svg_import_weights.argtypes = [i, i, i, i, vp, vp, vp, vp, vp, vp, vp]
    lib.svg_export_weights.argtypes = [i, i, i, i, vp, vp, vp, vp, vp, vp, vp]
    lib.svg_import_act_codes.argtypes = [vp, i, i, vp, vp]
    lib.svg_export_act_codes.argtypes = [vp, i, i, vp, vp]
    lib.svg_pass_plan.restype = ctypes.c_int
    lib.svg_pass_run.restype = ctypes.c_int
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.svg_weight_sizes.argtypes = [i, i, i, i, u64p, u64p, u64p]
    lib.svg_weight_sizes.restype = ctypes.c_int
    lib.svg_last_error.argtypes = []
    lib.svg_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


class SvgError(RuntimeError):
    """A non-zero status from libsvgemm."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libsvgemm status {status}: {message}")
        self.status = status


def last_error() -> str:
    return lib.svg_last_error().decode()


def _check(status: int):
    if status != SVG_OK:
        raise SvgError(status, last_error())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream, t):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


# ------------------------------------------------------------ entry points
def weight_sizes(N, K, fmt, group):
    """Bytes of the tiled weight storage: (wq, scales, zeros)."""
    a, b, c = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib.svg_weight_sizes(N, K, _fmt(fmt), group, ctypes.byref(a), ctypes.byref(b),
                                ctypes.byref(c)))
    return a.value, b.value, c.value


def _check_storage(N, K, f, group, wq, w_scale, w_zero):
    wb, sb, zb = weight_sizes(N, K, f, group)
    _dev(wq, "wq", torch.int8 if f == W8 else torch.uint8)
    _dev(w_scale, "w_scale", torch.float16)
    if wq.numel() < wb or w_scale.numel() * 2 < sb:
        raise ValueError(f"weight storage too small: need {wb} code bytes and {sb} scale bytes")
    if f != W8:
        if w_zero is None:
            raise ValueError("W4 formats need w_zero")
        _dev(w_zero, "w_zero", torch.uint8 if f == W4_Z4 else torch.float16)
        if w_zero.numel() * w_zero.element_size() < zb:
            raise ValueError(f"w_zero too small: need {zb} bytes")


def rht_rotate_weights(W, signs, fmt, group, wq, w_scale, w_zero=None, w_rot_debug=None,
                       block=BLOCK, stream=None):
    """Rotate and quantize fp32 weights W[N, K] into the tiled storage
    (wq, w_scale, w_zero) sized by weight_sizes()."""
    f = _fmt(fmt)
    _dev(W, "W", torch.float32)
    _dev(signs, "signs", torch.int8)
    N, K = W.shape
    _check_storage(N, K, f, group, wq, w_scale, w_zero)
    if w_rot_debug is not None:
        _dev(w_rot_debug, "w_rot_debug", torch.float32)
    _check(lib.rht_rotate_weights(_p(W), N, K, _p(signs), block, f, group, _p(wq), _p(w_scale),
                                  _p(w_zero), _p(w_rot_debug), _stream(stream, W)))


def act_rht_quant_i8(X, signs, xq, x_scale, block=BLOCK, stream=None):
    """Rotate fp32 activations X[M, K] and quantize each row to int8."""
    _dev(X, "X", torch.float32)
    _dev(signs, "signs", torch.int8)
    _dev(xq, "xq", torch.int8)
    _dev(x_scale, "x_scale", torch.float32)
    M, K = X.shape
    if tuple(xq.shape) != (M, K) or tuple(x_scale.shape) != (M,):
        raise ValueError("xq must be [M, K] and x_scale [M]")
    _check(lib.act_rht_quant_i8(_p(X), M, K, _p(signs), block, _p(xq), _p(x_scale),
                                _stream(stream, X)))


def w4a8_linear(xq, x_scale, wq, w_scale, w_zero, fmt, group, N, y, partials_debug=None,
                stream=None):
    """y[M, N] = dequantized (xq . W^T) for tiled W4 weights of N rows."""
    f = _fmt(fmt)
    _dev(xq, "xq", torch.int8)
    _dev(x_scale, "x_scale", torch.float32)
    _dev(y, "y", torch.float32)
    M, K = xq.shape
    _check_storage(N, K, f, group, wq, w_scale, w_zero)
    if tuple(y.shape) != (M, N) or tuple(x_scale.shape) != (M,):
        raise ValueError("y must be [M, N] and x_scale [M]")
    if partials_debug is not None:
        _dev(partials_debug, "partials_debug", torch.int32)
        if tuple(partials_debug.shape) != (M, N, K // group):
            raise ValueError("partials_debug must be [M, N, K/g]")
    _check(lib.w4a8_linear(_p(xq), _p(x_scale), M, K, _p(wq), _p(w_scale), _p(w_zero), f, group,
                           N, _p(y), _p(partials_debug), _stream(stream, xq)))


def w8a8_linear(xq, x_scale, wq, w_scale, N, y, partials_debug=None, stream=None):
    """y[M, N] = dequantized (xq . W^T) for tiled W8 weights of N rows."""
    _dev(xq, "xq", torch.int8)
    _dev(x_scale, "x_scale", torch.float32)
    _dev(y, "y", torch.float32)
    M, K = xq.shape
    _check_storage(N, K, W8, 0, wq, w_scale, None)
    if tuple(y.shape) != (M, N) or tuple(x_scale.shape) != (M,):
        raise ValueError("y must be [M, N] and x_scale [M]")
    if partials_debug is not None:
        _dev(partials_debug, "partials_debug", torch.int32)
        if tuple(partials_debug.shape) != (M, N):
            raise ValueError("partials_debug must be [M, N]")
    _check(lib.w8a8_linear(_p(xq), _p(x_scale), M, K, _p(wq), _p(w_scale), N, _p(y),
                           _p(partials_debug), _stream(stream, xq)))


def _check_fused(X, signs, xq, x_scale):
    _dev(X, "X", torch.float32)
    _dev(signs, "signs", torch.int8)
    if tuple(xq.shape) != tuple(X.shape):
        raise ValueError("xq must have the shape of X")


def act_quant_w4a8_linear(X, signs, xq, x_scale, wq, w_scale, w_zero, fmt, group, N, y,
                          partials_debug=None, block=BLOCK, stream=None, workspace=None):
    """act_rht_quant_i8 then w4a8_linear (one launch for M = 1): fp32 X[M, K]
    in, xq / x_scale (written) and y[M, N] out.  With a workspace (from
    linear_workspace()) the rows of a verify batch are quantized inside the
    linear's own launch (act_quant_w4a8_linear_ws)."""
    _check_fused(X, signs, xq, x_scale)
    f = _fmt(fmt)
    _dev(xq, "xq", torch.int8)
    _dev(x_scale, "x_scale", torch.float32)
    _dev(y, "y", torch.float32)
    M, K = X.shape
    _check_storage(N, K, f, group, wq, w_scale, w_zero)
    if tuple(y.shape) != (M, N) or tuple(x_scale.shape) != (M,):
        raise ValueError("y must be [M, N] and x_scale [M]")
    if partials_debug is not None:
        _dev(partials_debug, "partials_debug", torch.int32)
        if tuple(partials_debug.shape) != (M, N, K // group):
            raise ValueError("partials_debug must be [M, N, K/g]")
    if workspace is not None:
        _check_linear_workspace(workspace)
        _check(lib.act_quant_w4a8_linear_ws(_p(X), M, K, _p(signs), block, _p(xq), _p(x_scale), _p(wq),
                                            _p(w_scale), _p(w_zero), f, group, N, _p(y), _p(partials_debug),
                                            _p(workspace), _stream(stream, X)))
        return
    _check(lib.act_quant_w4a8_linear(_p(X), M, K, _p(signs), block, _p(xq), _p(x_scale), _p(wq),
                                     _p(w_scale), _p(w_zero), f, group, N, _p(y), _p(partials_debug),
                                     _stream(stream, X)))


def act_quant_w8a8_linear(X, signs, xq, x_scale, wq, w_scale, N, y, partials_debug=None,
                          block=BLOCK, stream=None, workspace=None):
    """act_rht_quant_i8 then w8a8_linear (one launch for M = 1; with a
    workspace, one launch at every M: act_quant_w8a8_linear_ws)."""
    _check_fused(X, signs, xq, x_scale)
    _dev(xq, "xq", torch.int8)
    _dev(x_scale, "x_scale", torch.float32)
    _dev(y, "y", torch.float32)
    M, K = X.shape
    _check_storage(N, K, W8, 0, wq, w_scale, None)
    if tuple(y.shape) != (M, N) or tuple(x_scale.shape) != (M,):
        raise ValueError("y must be [M, N] and x_scale [M]")
    if partials_debug is not None:
        _dev(partials_debug, "partials_debug", torch.int32)
        if tuple(partials_debug.shape) != (M, N):
            raise ValueError("partials_debug must be [M, N]")
    if workspace is not None:
        _check_linear_workspace(workspace)
        _check(lib.act_quant_w8a8_linear_ws(_p(X), M, K, _p(signs), block, _p(xq), _p(x_scale), _p(wq),
                                            _p(w_scale), N, _p(y), _p(partials_debug), _p(workspace),
                                            _stream(stream, X)))
        return
    _check(lib.act_quant_w8a8_linear(_p(X), M, K, _p(signs), block, _p(xq), _p(x_scale), _p(wq),
                                     _p(w_scale), N, _p(y), _p(partials_debug), _stream(stream, X)))


# ------------------------------------------------------------- allocation
LINEAR_WORKSPACE_BYTES = 256


def linear_workspace(device="cuda"):
    """A zero-filled workspace for the fused calls' in-launch quantization
    (each call leaves it zero-filled, word 3 excepted: a sticky give-up flag;
    calls that may overlap need workspaces of their own)."""
    return torch.zeros(LINEAR_WORKSPACE_BYTES // 4, dtype=torch.int32, device=device)


def _check_linear_workspace(ws):
    _dev(ws, "workspace", torch.int32)
    if ws.numel() * 4 < LINEAR_WORKSPACE_BYTES:
        raise ValueError(f"workspace needs {LINEAR_WORKSPACE_BYTES} bytes")


def linear_workspace_gave_up(ws) -> bool:
    """Whether a bounded wait of a call on this workspace ever gave up."""
    return int(ws[3].item()) != 0


TREE_MAX_NODES, TREE_WORKSPACE_BYTES = 32, 512


def tree_workspace(device="cuda"):
    """A zero-filled workspace for tree_accept_greedy (each call leaves it
    zero-filled; calls that may overlap need workspaces of their own)."""
    return torch.zeros(TREE_WORKSPACE_BYTES, dtype=torch.uint8, device=device)


def tree_accept_greedy(logits, parent, draft, target, path, emit, n_emit, workspace, stream=None):
    """Greedy acceptance of a verified draft tree (include/svgemm.h): logits
    [T, V] fp32; parent, draft [T] int32; outputs target, path, emit [T] and
    n_emit [1] int32; workspace from tree_workspace()."""
    T, V = _tree_args(logits, parent, draft, target, path, emit, n_emit)
    _dev(workspace, "workspace", torch.uint8)
    if workspace.numel() < TREE_WORKSPACE_BYTES:
        raise ValueError("workspace needs TREE_WORKSPACE_BYTES bytes")
    _check(lib.tree_accept_greedy(_p(logits), T, V, _p(parent), _p(draft), _p(target), _p(path),
                                  _p(emit), _p(n_emit), _p(workspace), _stream(stream, logits)))


def _tree_args(logits, parent, draft, target, path, emit, n_emit):
    _dev(logits, "logits", torch.float32)
    T, V = logits.shape
    for name, t in (("parent", parent), ("draft", draft), ("target", target), ("path", path),
                    ("emit", emit)):
        _dev(t, name, torch.int32)
        if tuple(t.shape) != (T,):
            raise ValueError(f"{name} must have shape [{T}]")
    _dev(n_emit, "n_emit", torch.int32)
    if n_emit.numel() < 1:
        raise ValueError("n_emit needs 1 element")
    return T, V


def tree_accept_greedy_static(logits, parent, draft, target, path, emit, n_emit, stream=None):
    """tree_accept_greedy on the library's own static workspace (nothing
    allocated; calls that may overlap on one device must not be made)."""
    T, V = _tree_args(logits, parent, draft, target, path, emit, n_emit)
    _check(lib.tree_accept_greedy_static(_p(logits), T, V, _p(parent), _p(draft), _p(target), _p(path),
                                         _p(emit), _p(n_emit), _stream(stream, logits)))


def _gdn_shapes(state, k, v, alpha, beta):
    for name, t in (("state", state), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta)):
        _dev(t, name, torch.float32)
    H, dv, dk = state.shape
    T = k.shape[0]
    if (tuple(k.shape) != (T, H, dk) or tuple(v.shape) != (T, H, dv) or tuple(alpha.shape) != (T, H)
            or tuple(beta.shape) != (T, H)):
        raise ValueError("need state [H, dv, dk], k [T, H, dk], v [T, H, dv], alpha and beta [T, H]")
    return T, H, dk, dv


def tree_deltanet_verify(state, q, k, v, alpha, beta, parent, out, stream=None):
    """Outputs of a gated delta-rule layer at every node of a draft tree
    (include/svgemm.h); `state` [H, dv, dk] is only read."""
    T, H, dk, dv = _gdn_shapes(state, k, v, alpha, beta)
    _dev(q, "q", torch.float32)
    _dev(parent, "parent", torch.int32)
    _dev(out, "out", torch.float32)
    if tuple(q.shape) != (T, H, dk) or tuple(parent.shape) != (T,) or tuple(out.shape) != (T, H, dv):
        raise ValueError("need q [T, H, dk], parent [T] and out [T, H, dv]")
    _check(lib.tree_deltanet_verify(_p(state), _p(q), _p(k), _p(v), _p(alpha), _p(beta), _p(parent),
                                    T, H, dk, dv, _p(out), _stream(stream, state)))


def tree_deltanet_commit(state, k, v, alpha, beta, path, n_emit, stream=None):
    """Advance `state` in place by the root and the accepted path written by
    tree_accept_greedy (path, n_emit)."""
    T, H, dk, dv = _gdn_shapes(state, k, v, alpha, beta)
    _dev(path, "path", torch.int32)
    _dev(n_emit, "n_emit", torch.int32)
    if path.numel() < T - 1 or n_emit.numel() < 1:
        raise ValueError("path needs T - 1 entries and n_emit one")
    _check(lib.tree_deltanet_commit(_p(state), _p(k), _p(v), _p(alpha), _p(beta), _p(path), _p(n_emit),
                                    T, H, dk, dv, _stream(stream, state)))


# ------------------------------------------------------- layout conversions
def _check_canonical(N, K, f, group, codes, scale, zero):
    if f == W8:
        _dev(codes, "codes", torch.int8)
        if tuple(codes.shape) != (N, K) or tuple(scale.shape) != (N,):
            raise ValueError("W8: codes must be [N, K] int8 and scale [N] fp16")
    else:
        _dev(codes, "codes", torch.uint8)
        ng = K // group
        if tuple(codes.shape) != (N, K // 2) or tuple(scale.shape) != (N, ng):
            raise ValueError("W4: codes must be [N, K/2] uint8 and scale [N, K/group] fp16")
        if zero is None:
            raise ValueError("W4 formats need zero")
        if f == W4_Z4:
            _dev(zero, "zero", torch.uint8)
            if tuple(zero.shape) != (N, (ng + 1) // 2):
                raise ValueError("4-bit zeros must be [N, ceil(K/group/2)] uint8")
        else:
            _dev(zero, "zero", torch.float16)
            if tuple(zero.shape) != (N, ng):
                raise ValueError("fp16 zeros must be [N, K/group]")
    _dev(scale, "scale", torch.float16)


def import_weights(codes, scale, zero, fmt, group, K, wq, w_scale, w_zero=None, stream=None):
    """Canonical row-major weights (codes, scale, zero) -> the tiled storage
    (wq, w_scale, w_zero) sized by weight_sizes()."""
    f = _fmt(fmt)
    N = codes.shape[0]
    _check_canonical(N, K, f, group, codes, scale, zero)
    _check_storage(N, K, f, group, wq, w_scale, w_zero)
    _check(lib.svg_import_weights(f, group, N, K, _p(codes), _p(scale), _p(zero), _p(wq), _p(w_scale),
                                  _p(w_zero), _stream(stream, wq)))


def export_weights(wq, w_scale, w_zero, fmt, group, N, K, codes, scale, zero=None, stream=None):
    """The tiled storage -> canonical row-major (codes, scale, zero)."""
    f = _fmt(fmt)
    _check_canonical(N, K, f, group, codes, scale, zero)
    _check_storage(N, K, f, group, wq, w_scale, w_zero)
    _check(lib.svg_export_weights(f, group, N, K, _p(wq), _p(w_scale), _p(w_zero), _p(codes), _p(scale),
                                  _p(zero), _stream(stream, wq)))


def import_act_codes(rows, xq, stream=None):
    """Activation codes [M, K] int8 rows -> xq in the slab layout."""
    _dev(rows, "rows", torch.int8)
    _dev(xq, "xq", torch.int8)
    M, K = rows.shape
    if xq.numel() != M * K:
        raise ValueError("xq must hold M * K codes")
    _check(lib.svg_import_act_codes(_p(rows), M, K, _p(xq), _stream(stream, rows)))


def export_act_codes(xq, rows, stream=None):
    """xq in the slab layout -> activation codes [M, K] int8 rows."""
    _dev(rows, "rows", torch.int8)
    _dev(xq, "xq", torch.int8)
    M, K = rows.shape
    if xq.numel() != M * K:
        raise ValueError("xq must hold M * K codes")
    _check(lib.svg_export_act_codes(_p(xq), M, K, _p(rows), _stream(stream, rows)))


def empty_weights(N, K, fmt, group, device="cuda"):
    """Uninitialised tiled storage for rht_rotate_weights: flat (wq, w_scale,
    w_zero) tensors (w_zero is None for W8)."""
    f = _fmt(fmt)
    wb, sb, zb = weight_sizes(N, K, f, group)
    wq = torch.empty((wb,), dtype=torch.int8 if f == W8 else torch.uint8, device=device)
    sc = torch.empty((sb // 2,), dtype=torch.float16, device=device)
    if f == W8:
        return wq, sc, None
    if f == W4_Z4:
        return wq, sc, torch.empty((zb,), dtype=torch.uint8, device=device)
    return wq, sc, torch.empty((zb // 2,), dtype=torch.float16, device=device)


def stacked_slices(wq, w_scale, w_zero, rows_before, N, K, fmt, group):
    """Views of the tiled storage of a matrix stacked after `rows_before` rows
    (a multiple of 16) of other matrices in one buffer, N rows of its own."""
    if rows_before % 16:
        raise ValueError("stacked matrices must start on a 16-row tile")
    f = _fmt(fmt)
    w0, s0, z0 = weight_sizes(rows_before, K, f, group) if rows_before else (0, 0, 0)
    w1, s1, z1 = weight_sizes(N, K, f, group)
    if f == W8:
        # W8 scales are per row, in row order
        return wq[w0:w0 + w1], w_scale[rows_before:rows_before + N], None
    es = w_zero.element_size()
    return (wq[w0:w0 + w1], w_scale[s0 // 2:(s0 + s1) // 2], w_zero[z0 // es:(z0 + z1) // es])


# ------------------------------------------------------------ one-launch pass
class PassStepC(ctypes.Structure):
    """svg_pass_step (include/svgemm.h)."""
    _fields_ = [("X", ctypes.c_void_p), ("signs", ctypes.c_void_p), ("xq", ctypes.c_void_p),
                ("x_scale", ctypes.c_void_p), ("wq", ctypes.c_void_p), ("w_scale", ctypes.c_void_p),
                ("w_zero", ctypes.c_void_p), ("y", ctypes.c_void_p), ("partials_debug", ctypes.c_void_p),
                ("N", ctypes.c_int), ("K", ctypes.c_int), ("after", ctypes.c_int)]


class PassInfoC(ctypes.Structure):
    """svg_pass_info (include/svgemm.h)."""
    _fields_ = [("nsteps", ctypes.c_int), ("M", ctypes.c_int), ("fmt", ctypes.c_int), ("group", ctypes.c_int),
                ("block", ctypes.c_int), ("plan_bytes", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64)]


class LinearPass:
    """A pass of dependent W4A8 linears run as ONE launch (svg_pass_plan /
    svg_pass_run).  `steps`: dicts with X [M, K] fp32, signs [K] int8, xq
    [M, K] int8 and x_scale [M] fp32 (outputs), wq / w_scale / w_zero (the
    tiled storage), N, y [M, N] fp32, optional partials_debug [M, N, K/group]
    int32, and `after` (read X only once every earlier step has finished).
    The plan image is uploaded once; the tensors must stay alive and in place
    (the object keeps references)."""

    def __init__(self, steps, fmt, group, block=BLOCK, device=None):
        if not steps:
            raise ValueError("a pass needs at least one step")
        f = _fmt(fmt)
        M = steps[0]["X"].shape[0]
        arr = (PassStepC * len(steps))()
        self._keep = []
        for i, st in enumerate(steps):
            X, sg, xq, xs, y = st["X"], st["signs"], st["xq"], st["x_scale"], st["y"]
            _dev(X, "X", torch.float32)
            _dev(sg, "signs", torch.int8)
            _dev(xq, "xq", torch.int8)
            _dev(xs, "x_scale", torch.float32)
            _dev(y, "y", torch.float32)
            m, K = X.shape
            N = int(st["N"])
            if m != M:
                raise ValueError("every step of a pass has the same M")
            if tuple(xq.shape) != (M, K) or tuple(xs.shape) != (M,) or tuple(y.shape) != (M, N):
                raise ValueError("step shapes: xq [M, K], x_scale [M], y [M, N]")
            _check_storage(N, K, f, group, st["wq"], st["w_scale"], st["w_zero"])
            dbg = st.get("partials_debug")
            if dbg is not None:
                _dev(dbg, "partials_debug", torch.int32)
                if tuple(dbg.shape) != (M, N, K // group):
                    raise ValueError("partials_debug must be [M, N, K/g]")
            arr[i] = PassStepC(X.data_ptr(), sg.data_ptr(), xq.data_ptr(), xs.data_ptr(), st["wq"].data_ptr(),
                               st["w_scale"].data_ptr(), st["w_zero"].data_ptr(), y.data_ptr(),
                               dbg.data_ptr() if dbg is not None else None, N, K, int(st.get("after", 1)))
            self._keep.append(st)
        self.info = PassInfoC()
        _check(lib.svg_pass_plan(arr, len(steps), M, f, group, block, None, 0, ctypes.byref(self.info)))
        host = ctypes.create_string_buffer(self.info.plan_bytes)
        _check(lib.svg_pass_plan(arr, len(steps), M, f, group, block, host, self.info.plan_bytes,
                                 ctypes.byref(self.info)))
        dev = device if device is not None else steps[0]["X"].device
        self.plan = torch.frombuffer(bytearray(host.raw), dtype=torch.uint8).to(dev)
        self.workspace = torch.zeros(self.info.workspace_bytes, dtype=torch.uint8, device=dev)
        if self.workspace.data_ptr() % 256 or self.plan.data_ptr() % 8:
            raise RuntimeError("device allocations are not aligned as the pass needs")

    def run(self, stream=None):
        _check(lib.svg_pass_run(_p(self.plan), ctypes.byref(self.info), _p(self.workspace),
                                _stream(stream, self.plan)))

    def gave_up(self) -> bool:
        """Whether a run of this pass ever gave up a bounded wait (word 0 of
        its workspace; its outputs are then undefined)."""
        return bool(int(self.workspace[:4].view(torch.int32).cpu()[0]))
