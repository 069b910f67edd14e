"""Shared GPU-test plumbing: move seeded inputs to the device, run the library
entry points through the binding, and fetch results.  No arithmetic of the
method lives here: the expected values come from oracle/ only."""
import sys

import numpy as np
import torch

import speculative_verify_gemm_amd as svg

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def gpu_quant_acts(x, signs, block=32):
    M, K = x.shape
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    xs = torch.empty((M,), dtype=torch.float32, device=DEV)
    svg.act_rht_quant_i8(to_dev(x), to_dev(signs), xq, xs, block=block)
    return xq, xs


def gpu_prepare(W, signs, fmt, group, debug=False, poison=True, block=32):
    """W: numpy [N,K] fp32 or a device tensor.  The storage is first filled
    with a non-zero byte so that padding the library fails to write shows."""
    Wd = W if isinstance(W, torch.Tensor) else to_dev(W)
    N, K = Wd.shape
    wq, ws, wz = svg.empty_weights(N, K, fmt, group)
    if poison:
        for t in (wq, ws, wz):
            if t is not None:
                t.view(torch.uint8).fill_(0x5A)
    rot = torch.empty((N, K), dtype=torch.float32, device=DEV) if debug else None
    svg.rht_rotate_weights(Wd, to_dev(signs), fmt, group, wq, ws, wz, rot, block=block)
    return dict(wq=wq, ws=ws, wz=wz, rot=rot, fmt=fmt, group=group, N=N, K=K, block=block)


def gpu_linear(xq, xs, w, debug=True):
    M, K = xq.shape
    N = w["N"]
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    if w["fmt"] == "w8":
        dbg = torch.empty((M, N), dtype=torch.int32, device=DEV) if debug else None
        svg.w8a8_linear(xq, xs, w["wq"], w["ws"], N, y, dbg)
    else:
        dbg = torch.empty((M, N, K // w["group"]), dtype=torch.int32, device=DEV) if debug else None
        svg.w4a8_linear(xq, xs, w["wq"], w["ws"], w["wz"], w["fmt"], w["group"], N, y, dbg)
    return y, dbg


def oracle_storage(ow, fmt, K):
    """The oracle's encoded weights in the library's tiled storage (host arrays)."""
    import storage_layout as SL
    if fmt == "w8":
        return SL.pack_w8_codes(ow["q"]), ow["s"], None
    g = ow["group"]
    z = SL.pack_z4(ow["z"], K, g) if fmt == "w4_z4" else SL.zeros_as_f16(ow["z"], K, g)
    return SL.pack_w4_codes(ow["q"]), SL.tile_group_params(ow["s"], K, g), z


def oracle_weights_to_dev(ow, fmt):
    """Device copies of the oracle's encoded weights, in the library layout."""
    N, K = ow["q"].shape
    wq, ws, wz = oracle_storage(ow, fmt, K)
    return dict(wq=to_dev(wq), ws=to_dev(ws), wz=None if wz is None else to_dev(wz), fmt=fmt,
                group=ow.get("group", 0), N=N, K=K)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def f16_bits(a):
    return np.asarray(a).view(np.uint16) if np.asarray(a).dtype == np.float16 else np.asarray(a)


def gpu_fused(x, signs, w, debug=True):
    """act_quant_w4a8_linear / act_quant_w8a8_linear on host inputs x [M,K]:
    returns (xq, x_scale, y, partials)."""
    xd = x if isinstance(x, torch.Tensor) else to_dev(x)
    sd = signs if isinstance(signs, torch.Tensor) else to_dev(signs)
    M, K = xd.shape
    N = w["N"]
    xq = torch.empty((M, K), dtype=torch.int8, device=DEV)
    xs = torch.empty((M,), dtype=torch.float32, device=DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    block = w.get("block", 32)
    if w["fmt"] == "w8":
        dbg = torch.empty((M, N), dtype=torch.int32, device=DEV) if debug else None
        svg.act_quant_w8a8_linear(xd, sd, xq, xs, w["wq"], w["ws"], N, y, dbg, block=block)
    else:
        dbg = torch.empty((M, N, K // w["group"]), dtype=torch.int32, device=DEV) if debug else None
        svg.act_quant_w4a8_linear(xd, sd, xq, xs, w["wq"], w["ws"], w["wz"], w["fmt"], w["group"], N, y, dbg,
                                  block=block)
    return xq, xs, y, dbg


def tie_rows(M, K, seed, exp=-3, nudge=False):
    """Activation rows whose rotated values are exact half-integer multiples of
    the row scale 2^exp (ties of the int8 rounding), one value 127 * 2^exp per
    row so that the scale is exactly 2^exp; with nudge, each target moved by
    one fp32 ulp up or down (near-ties).  Built as x = D H u / 32 blockwise
    in fp64 with the oracle's butterfly (H H = 32 I), then cast to fp32.
    Input construction only: the expected codes come from the oracle."""
    from oracle import svg_oracle as O
    rng = np.random.default_rng(seed)
    u = (rng.integers(-127, 127, size=(M, K)) + 0.5) * 2.0 ** exp
    u[:, 0] = 127 * 2.0 ** exp
    if nudge:
        up = rng.integers(0, 2, size=(M, K)).astype(bool)
        u32 = u.astype(np.float32)
        u = np.where(up, np.nextafter(u32, np.float32(np.inf)), np.nextafter(u32, np.float32(-np.inf)))
        u = u.astype(np.float64)
        u[:, 0] = 127 * 2.0 ** exp
    signs = np.where(rng.integers(0, 2, size=K) == 0, 1, -1).astype(np.int8)
    x = O.fwht32(u) * signs.astype(np.float64) / 32.0
    return x.astype(np.float32), signs


# the launches of one stack layer as the benchmark issues them: member
# matrices stacked along N into one storage, and the input space they read
STACK_LAUNCHES = {"qkv": (("q", "k", "v"), "attn_in"), "o": (("o",), "attn_out"),
                  "gateup": (("gate", "up"), "mlp_in"), "down": (("down",), "mlp_mid")}


def stack_launch(layer, launch, fmt, group):
    """Device storage of one stacked launch of a stack layer, rotated and
    quantized member by member into consecutive 16-row tiles (as bench.py
    builds it).  Returns (w, member weights on the device, signs, space)."""
    import synth
    members, space = STACK_LAUNCHES[launch]
    signs = synth.stack_signs(layer, space)
    Ws = [synth.stack_weight(layer, m, device=DEV) for m in members]
    N, K = sum(W.shape[0] for W in Ws), Ws[0].shape[1]
    wq, ws, wz = svg.empty_weights(N, K, fmt, group)
    sd = to_dev(signs)
    r0 = 0
    for W in Ws:
        mq, ms, mz = svg.stacked_slices(wq, ws, wz, r0, W.shape[0], K, fmt, group)
        svg.rht_rotate_weights(W, sd, fmt, group, mq, ms, mz)
        r0 += W.shape[0]
    return dict(wq=wq, ws=ws, wz=wz, fmt=fmt, group=group, N=N, K=K), Ws, signs, space


def stacked_rows(Ws, rows):
    """Host copy (fp32) of rows `rows` of the matrices Ws stacked along N."""
    out, r0 = [], 0
    for W in Ws:
        n = W.shape[0]
        sel = [r - r0 for r in rows if r0 <= r < r0 + n]
        if sel:
            out.append(W[torch.tensor(sel, device=W.device)].cpu().numpy())
        r0 += n
    return np.concatenate(out, axis=0)
