"""Seeded synthetic inputs for the RHT + W4A8/W8A8 quantized linear.

This module draws inputs only: fp32 weight matrices, fp32 activation rows and
the +/-1 sign vectors of the random Hadamard transform (the method's random
numbers, which both the HIP library and the CPU oracle take as an argument).
It holds none of the method's arithmetic and imports neither side.

Every tensor has its own numpy SeedSequence child of ROOT_SEED, keyed by
(workload, layer, slot, tensor kind), so any tensor can be regenerated alone.

Workloads (shapes and value distributions):

* ``single_1k``  -- M=1, K=N=1024.  x ~ N(0,1) with 4 distinct channels x50;
  W ~ N(0, 0.02); W4, zero as uint4, group 32.
* ``decode_12k`` -- M=1, K=4096, N=12288.  x ~ Student-t(3);
  W ~ N(0, 0.02) with round(0.001*N*K) distinct entries x20; W4, fp16 zero,
  group 64.
* ``stack_w4g64`` -- a 32-layer projection stack (q, k, v, o: 4096x4096;
  gate, up: 12288x4096; down: 4096x12288), W drawn as in ``decode_12k``;
  x per layer input space ~ N(0,1) with 4 channels x50; M=16; W4 fp16 zero g64.
* ``stack_w8``   -- the same stack as 8-bit symmetric per-row weights, M=32,
  x ~ Student-t(3).
* ``stack_w4g128`` -- the same stack, W4 fp16 zero, group 128; x ~ Student-t(3)
  with round(0.01*K) channels x100; M in {1, 2, 4, 8, 16, 32} (the first M
  rows of a 32-row draw).

Stack weights are large (7.0e9 values), so they are drawn on the device with
torch's counter-based generator seeded from the same SeedSequence tree
(``stack_weight``); the host never materialises the stack.  Small workloads use
numpy on the host.
"""
from __future__ import annotations

import numpy as np

ROOT_SEED = 20261202

# Integer ids used in SeedSequence spawn keys.
_WORKLOAD_ID = {"single_1k": 1, "decode_12k": 2, "stack": 3,
                "stack_w4g64": 3, "stack_w8": 4, "stack_w4g128": 5, "test": 9}
_KIND_ID = {"W": 1, "x": 2, "signs": 3, "W_outlier": 4, "x_outlier": 5}

# Projection stack: name -> (N, K, input space).  Matrices of one input space
# consume the same activation row and therefore share one sign vector.
STACK_LAYERS = 32
STACK_MATRICES = (
    ("q", 4096, 4096, "attn_in"),
    ("k", 4096, 4096, "attn_in"),
    ("v", 4096, 4096, "attn_in"),
    ("o", 4096, 4096, "attn_out"),
    ("gate", 12288, 4096, "mlp_in"),
    ("up", 12288, 4096, "mlp_in"),
    ("down", 4096, 12288, "mlp_mid"),
)
STACK_SPACES = (("attn_in", 4096), ("attn_out", 4096), ("mlp_in", 4096),
                ("mlp_mid", 12288))
_MATRIX_ID = {name: i for i, (name, *_r) in enumerate(STACK_MATRICES)}
_SPACE_ID = {name: 16 + i for i, (name, _k) in enumerate(STACK_SPACES)}

# Workload table: the shapes and formats each workload is quoted on.
WORKLOADS = {
    "single_1k": dict(M=1, K=1024, N=1024, fmt="w4_z4", group=32,
                      x="normal_outlier", x_outliers=4, x_mult=50.0,
                      w_outlier_frac=0.0),
    "decode_12k": dict(M=1, K=4096, N=12288, fmt="w4_z16", group=64,
                       x="student_t3", w_outlier_frac=1e-3, w_mult=20.0),
    "stack_w4g64": dict(M=16, fmt="w4_z16", group=64, x="normal_outlier",
                        x_outliers=4, x_mult=50.0),
    "stack_w8": dict(M=32, fmt="w8", group=0, x="student_t3"),
    "stack_w4g128": dict(M=32, fmt="w4_z16", group=128, x="student_t3_outlier",
                         x_outlier_frac=0.01, x_mult=100.0,
                         m_sweep=(1, 2, 4, 8, 16, 32)),
}
W_STD = 0.02
STACK_W_OUTLIER_FRAC = 1e-3
STACK_W_MULT = 20.0


def seed_sequence(workload: str, layer: int, slot: int, kind: str) -> np.random.SeedSequence:
    """The SeedSequence child of one tensor."""
    return np.random.SeedSequence(
        ROOT_SEED, spawn_key=(_WORKLOAD_ID[workload], int(layer), int(slot),
                              _KIND_ID[kind]))


def rng_for(workload: str, layer: int, slot: int, kind: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed_sequence(workload, layer, slot, kind)))


def torch_seed_for(workload: str, layer: int, slot: int, kind: str) -> int:
    """A 63-bit seed for torch's generator, derived from the same tree."""
    st = seed_sequence(workload, layer, slot, kind).generate_state(2, dtype=np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


# ---------------------------------------------------------------- host draws
def rademacher(K: int, rng: np.random.Generator) -> np.ndarray:
    """K independent +/-1 values as int8."""
    return np.where(rng.integers(0, 2, size=K, dtype=np.int8) == 1, 1, -1).astype(np.int8)


def normal_weights(N: int, K: int, rng: np.random.Generator, std: float = W_STD,
                   outlier_frac: float = 0.0, mult: float = 20.0,
                   rng_outlier: np.random.Generator | None = None) -> np.ndarray:
    """W[N, K] ~ N(0, std) fp32; round(outlier_frac*N*K) distinct entries x mult."""
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(std)
    count = int(round(outlier_frac * N * K))
    if count:
        r = rng_outlier if rng_outlier is not None else rng
        idx = r.choice(N * K, size=count, replace=False)
        W.reshape(-1)[idx] *= np.float32(mult)
    return W


def normal_outlier_acts(M: int, K: int, rng: np.random.Generator, n_out: int,
                        mult: float) -> np.ndarray:
    """x[M, K] ~ N(0, 1) fp32 with n_out distinct channels scaled by mult."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    ch = rng.choice(K, size=n_out, replace=False)
    x[:, ch] *= np.float32(mult)
    return x


def student_t3_acts(M: int, K: int, rng: np.random.Generator, outlier_frac: float = 0.0,
                    mult: float = 100.0) -> np.ndarray:
    """x[M, K] ~ standard Student-t with 3 degrees of freedom, fp32; optionally
    round(outlier_frac*K) distinct channels scaled by mult."""
    x = rng.standard_t(3.0, size=(M, K)).astype(np.float32)
    n_out = int(round(outlier_frac * K))
    if n_out:
        ch = rng.choice(K, size=n_out, replace=False)
        x[:, ch] *= np.float32(mult)
    return x


def single_inputs(workload: str):
    """(x[M,K] fp32, W[N,K] fp32, signs[K] int8, spec dict) for a single-matrix
    workload ("single_1k" or "decode_12k")."""
    spec = dict(WORKLOADS[workload])
    M, K, N = spec["M"], spec["K"], spec["N"]
    signs = rademacher(K, rng_for(workload, 0, 0, "signs"))
    W = normal_weights(N, K, rng_for(workload, 0, 0, "W"),
                       outlier_frac=spec.get("w_outlier_frac", 0.0),
                       mult=spec.get("w_mult", 20.0),
                       rng_outlier=rng_for(workload, 0, 0, "W_outlier"))
    x = make_acts(workload, spec, M, K, rng_for(workload, 0, 0, "x"))
    return x, W, signs, spec


def make_acts(workload: str, spec: dict, M: int, K: int, rng: np.random.Generator) -> np.ndarray:
    kind = spec["x"]
    if kind == "normal_outlier":
        return normal_outlier_acts(M, K, rng, spec["x_outliers"], spec["x_mult"])
    if kind == "student_t3":
        return student_t3_acts(M, K, rng)
    if kind == "student_t3_outlier":
        return student_t3_acts(M, K, rng, spec["x_outlier_frac"], spec["x_mult"])
    raise ValueError(kind)


def stack_signs(layer: int, space: str) -> np.ndarray:
    """Sign vector of one input space of one stack layer (shared by every
    workload built on the stack, like the stack's weights)."""
    K = dict(STACK_SPACES)[space]
    return rademacher(K, rng_for("stack", layer, _SPACE_ID[space], "signs"))


def stack_acts(workload: str, layer: int, space: str, M: int | None = None) -> np.ndarray:
    """Activation rows x[M, K] of one input space of one stack layer."""
    spec = WORKLOADS[workload]
    K = dict(STACK_SPACES)[space]
    Mdraw = 32 if workload == "stack_w4g128" else spec["M"]
    x = make_acts(workload, spec, Mdraw, K, rng_for(workload, layer, _SPACE_ID[space], "x"))
    return x if M is None else x[:M]


def random_case(M: int, N: int, K: int, seed: int, w_std: float = W_STD,
                x_kind: str = "normal_outlier"):
    """Small seeded case for parity tests: (x, W, signs)."""
    rx = rng_for("test", seed, 1, "x")
    rw = rng_for("test", seed, 2, "W")
    rs = rng_for("test", seed, 3, "signs")
    signs = rademacher(K, rs)
    W = normal_weights(N, K, rw, std=w_std, outlier_frac=1e-3 if N * K >= 1000 else 0.0,
                       mult=20.0)
    if x_kind == "normal_outlier":
        x = normal_outlier_acts(M, K, rx, min(4, K), 50.0)
    else:
        x = student_t3_acts(M, K, rx)
    return x, W, signs


# ---------------------------------------------------------------- draft trees
def draft_tree(T: int, V: int, seed: int, shape: str = "bushy", accept: int | None = None,
               ties: bool = False):
    """A verified draft tree of T nodes over a V-token vocabulary:
    (logits[T, V] fp32, parent[T] int32, draft[T] int32).

    Node 0 is the root (parent -1); node i >= 1 hangs under an earlier node:
    "chain" (parent i - 1), "star" (parent 0) or "bushy" (uniform over the
    four nodes before it).  Drafted tokens are uniform over the vocabulary.
    Logits are N(0, 1).  With `accept` = d, the root path of a random node of
    depth >= d is made to agree for its first d steps (the parent's row gets
    logit 10 at the child's token) and to disagree at step d + 1 (logit -10),
    so that the accepted depth is about d (a sibling can still agree by
    chance).  With `ties`, a few rows get their largest value copied to a
    random index (an exact fp32 tie, unless that index already held it)."""
    rng = rng_for("test", seed, 7, "x")
    parent = np.full(T, -1, dtype=np.int32)
    for i in range(1, T):
        if shape == "chain":
            parent[i] = i - 1
        elif shape == "star":
            parent[i] = 0
        else:
            parent[i] = rng.integers(max(0, i - 4), i)
    draft = rng.integers(0, V, size=T).astype(np.int32)
    logits = rng.standard_normal((T, V), dtype=np.float32)
    if accept is not None:
        depth = np.zeros(T, dtype=np.int64)
        for i in range(1, T):
            depth[i] = depth[parent[i]] + 1
        deep = np.flatnonzero(depth >= min(accept, int(depth.max())))
        node = int(rng.choice(deep))
        path = [node]
        while path[-1] != 0:
            path.append(int(parent[path[-1]]))
        path = path[::-1]
        for step, (a, b) in enumerate(zip(path, path[1:])):
            logits[a, draft[b]] = np.float32(10.0 if step < accept else -10.0)
    if ties and V > 1:
        for r in rng.choice(T, size=max(1, T // 4), replace=False):
            logits[r, int(rng.integers(0, V))] = logits[r].max()
    return logits, parent, draft


# ------------------------------------------------- recurrent layer on a tree
def deltanet_case(T: int, H: int, d_k: int, d_v: int, seed: int, shape: str = "bushy"):
    """Inputs of a gated delta-rule layer over a draft tree of T nodes and H
    heads: (S0[H, d_v, d_k], q[T, H, d_k], k[T, H, d_k], v[T, H, d_v],
    alpha[T, H], beta[T, H], parent[T]), fp32 / int32.

    The tree shapes are those of draft_tree.  q, v ~ N(0, 1); keys N(0, 1)
    scaled to unit length (the layer's keys are normalised); decay gates
    alpha uniform in [0.9, 1); write strengths beta = sigmoid(N(0, 1)); the
    live state S0 ~ N(0, 0.5)."""
    rng = rng_for("test", seed, 8, "x")
    _logits, parent, _draft = draft_tree(T, 2, seed, shape=shape)
    q = rng.standard_normal((T, H, d_k), dtype=np.float32)
    k = rng.standard_normal((T, H, d_k), dtype=np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True).astype(np.float32)
    v = rng.standard_normal((T, H, d_v), dtype=np.float32)
    alpha = rng.uniform(0.9, 1.0, size=(T, H)).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))).astype(np.float32)
    S0 = (0.5 * rng.standard_normal((H, d_v, d_k))).astype(np.float32)
    return S0, q, k.astype(np.float32), v, alpha, beta, parent


# -------------------------------------------------------------- device draws
def stack_weight(layer: int, name: str, device="cuda"):
    """fp32 W[N, K] of one stack matrix, drawn with torch on `device`:
    N(0, 0.02) plus round(0.001*N*K) distinct entries x20."""
    import torch
    N, K = {m: (n, k) for m, n, k, _s in STACK_MATRICES}[name]
    slot = _MATRIX_ID[name]
    g = torch.Generator(device=device)
    g.manual_seed(torch_seed_for("stack", layer, slot, "W"))
    W = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    W.mul_(W_STD)
    count = int(round(STACK_W_OUTLIER_FRAC * N * K))
    go = torch.Generator(device=device)
    go.manual_seed(torch_seed_for("stack", layer, slot, "W_outlier"))
    idx = torch.randperm(N * K, generator=go, device=device)[:count]
    W.view(-1)[idx] *= STACK_W_MULT
    return W


def stack_matrix_names():
    return [m for m, *_r in STACK_MATRICES]
