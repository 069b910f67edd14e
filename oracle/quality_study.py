"""Quantization error with and without the random Hadamard transform, for the
pages' 32-value block and the wave-wide 64-value block (CPU, oracle only).

TEST INFRASTRUCTURE / measurement script: it runs the oracle on the seeded
synthetic workloads and prints a table; nothing here is on the product path.

    python -m oracle.quality_study            # from the repository root

Source of the claim measured: "Karpathy's Trick for Faster Local LLMs Finally
Has Proper Tooling" (blog.dailydoseofds.com), section "How Uzu optimizes bytes
and tokens per pass": one scale per group is sized to the group's largest
magnitude, so a few large values leave the small ones few levels; the
transform mixes every value of a block into every position, turning one
outlier into many moderate values, and is exactly reversible, so only the
rounding changes.

For each workload and transform (none; block 32; block 64) the layer is
quantized exactly as the library does it -- int8 per-token activations,
W4 asymmetric per group or W8 symmetric per row, exact integer partial sums,
fp64 output -- and compared with the unquantized fp64 product x . W^T:

    rel_err = ||y_q - x W^T||_F / ||x W^T||_F

plus the two operands' own errors (normwise, of the dequantized rotated
operand against the rotated one; rotation preserves the norm).  "none" skips
the sign flip and the Hadamard and keeps the activation scale sigma.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import svg_oracle as O

F32 = np.float32


def _rotate(a, signs, block):
    return np.asarray(a, F32) if block is None else O.rht(a, signs, F32, block)


def layer_error(x, W, signs, fmt, group, block):
    """(rel_err of y, act rel_err, weight rel_err) for one transform choice
    (block None = no transform)."""
    ux = _rotate(x, signs, block)
    uw = _rotate(W, signs, block)
    qx, sx = O.act_quant_i8(ux, block or 1)     # scale carries 1/block (1: no transform)
    scale_back = block or 1                     # sx * block = sigma
    act_err = (np.linalg.norm(qx.astype(np.float64) * (sx.astype(np.float64) * scale_back)[:, None] - ux)
               / np.linalg.norm(ux.astype(np.float64)))
    if fmt == "w8":
        q, s = O.quant_w8(uw)
        wdq = q.astype(np.float64) * s.astype(np.float64)[:, None]
        y = O.w8a8_output(sx, O.w8_partials(qx, q), s)
    else:
        q, s, z = O.quant_w4(uw, group)
        G = W.shape[1] // group
        wdq = ((q.astype(np.float64).reshape(-1, G, group) - z.astype(np.float64)[:, :, None])
               * s.astype(np.float64)[:, :, None]).reshape(W.shape)
        y = O.w4a8_output(sx, O.w4_group_partials(qx, q, z, group), s)
    w_err = np.linalg.norm(wdq - uw) / np.linalg.norm(uw.astype(np.float64))
    y_ref = x.astype(np.float64) @ W.astype(np.float64).T
    return float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref)), float(act_err), float(w_err)


def workloads(n_rows=512):
    """The seeded stand-ins of the pages' workloads (synth), with weight
    matrices cut to n_rows output rows so the study runs in seconds."""
    import synth
    out = []
    for name in ("single_1k", "decode_12k"):
        x, W, signs, spec = synth.single_inputs(name)
        out.append((name, x, W[:n_rows], signs, spec["fmt"], spec["group"]))
    for name, fmt, group in (("stack_w4g64", "w4_z16", 64), ("stack_w8", "w8", 0),
                             ("stack_w4g128", "w4_z16", 128)):
        x = synth.stack_acts(name, 0, "attn_in", M=16)
        signs = synth.stack_signs(0, "attn_in")
        rng = synth.rng_for("stack", 0, 0, "W")
        W = synth.normal_weights(n_rows, x.shape[1], rng, outlier_frac=1e-3, mult=20.0)
        out.append((name, x, W, signs, fmt, group))
    return out


def study(n_rows=512):
    rows = []
    for name, x, W, signs, fmt, group in workloads(n_rows):
        for block in (None, 32, 64):
            e, ea, ew = layer_error(x, W, signs, fmt, group, block)
            rows.append(dict(workload=name, fmt=fmt, group=group, transform=block, rel_err=e,
                             act_err=ea, weight_err=ew))
    return rows


def main(argv=None):
    rows = study()
    print("| workload | weights | transform | output rel. error | activation error | weight error |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        t = "none" if r["transform"] is None else f"RHT, block {r['transform']}"
        wf = "W8" if r["fmt"] == "w8" else f"W4 g{r['group']}"
        print(f"| {r['workload']} | {wf} | {t} | {r['rel_err']:.4f} | {r['act_err']:.4f} | {r['weight_err']:.4f} |")
    return 0


if __name__ == "__main__":
    sys.exit(main())
