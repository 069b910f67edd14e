"""The quantization-quality study (CPU, oracle only): on the seeded
outlier-laden workloads the random Hadamard transform must lower the error of
the quantized layer, and the wave-wide 64-block must do about as well as the
pages' 32-block.

Source of the claim: "Karpathy's Trick for Faster Local LLMs Finally Has
Proper Tooling" (blog.dailydoseofds.com), section "How Uzu optimizes bytes and
tokens per pass": a group's scale follows its largest value, and the transform
spreads an outlier over the whole block.
"""
import pytest

from oracle import quality_study as Q


@pytest.fixture(scope="module")
def rows():
    return Q.study(n_rows=128)


def _by(rows):
    out = {}
    for r in rows:
        out.setdefault(r["workload"], {})[r["transform"]] = r
    return out


def test_transform_lowers_the_layer_error(rows):
    for name, t in _by(rows).items():
        for block in (32, 64):
            assert t[block]["rel_err"] < t[None]["rel_err"], (name, block)


def test_transform_spreads_activation_outliers(rows):
    # every workload's activations carry outlier channels or heavy tails
    for name, t in _by(rows).items():
        for block in (32, 64):
            assert t[block]["act_err"] < 0.5 * t[None]["act_err"], (name, block)


def test_wave_wide_block_is_as_good(rows):
    # the 64-block spreads activation outliers further; the layer error is
    # about the same (within sampling noise on 128 output rows per workload)
    ratios = []
    for name, t in _by(rows).items():
        assert t[64]["act_err"] <= 1.05 * t[32]["act_err"], name
        assert t[64]["rel_err"] < 1.25 * t[32]["rel_err"], name
        ratios.append(t[64]["rel_err"] / t[32]["rel_err"])
    assert sum(ratios) / len(ratios) < 1.05
