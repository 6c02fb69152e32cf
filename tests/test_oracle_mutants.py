"""Planted mistakes in the oracle must fail its independent pins.

Each case copies ``oracle/qlin_oracle.c``, changes one step the way a
plausible misreading would (a reciprocal multiply for the quantizer's
division, the butterfly's strides in descending order, rounding up on
u <= frac, the two forward scales multiplied together first, a wrong Philox
multiplier, the SGD update associated another way, a swapped butterfly sign,
the scale taken as amax / 128), builds it into a temporary library with the
oracle's own compiler flags, loads it into a separate instance of the
``oracle`` module and runs the pins of ``test_oracle_replicas.py`` on it: at least one must fail.
The digests the oracle wrote itself are not among them.  Everything here runs
on the CPU; the real oracle and its library are not touched.

Passages: OneTrainer PR #1681, summary and verification paragraph (rotation
along the contraction dimension by an orthogonal block-Hadamard buffer;
per-row absmax activation quantization); mini_trainer "quantized-training"
guide, opening and update paragraphs (integer products with float scales;
stochastic requantization of the updated represented weight).
"""
import importlib.util
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_replicas as rep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qlin_oracle.c")


def _forward_scale_product(s):
    old = ("    v = v * srow[i];\n    if (op == 0) {\n        v = v * scol[j];\n")
    new = ("    if (op == 0) {\n        v = v * (srow[i] * scol[j]);\n")
    tail_old = "    return v;\n}\n\nstatic float dequant("
    tail_new = "    else\n        v = v * srow[i];\n    return v;\n}\n\nstatic float dequant("
    assert old in s and tail_old in s
    return s.replace(old, new).replace(tail_old, tail_new)


def _sub(old, new):
    def f(s):
        assert s.count(old) == 1, old
        return s.replace(old, new)
    return f


# name -> (source edit, pins that must catch it)
MUTANTS = {
    "reciprocal_division": (
        _sub("float v = rne(g[j] / s);", "float v = rne(g[j] * (1.0f / s));"),
        [rep.test_quantizer_replica_near_ties]),
    "descending_butterfly": (
        _sub("for (int h = 1; h < b; h <<= 1) {", "for (int h = b >> 1; h >= 1; h >>= 1) {"),
        [lambda o: rep.test_rotation_replica(o, 8), lambda o: rep.test_rotation_replica(o, 128)]),
    "swapped_butterfly_sign": (
        _sub("y[i + h] = lo - hi;", "y[i + h] = hi - lo;"),
        [lambda o: rep.test_rotation_replica(o, 8)]),
    "round_up_on_equal": (
        _sub("float v = f + (u < frac ? 1.0f : 0.0f);", "float v = f + (u <= frac ? 1.0f : 0.0f);"),
        [rep.test_sgd_requant_exact_ties]),
    "forward_scale_product": (
        _forward_scale_product,
        [rep.test_forward_epilogue_replica]),
    "philox_multiplier": (
        _sub("0xD2511F53u, 0xCD9E8D57u", "0xD2511F53u, 0xCD9E8D58u"),
        [rep.test_philox4x32_matches_triton]),
    "sgd_association": (
        _sub("w[j] = cur - upd;", "w[j] = s * ((float)qw[n * K + j] - upd / s);"),
        [rep.test_sgd_requant_replica]),
    "scale_divisor_128": (
        _sub("float s = amax / 127.0f;", "float s = amax / 128.0f;"),
        [rep.test_quantizer_replica_random_rows, rep.test_quantizer_replica_near_ties]),
}


def _mutant_oracle(name, edit, tmp_path):
    src = open(SRC).read()
    text = edit(src)
    assert text != src
    c = tmp_path / f"{name}.c"
    c.write_text(text)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *oracle.CFLAGS, str(c), "-o", str(so), "-lm"], check=True)
    spec = importlib.util.spec_from_file_location(f"oracle_mutant_{name}",
                                                  os.path.join(ROOT, "oracle", "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.lib(str(so))
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    edit, pins = MUTANTS[name]
    mod = _mutant_oracle(name, edit, tmp_path)
    caught = 0
    for pin in pins:
        try:
            pin(mod)
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake '{name}'"
