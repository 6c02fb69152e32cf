"""Host-side logic of bench.py: the kernel-source digest that ties the committed
counter summaries to the sources they were taken on."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_only_drops_comments_keeps_literals(bench):
    src = ('int a = 1; // trailing\n/* block\n comment */ asm("s_nop 1 // kept");\n'
           "char q = '\"'; const char *s = \"/* kept */\";\n")
    assert bench.code_only(src) == ('int a = 1; asm("s_nop 1 // kept"); '
                                    "char q = '\"'; const char *s = \"/* kept */\";")


def test_digest_ignores_comments_and_layout(bench):
    csrc = os.path.join(ROOT, "w8a8_integer_linear_amd", "csrc")
    names = sorted(os.listdir(csrc))
    texts = {}
    for n in names:
        with open(os.path.join(csrc, n), encoding="utf-8") as f:
            texts[n] = f.read()
    base = bench.source_digest(lambda n: texts[n])
    assert base == bench.source_digest()
    target = next(n for n in names if n.endswith(".hip"))
    commented = dict(texts)
    commented[target] = "// a new comment\n" + texts[target].replace("\n", "\n\n", 3)
    assert bench.source_digest(lambda n: commented[n]) == base
    changed = dict(texts)
    changed[target] = texts[target] + "\nstatic int qlin_digest_probe = 1;\n"
    assert bench.source_digest(lambda n: changed[n]) != base
