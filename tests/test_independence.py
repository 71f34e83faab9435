"""The oracle and the HIP path share nothing: neither imports, includes or
names the other, and the product path has no CPU fallback."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def files(d, exts):
    for dp, _, fs in os.walk(os.path.join(ROOT, d)):
        if "_build" in dp or "__pycache__" in dp:
            continue
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(dp, f)


def test_product_never_touches_the_oracle():
    for p in list(files("gram_memory_layer_amd", (".py", ".hip", ".h", ".cpp"))) + \
            list(files("include", (".h",))):
        src = open(p).read()
        assert not re.search(r"\boracle\b|engram_oracle|liboracle|\beo_", src), p


def test_oracle_never_touches_the_product():
    for p in files("oracle", (".py", ".c", ".h")):
        src = open(p).read()
        assert "gram_memory_layer_amd" not in src and "libengram" not in src, p
        assert "engram.h" not in src and "hip_runtime" not in src and "hipcc" not in src, p


def test_input_generators_hold_no_method_arithmetic():
    src = open(os.path.join(ROOT, "synth", "__init__.py")).read()
    for name in ("import gram_memory_layer_amd", "import oracle", "from oracle", "sigmoid",
                 "rsqrt", " % prime", "^="):
        assert name not in src, name
