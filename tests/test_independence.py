"""The oracle and the HIP path share no code: neither imports, includes or loads the other."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _files(folder, exts):
    for dp, _, fns in os.walk(os.path.join(ROOT, folder)):
        for fn in fns:
            if fn.endswith(exts):
                yield os.path.join(dp, fn)


def test_product_never_touches_the_oracle():
    for f in _files("adam_ob_compress_amd", (".py", ".hip", ".cpp", ".h")):
        text = open(f).read()
        assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
        assert "ob_oracle" not in text and "libob_oracle" not in text, f
        assert '#include "../../oracle' not in text, f
    for f in _files("include", (".h",)):
        assert "oracle" not in open(f).read().lower(), f


def test_oracle_never_touches_the_product():
    for f in _files("oracle", (".py", ".c", ".h")):
        text = open(f).read()
        assert not re.search(r"^\s*(import|from)\s+adam_ob_compress_amd\b", text, re.M), f
        assert "libobadam" not in text and "ob_adam.h" not in text and "ob_internal" not in text, f
