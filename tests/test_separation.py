"""The product and the oracle share nothing: no file of the package (Python
binding, PyTorch layer, HIP sources, C ABI header) imports, includes or
names the oracle, and the oracle includes nothing of the package."""
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "rmsnorm_layernorm_fwd_amd")


def _files(top, exts):
    for d, _, names in os.walk(top):
        for f in names:
            if f.endswith(exts):
                yield os.path.join(d, f)


def test_package_does_not_use_the_oracle():
    srcs = list(_files(PKG, (".py", ".hip", ".hpp", ".h"))) + list(
        _files(os.path.join(ROOT, "include"), (".h",)))
    assert len(srcs) > 10
    for p in srcs:
        with open(p, encoding="utf-8") as fh:
            text = fh.read()
        assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), p
        assert not re.search(r"#\s*include\s*[<\"][^>\"]*oracle", text), p
        assert "oracle.c" not in text and "liboracle" not in text, p


def test_oracle_does_not_use_the_package():
    srcs = list(_files(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")))
    assert srcs
    for p in srcs:
        with open(p, encoding="utf-8") as fh:
            text = fh.read()
        assert "rmsnorm_layernorm_fwd_amd" not in text, p
        assert not re.search(r"#\s*include\s*[<\"][^>\"]*(normrope|nr_device|nr_internal)", text), p
        assert "libnormrope" not in text, p
