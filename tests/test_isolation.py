"""The oracle and the product path stay apart: no source of the HIP library,
its header or its binding names the oracle; the oracle's sources use
nothing of the package or the library; and the three places allowed to run
the oracle (the tests, the smoke check and the bench's CPU baseline) reach
it only from inside those functions."""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "dac_vocoder_decoding_amd")


def _sources(top, exts):
    for d, _, files in os.walk(top):
        if "__pycache__" in d or "_build" in d:
            continue
        for f in files:
            if f.endswith(exts):
                yield os.path.join(d, f)


def _imports(path):
    tree = ast.parse(open(path).read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            yield from (a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_product_sources_never_name_the_oracle():
    """The seeded input generators (inputs.py) serve both sides and may
    mention the oracle in prose; they import neither side's arithmetic."""
    paths = list(_sources(PKG, (".py", ".hip", ".h", ".cpp"))) + list(_sources(os.path.join(ROOT, "include"), (".h",)))
    assert any(p.endswith("runtime.hip") for p in paths)
    for p in paths:
        if p.endswith("inputs.py"):
            assert not any(m.split(".")[0] == "oracle" for m in _imports(p)), p
            continue
        assert not re.search(r"\boracle\b", open(p).read(), re.I), p


def test_oracle_sources_use_nothing_of_the_product():
    for p in _sources(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")):
        if p.endswith(".py"):
            assert not any(m.split(".")[0] == "dac_vocoder_decoding_amd" for m in _imports(p)), p
            continue
        text = open(p).read()
        assert "vocoder.h" not in text and "libvocoder" not in text and "dac_vocoder" not in text, p
        assert not re.findall(r'#include\s+"', text), p      # system headers only


def _oracle_imports(path):
    """(enclosing top-level function or None) of every import of the oracle."""
    tree = ast.parse(open(path).read())
    found = []
    for top in tree.body:
        for node in ast.walk(top):
            if isinstance(node, (ast.Import, ast.ImportFrom)):
                names = [getattr(node, "module", None) or ""] + [a.name for a in node.names]
                if any(n.split(".")[0] == "oracle" for n in names):
                    found.append(top.name if isinstance(top, ast.FunctionDef) else None)
    return found


def test_oracle_reached_only_from_the_allowed_functions():
    assert set(_oracle_imports(os.path.join(ROOT, "bench.py"))) == {"cpu_baseline"}
    assert set(_oracle_imports(os.path.join(ROOT, "__graft_entry__.py"))) <= {"build", "smoke"}
