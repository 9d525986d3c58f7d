"""The product path never touches the oracle.

The oracle (oracle/) is test infrastructure: only the tests, the smoke entry and
bench.py's cpu_baseline leg may import or call it.  These checks parse the
sources (no GPU, nothing is executed) and fail on any other reference."""
import ast
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "transformer_lm_pretraining_amd")


def oracle_refs(tree):
    """(line, enclosing top-level function or None) of every import of, or name
    reference to, the oracle package in a module's syntax tree."""
    out = []

    def visit(node, func):
        if isinstance(node, (ast.FunctionDef, ast.AsyncFunctionDef)) and func is None:
            func = node.name
        hit = False
        if isinstance(node, ast.Import):
            hit = any(a.name == "oracle" or a.name.startswith("oracle.") for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            hit = node.level == 0 and node.module is not None and \
                (node.module == "oracle" or node.module.startswith("oracle."))
        elif isinstance(node, ast.Name):
            hit = node.id == "oracle"
        if hit:
            out.append((node.lineno, func))
        for ch in ast.iter_child_nodes(node):
            visit(ch, func)

    visit(tree, None)
    return out


def parse(path):
    with open(path) as f:
        return ast.parse(f.read(), filename=path)


def test_bench_uses_the_oracle_only_in_cpu_baseline():
    refs = oracle_refs(parse(os.path.join(ROOT, "bench.py")))
    assert refs, "bench.py's cpu_baseline leg times the oracle"
    outside = [(line, fn) for line, fn in refs if fn != "cpu_baseline"]
    assert not outside, f"bench.py references the oracle outside cpu_baseline at {outside}"


@pytest.mark.parametrize("name", sorted(f for f in os.listdir(PKG) if f.endswith(".py")))
def test_package_never_references_the_oracle(name):
    refs = oracle_refs(parse(os.path.join(PKG, name)))
    assert not refs, f"{name} references the oracle at lines {[r[0] for r in refs]}"


def test_package_sources_never_name_the_oracle_directory():
    """The HIP sources and headers include nothing from oracle/."""
    hits = []
    for d in (os.path.join(PKG, "csrc"), os.path.join(ROOT, "include")):
        for f in os.listdir(d):
            with open(os.path.join(d, f), errors="replace") as fh:
                for i, line in enumerate(fh, 1):
                    if "#include" in line and "oracle" in line:
                        hits.append((f, i))
    assert not hits, hits


def test_the_guard_sees_a_planted_reference():
    """A planted import in a function other than cpu_baseline is caught."""
    src = "def cpu_baseline():\n    import oracle\n\ndef main():\n    import oracle\n    oracle.lr_at(1)\n"
    refs = oracle_refs(ast.parse(src))
    assert [(l, f) for l, f in refs if f != "cpu_baseline"] == [(5, "main"), (6, "main")]
