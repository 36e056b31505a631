"""The oracle and the product path share no code: neither imports the other."""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def imported_modules(path):
    tree = ast.parse(open(path).read(), filename=path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            if node.level == 0 and node.module:
                yield node.module


def py_files(d):
    for base, _, files in os.walk(os.path.join(ROOT, d)):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(base, f)


def test_oracle_imports_nothing_from_the_product():
    for p in py_files("oracle"):
        for m in imported_modules(p):
            assert not m.startswith("weight_merge_amd"), (p, m)
            assert m.split(".")[0] in {"numpy", "__future__", "math", "typing"} or m.startswith("."), (p, m)


def test_product_never_imports_the_oracle():
    for p in py_files("weight_merge_amd"):
        for m in imported_modules(p):
            assert not m.startswith("oracle"), (p, m)
        src = open(p).read()
        for pat in ("import oracle", "from oracle", "__import__(\"oracle", "import_module(\"oracle"):
            assert pat not in src, (p, pat)
