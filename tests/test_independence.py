"""The oracle and the product path stay apart, checked statically on the sources:

* nothing in the package (the binding, the HIP sources, the build) imports,
  includes or names the oracle;
* the oracle imports nothing of the package, not even the seeded generators
  (the tests hand it the generated values);
* outside tests/, only bench.py's CPU-baseline leg and __graft_entry__.smoke()
  reach the oracle, inside those functions."""
import ast
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "ssm_recurrent_decode_amd")


def _imports(path):
    tree = ast.parse(open(path).read(), path)
    out = []
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            out += [(a.name, node) for a in node.names]
        elif isinstance(node, ast.ImportFrom):
            out.append(((node.module or ""), node))
    return tree, out


def test_package_never_reaches_the_oracle():
    for path in glob.glob(os.path.join(PKG, "**", "*.py"), recursive=True):
        _, imps = _imports(path)
        for name, _ in imps:
            assert not name.split(".")[0] == "oracle", path
    for path in glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*")):
        text = open(path).read()
        assert not re.search(r"#\s*include\s*[<\"][^>\"]*oracle", text), path


def test_oracle_imports_nothing_of_the_package():
    for path in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        _, imps = _imports(path)
        for name, node in imps:
            top = name.split(".")[0]
            assert top not in ("ssm_recurrent_decode_amd", "torch", "bench", "tests"), (path, name)
            if isinstance(node, ast.ImportFrom) and node.level:
                assert node.level == 1, (path, name)  # only siblings inside oracle/


def _functions_importing_oracle(path):
    tree, imps = _imports(path)
    owners = set()
    for fn in ast.walk(tree):
        if isinstance(fn, (ast.FunctionDef, ast.AsyncFunctionDef)):
            for node in ast.walk(fn):
                if isinstance(node, (ast.Import, ast.ImportFrom)):
                    names = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                    if any(n.split(".")[0] == "oracle" for n in names):
                        owners.add(fn.name)
    top_level = [name for name, node in imps if name.split(".")[0] == "oracle" and node in tree.body]
    return owners, top_level


def test_only_the_allowed_legs_call_the_oracle():
    owners, top = _functions_importing_oracle(os.path.join(ROOT, "bench.py"))
    assert not top and owners <= {"_cpu_baseline", "_cpu_worker", "_cpu_spec_baseline", "_cpu_standard_baseline"}, (owners, top)
    owners, top = _functions_importing_oracle(os.path.join(ROOT, "__graft_entry__.py"))
    assert not top and owners <= {"smoke"}, (owners, top)
