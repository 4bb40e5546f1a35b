"""The oracle and the product path stay apart (CPU).

The fp64 oracle is test infrastructure: the package never imports it, the
oracle never imports the package or torch, the native sources include
nothing from it, and without the built library the package refuses to load
instead of computing anything some other way.
"""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "post_weight_quantization_amd")


def _sources(folder, exts):
    for dirpath, _, files in os.walk(folder):
        if "__pycache__" in dirpath:
            continue
        for f in files:
            if f.endswith(exts):
                yield os.path.join(dirpath, f)


def test_package_sources_never_name_the_oracle():
    for path in _sources(PKG, (".py", ".hip", ".h", ".cpp")):
        text = open(path, encoding="utf-8").read()
        assert not re.search(r"\b(import|from)\s+oracle\b", text), path
        assert "oracle/" not in text and "oracle." not in text, path


def test_oracle_never_imports_the_package_or_torch():
    for path in _sources(os.path.join(ROOT, "oracle"), (".py",)):
        text = open(path, encoding="utf-8").read()
        assert "post_weight_quantization_amd" not in text, path
        assert not re.search(r"^\s*(import|from)\s+torch\b", text, re.M), path


def test_importing_the_package_loads_no_oracle():
    code = ("import sys; import post_weight_quantization_amd, post_weight_quantization_amd.api, "
            "post_weight_quantization_amd.layer, post_weight_quantization_amd.capture; "
            "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]; "
            "print(bad); sys.exit(1 if bad else 0)")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr


def test_missing_library_fails_loudly():
    code = "import post_weight_quantization_amd._native"
    env = dict(os.environ, KQ_LIB_PATH=os.path.join(ROOT, "no_such_dir", "libkq.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "not built" in r.stderr


def _oracle_imports_by_function(path):
    import ast
    tree = ast.parse(open(path, encoding="utf-8").read())
    found = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            # the outermost function a statement sits in
            name = child.name if fn is None and isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else fn
            if isinstance(child, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in child.names):
                found.append(name)
            if isinstance(child, ast.ImportFrom) and (child.module or "").split(".")[0] == "oracle":
                found.append(name)
            visit(child, name)

    visit(tree, None)
    return found


def test_bench_and_entry_use_the_oracle_only_where_allowed():
    """bench.py reaches the oracle only from its CPU-baseline leg, the entry
    module only from smoke()."""
    assert set(_oracle_imports_by_function(os.path.join(ROOT, "bench.py"))) == {"cpu_baseline"}
    assert set(_oracle_imports_by_function(os.path.join(ROOT, "__graft_entry__.py"))) <= {"smoke"}


def test_every_source_is_built_for_gfx950_without_packed_fp32():
    import importlib.util
    spec = importlib.util.spec_from_file_location("kq_build", os.path.join(PKG, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    hip = {f for f in os.listdir(os.path.join(PKG, "csrc")) if f.endswith(".hip")}
    assert hip == set(b.SOURCES) | set(b.PEAKS_SOURCES)
    flags = " ".join(b.FLAGS)
    assert "--offload-arch=gfx950" in flags
    assert "-Xclang -target-feature -Xclang -packed-fp32-ops" in flags
