"""Structural checks of the product/oracle boundary (CPU only).

The oracle is test infrastructure: the product package and its native sources
never import or include it, the workload generator holds no attention arithmetic,
and bench.py touches the oracle only inside its CPU-baseline leg.  The binding
fails loudly when the native library is missing instead of falling back.
"""
import ast
import pathlib
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parents[1]
PKG = ROOT / "segmented_attention_seq_amd"


def _imports(tree):
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield node, a.name
        elif isinstance(node, ast.ImportFrom):
            yield node, node.module or ""


def test_package_never_imports_oracle():
    for path in PKG.rglob("*.py"):
        tree = ast.parse(path.read_text())
        for _, name in _imports(tree):
            assert not name.split(".")[0] == "oracle", f"{path} imports {name}"


def test_native_sources_never_reference_oracle():
    for path in list(PKG.rglob("*.hip")) + list(PKG.rglob("*.cpp")) + list(PKG.rglob("*.h")) + \
            list((ROOT / "include").rglob("*.h")):
        text = path.read_text()
        assert "oracle" not in text.lower(), f"{path} mentions the oracle"


def test_bench_uses_oracle_only_in_cpu_baseline():
    tree = ast.parse((ROOT / "bench.py").read_text())
    funcs = {n.name: n for n in ast.walk(tree) if isinstance(n, ast.FunctionDef)}
    for node, name in _imports(tree):
        if name.split(".")[0] != "oracle":
            continue
        owner = [f for f, fn in funcs.items() if fn.lineno <= node.lineno <= fn.end_lineno]
        assert owner == ["cpu_baseline"], f"oracle imported at bench.py line {node.lineno} in {owner}"


def test_oracle_never_imports_the_product():
    for path in (ROOT / "oracle").rglob("*.py"):
        tree = ast.parse(path.read_text())
        for _, name in _imports(tree):
            assert name.split(".")[0] not in ("segmented_attention_seq_amd", "torch"), f"{path} imports {name}"


def test_binding_fails_loudly_without_the_library(tmp_path):
    # a copy of the package without libakv.so must raise on import, not fall back
    dst = tmp_path / "segmented_attention_seq_amd"
    dst.mkdir()
    for f in ("__init__.py", "akv.py", "workload.py"):
        (dst / f).write_text((PKG / f).read_text())
    code = "import segmented_attention_seq_amd.akv"
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "libakv" in (r.stderr + r.stdout)


def test_binding_and_torch_share_one_hip_runtime():
    """Importing the binding first (before torch) must still map a single HIP
    runtime: the one torch loads, which libakv.so then binds to by soname."""
    code = ("import os\n"
            "from segmented_attention_seq_amd import akv\n"
            "import torch\n"
            "m = open(f'/proc/{os.getpid()}/maps').read()\n"
            "libs = {l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}\n"
            "print(len(libs), sorted(libs))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[0] == "1", r.stdout



def test_traffic_key_ignores_comments_only(tmp_path, monkeypatch):
    """bench.py reports the attention's HBM traffic only for the kernel code the
    counters were taken on: a comment edit keeps the key, a code edit changes it."""
    sys.path.insert(0, str(ROOT))
    import bench
    src = ["// header\n__global__ void k(int* p) { /* store */ p[0] = 1; }\n", "#define X 2 // two\n"]
    paths = []
    for i, text in enumerate(src):
        p = tmp_path / f"f{i}.h"
        p.write_text(text)
        paths.append(str(p))
    monkeypatch.setattr(bench, "ATTN_SRCS", paths)
    h0 = bench.attn_src_hash()
    (tmp_path / "f0.h").write_text("// other words\n__global__ void k(int* p) {\n  p[0] = 1;  // one\n}\n")
    assert bench.attn_src_hash() == h0
    (tmp_path / "f1.h").write_text("#define X 3 // two\n")
    assert bench.attn_src_hash() != h0


def test_bench_refuses_more_than_one_gpu():
    """The bench measures one GPU; asking for more exits with a message before any
    GPU or library work."""
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr

