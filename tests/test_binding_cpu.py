"""The Python binding has no CPU path: every entry point refuses host tensors with an error
instead of computing anything (CPU only; the library loads without a GPU)."""
import pytest
import torch

import fp8_mla_split_amd as mla


def _cpu(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def test_every_entry_point_refuses_host_tensors():
    q8 = _cpu(1, 1, 16, 576, dtype=torch.uint8)
    pool = _cpu(1, 64, 576, dtype=torch.uint8)
    table = _cpu(1, 1, dtype=torch.int32)
    lens = _cpu(1, dtype=torch.int32)
    po = _cpu(1, 4, 16, 512, dtype=torch.float16)
    pl = _cpu(1, 4, 16)
    calls = [
        lambda: mla.quantize_fp8_sat(_cpu(64), 1.0),
        lambda: mla.quantize_fp8_sat_dynamic(_cpu(64)),
        lambda: mla.quantize_fp8_sat_dynamic(_cpu(64, dtype=torch.bfloat16)),
        lambda: mla.kv_append_fp8_sat(_cpu(1, 1, 576), pool, table, lens, 1.0),
        lambda: mla.kv_append_rope_fp8_sat(_cpu(1, 1, 576), pool, table, lens, 1.0,
                                           _cpu(64, 32), _cpu(64, 32)),
        lambda: mla.decode_noalloc(q8, pool, table, lens, 1.0, 1.0, 0.07, 64, 4),
        lambda: mla.decode_splitkv(q8, pool, table, lens, 1.0, 1.0, 0.07, 64, 4, 0),
        lambda: mla.splitkv_combine(po, pl, 1, 16, 1.0),
        lambda: mla.splitkv_combine_partial(po, pl, 1, 16, _cpu(1, 16, 512,
                                                                dtype=torch.float16),
                                            _cpu(1, 16)),
    ]
    for call in calls:
        with pytest.raises(ValueError):
            call()


def test_status_codes_are_named():
    assert mla.status_string(0) == "MLA_OK"
    assert mla.status_string(3) == "MLA_ERR_WORKSPACE"
    err = mla.MLAError(2, "where")
    assert "MLA_ERR_UNSUPPORTED" in str(err) and err.code == 2


def test_the_product_never_imports_the_oracle():
    """The oracle is test infrastructure: no module of the package or of the input generators
    imports it, and the two top-level scripts import it only inside the functions allowed to
    (the benchmark's CPU baseline and the smoke check)."""
    import ast
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

    def oracle_imports(tree):
        for node in ast.walk(tree):
            if isinstance(node, ast.Import) and any(a.name.split(".")[0] == "oracle"
                                                    for a in node.names):
                yield node
            if isinstance(node, ast.ImportFrom) and (node.module or "").split(".")[0] == "oracle":
                yield node

    for pkg in ("fp8_mla_split_amd", "synthetic"):
        for dirpath, _, files in os.walk(os.path.join(root, pkg)):
            for f in files:
                if f.endswith(".py"):
                    tree = ast.parse(open(os.path.join(dirpath, f)).read())
                    assert not list(oracle_imports(tree)), os.path.join(dirpath, f)
    for script, allowed in (("bench.py", {"cpu_baseline"}), ("__graft_entry__.py", {"smoke"})):
        tree = ast.parse(open(os.path.join(root, script)).read())
        inside = set()
        for fn in ast.walk(tree):
            if isinstance(fn, ast.FunctionDef) and list(oracle_imports(fn)):
                inside.add(fn.name)
        total = len(list(oracle_imports(tree)))
        nested = sum(len(list(oracle_imports(fn))) for fn in ast.walk(tree)
                     if isinstance(fn, ast.FunctionDef) and fn.name in allowed)
        assert inside <= allowed and total == nested, (script, inside)


def test_a_package_without_its_library_fails_loudly(tmp_path):
    """No fallback: a copy of the package without libmla.so raises on first use, naming the
    build step, rather than computing anything another way."""
    import os
    import shutil
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    dst = tmp_path / "fp8_mla_split_amd"
    shutil.copytree(os.path.join(root, "fp8_mla_split_amd"), dst,
                    ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    code = ("import fp8_mla_split_amd as m\n"
            "try:\n"
            "    m.decode_splitkv\n"
            "except ImportError as e:\n"
            "    print('IMPORT-ERROR', e)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True,
                       text=True, timeout=300)
    assert "IMPORT-ERROR" in r.stdout and "fp8_mla_split_amd.build" in r.stdout, r.stdout + r.stderr
