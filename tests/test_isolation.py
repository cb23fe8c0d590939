"""The product path and the oracle stay apart (no GPU needed).

The HIP library and its binding never import, include or load anything
under oracle/; the oracle never reaches into the package or its kernels;
the benchmark touches the oracle only inside its CPU-baseline leg; and the
binding refuses to run rather than fall back when the library is missing or
the tensors are not on the GPU."""
import ast
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "chunked_gated_delta_02_amd")


def _files(d, exts):
    out = []
    for dp, _, fs in os.walk(d):
        if "__pycache__" in dp:
            continue
        out += [os.path.join(dp, f) for f in fs if f.endswith(exts)]
    return sorted(out)


def _imports(path):
    """(module name, enclosing top-level function or None) of every import."""
    tree = ast.parse(open(path).read(), path)
    found = []

    def visit(node, fn):
        for child in ast.iter_child_nodes(node):
            f = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) and fn is None else fn
            if isinstance(child, ast.Import):
                found.extend((a.name, fn) for a in child.names)
            elif isinstance(child, ast.ImportFrom):
                base = "." * child.level + (child.module or "")
                found.append((base, fn))
                found.extend((base + "." + a.name, fn) for a in child.names)
            visit(child, f)

    visit(tree, None)
    return found


def test_package_never_imports_the_oracle():
    pys = _files(PKG, (".py",))
    assert len(pys) >= 4
    for p in pys:
        for mod, _ in _imports(p):
            assert not re.search(r"(^|\.)oracle\b", mod), (p, mod)


def test_kernels_and_header_include_nothing_of_the_oracle():
    srcs = _files(os.path.join(PKG, "csrc"), (".hip", ".h", ".cpp")) + _files(os.path.join(ROOT, "include"), (".h",))
    assert len(srcs) >= 5
    for p in srcs:
        for line in open(p):
            if line.lstrip().startswith("#include"):
                assert "oracle" not in line, (p, line)


def test_oracle_never_reaches_into_the_package():
    for p in _files(os.path.join(ROOT, "oracle"), (".py",)):
        for mod, _ in _imports(p):
            assert not mod.startswith(("chunked_gated_delta_02_amd", "tests", "bench")), (p, mod)
        text = open(p).read()
        assert "libgdr.so" not in text and "csrc" not in text, p
    for p in _files(os.path.join(ROOT, "oracle"), (".c", ".h")):
        for line in open(p):
            if line.lstrip().startswith("#include"):
                assert re.match(r'\s*#include\s*<[a-z]+\.h>', line), (p, line)


def test_bench_uses_the_oracle_only_in_its_cpu_baseline_leg():
    uses = [(m, fn) for m, fn in _imports(os.path.join(ROOT, "bench.py")) if re.search(r"(^|\.)oracle\b", m)]
    assert uses, "the CPU-baseline leg times the oracle"
    assert {fn for _, fn in uses} == {"cpu_baseline"}



def test_entry_points_use_the_oracle_only_to_build_it_and_in_smoke():
    uses = [(m, fn) for m, fn in _imports(os.path.join(ROOT, "__graft_entry__.py")) if "oracle" in m]
    assert uses
    assert {fn for _, fn in uses} <= {"build", "smoke"}


def test_missing_library_fails_loudly(tmp_path):
    from chunked_gated_delta_02_amd import _lib
    with pytest.raises(RuntimeError, match="not built"):
        _lib._open(str(tmp_path / "libgdr.so"))


def test_cpu_tensors_are_refused_not_computed():
    from chunked_gated_delta_02_amd import ops
    B, T, H, D = 1, 8, 1, 64
    q = torch.zeros(B, T, H, D, dtype=torch.bfloat16)
    beta = torch.zeros(B, T, H)
    with pytest.raises(ValueError, match="GPU"):
        ops.chunk_gdr_fwd(q, q.clone(), q.clone(), beta, beta.clone())


def test_mismatched_value_shapes_are_refused_before_any_launch(monkeypatch):
    # v (and dO) must share B, T and H with q: the kernels address them with
    # q's sizes.  The checks run on the host, before the library is reached.
    from chunked_gated_delta_02_amd import _lib, ops
    calls = []
    for name in ("gdr_chunk_fwd", "gdr_chunk_bwd", "gdr_check"):
        monkeypatch.setattr(_lib, name, lambda *a, _n=name, **k: calls.append(_n))
    B, T, H, D = 1, 8, 2, 64
    q = torch.zeros(B, T, H, D, dtype=torch.bfloat16)
    beta = torch.zeros(B, T, H)
    for bad_v in (torch.zeros(B, T - 1, H, D, dtype=torch.bfloat16),
                  torch.zeros(B, T, H - 1, D, dtype=torch.bfloat16),
                  torch.zeros(B + 1, T, H, D, dtype=torch.bfloat16)):
        with pytest.raises(ValueError, match="B, T, H"):
            ops.chunk_gdr_fwd(q, q.clone(), bad_v, beta, beta.clone())
        with pytest.raises(ValueError, match="B, T, H"):
            ops.chunk_gdr_bwd(q, q.clone(), bad_v, beta, beta.clone(), bad_v.clone())
    v = torch.zeros(B, T, H, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="do must match v"):
        ops.chunk_gdr_bwd(q, q.clone(), v, beta, beta.clone(), v[:, :4].clone())
    assert calls == []
