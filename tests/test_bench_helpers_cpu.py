"""CPU checks of bench.py's host-side helpers: the digest that ties a
recorded counter row to the kernel source it was measured on."""

import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_digest_ignores_comments_and_space_only(tmp_path):
    b = _bench()
    base = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    variants = {
        "comment": "int f(int x) {\n  return x + 1;  // a different comment\n}\n// trailer\n",
        "space": "int f(int x)\n{\n    return x + 1;\n\n}\n",
        "code": "int f(int x) {\n  return x + 2;  // one more\n}\n",
        "token_split": "int f(int x) {\n  return x +1;\n}\n",
    }
    p = tmp_path / "k.hip"
    p.write_text(base)
    d0 = b.code_digest(str(p))
    got = {}
    for name, text in variants.items():
        p.write_text(text)
        got[name] = b.code_digest(str(p))
    assert got["comment"] == d0 and got["space"] == d0
    assert got["code"] != d0
    # white space between tokens is normalised, not removed: "x +1" differs
    # from "x + 1" only where a token boundary moves, which is still a change
    assert got["token_split"] != d0


def test_recorded_traffic_rows_match_the_current_sources():
    # every counter row in profiles/traffic.md was taken on the code that is
    # in the tree now (bench.py reports it only then)
    b = _bench()
    keys = {"gemm.hip": [], "elementwise.hip": []}
    for line in open(os.path.join(ROOT, "profiles", "traffic.md")):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 9 and cells[0] and cells[0][0].islower() and cells[1].isdigit():
            src = "gemm.hip" if cells[5].startswith("`void gemm_kernel") else "elementwise.hip"
            keys[src].append(cells[0])
    assert keys["gemm.hip"] and keys["elementwise.hip"]
    for src, ks in keys.items():
        for k in ks:
            assert b.recorded_traffic(k, src) is not None, (k, src)
