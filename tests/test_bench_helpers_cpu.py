"""CPU checks of bench.py's host-side helpers and of the committed profile
summaries: the digest that ties a recorded counter row to the kernel source
it was measured on, the algorithmic bytes and ratios of those rows, and the
kernel-trace summary's FLOP arithmetic and agreement with the live timing of
the same run."""

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


def _algorithmic_bytes(key):
    """Bytes a kernel must move at least, from the sizes in its traffic key:
    E4M3 codes 1 byte, BF16 2; the fused gate/up kernel writes its SwiGLU
    output as codes, the down GEMM writes BF16."""
    name, dims = key.rsplit("_", 1)
    d = [int(v) for v in dims.split("x")]
    if name == "gate_up_swiglu_exact":
        M, I, H = d
        return M * H + 2 * I * H + M * I
    if name == "down_exact":
        M, N, K = d
        return M * K + N * K + 2 * M * N
    R, C = d
    per = {"quant_static": 3, "rw_ceiling_quant_mix": 3, "silu_mul": 5, "silu_mul_1in": 5,
           "rw_ceiling_silu_mix": 5, "amax": 2}[name]
    return per * R * C


def test_committed_traffic_rows_add_up():
    # each row's algorithmic bytes follow from its sizes, and its ratio
    # column from its byte columns
    rows = 0
    for line in open(os.path.join(ROOT, "profiles", "traffic.md")):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 9 and cells[0] and cells[0][0].islower() and cells[1].isdigit():
            fetch, write, alg = int(cells[1]), int(cells[2]), int(cells[3])
            assert alg == _algorithmic_bytes(cells[0]), cells[0]
            assert abs((fetch + write) / alg - float(cells[8])) < 1e-3, cells[0]
            rows += 1
    assert rows >= 8


def test_kernel_trace_summary_agrees_with_the_live_roofline():
    # the committed trace of the headline kernel: its FLOP count is the
    # gated MLP's 2 x 2*M*I*H, its TFLOP/s follows from the trace average,
    # and the live HIP-event figure of the same run lies within 5% of it
    import re
    text = open(os.path.join(ROOT, "profiles", "large_mlp_M16384_H5120_I25600_kernel_trace.md")).read()
    m = re.search(r"([\d.]+) µs average over \d+ launches in this trace -> ([\d.]+) TFLOP/s for its "
                  r"2 x 2MIH = ([\d.e+]+) FLOP", text)
    assert m, "dominant-kernel line not found"
    avg_us, tflops, flops = float(m.group(1)), float(m.group(2)), float(m.group(3))
    M, H, I = 16384, 5120, 25600
    assert abs(flops / (2 * 2 * M * I * H) - 1) < 1e-4
    assert abs(flops / (avg_us * 1e-6) / 1e12 - tflops) < 0.1
    live = re.search(r"fused kernel ([\d.]+) µs per launch", text)
    assert live, "live roofline line not found"
    assert abs(float(live.group(1)) / avg_us - 1) < 0.05
