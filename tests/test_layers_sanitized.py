"""The per-layer config resolvers (host C++, csrc/ar_layers.cpp) built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer into a small driver
(tests/layers_driver.cpp), run on the rule sets of test_layer_config.py plus
malformed inputs, and compared with the oracle's resolution. A sanitizer report
fails the run (-fno-sanitize-recover, non-zero exit). CPU only."""
import os
import shutil
import subprocess

import pytest

import oracle as O
from test_layer_config import DEF, NAMES, RULES

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "autoround_signsgd_rounding_amd", "csrc", "ar_layers.cpp")
DRIVER = os.path.join(HERE, "layers_driver.cpp")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("asan") / "layers_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), SRC, DRIVER, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _rule_lines(rules):
    return [f"R\t{key}\t{cfg.get('bits', -1)}\t{cfg.get('group_size', 0)}\t"
            f"{int(cfg['sym']) if 'sym' in cfg else -1}" for key, cfg in rules]


def _run(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                       env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    return r.stdout.splitlines()


def _expect(fn):
    try:
        b, g, s = fn()
        return f"{b} {g} {int(s)}"
    except ValueError:
        return "ERR 1"


def test_layer_rules_under_sanitizers(driver):
    lines = _rule_lines(RULES) + [f"D\t{DEF[0]}\t{DEF[1]}\t{int(DEF[2])}"]
    want = []
    for q in (1, 0):
        for name in NAMES:
            lines.append(f"L\t{q}\t{name}")
            want.append(_expect(lambda: O.resolve_layer_config(RULES, DEF, bool(q), name)))
    fused = [("m.qk", ["m.q_proj", "m.k_proj"]), ("m.qkv_proj", ["m.q_proj", "m.k_proj",
                                                                "m.v_proj"]),
             ("e.experts", None), ("f.experts", None), ("model.layers.0.mlp", None),
             ("experts", [])]
    for layer, subs in fused:
        n = -1 if subs is None else len(subs)
        lines.append("\t".join(["F", "1", layer, str(n)] + list(subs or [])))
        want.append(_expect(lambda: O.resolve_fused_config(RULES, DEF, True, layer, subs)))
    assert _run(driver, lines) == want


def test_malformed_inputs_under_sanitizers(driver):
    """Keys that are long, hold every pattern character, or do not compile;
    names that are empty or long; an empty rule list."""
    long_name = "model." + "layers." * 400 + "q_proj"
    rules = [("(" * 50, {"bits": 2}), ("[", {"bits": 3}), ("a{2,1}", {"bits": 2}),
             (r"\\", {"bits": 8}), ("*+?^$()[]{}|\\", {"bits": 8}),
             (r"model\.(layers\.)+q_proj", {"bits": 3, "group_size": 32}),
             ("", {"sym": True}), (long_name, {"bits": 2})]
    names = ["", "x", long_name, "model.layers.q_proj", "(((", "\\"]
    lines = [f"D\t{DEF[0]}\t{DEF[1]}\t{int(DEF[2])}"]
    want = []
    for name in names:     # no rules yet
        lines.append(f"L\t1\t{name}")
        want.append(_expect(lambda: O.resolve_layer_config([], DEF, True, name)))
    lines += _rule_lines(rules)
    for q in (1, 0):
        for name in names:
            lines.append(f"L\t{q}\t{name}")
            want.append(_expect(lambda: O.resolve_layer_config(rules, DEF, bool(q), name)))
    lines.append("F\t1\tmodel\t-1")
    want.append(_expect(lambda: O.resolve_fused_config(rules, DEF, True, "model")))
    assert _run(driver, lines) == want
