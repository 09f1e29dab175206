"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

A sanitized build of oracle/moe_oracle.c (gcc -fsanitize=address,undefined,
every finding fatal) is loaded into a child Python process in place of the
normal build, which then runs the whole layer on small inputs of every mode:
fp32, bf16 with a clamp, capacity drops, sigmoid and sqrt-softplus gating,
MXFP4 weights with scale codes at the ends of the e8m0 range, MXFP8
activations and a shared expert. The child exits non-zero on any finding.
(The oracle's pin tests, run the same way by hand, pass too.)"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, ROOT)
import numpy as np
import oracle
oracle._SO = SO
oracle.build = lambda force=False: SO
from mixture_experts_layer_25_amd import synthetic as syn

cases = [
    syn.CONFIGS["tiny_fp32"],
    syn.small_variant(syn.CONFIGS["mixtral"], T=40, D=64, F=96),
    syn.small_variant(syn.CONFIGS["capacity"], T=60, D=64, F=64),
    syn.Config("sig", T=33, D=64, E=6, k=3, F=32, gating=syn.GATE_SIGMOID, renorm=1,
               bias="normal", bias_sigma=0.3),
    syn.small_variant(syn.CONFIGS["fine384_mxfp4"], T=24, D=64, F=64, E=16, shared_F=32),
    syn.small_variant(syn.CONFIGS["fine384_mxfp4_a8"], T=24, D=64, F=64, E=16, shared_F=32),
]
for cfg in cases:
    inp = syn.make_inputs(cfg)
    if syn.is_mx(cfg.wdt):
        inp.S_gate[:, 0, 0:4] = 0
        inp.S_gate[:, 0, 4:8] = 254
        inp.W_gate[:, 0, 4:8, :] = 0
    ref = oracle.forward(inp)
    assert np.isfinite(ref["y_exact"]).all(), cfg.name
    print("ok", cfg.name, flush=True)
"""


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_asan_and_ubsan():
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("sanitizer runtimes not installed")
    with tempfile.TemporaryDirectory() as d:
        so = os.path.join(d, "liboracle_san.so")
        subprocess.check_call([
            "gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
            "-fno-omit-frame-pointer", "-march=x86-64-v3", "-ffp-contract=off",
            "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
            os.path.join(ROOT, "oracle", "moe_oracle.c"), "-o", so, "-lm"])
        env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
                   ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
        code = f"ROOT = {ROOT!r}\nSO = {so!r}\n" + CHILD
        p = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True,
                           text=True, timeout=600)
        assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-4000:]
        assert p.stdout.count("ok ") == 6
