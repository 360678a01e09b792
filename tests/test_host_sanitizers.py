"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

intattn_host.cpp (parameter derivation) and intattn_api.cpp (argument
validation and kernel choice) are compiled by g++ with
-fsanitize=address,undefined (any report aborts the run) together with
tests/host_sanitize_check.cpp, whose stub launchers stand in for the HIP
kernels and record which kernel family each call picks. The run derives the
integers for a seeded sweep of scale sets (compared here with the oracle's),
then checks every entry point's argument validation and kernel choice. CPU
only: no device code is built or run.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import intattn_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "integer_only_quantized_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _param_sets():
    """(D, s_q, s_k, s_v, s_o, clip, lut_size, prob_bits, lut_bits): a seeded
    sweep over every table size, entry width and probability width, plus
    scale sets at and beyond the edges of the accepted range."""
    rng = np.random.default_rng(2024)
    f32 = lambda x: float(np.float32(x))
    sets = []
    for i in range(1500):
        D = (64, 128)[i % 2]
        n = (32, 64, 128)[i % 3]
        pb = (8, 16)[(i // 3) % 2]
        lb = (16, 8)[(i // 6) % 2]
        sq, sk, sv, so = (f32(10 ** rng.uniform(-4.0, 1.5)) for _ in range(4))
        clip = f32(rng.uniform(1.0, 12.0)) if i % 5 else O.DEFAULT_CLIP
        sets.append((D, sq, sk, sv, so, clip, n, pb, lb))
    for s in (1e-6, 1e-4, 3e-4, 0.5, 1.0, 3.0, 30.0, 300.0):
        sets.append((64, f32(s), f32(s), 0.05, 0.05, O.DEFAULT_CLIP, 32, 8, 16))
    sets.append((64, 0.05, 0.05, 1e-30, 1.0, O.DEFAULT_CLIP, 32, 8, 16))
    return sets


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "host_sanitize_check"
    cmd = (["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off"] + SAN +
           ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
            os.path.join(CSRC, "intattn_host.cpp"), os.path.join(CSRC, "intattn_api.cpp"),
            os.path.join(HERE, "host_sanitize_check.cpp"), "-o", str(exe)])
    subprocess.run(cmd, check=True)
    sets = _param_sets()
    stdin = "".join(" ".join(x.hex() if isinstance(x, float) else str(x) for x in s) + "\n" for s in sets)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([str(exe)], input=stdin, capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
    assert "runtime error" not in res.stderr and "Sanitizer" not in res.stderr, res.stderr[-3000:]
    lines = res.stdout.splitlines()
    assert lines[-1] == "ok", lines[-20:]
    n_ok = 0
    for s, line in zip(sets, lines):
        D, sq, sk, sv, so, clip, n, pb, lb = s
        got = [int(t) for t in line.split()]
        try:
            prm = O.derive_params(D, sq, sk, sv, so, clip, n, pb, lb)
        except O.OracleRangeError:
            assert got[0] != 0, (s, got)
            continue
        assert got[0] == 0, (s, got)
        lut = [x * 128 for x in prm.lut] if lb == 8 else list(prm.lut)
        assert got[1:5] == [prm.idx_mul, prm.x_clip, prm.req_shift, prm.req_mul], (s, got[:5])
        assert got[5:] == lut, s
        n_ok += 1
    assert n_ok > 500, n_ok
