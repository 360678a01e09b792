"""The device path is integer-only: no floating-point instruction in any
kernel of the attention path, checked on the gfx950 code the build produced.

Every HIP object the build writes carries its device code object; it is
unbundled and disassembled with the ROCm LLVM tools, and each kernel's
instruction stream is scanned for floating-point opcodes (f16/f32/f64
arithmetic, conversions to or from float, reciprocal, square root, exp, log).
Two kernels are float by definition and are exempt: the float32 softmax
comparator (dequantise -> softmax -> requantise) and the cache update, whose
inputs are float32 keys and values. The scan must find floating point in
them, so that a broken scan cannot pass.
"""
import os
import re
import shutil
import subprocess

import pytest

from integer_only_quantized_amd import build as B

LLVM = "/opt/rocm/llvm/bin"
TOOLS = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
FP_OP = re.compile(r"^(v_\w*_f(16|32|64)\w*|v_cvt_\w*f(16|32|64)\w*|v_rcp\w*|v_rsq\w*|v_sqrt\w*|v_exp\w*|"
                   r"v_log\w*|v_div_\w*|v_ldexp\w*|v_frexp\w*|v_fma\w*|v_mac_f\w*|v_trig\w*|v_fract\w*|"
                   r"v_pk_\w*f(16|32)\w*)$")
FLOAT_KERNELS = ("ia_fp_softmax_kernel", "ia_kv_append_kernel")
INTEGER_KERNELS = ("ia_short_kernel", "ia_long_kernel", "ia_decode_kernel", "ia_general_kernel",
                   "ia_qk_kernel", "ia_index_softmax_kernel", "ia_pv_kernel")


def _functions(obj, tmp):
    fb, host, co = (os.path.join(tmp, n) for n in ("fb.bin", "host.o", "dev.co"))
    subprocess.run([TOOLS[0], f"--dump-section=.hip_fatbin={fb}", obj, host], check=True)
    subprocess.run([TOOLS[1], "--unbundle", "--type=o", f"--input={fb}",
                    f"--targets=hipv4-amdgcn-amd-amdhsa--{B.ARCH}", f"--output={co}"], check=True)
    dis = subprocess.run([TOOLS[2], "-d", f"--mcpu={B.ARCH}", "--no-show-raw-insn", co],
                         capture_output=True, text=True, check=True).stdout
    funcs, cur = {}, None
    for line in dis.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        t = line.strip()
        if cur and t and not t.startswith((".", ";")):
            funcs[cur].append(t.split()[0])
    return funcs


@pytest.mark.skipif(not all(os.path.exists(t) for t in TOOLS), reason="needs the ROCm LLVM tools")
def test_no_floating_point_in_integer_kernels(tmp_path):
    seen, fp_seen = set(), set()
    for src in B.HIP_SOURCES:
        obj = os.path.join(B.BUILD_DIR, os.path.splitext(src)[0] + ".o")
        assert os.path.exists(obj), f"{obj} missing: build the library first"
        d = tmp_path / os.path.splitext(src)[0]
        d.mkdir()
        for name, ops in _functions(obj, str(d)).items():
            fp = sorted({o for o in ops if FP_OP.match(o)})
            kind = next((k for k in FLOAT_KERNELS + INTEGER_KERNELS if k in name), None)
            if kind in FLOAT_KERNELS:
                if fp:
                    fp_seen.add(kind)
                continue
            if kind:
                seen.add(kind)
            assert not fp, f"{name} ({src}) has floating-point instructions: {fp}"
    assert seen == set(INTEGER_KERNELS), f"kernels not found: {set(INTEGER_KERNELS) - seen}"
    assert fp_seen == set(FLOAT_KERNELS), "the scan found no floating point in the float kernels"
