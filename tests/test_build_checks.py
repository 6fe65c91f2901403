"""CPU checks of the compiled device code (gfx950 assembly of this repo's own
source, built here with the library's flags).

* No decode kernel calls a device function: code off the tile loop (the
  fused append's tail wave) reads the kernel's arguments afresh from the
  kernel-argument segment, and that segment's address is only defined
  inside the kernel itself, so every such helper must be inlined.  A call (s_swappc_b64) would mean a helper was compiled
  as a separate function, reading its arguments from address 0.
* The int8 codec's tile loops keep every scalar value in registers: no
  scalar-register spill reloads (v_readlane_b32) inside the static-grid and
  plain persistent-grid tile loops, the blocks that hold the Q.K and P.V
  matrix-core instructions.
"""
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "decode_attention_int8_amd", "csrc", "q8kv.hip")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.fixture(scope="module")
def device_asm():
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_q8kv_build_flags", os.path.join(ROOT, "decode_attention_int8_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    flags = [f for f in mod.FLAGS if f not in ("-fPIC", "-shared")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "q8kv.s")
        cmd = [HIPCC] + flags + [SRC, "--cuda-device-only", "-S", "-o", out]
        subprocess.run(cmd, check=True, capture_output=True)
        text = open(out).read()
    funcs = {}
    for m in re.finditer(r"^(_Z\S+):\s*;.*?$(.*?)^\.Lfunc_end", text, re.M | re.S):
        funcs[m.group(1)] = m.group(2)
    return funcs


def test_no_device_function_calls(device_asm):
    kernels = [n for n in device_asm if "q8kv_decode_kernel" in n]
    assert len(kernels) >= 30
    calls = [n for n, body in device_asm.items() if "s_swappc_b64" in body]
    assert not calls, f"device function calls in {calls[:3]}"


def tile_loop_blocks(body):
    """Basic blocks holding matrix-core instructions: (label, text)."""
    parts = re.split(r"^(\.LBB\S+):", body, flags=re.M)
    blocks = [("entry", parts[0])] + list(zip(parts[1::2], parts[2::2]))
    return [(lab, txt) for lab, txt in blocks if "v_mfma" in txt]


@pytest.mark.parametrize("mode", ["1", "0"])
def test_int8_tile_loop_has_no_scalar_reloads(device_asm, mode):
    name = f"_ZN12_GLOBAL__N_118q8kv_decode_kernelILi128ELi{mode}ELb0ELi0ELi4EEEvNS_10DecodeArgsE"
    blocks = tile_loop_blocks(device_asm[name])
    assert blocks
    for lab, txt in blocks:
        assert "v_readlane_b32" not in txt, f"{name}: scalar spill reload in {lab}"
