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
* The LDS-staged kernels' multi-read asm blocks (a tile's LDS reads, issued
  together and waited for once) never write a read's destination over the
  address register of a later read in the same block: a read that returns
  early would otherwise redirect the reads still to be issued.
* The staged tile loops hold no compiler-inserted wait for every load in
  flight (vmcnt(0)) ahead of their LDS reads other than the kernel's own
  waits in asm.
* Every decode kernel's argument block sits where kernel_args() reads it,
  behind the leading scalar arguments (the kernel metadata's offsets).
* No int8 or FP8 decode kernel at hd 64 or 128 spills to scratch memory, and the
  persistent int8 and FP8 kernels' rolled tile loop issues a tile's P.V
  behind the next tile's K loads without waiting for them.
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
    # the kernel metadata (argument offsets and sizes), under a key no kernel has
    funcs["__metadata__"] = text[text.find("amdhsa.kernels:"):]
    return funcs


def kernel_body(device_asm, prefix):
    """The body of the one kernel whose mangled name starts with prefix (the
    template arguments; the parameter list follows)."""
    names = [n for n in device_asm if n.startswith(prefix)]
    assert len(names) == 1, (prefix, names)
    return names[0], device_asm[names[0]]


def test_decode_argument_block_behind_the_leading_arguments(device_asm):
    """kernel_args() reads a decode kernel's argument block kArgsOffset bytes
    into the argument segment, behind the leading scalar arguments: every
    decode kernel's metadata must place its by-value argument block there."""
    off = int(re.search(r"static_assert\(kArgsOffset == (\d+)", open(SRC).read()).group(1))
    n = 0
    for entry in re.split(r"\n  - \.agpr_count:", device_asm["__metadata__"]):
        m = re.search(r"\.name:\s+(\S*q8kv_decode_kernel\S*)", entry)
        if not m:
            continue
        args = re.findall(r"\.offset:\s+(\d+)\s+\.size:\s+(\d+)\s+\.value_kind:\s+by_value", entry)
        blocks = [(int(o), int(sz)) for o, sz in args if int(sz) > 8]
        assert len(blocks) == 1 and blocks[0][0] == off, (m.group(1), blocks, off)
        n += 1
    assert n >= 30


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
    name, body = kernel_body(device_asm, f"_ZN12_GLOBAL__N_118q8kv_decode_kernelILi128ELi{mode}ELb0ELi0ELi4ELb0EEEv")
    blocks = tile_loop_blocks(body)
    assert blocks
    for lab, txt in blocks:
        assert "v_readlane_b32" not in txt, f"{name}: scalar spill reload in {lab}"


def _vregs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)", tok)
    return {int(m.group(1))}


def test_multi_read_asm_blocks_keep_their_addresses(device_asm):
    checked = 0
    for name, body in device_asm.items():
        for blk in re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", body, re.S):
            reads = [l.strip().replace(",", " ").split() for l in blk.split("\n")
                     if l.strip().startswith("ds_read_b128")]
            if len(reads) < 2:
                continue
            checked += 1
            for k, r in enumerate(reads):
                dst = _vregs(r[1])
                for later in reads[k + 1:]:
                    assert not dst & _vregs(later[2]), f"{name}: {' '.join(r)} overwrites the address of {' '.join(later)}"
    assert checked >= 8


@pytest.mark.parametrize("hd,nw", [("128", "4"), ("128", "8"), ("64", "4")])
def test_staged_tile_loop_waits_are_its_own(device_asm, hd, nw):
    """Up to the last matrix-core instruction (the end of the tile loop),
    every wait for all loads in flight is one of the kernel's own asm waits."""
    name, body = kernel_body(device_asm, f"_ZN12_GLOBAL__N_118q8kv_decode_kernelILi{hd}ELi1ELb0ELi0ELi{nw}ELb1EEEv")
    lines = body.split("\n")
    assert any("global_load_lds_dwordx4" in l for l in lines)
    last_mfma = max(i for i, l in enumerate(lines) if "v_mfma" in l)
    for i in range(last_mfma):
        if "s_waitcnt vmcnt(0)" in lines[i]:
            assert ";;#ASMSTART" in lines[i - 1], f"{name}: compiler wait for every load at line {i}: {lines[i]}"


def test_int8_and_fp8_decode_kernels_do_not_spill(device_asm):
    """No int8- or FP8-codec decode kernel at hd 64 or 128 keeps a value in
    scratch memory (the rolled persistent kernels run at two waves per SIMD
    at hd 128 for that reason)."""
    names = [n for n in device_asm if re.search(r"q8kv_decode_kernelILi(64|128)ELi\dELb\dELi[01]E", n)]
    assert len(names) >= 10
    for n in names:
        assert "scratch_" not in device_asm[n], f"{n}: scratch (spill) access"


@pytest.mark.parametrize("new,codec,pv", [("0", "0", "v_mfma_f32_16x16x32_f16"),
                                          ("1", "0", "v_mfma_f32_16x16x32_f16"),
                                          ("0", "1", "v_mfma_f32_16x16x32_bf16")])
def test_rolled_tile_loop_keeps_the_next_k_half_in_flight(device_asm, new, codec, pv):
    """In the persistent int8 and FP8 kernels the P.V matrix-core
    instructions of a tile are issued behind loads of the next tile that
    they do not wait for: between the last load before them and the P.V
    instruction every wait leaves at least the next tile's four K chunks in
    flight."""
    name, body = kernel_body(device_asm, f"_ZN12_GLOBAL__N_118q8kv_decode_kernelILi128ELi0ELb{new}ELi{codec}ELi4ELb0EEEv")
    lines = body.split("\n")
    found = False
    since_load, low = None, None
    for l in lines:
        t = l.strip()
        if t.startswith("global_load_dwordx4"):
            since_load, low = True, 63
        elif since_load and t.startswith("s_waitcnt") and "vmcnt(" in t:
            low = min(low, int(re.search(r"vmcnt\((\d+)\)", t).group(1)))
        elif since_load and t.startswith(pv):
            found = found or low >= 4
            since_load = None
    assert found, f"{name}: every P.V waits for all loads in flight"
