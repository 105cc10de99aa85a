"""Properties of the split kernel's gfx950 machine code, read from the built
library's own code objects (no GPU): hand-counted waits and register spills.

The library is disassembled with the ROCm LLVM tools: the device code bundles
in the library's `.hip_fatbin` section are split, unbundled for gfx950 and
printed with llvm-objdump.
"""

import os
import re
import subprocess
import tempfile

import pytest

import mla_latent_kv_10_amd as m
from mla_latent_kv_10_amd import build as B

LLVM = "/opt/rocm/llvm/bin"
TOOLS = ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = f"hipv4-amdgcn-amd-amdhsa--{B.ARCH}"
KERNEL_RE = re.compile(r"decode_kernelILi(\d)ELb(\d)ELi(\d)ELb(\d)E")
# k-steps of 16 key dims per 32-row MFMA block: the q loads of a row group
NQ = {1: 576 // 16, 2: 512 // 16}
VMEM_LOAD = re.compile(r"^(global_load|buffer_load|flat_load)")


@pytest.fixture(scope="module")
def functions():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("library not built")
    return _decode_functions(B.LIB_PATH)


def _decode_functions(lib):
    """{(format, sparse, variant, mixed): [(address, instruction, branch target)]} of the decode kernels."""
    for t in TOOLS:
        if not os.path.exists(os.path.join(LLVM, t)):
            pytest.skip(f"{t} not found")
    text = ""
    with tempfile.TemporaryDirectory() as d:
        fat = os.path.join(d, "fat.bin")
        subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", lib],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
        starts = [i for i in range(len(data)) if data.startswith(BUNDLE_MAGIC, i)]
        assert starts, "no offload bundle in the library"
        for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
            src, co = os.path.join(d, f"b{n}.bin"), os.path.join(d, f"b{n}.co")
            open(src, "wb").write(data[a:b])
            subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--type=o", f"--targets={TARGET}",
                            f"--input={src}", f"--output={co}", "--unbundle"], check=True, capture_output=True)
            text += subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", f"--mcpu={B.ARCH}", co],
                                   check=True, capture_output=True, text=True).stdout
    funcs, base, cur = {}, {}, None
    for line in text.splitlines():
        h = re.match(r"^([0-9a-f]+) <(.*)>:", line)
        if h:
            cur = h.group(2)
            funcs[cur], base[cur] = [], int(h.group(1), 16)
            continue
        i = re.match(r"^\s+(.*?)\s*//\s*([0-9A-F]+):", line)
        if cur and i:
            target = None
            if i.group(1).startswith(("s_branch", "s_cbranch")):
                t = re.search(r"<[^+>]*\+0x([0-9a-f]+)>", line)
                target = base[cur] + int(t.group(1), 16) if t else None
            funcs[cur].append((int(i.group(2), 16), i.group(1), target))
    decode = {tuple(int(x) for x in KERNEL_RE.search(n).groups()): body
              for n, body in funcs.items() if KERNEL_RE.search(n)}
    # 3 formats x (dense, dense with position-spanning row groups, sparse) x 3 row-group sizes
    assert len(decode) == 27, sorted(decode)
    return decode


def _loops(body):
    """Backward-branch regions [target, branch] of a function."""
    return sorted({(t, a) for a, _, t in body if t is not None and t <= a})


def _count(body, lo, hi, pattern):
    return sum(1 for a, ins, _ in body if lo <= a <= hi and re.match(pattern, ins))


def test_no_register_spill_inside_a_tile_loop(functions):
    """Every innermost loop that runs MFMAs (the per-tile loop) is free of
    scratch accesses; what the compiler spills is saved and restored once per
    sequence segment, outside it."""
    for key, body in functions.items():
        loops = [r for r in _loops(body) if _count(body, r[0], r[1], r"v_mfma") > 0]
        tile_loops = [r for r in loops
                      if not any(o != r and r[0] <= o[0] and o[1] <= r[1] for o in loops)]
        assert tile_loops, key
        for lo, hi in tile_loops:
            assert _count(body, lo, hi, r"scratch_") == 0, (key, hex(lo), hex(hi))


@pytest.mark.parametrize("fmt", [1, 2])
def test_sparse_ring_wait_counts_only_later_loads(functions, fmt):
    """The sparse FP8 pipeline loads three index words into an LDS ring with
    loads the compiler does not track, then waits with vmcnt(NQ) before reading
    them: that is only sound if at least NQ VMEM loads (the q loads) are
    issued between the third ring load and the wait."""
    body = functions[(fmt, 1, 0, 0)]
    ring = [i for i, (_, ins, _) in enumerate(body) if re.match(r"^buffer_load_dword\s.*\blds\b", ins)]
    assert len(ring) >= 3
    third = ring[2]
    want = f"s_waitcnt vmcnt({NQ[fmt]})"
    wait = next(i for i in range(third, len(body)) if body[i][1] == want)
    loads = [ins for _, ins, _ in body[third + 1:wait] if VMEM_LOAD.match(ins)]
    assert len(loads) >= NQ[fmt], (len(loads), NQ[fmt])
    # and no wait in between that the count would rely on being absent
    assert not any(ins.startswith("s_waitcnt vmcnt") for _, ins, _ in body[third + 1:wait])


def test_library_is_the_one_the_binding_loads():
    assert os.path.samefile(m.lib()._name, B.LIB_PATH)


def test_race_check_build_drains_every_pipeline():
    """The race-check library waits vmcnt(0) more often in every decode kernel."""
    if not os.path.exists(B.DRAIN_LIB_PATH):
        pytest.skip("race-check library not built")
    main = _decode_functions(B.LIB_PATH)
    drain = _decode_functions(B.DRAIN_LIB_PATH)
    assert sorted(main) == sorted(drain)
    for key in main:
        n_main = sum(1 for _, ins, _ in main[key] if ins == "s_waitcnt vmcnt(0)")
        n_drain = sum(1 for _, ins, _ in drain[key] if ins == "s_waitcnt vmcnt(0)")
        assert n_drain > n_main, (key, n_main, n_drain)
