"""Generated-code guards for the HIP kernels (CPU only: hipcc cross-compiles gfx950 here).

Two properties that no parity test can see but that bound the kernels' speed:

- no kernel spills to scratch (private) memory;
- no 16-byte load is issued right after a wait for every outstanding memory operation
  (``s_waitcnt vmcnt(0)``), in the row-copy kernels (which must have such loads) or any other.  That pattern means the compiler could not keep the
  thread's loads in flight together and issued them one at a time; it appeared when each load sat
  under a per-lane condition, and cost the network and unpack kernels 5-10%.
"""
import importlib.util
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_moe_route_top_amd", "csrc")


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "moe_build_flags", os.path.join(ROOT, "combine_moe_route_top_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _hipcc():
    b = _build_module()
    if not (os.path.exists(b.HIPCC) or shutil.which(b.HIPCC)):
        pytest.skip("hipcc not available")
    return b


_ASM = {}


def _device_asm(tmp_path, source):
    """gfx950 assembly of one source and the compiler's resource-usage remarks (compiled once per
    test session)."""
    if source not in _ASM:
        _ASM[source] = _compile(tmp_path, source)
    return _ASM[source]


def _compile(tmp_path, source):
    b = _hipcc()
    flags = [f for f in b.FLAGS if f not in ("-fPIC", "-shared")]
    out = os.path.join(str(tmp_path), os.path.basename(source) + ".s")
    cmd = [b.HIPCC, *flags, "--offload-device-only", "-S", "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, source), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read(), r.stderr


def _functions(asm):
    """(mangled name, instruction lines) of every kernel in the assembly."""
    for name in re.findall(r"^\s*\.type\s+(_ZN3moe\w+),@function", asm, re.M):
        i = asm.index(name + ":")
        j = asm.index(".Lfunc_end", i)
        lines = [l.strip() for l in asm[i:j].splitlines()]
        yield name, [l for l in lines if l and not l.startswith((";", "."))]


SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))


@pytest.mark.parametrize("source", SOURCES)
def test_no_kernel_spills_to_scratch(tmp_path, source):
    asm, remarks = _device_asm(tmp_path, source)
    sizes = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", remarks)]
    if not sizes:  # a source with host code only (the entry points)
        assert not list(_functions(asm)), "kernels found but no resource-usage remarks"
        return
    assert max(sizes) == 0, f"{source}: a kernel uses {max(sizes)} bytes of scratch per lane"


COPY_KERNELS = {
    "dispatch.hip": r"k_net_dispatch|k_unpack",
    "combine.hip": r"k_combine_pack|k_combine_net",
    "combine_acc.hip": r"k_acc_net",
}


@pytest.mark.parametrize("source", sorted(COPY_KERNELS))
def test_row_copy_loads_stay_in_flight(tmp_path, source):
    asm, _ = _device_asm(tmp_path, source)
    checked, serial = 0, []
    for name, lines in _functions(asm):
        if not re.search(COPY_KERNELS[source], name):
            continue
        for k, line in enumerate(lines):
            if re.match(r"(global|flat|buffer)_load_dwordx4", line):
                checked += 1
                if any(re.match(r"s_waitcnt vmcnt\(0\)", p) for p in lines[max(0, k - 2):k]):
                    serial.append(name)
    assert checked > 0, "no 16-byte loads found in the row-copy kernels"
    assert not serial, f"loads issued after a full wait in {sorted(set(serial))[:4]}"


@pytest.mark.parametrize("source", SOURCES)
def test_no_16_byte_load_waits_for_every_earlier_load(tmp_path, source):
    # the same property for every kernel, row copies or not (weighted sums, packs, prefill): a
    # 16-byte load right after a full wait would mean the loads of a thread go out one at a time
    asm, _ = _device_asm(tmp_path, source)
    serial = []
    for name, lines in _functions(asm):
        for k, line in enumerate(lines):
            if re.match(r"(global|flat|buffer)_load_dwordx4", line) and \
                    any(re.match(r"s_waitcnt vmcnt\(0\)", p) for p in lines[max(0, k - 2):k]):
                serial.append(name)
    assert not serial, f"{source}: loads issued after a full wait in {sorted(set(serial))[:4]}"


def test_lds_staged_stream_build_uses_direct_to_lds_loads(tmp_path):
    # the build option MOE_STREAM_LDS=1 stages row chunks through LDS with gfx950 direct-to-LDS
    # 16-byte loads in every row-copy kernel, spills nothing, and reads each chunk back only after
    # a wait for the loads (the compiler orders the LDS read after the direct load)
    b = _hipcc()
    flags = [f for f in b.FLAGS if f not in ("-fPIC", "-shared")]
    out = os.path.join(str(tmp_path), "dispatch_lds.s")
    cmd = [b.HIPCC, *flags, "-DMOE_STREAM_LDS=1", "-DMOE_STREAM_MAX_U=4", "--offload-device-only", "-S",
           "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "dispatch.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = open(out).read()
    sizes = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert sizes and max(sizes) == 0
    seen = 0
    for name, lines in _functions(asm):
        if not re.search(r"k_net_dispatch|k_unpack", name):
            continue
        assert not any(re.match(r"(global|flat|buffer)_load_dwordx4", l) for l in lines), name
        loads = [k for k, l in enumerate(lines) if l.startswith("global_load_lds_dwordx4")]
        reads = [k for k, l in enumerate(lines) if l.startswith("ds_read_b128")]
        assert loads and reads, name
        first_read = reads[0]
        assert any(re.match(r"s_waitcnt vmcnt\(0\)", l) for l in lines[loads[0]:first_read]), name
        seen += 1
    assert seen > 0
