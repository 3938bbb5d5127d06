"""Assumptions the kernels' source makes about the code the compiler emits,
checked on the gfx950 device assembly of every HIP source (compiled here,
no GPU needed):

- M0 (the LDS base of the direct global -> LDS loads) is written only by the
  inline-assembly load statements, each of which sets it right before its
  own global_load_lds_dwordx4 (or dword); no compiler-generated instruction uses M0,
  so the value a load statement sets cannot be clobbered between the two.
- No packed fp32 VALU instruction (v_pk_fma_f32, v_pk_mul_f32,
  v_pk_add_f32) is emitted anywhere (the sources are built with the
  packed-fp32-ops target feature off).
- The bf16 D = 64 kernels (forward band kernels and the backward kernels of
  shared projections) use no scratch memory.
"""

import os
import re
import subprocess
import tempfile

import pytest

from long_context_sparse_band_amd import build

PKG = os.path.dirname(build.LIB)


def _asm(src, out_dir):
    cmd = build.command(os.path.join(out_dir, "unused.so"))
    # Keep the compiler, arch, optimisation, feature and include flags; emit
    # the device assembly of one source instead of linking the library.
    flags = [a for a in cmd[1:] if a not in ("-shared", "-fPIC", "-o") and not a.endswith(".hip")
             and not a.endswith(".so")]
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    return subprocess.Popen([cmd[0], *flags, "--cuda-device-only", "-S", src, "-o", out],
                            stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True), out


@pytest.fixture(scope="module")
def device_asm():
    with tempfile.TemporaryDirectory() as d:
        jobs = [(_asm(s, d), s) for s in build.sources()]
        texts = {}
        for (proc, out), src in jobs:
            log, _ = proc.communicate(timeout=900)
            assert proc.returncode == 0, log[-3000:]
            texts[os.path.basename(src)] = open(out).read()
        yield texts


def _functions(text):
    """(name, body) of each kernel in an assembly listing."""
    parts = re.split(r"^(\S+):\s*;\s*@\1\s*$", text, flags=re.M)
    return [(parts[i], parts[i + 1]) for i in range(1, len(parts) - 1, 2)]


def test_m0_only_in_direct_load_statements(device_asm):
    for name, text in device_asm.items():
        in_asm = False
        block = []
        for line in text.splitlines():
            s = line.strip()
            if s == ";;#ASMSTART":
                in_asm, block = True, []
                continue
            if s == ";;#ASMEND":
                if any(re.search(r"\bm0\b", b) for b in block):
                    ops = [b.split()[0] for b in block if b and not b.startswith(";")]
                    assert ops in (["s_mov_b32", "global_load_lds_dwordx4"],
                                   ["s_add_u32", "global_load_lds_dwordx4"],
                                   ["s_mov_b32", "global_load_lds_dword"]), (name, block)
                    assert re.match(r"s_(mov_b32|add_u32)\s+m0\s*,", block[0]), (name, block)
                in_asm = False
                continue
            if in_asm:
                block.append(s)
            elif s and not s.startswith((";", ".")) and re.search(r"\bm0\b", s.split(";")[0]):
                pytest.fail(f"{name}: compiler-generated use of M0: {s}")


def test_no_packed_fp32_valu(device_asm):
    for name, text in device_asm.items():
        hits = re.findall(r"^\s*(v_pk_(?:fma|mul|add)_f32)\b", text, flags=re.M)
        assert not hits, (name, hits[:5])


def _lean_rows(fn):
    # The query side's four-wavefront instantiation (128 registers) keeps a
    # few bytes in scratch, stored before its step loop and read after it.
    return "bwd_rows_kernel" in fn and "ELi4E" in fn


def _small_spill(fn):
    # The key side with 128-key items (taken only when LFATTN_BWD_ROWS=128)
    # keeps one value in scratch, read on the gathered-global-row load path.
    return "bwd_keys_kernelILi64ELi1ELb0E" in fn


def test_d64_bf16_kernels_use_no_scratch(device_asm):
    checked = lean = 0
    for name, text in device_asm.items():
        for fn, body in _functions(text):
            d64_band = "band32_kernel" in fn and "ILi64E" in fn
            # (the key side's separate-projection instantiation, Lb1E, may spill)
            d64_bwd = "bwd_" in fn and "kernel" in fn and "ILi64E" in fn and "Lb1E" not in fn
            if not (d64_band or d64_bwd):
                continue
            checked += 1
            if _small_spill(fn):
                continue
            if _lean_rows(fn):
                # No scratch load between its first and last MFMA (the loop).
                lines = body.splitlines()
                mf = [i for i, l in enumerate(lines) if "v_mfma" in l]
                assert mf, fn
                inside = lines[mf[0]:mf[-1] + 1]
                assert not any(re.match(r"\s*scratch_load", l) for l in inside), fn
                lean += 1
                continue
            assert not re.search(r"^\s*scratch_", body, flags=re.M), fn
        for m in re.finditer(r"\.name:\s+(\S+)\n(?:.*\n)*?\s+\.private_segment_fixed_size:\s+(\d+)",
                             text):
            fn, size = m.group(1), int(m.group(2))
            if "ILi64E" in fn and ("band32_kernel" in fn or ("bwd_" in fn and "Lb1E" not in fn)):
                assert size <= (16 if _lean_rows(fn) or _small_spill(fn) else 0), (fn, size)
    assert checked >= 4 and lean == 2
