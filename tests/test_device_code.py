"""Properties of the gfx950 device code, read from the compiler's own assembly
of the library's HIP sources (no GPU needed):

- no packed fp32 arithmetic (the build turns the packed-fp32-ops feature off);
- no flat (generic address space) memory instructions: flat accesses also
  count against the LDS wait counter, so an LDS read or cross-lane shuffle
  after one waits for it (KV page pointers built from page-table entries were
  generic until they were cast to the global address space);
- no kernel uses scratch (private segment) memory: register arrays that the
  compiler cannot keep in registers spill there.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from qwen3_kv_cache_amd import build as qbuild

HIP_SOURCES = [s for s in qbuild.SOURCES if s.endswith(".hip")]


def _page_define():
    from qwen3_kv_cache_amd import qdec
    return f"-DQDEC_PAGE={qdec.QDEC_PAGE}"


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if not os.path.exists(qbuild.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm")
    flags = [f for f in qbuild.FLAGS if f not in ("-fPIC", "-shared")]

    def compile_one(src):
        dst = out / (src + ".s")
        cmd = [qbuild.HIPCC, *flags, _page_define(), "--cuda-device-only", "-S",
               os.path.join(qbuild.CSRC, src), "-o", str(dst)]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return src, dst.read_text()

    with ThreadPoolExecutor(len(HIP_SOURCES)) as ex:
        return dict(ex.map(compile_one, HIP_SOURCES))


def _functions(asm):
    """(kernel symbol, body text up to its end of program) pairs."""
    out = []
    for m in re.finditer(r"^(_Z\w+):", asm, re.M):
        end = asm.find("s_endpgm", m.end())
        out.append((m.group(1), asm[m.end():end if end > 0 else len(asm)]))
    return out


def test_every_source_has_kernels(device_asm):
    for src, asm in device_asm.items():
        assert len(_functions(asm)) > 0, src


def test_no_packed_fp32_arithmetic(device_asm):
    for src, asm in device_asm.items():
        hits = re.findall(r"\bv_pk_(?:add|mul|fma)_f32\b", asm)
        assert not hits, (src, hits[:5])


def test_no_flat_memory_instructions(device_asm):
    for src, asm in device_asm.items():
        bad = [name for name, body in _functions(asm) if re.search(r"^\s+flat_(?:load|store|atomic)", body, re.M)]
        assert not bad, (src, bad[:5])


def test_no_kernel_uses_scratch(device_asm):
    for src, asm in device_asm.items():
        sizes = re.findall(r"\.amdhsa_kernel\s+(\S+)\n(?:.*\n)*?\s+\.amdhsa_private_segment_fixed_size\s+(\d+)", asm)
        assert sizes, src
        bad = [name for name, n in sizes if int(n) != 0]
        assert not bad, (src, bad[:5])
