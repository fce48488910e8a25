"""The run-time specialized kernels (fa_jit_code_object, hipRTC) on the CPU: they
compile for gfx950 without a GPU, contain no packed-fp32 VALU instructions (the
library's own build forbids them), do not spill, and fold the shape into constants."""

import os
import re
import shutil
import subprocess

import pytest

fa = pytest.importorskip("tiled_online_softmax_amd", reason="libfa.so not built")

OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"
READELF = "/opt/rocm/llvm/bin/llvm-readelf"

CASES = [(fa.FA_DTYPE_BF16, 128, True, 4, 16, 4096), (fa.FA_DTYPE_BF16, 64, False, 1, 2, 1000),
         (fa.FA_DTYPE_F32, 64, False, 8, 1, 1024), (fa.FA_DTYPE_F32, 16, True, 1, 1, 100)]


def _disassemble(co, tmp_path):
    path = tmp_path / "k.co"
    path.write_bytes(co)
    return subprocess.run([OBJDUMP, "-d", "--mcpu=gfx950", str(path)], capture_output=True, text=True,
                          check=True).stdout


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_specialized_code_object(case, tmp_path):
    co = fa.jit_code_object(*case)
    assert co[:4] == b"\x7fELF"
    if not os.path.exists(OBJDUMP):
        pytest.skip("llvm-objdump not available")
    asm = _disassemble(co, tmp_path)
    assert "v_mfma" in asm
    assert not re.search(r"v_pk_(add|mul|fma)_f32", asm)
    notes = subprocess.run([READELF, "--notes", str(tmp_path / "k.co")], capture_output=True, text=True).stdout
    spills = [int(x) for x in re.findall(r"\.vgpr_spill_count:\s+(\d+)", notes)]
    assert spills and max(spills) == 0


def test_shapes_give_different_code(tmp_path):
    """N is a compile-time constant: two sizes compile to different code."""
    a = fa.jit_code_object(fa.FA_DTYPE_BF16, 64, False, 1, 2, 1000)
    b = fa.jit_code_object(fa.FA_DTYPE_BF16, 64, False, 1, 2, 1024)
    assert a != b


@pytest.mark.parametrize("causal,heads,split", [(False, 192, True), (False, 193, False),
                                                (True, 384, True), (True, 385, False)])
def test_key_split_selection(causal, heads, split):
    """The bf16 forward compiles the key-split form (template argument KS = 2) exactly when
    B*H*ceil(N/128) is at most 192 workgroups, or 384 when causal; fa_fwd_specialized and
    fa_fwd make the same choice. The kernel symbol in the code object names the form."""
    co = fa.jit_code_object(fa.FA_DTYPE_BF16, 128, causal, 1, heads, 128)
    ks = re.findall(rb"fa_fwd_bf16_kernelILi128ELb[01]ELi4ELi64ELi([12])E", co)
    assert ks, "bf16 kernel symbol not found in the code object"
    assert set(ks) == {b"2" if split else b"1"}
