"""Checks on the gfx950 assembly of the kernels (CPU only: hipcc cross-compiles).

Buffer loads that write LDS directly count against vmcnt.  A barrier that
publishes tiles to the other waves of the workgroup must therefore be preceded
by a wait that drains vmcnt; otherwise a wave can read a K or V tile while it
is still arriving.  This compiler has dropped that wait at a barrier heading a
loop, which showed on the GPU only as sporadic rows with a wrong LSE, so the
property is checked on the generated code for every kernel instantiation.
"""
import re

import pytest

from exact_attention_65_amd import build as fabuild


@pytest.fixture(scope="module")
def asm() -> str:
    return fabuild.device_asm("fa_fwd.hip")


@pytest.fixture(scope="module")
def bwd_asm() -> str:
    return fabuild.device_asm("fa_bwd.hip")


def _kernels(text: str):
    """(name, body) of every kernel in the assembly."""
    out = []
    for m in re.finditer(r"^(_ZN2fa\w*kernel\w*):", text, re.M):
        start = m.end()
        end = text.find(".Lfunc_end", start)  # blocks may follow an s_endpgm
        out.append((m.group(1), text[start:end]))
    return out


def _barrier_waits(body: str):
    """For every s_barrier after the first LDS-writing buffer load: whether the
    closest s_waitcnt before it (with no memory instruction in between) drains vmcnt."""
    lines = [ln.strip() for ln in body.splitlines() if ln.strip() and not ln.strip().startswith(";")]
    seen_dma = False
    res = []
    for i, ln in enumerate(lines):
        if ln.startswith("buffer_load") and ln.endswith(" lds"):
            seen_dma = True
        if ln.startswith("s_barrier") and seen_dma:
            ok = False
            for prev in reversed(lines[max(0, i - 12):i]):
                if prev.startswith("s_waitcnt"):
                    ok = "vmcnt(0)" in prev or prev.split()[1:] == ["0"]
                    break
                if prev.startswith(("buffer_", "global_", "ds_")):
                    break
            res.append((i, ok))
    return res


def test_bf16_kernels_present(asm):
    names = [n for n, _ in _kernels(asm)]
    assert sum("fwd_bf16" in n and "rows16" not in n for n in names) == 16, names
    assert sum("fwd_f16" in n and "rows16" not in n for n in names) == 16, names
    assert sum("rows16_kernel" in n for n in names) == 28, names
    assert sum("rows16x8_kernel" in n for n in names) == 4, names
    assert sum("combine" in n for n in names) == 8, names


def test_every_tile_barrier_drains_vmcnt(asm):
    kernels = [(n, b) for n, b in _kernels(asm) if "fwd_bf16" in n or "fwd_f16" in n]
    assert len(kernels) == 64
    for name, body in kernels:
        waits = _barrier_waits(body)
        assert waits, f"{name}: no barrier after a tile load"
        bad = [i for i, ok in waits if not ok]
        assert not bad, f"{name}: barrier(s) at asm line(s) {bad} do not wait for the LDS tile loads"


def test_backward_kernels_present(bwd_asm):
    names = [n for n, _ in _kernels(bwd_asm)]
    # (bf16, fp16) x D (64, 96, 128) x causal for each of the three tile kernels (dq, dk/dv, both in
    # one grid), and (bf16, fp16) x D for the Delta kernel; at D = 256 (bf16, fp16) x causal for the
    # dq kernel and the 16-key dk/dv kernel
    assert sum("bwd_dq" in n for n in names) == 16, names
    assert sum("bwd_dkdv_kernel" in n for n in names) == 12, names
    assert sum("bwd_dkdv16_kernel" in n for n in names) == 4, names
    assert sum("bwd_fused" in n for n in names) == 12, names
    assert sum("bwd_delta" in n for n in names) == 6, names


def test_backward_tile_barriers_drain_vmcnt(bwd_asm):
    # every backward kernel but the Delta one streams tiles through LDS
    for name, body in [(n, b) for n, b in _kernels(bwd_asm) if "bwd_delta" not in n]:
        waits = _barrier_waits(body)
        assert waits, f"{name}: no barrier after a tile load"
        bad = [i for i, ok in waits if not ok]
        assert not bad, f"{name}: barrier(s) at asm line(s) {bad} do not wait for the LDS tile loads"


def test_backward_kernels_do_not_spill(bwd_asm):
    for m in re.finditer(r"\.name:\s+(_ZN2fa\w*bwd\w*)\s.*?\.vgpr_spill_count:\s+(\d+)", bwd_asm, re.S):
        assert int(m.group(2)) == 0, m.group(1)


@pytest.fixture(scope="module")
def fp8_asm() -> str:
    return fabuild.device_asm("fa_fp8.hip")


def test_fp8_kernels_barriers_drain_vmcnt_and_do_not_spill(fp8_asm):
    kernels = _kernels(fp8_asm)
    # D 64 and 128 x causal on the 32-row kernel, D = 256 x causal on the 16-row one
    assert sum("fp8_kernel" in n for n, _ in kernels) == 4, [n for n, _ in kernels]
    assert sum("fp8_rows16_kernel" in n for n, _ in kernels) == 2, [n for n, _ in kernels]
    for name, body in kernels:
        waits = _barrier_waits(body)
        assert waits, f"{name}: no barrier after a tile load"
        bad = [i for i, ok in waits if not ok]
        assert not bad, f"{name}: barrier(s) at asm line(s) {bad} do not wait for the LDS tile loads"
    # no FP8 kernel spills a register
    for m in re.finditer(r"\.name:\s+(_ZN2fa\w*fp8\w*)\s.*?\.vgpr_spill_count:\s+(\d+)", fp8_asm, re.S):
        assert int(m.group(2)) == 0, m.group(1)


@pytest.mark.parametrize("source", ["fa_fwd.hip", "fa_bwd.hip", "fa_fp8.hip"])
def test_no_kernel_uses_scratch_memory(source):
    """Register arrays that the compiler cannot keep in registers go to scratch
    memory, silently and at a large cost (it happened at head dimension 256)."""
    text = fabuild.device_asm(source)
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)\n(?:.*\n){0,40}?\s+\.name:\s+(\S+)", text)
    assert sizes, "no kernel metadata found"
    assert all(int(n) == 0 for n, _ in sizes), [(k, n) for n, k in sizes if int(n)]
