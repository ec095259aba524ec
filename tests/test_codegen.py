"""CPU-only checks of the machine code hipcc makes for the prefill gate/up
and down kernels (csrc/ffn_dma.hip), and for the tiled kernel on int8 codes
(csrc/ffn_bf16.hip, last test), compiled with the exact flags the build uses.

Their main loop is scheduled by hand; the properties its speed rests on are
properties of the generated gfx950 code, so they are checked there: every
MFMA accumulates in place (destination = accumulator input), no accumulator
is copied between register files inside the loop, nothing spills to scratch,
and the only memory waits in the loop are the one per K step that the design
calls for, together with the barrier's lgkmcnt(0): "vmcnt <= 4" in odd steps,
and "<= 8" in even ones with fragment-order weights (4-step loop trips) or
"<= 12" (no wait) with row-major weights (12-step loop trips); "<= 8" and
"<= 10" in the loops of the paired last m-tiles (gate/up, fragment order).
"""
import os
import re
import shutil
import subprocess

import pytest

from sparse_mixture_experts_06_amd import build as B

SRC = os.path.join(B.CSRC, "ffn_dma.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "ffn_dma.s")
    cmd = B.compile_command(SRC, out, ["--cuda-device-only", "-S"])
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return open(out).read()


def _loops(text):
    """(body lines) of every innermost loop that holds MFMAs."""
    lines = text.split("\n")
    found = []
    for i, line in enumerate(lines):
        if "Loop Header" not in line:
            continue
        label = line.split(":")[0]
        for j in range(i + 1, len(lines)):
            if re.search(r"s_cbranch\S*\s+" + re.escape(label) + r"\s*$", lines[j]):
                body = lines[i:j + 1]
                if any("v_mfma" in b for b in body):
                    found.append(body)
                break
    return found


def _kernels(text):
    """{kernel symbol: its code} for every kernel in the file."""
    starts = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\w+):", text, re.M)]
    out = {}
    for i, (pos, name) in enumerate(starts):
        end = starts[i + 1][0] if i + 1 < len(starts) else len(text)
        out[name] = text[pos:end]
    return out


# template arguments PACKED (fragment-order b1 or row-major b0 weights) and
# SCALED (row scales of int8 codes widened to bf16); K steps per loop trip and
# the even steps' wait
LAYOUTS = {"packed": ("ILb1ELb0E", 4, 8), "packed_scaled": ("ILb1ELb1E", 4, 8),
           "row_major": ("ILb0ELb0E", 12, 12)}


def test_all_kernels_are_present(asm):
    names = list(_kernels(asm))
    for kernel in ("gate_up_dma_kernel", "down_dma_kernel"):
        for tag, _, _ in LAYOUTS.values():
            assert any(kernel + tag in n for n in names), (kernel, tag, names)


@pytest.mark.parametrize("layout", list(LAYOUTS))
@pytest.mark.parametrize("kernel", ["gate_up_dma_kernel", "down_dma_kernel"])
def test_loops_keep_accumulators_in_place(asm, kernel, layout):
    tag, steps, even_wait = LAYOUTS[layout]
    code = [c for n, c in _kernels(asm).items() if kernel + tag in n]
    assert len(code) == 1
    loops = _loops(code[0])
    # one loop per token-fragment count the kernel is instantiated for (8, 6,
    # 4, 2); fragment order adds the paired tile's loops (both projections),
    # one per count and per half of the workgroup (its weight-half reads are
    # constants)
    paired = [b for b in loops if any("vmcnt(10)" in x for x in b)]
    single = [b for b in loops if b not in paired]
    assert len(single) == 4
    assert len(paired) == (8 if tag.startswith("ILb1") else 0)
    for body in loops:
        pair = body in paired
        mfma = [b.split() for b in body if "v_mfma" in b]
        # K steps x (4 x 8, 6, 4, 2) tiles
        assert len(mfma) in tuple(steps * 4 * j for j in (8, 6, 4, 2))
        untied = [m for m in mfma if m[1].rstrip(",") != m[-1]]
        assert not untied, untied[:3]
        assert not [b for b in body if "accvgpr" in b]
        assert not [b for b in body if "scratch_" in b]
        waits = {re.sub(r"\s+", " ", b.strip()) for b in body if "s_waitcnt" in b}
        # paired tile: 4 weight loads a step, 2 token loads in odd steps, so
        # "<= 8" in odd steps and "<= 10" in even ones
        odd, even = ("vmcnt(8)", "vmcnt(10)") if pair else ("vmcnt(4)", f"vmcnt({even_wait})")
        assert waits == {f"s_waitcnt {odd} lgkmcnt(0)", f"s_waitcnt {even} lgkmcnt(0)"}, waits
        assert sum(odd in b for b in body) == steps // 2
        assert sum(even in b for b in body) == steps // 2
        # per 4 K steps: fragment order, 2 weight loads each and 4 token loads in the two odd
        # ones (paired: 4 weight loads each, 2 token loads in the odd ones); row-major, 4 token
        # and 4 weight loads in the two odd ones
        loads = sum("buffer_load_dwordx4" in b and " lds" in b for b in body)
        assert loads == (5 if pair else 4) * steps


def test_kernels_have_no_scratch_and_two_waves_per_simd(asm):
    # fragment order: no scratch at all; row-major (256 registers): at most a
    # few dwords saved before the K loop and restored after it (no scratch
    # access inside the loops, checked above)
    kernels = _kernels(asm)
    for name, code in kernels.items():
        n = sum("scratch_" in line for line in code.split("\n"))
        assert n == 0 if "ILb1E" in name else n <= 4, (name, n)
    sizes = re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)
    assert sizes and all(int(s) <= 16 for s in sizes)
    # the 8-wave workgroup needs two waves per SIMD: at most 256 registers per lane each
    occ = [int(o) for o in re.findall(r"; Occupancy: (\d+)", asm)]
    assert occ and min(occ) >= 2, occ


@pytest.fixture(scope="module")
def asm_bf16(tmp_path_factory):
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asm") / "ffn_bf16.s")
    cmd = B.compile_command(os.path.join(B.CSRC, "ffn_bf16.hip"), out,
                            ["--cuda-device-only", "-S"])
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return open(out).read()


# ring depth in 32-wide K steps, workgroups per CU, token stages (the
# template arguments after W8) and K steps per unrolled loop trip
W8_TILED = {"gate_up": ("wtiled_kernelILb1ELb1ELb1ELi4ELi2ELi1E", 4, 2, 4),
            "down": ("wtiled_kernelILb0ELb1ELb1ELi8ELi1ELi2E", 8, 1, 8)}


@pytest.mark.parametrize("proj", list(W8_TILED))
def test_int8_tiled_kernel_code(asm_bf16, proj):
    """The weights-in-registers tiled kernel on int8 codes (csrc/ffn_bf16.hip,
    template argument W8): accumulators stay in place, nothing spills (gate/up
    fits the 256 registers of two workgroups per CU), every code is converted
    once (one v_cvt_f32_i32 per code, one v_perm_b32 per pair: 4 operands of
    8 codes per K step of the unrolled trip, plus the first step's 4 before
    the loop), and the weight loads are the 16-byte non-temporal ones, one
    per 64-wide stage and row tile (RING/2 stages ahead before the loop, one
    per two K steps in it)."""
    tag, ring, occ, steps = W8_TILED[proj]
    code = [c for n, c in _kernels(asm_bf16).items() if tag in n]
    assert len(code) == 1
    lines = code[0].split("\n")
    mfma = [l.split() for l in lines if "v_mfma" in l]
    assert len(mfma) == steps * 32
    assert not [m for m in mfma if m[1].rstrip(",") != m[-1]]
    assert not [l for l in lines if "scratch_" in l]
    perm = sum("v_perm_b32" in l for l in lines)
    cvt = sum("v_cvt_f32_i32" in l for l in lines)
    assert perm == (steps + 1) * 4 * 4 and cvt == 2 * perm, (perm, cvt)
    assert sum("global_load_dwordx4" in l and " nt" in l for l in lines) == (ring // 2 + steps // 2) * 4
    occupancy = re.search(r"; Occupancy: (\d+)", code[0])
    assert occupancy and int(occupancy.group(1)) >= occ
