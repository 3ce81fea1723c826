"""Host-side checks of the gfx950 instruction listing of the 128-row decode
kernel, whose score MFMAs are issued from inline assembly in their VGPR form.

The compiler's hazard checker does not see those MFMAs, and it treats an asm
output as written when the asm statement issues, while the MFMA writes it
some cycles later.  So the listing must show, for every such MFMA:
  * no other instruction reads or writes its destination registers before
    the next MFMA of the same accumulation chain or a drain of at least 20
    wait states (s_nop), and
  * no VALU instruction wrote one of its source registers in the few wait
    states before it.
A planted violation checks that the scanner sees them."""
import os
import re
import subprocess

import pytest

from paged_mla_decode_03_amd import build as libbuild

SRC = os.path.join(libbuild.CSRC, "mla_decode_wide.hip")
KERNELS = ["_ZN3mla22mla_decode_wide_kernelILb1EEEvNS_12DecodeParamsE",
           "_ZN3mla22mla_decode_wide_kernelILb0EEEvNS_12DecodeParamsE"]
DRAIN_WAIT_STATES = 20
VALU_TO_MFMA_WAIT_STATES = 4


def _regs(text):
    """VGPR numbers named in an operand list (v7, v[8:11])."""
    out = set()
    for m in re.finditer(r"\bv(\d+)\b|\bv\[(\d+):(\d+)\]", text):
        if m.group(1):
            out.add(int(m.group(1)))
        else:
            out |= set(range(int(m.group(2)), int(m.group(3)) + 1))
    return out


def _instructions(listing, kernel):
    body = re.search(rf"^{kernel}:[^\n]*\n(.*?)\n\s*s_endpgm", listing, re.S | re.M)
    assert body, kernel
    out = []
    for line in body.group(1).split("\n"):
        t = line.split(";")[0].strip()
        if not t or t.endswith(":") or t.startswith("."):
            continue
        op, _, rest = t.partition(" ")
        out.append((op, rest.strip()))
    return out


def _wait_states(op, rest):
    return int(rest) + 1 if op == "s_nop" else 1


def scan(instrs):
    """List of violations (index, text) in one kernel's instructions."""
    found = []
    for i, (op, rest) in enumerate(instrs):
        if not (op.startswith("v_mfma") and rest.startswith("v[")):
            continue
        args = [a.strip() for a in rest.split(",")]
        dst, srcs = _regs(args[0]), _regs(",".join(args[1:]))
        # sources: no VALU write shortly before
        ws = 0
        for op2, rest2 in reversed(instrs[max(0, i - 12):i]):
            if ws >= VALU_TO_MFMA_WAIT_STATES:
                break
            if op2.startswith("v_") and not op2.startswith("v_mfma") and _regs(rest2.split(",")[0]) & srcs:
                found.append((i, f"VALU write of an MFMA source: {op2} {rest2}"))
            ws += _wait_states(op2, rest2)
        # destination: untouched until the chain's next link or a drain
        ws = 0
        for op2, rest2 in instrs[i + 1:i + 400]:
            if op2 == "s_nop":
                ws += _wait_states(op2, rest2)
                if ws >= DRAIN_WAIT_STATES:
                    break
                continue
            if op2.startswith("v_mfma"):
                a2 = [a.strip() for a in rest2.split(",")]
                if _regs(a2[0]) == dst and _regs(a2[3]) == dst:
                    break                                  # next link of the same chain
                if _regs(a2[0]) & dst or _regs(",".join(a2[1:])) & dst:
                    found.append((i, f"MFMA touches an in-flight destination: {op2} {rest2}"))
                    break
            elif _regs(rest2) & dst:
                found.append((i, f"touches an in-flight MFMA destination: {op2} {rest2}"))
                break
            if op2 in ("s_branch", "s_setpc_b64", "s_endpgm"):
                break
    return found


@pytest.fixture(scope="module")
def listing(tmp_path_factory):
    try:
        hipcc = libbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "wide.s"
    cmd = [hipcc, f"--offload-arch={libbuild.ARCH}", "-O3", "-std=c++20", "--cuda-device-only", "-S",
           *libbuild.DEVICE_FLAGS, SRC, "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    return out.read_text()


@pytest.mark.parametrize("kernel", KERNELS)
def test_asm_mfma_hazards(listing, kernel):
    instrs = _instructions(listing, kernel)
    n = sum(1 for op, rest in instrs if op.startswith("v_mfma") and rest.startswith("v["))
    assert n == 144, n                       # the score MFMAs of one page
    assert scan(instrs) == []


def test_scanner_sees_planted_violations(listing):
    instrs = _instructions(listing, KERNELS[0])
    i = next(k for k, (op, rest) in enumerate(instrs) if op.startswith("v_mfma") and rest.startswith("v["))
    args = [a.strip() for a in instrs[i][1].split(",")]
    d0, s0 = min(_regs(args[0])), min(_regs(args[1]))
    read_dst = instrs[:i + 1] + [("v_add_f32_e32", f"v0, 1.0, v{d0}")] + instrs[i + 1:]
    assert scan(read_dst)
    write_src = instrs[:i] + [("v_mov_b32_e32", f"v{s0}, 0")] + instrs[i:]
    assert scan(write_src)


@pytest.mark.parametrize("kernel", KERNELS)
def test_lds_fits_and_no_scratch_in_score_stream(listing, kernel):
    """160 KB of LDS at most, and no spill traffic between a page's first and
    last score MFMA (a spilled accumulator would also break the rules above)."""
    head = listing[:listing.index(f".name:           {kernel}")]
    lds = int(re.findall(r"\.group_segment_fixed_size:\s+(\d+)", head)[-1])   # this kernel's metadata entry
    assert lds <= 160 * 1024
    instrs = _instructions(listing, kernel)
    idx = [k for k, (op, rest) in enumerate(instrs) if op.startswith("v_mfma") and rest.startswith("v[")]
    assert not [op for op, _ in instrs[idx[0]:idx[-1] + 1] if op.startswith("scratch_")]
