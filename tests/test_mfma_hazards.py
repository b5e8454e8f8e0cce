"""Wait states between the FP8 / FP4 block-scaled MFMAs that write ordinary
VGPRs and the first vector-ALU or memory instruction that reads their result.

The library is built with MFMA results in ordinary VGPRs (the GEMM promotes
every partial product with VALU FMAs).  The hardware does not interlock a
VALU read of such a result: the compiler must place enough independent
instructions or s_nop wait states in between.  For the 8-pass
v_mfma_scale_f32_16x16x128_f8f6f4 (FP8 x FP8, and FP8 x FP4, which issues at
the same rate on this chip) that is 11 wait states.  This test disassembles
the gfx950 code object of the built library (code built here) and walks
every path from each such MFMA, through branches, until the first
instruction that reads a register it wrote; reads by another MFMA (srcC
chaining, which the matrix core checks itself) are not counted.  It pins
that every path leaves at least 11 wait states, and the checker itself on
small listings with a planted short distance.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "moe_layer_router_amd", "libmoe_layer.so")
LLVM = "/opt/rocm/llvm/bin"
REQUIRED = 11          # wait states after an 8-pass XDL MFMA before a VALU read of its VGPR result
STORE = re.compile(r"^(buffer_store|global_store|flat_store|scratch_store|ds_write|ds_store)")


def _regs(s):
    out = set()
    for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", s):
        out.update(range(int(a), int(b) + 1))
    out.update(int(a) for a in re.findall(r"\bv(\d+)\b", s))
    return out


def _dst_src(mn, ops):
    parts = [p.strip() for p in re.split(r",(?![^\[]*\])", ops)] if ops else []
    if mn.startswith("s_") or not parts:
        return set(), set()
    if STORE.match(mn) or mn.startswith(("v_readlane", "v_readfirstlane")):
        return set(), set().union(*[_regs(p) for p in parts])
    dst = _regs(parts[0])
    src = set().union(*[_regs(p) for p in parts[1:]]) if len(parts) > 1 else set()
    return dst, src


def parse(listing):
    """(instructions [(addr, mnemonic, operands, function)], branch targets {addr: addr})."""
    funcs, ins, tgt, cur = {}, [], {}, None
    for line in listing.split("\n"):
        m = re.match(r"^([0-9a-f]+) <(\S+)>:", line)
        if m:
            cur = m.group(2)
            funcs[cur] = int(m.group(1), 16)
            continue
        m = re.match(r"^\t(\S+)\s*(.*?)\s*//\s*([0-9A-F]+):(.*)$", line)
        if m and cur:
            addr = int(m.group(3), 16)
            ins.append((addr, m.group(1), m.group(2), cur))
            t = re.search(r"<(\S+)\+0x([0-9a-f]+)>", m.group(4))
            if m.group(1).startswith(("s_branch", "s_cbranch")) and t:
                tgt[addr] = funcs[t.group(1)] + int(t.group(2), 16)
    return ins, tgt


def distances(listing, mnemonic, horizon=REQUIRED + 8):
    """For each VGPR-destination `mnemonic`: the fewest wait states on any
    path to a non-MFMA instruction reading its result (None when none does
    within `horizon`).  An instruction counts 1, s_nop N counts N + 1."""
    ins, tgt = parse(listing)
    idx = {a: i for i, (a, *_r) in enumerate(ins)}
    out = []
    for i, (a, mn, ops, f) in enumerate(ins):
        if mn != mnemonic:
            continue
        dst, _ = _dst_src(mn, ops)
        if not dst:
            continue
        best, stack, seen = None, [(i + 1, 0)], set()
        while stack:
            j, w = stack.pop()
            while j < len(ins) and w < horizon and (j, w) not in seen:
                seen.add((j, w))
                a2, mn2, ops2, f2 = ins[j]
                if f2 != f or mn2 == "s_endpgm":
                    break
                _, src = _dst_src(mn2, ops2)
                if src & dst and not mn2.startswith("v_mfma"):
                    best = w if best is None else min(best, w)
                    break
                w += int(ops2.split()[0], 0) + 1 if mn2.startswith("s_nop") else 1
                if mn2.startswith("s_cbranch") and a2 in tgt:
                    stack.append((idx[tgt[a2]], w))
                elif mn2 == "s_branch" and a2 in tgt:
                    j = idx[tgt[a2]]
                    continue
                j += 1
        out.append((hex(a), f, best))
    return out


def _fake(body):
    """A listing in llvm-objdump's format: one function, one instruction per
    line at 0x1000 + 8 k; a branch given as (text, k) targets instruction k."""
    lines = ["0000000000001000 <_Z4testv>:"]
    for k, ins in enumerate(body):
        tail = ""
        if isinstance(ins, tuple):
            ins, to = ins
            tail = f" <_Z4testv+0x{8 * to:x}>"
        lines.append(f"\t{ins}  // {0x1000 + 8 * k:012X}: 00000000{tail}")
    return "\n".join(lines)


MF = "v_mfma_scale_f32_16x16x128_f8f6f4"


def test_checker_finds_a_short_distance():
    body = [f"{MF} v[0:3], v[8:15], v[16:23], 0, v30, v31", "v_mov_b32_e32 v40, v41", "s_nop 1",
            "v_fmac_f32_e32 v50, v2, v51"]
    assert distances(_fake(body), MF) == [("0x1000", "_Z4testv", 3)]


def test_checker_follows_branches_and_skips_mfma_chains():
    body = [f"{MF} v[0:3], v[8:15], v[16:23], 0, v30, v31",
            f"{MF} v[4:7], v[8:15], v[16:23], v[0:3], v30, v31",    # srcC chaining: not a VALU read
            ("s_cbranch_scc1 3", 6),
            "s_nop 7",
            "v_add_f32_e32 v60, v5, v61",                            # 1 + 8 wait states after the second
            "s_endpgm",
            "v_add_f32_e32 v60, v1, v61"]                            # branch target: 2 after the first
    assert distances(_fake(body), MF) == [("0x1000", "_Z4testv", 2), ("0x1008", "_Z4testv", 9)]


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
@pytest.mark.skipif(not shutil.which(os.path.join(LLVM, "llvm-objdump")), reason="llvm-objdump missing")
def test_fp8_mfma_results_read_after_enough_wait_states(tmp_path):
    fat, co = tmp_path / "fat.bin", tmp_path / "k.co"
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section=.hip_fatbin=" + str(fat), LIB,
                    str(tmp_path / "discard.so")], check=True)
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o", "--input=" + str(fat),
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", "--output=" + str(co)], check=True)
    listing = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", str(co)], check=True,
                             capture_output=True, text=True).stdout
    res = distances(listing, MF)
    read = [r for r in res if r[2] is not None]
    assert len(read) > 100, "no block-scaled MFMA result read found: the checker sees nothing"
    kernels = {f for _, f, _ in read}
    assert any("k_mega" in f for f in kernels) and any("k_gemm" in f for f in kernels)
    short = [r for r in read if r[2] < REQUIRED]
    assert not short, f"VGPR results read too early: {short[:5]}"
