"""Checks on the gfx950 assembly of the attention kernels (CPU only: hipcc cross-compiles).

Two compiler behaviours broke or slowed the kernels before; these checks keep them out:
  * an MFMA inside an EXEC-masked block whose skip branch the compiler removed still writes its
    accumulator when no lane is active, so every MFMA must sit outside EXEC-masked regions or
    behind an s_cbranch_execz;
  * a vmcnt(0) wait in front of the LDS transpose reads drains the global-to-LDS loads in flight
    for later stages (the reads are issued from an asm block that waits for its own results).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "draft_tree_verification_amd", "csrc")
HIPCC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "ev_attention.s"
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-S", "-o", str(out),
           os.path.join(CSRC, "ev_attention.hip")]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read().split("\n")


def _functions(lines):
    funcs, cur = {}, None
    for l in lines:
        m = re.match(r"^(_Z\S+):", l)
        if m:
            cur = m.group(1)
            funcs[cur] = []
        elif cur:
            funcs[cur].append(l.strip())
    return funcs


def test_no_mfma_in_unskipped_exec_masked_block(asm):
    bad, total = [], 0
    for name, body in _functions(asm).items():
        for i, ins in enumerate(body):
            if not ins.startswith("v_mfma"):
                continue
            total += 1
            for j in range(i - 1, -1, -1):
                t = body[j]
                if t.startswith(("s_and_saveexec", "s_andn2_b64 exec", "s_xor_b64 exec")):
                    if not any(b.startswith("s_cbranch_execz") for b in body[j + 1:i]):
                        bad.append((name[:60], ins))
                    break
                if t.startswith(("s_or_b64 exec", "s_mov_b64 exec", "s_endpgm")):
                    break
    assert total > 100, "expected the attention kernels' MFMAs in the assembly"
    assert not bad, f"MFMAs inside EXEC-masked blocks without a skip branch: {bad[:5]}"


def test_no_vmcnt0_drain_before_transpose_reads(asm):
    bad = []
    for name, body in _functions(asm).items():
        for i, ins in enumerate(body):
            if ins.startswith("s_waitcnt") and "vmcnt(0)" in ins:
                nxt = [b for b in body[i + 1:i + 4] if b and not b.startswith(";")]
                if nxt and nxt[0].startswith("ds_read_b64_tr_b16"):
                    bad.append(name[:60])
    assert not bad, f"vmcnt(0) right before the transpose reads in: {bad}"


def test_merge_kernels_use_no_scratch(asm):
    """The split-merge kernels keep their batches in registers (a scratch-backed batch array made
    every load a round trip through memory)."""
    text = "\n".join(asm)
    found = 0
    for m in re.finditer(r"\.agpr_count:\s+\d+.*?\.name:\s+(\S+).*?\.private_segment_fixed_size:\s+(\d+)", text, re.S):
        if "merge_kernel" in m.group(1):
            found += 1
            assert int(m.group(2)) == 0, f"{m.group(1)} uses {m.group(2)} bytes of scratch"
    assert found >= 4
