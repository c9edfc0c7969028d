"""Every gfx950 kernel compiles without register spills (no scratch memory).

A kernel that spills reads and writes per-lane scratch in memory on its hot
loop; the register budgets here are tight (1024-thread workgroups allow 128
VGPRs, the MFMA kernel is held to two wavefronts per SIMD), so a change that
adds live values can push one over without any test failing otherwise.
Cross-compiles on the host; no GPU needed.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess

import pytest

from moe_lora_adapter_amd import build

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _resource_usage(src):
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC, *flags, "-I", os.path.join(build.ROOT, "include"), "--cuda-device-only", "-c",
           src, "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).split()[0]] = int(m.group(2))
    return kernels


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")
def test_no_kernel_spills_registers():
    srcs = build.sources()
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        usage = dict(zip(srcs, ex.map(_resource_usage, srcs)))
    n = 0
    for src, kernels in usage.items():
        for name, u in kernels.items():
            n += 1
            assert u.get("ScratchSize", 0) == 0, f"{os.path.basename(src)}: {name} spills: {u}"
    assert n >= 40, f"expected every kernel instantiation, found {n}"


def _kernel_asm(src):
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC, *flags, "-I", os.path.join(build.ROOT, "include"), "--cuda-device-only", "-S",
           src, "-o", "-"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return res.stdout


@pytest.mark.skipif(not shutil.which(HIPCC) and not os.path.exists(HIPCC), reason="no hipcc")
def test_stream_stage_loop_keeps_the_ring_in_flight():
    """The decode stream kernel's stage loop waits for its ring stages with
    explicit counts (its DMA is inline assembly the compiler does not track).
    A full memory wait the compiler adds inside that loop -- one not at a
    workgroup barrier -- drains the ring on every stage; one crept in once
    through a poll loop in the K split and cost half the kernel's speed."""
    asm = _kernel_asm(os.path.join(build.ROOT, "moe_lora_adapter_amd", "csrc", "fused_stream.hip"))
    found = 0
    for m in re.finditer(r"^(_ZN\S*fused_stream_kernel\S*):", asm, re.M):
        found += 1
        body = asm[m.start():asm.index(".Lfunc_end", m.start())].splitlines()
        # each line's innermost loop (the header its block names) and its depth
        loop_of, depth, cur, d = [], [], None, 0
        for line in body:
            if re.match(r"^(\.LBB\S+|; %bb\.\d+):", line):
                h = re.search(r"Loop Header: Depth", line)
                inl = re.search(r"in Loop: Header=(\S+)", line)
                cur = line.split(":")[0].lstrip(".") if h else (inl.group(1) if inl else None)
                dm = re.search(r"Depth=(\d+)", line)
                d = int(dm.group(1)) if dm else 0
            loop_of.append(cur)
            depth.append(d)
        # stage loops: the loops inside a pass (depth 2) whose own blocks issue
        # ring loads (direct to LDS); the pass loop itself sets a pass up
        stage_loops = {loop_of[k] for k, line in enumerate(body)
                       if depth[k] == 2 and "buffer_load_dwordx4" in line and " lds" in line}
        assert stage_loops, f"{m.group(1)}: no stage loop found"
        bad = []
        for k, line in enumerate(body):
            if loop_of[k] in stage_loops and "vmcnt(0)" in line:
                nxt = " ".join(body[k + 1:k + 3])
                if "s_barrier" not in nxt:
                    bad.append(k)
        assert not bad, f"{m.group(1)}: full memory waits inside the stage loop at lines {bad}"
    assert found >= 6, f"expected the stream kernel instantiations, found {found}"
