"""The backward kernels' key loops wait for their tile loads only where the
kernels say so (no GPU: the library's device code is compiled to gfx950
assembly with hipcc and read).

The direct global->LDS tile loads of dK/dV and dQ are issued through inline
asm, so that the compiler does not make the first LDS read of each tile wait
for every load still in flight (the loads of the tiles prefetched ahead of
it).  This checks that the key loops of those kernels, as compiled, hold no
vector-memory wait other than the kernels' own counted waits (inline asm),
and no spill traffic, for both head dims.  The uncached-page-table copies of
the loops are skipped: their page-table reads are register loads that must be
waited for."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_sparse_attention_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


@pytest.fixture(scope="module")
def bwd_asm(tmp_path_factory):
    from paged_sparse_attention_amd import build
    out = str(tmp_path_factory.mktemp("isa") / "attn_bwd.s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [HIPCC, *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "attn_bwd.hip"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=600)
    return open(out).read().split("\n")


def kernel_body(lines, pattern):
    start = [i for i, l in enumerate(lines) if re.match(r"^_Z\S*" + pattern + r"\S*:", l)]
    assert len(start) == 1, pattern
    s = start[0]
    e = next(i for i in range(s, len(lines)) if lines[i].startswith(".Lfunc_end"))
    return lines[s:e]


def key_loops(body):
    """Top-level loops with MFMAs and no register loads from global memory."""
    loops = []
    for h, l in enumerate(body):
        if not (l.startswith(".LBB") and "Loop Header: Depth=1" in l):
            continue
        lab = l.split(":")[0]
        ends = [i for i, x in enumerate(body) if re.search(r"s_c?branch\w* " + re.escape(lab) + r"$", x.strip())]
        if not ends:
            continue
        seg = body[h:max(ends) + 1]
        if any("v_mfma" in x for x in seg) and not any(re.search(r"\bglobal_load_dword\b", x) for x in seg):
            loops.append(seg)
    return loops


def compiler_vm_waits(seg):
    out, in_asm = [], False
    for x in seg:
        if "ASMSTART" in x:
            in_asm = True
        elif "ASMEND" in x:
            in_asm = False
        elif not in_asm and re.search(r"\bs_waitcnt\b.*vmcnt", x):
            out.append(x.strip())
    return out


@pytest.mark.parametrize("kernel", ["dkdv_kernelIDF16bLi128E", "dkdv_kernelIDF16bLi64E",
                                    "dq_kernelIDF16bLi128E", "dq_kernelIDF16bLi64E"])
def test_key_loop_waits_only_for_its_own_loads(bwd_asm, kernel):
    body = kernel_body(bwd_asm, kernel)
    loops = key_loops(body)
    assert loops, "no key loop found"
    for seg in loops:
        text = "\n".join(seg)
        assert "global_load_lds_dwordx4" in text, "the loop issues no tile loads"
        assert compiler_vm_waits(seg) == [], compiler_vm_waits(seg)
        assert "scratch_" not in text, "spill traffic in the key loop"
