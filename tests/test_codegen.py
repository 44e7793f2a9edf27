"""The generated gfx950 code of the MFMA kernels keeps its LDS operand reads
ahead of the matrix products (no GPU: the sources are compiled to assembly
here).

The compiler's schedule of a full tile is fragile: small changes to the loop
around it have made it issue each LDS read just before the product that
consumes it and wait for it at once (`s_waitcnt lgkmcnt(0)` in front of most
MFMAs), which measured 38% slower for the d = 128 dK/dV kernel. These checks
catch that on the CPU. The bounds sit between the schedules measured fast and
the collapsed ones."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from exact_io_aware_07_amd import build

SOURCES = ("fa_bwd_mfma.hip", "fa_fwd_mfma.hip")


def _hipcc():
    try:
        return build.hipcc()
    except RuntimeError:
        return None


@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None or shutil.which(hipcc) is None and not os.path.exists(hipcc):
        pytest.skip("hipcc is not available")
    out = tmp_path_factory.mktemp("asm")

    def compile_one(name):
        dst = str(out / (name + ".s"))
        cmd = [hipcc, *build.COMMON, *build.DEVICE_FLAGS, "--cuda-device-only", "-S",
               os.path.join(build.CSRC, name), "-o", dst]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        return open(dst).read()

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        return dict(zip(SOURCES, ex.map(compile_one, SOURCES)))


def full_tile_blocks(asm, kernel_prefix):
    """Instructions of each basic block with the most MFMAs (the unrolled
    full tiles of the main loop) in the first kernel whose mangled name
    starts with kernel_prefix."""
    lines = asm.split("\n")
    start = next(i for i, l in enumerate(lines) if re.match(r"^_ZN2fa12_GLOBAL__N_1\d*" + kernel_prefix, l))
    blocks, cur = [], None
    for l in lines[start + 1:]:
        if re.match(r"^\.Lfunc_end", l):
            break
        if re.match(r"^\.LBB\S+:", l):
            cur = []
            blocks.append(cur)
            continue
        s = l.strip()
        if cur is not None and s and not s.startswith((";", ".")):
            cur.append(s)
    most = max(sum(i.startswith("v_mfma") for i in b) for b in blocks)
    return [b for b in blocks if sum(i.startswith("v_mfma") for i in b) == most]


def read_ahead(block):
    """(MFMAs, mean lgkmcnt of the block's LDS waits, MFMAs issued right
    after a wait for every LDS read)."""
    n_mfma = sum(i.startswith("v_mfma") for i in block)
    waits = [int(m.group(1)) for i in block for m in [re.search(r"lgkmcnt\((\d+)\)", i)] if m]
    after0 = sum(1 for j, i in enumerate(block)
                 if i.startswith("v_mfma") and j > 0 and "lgkmcnt(0)" in block[j - 1])
    return n_mfma, sum(waits) / max(len(waits), 1), after0


# kernel (mangled prefix), products per full tile, least mean lgkmcnt, most
# products right after lgkmcnt(0)
CASES = [
    ("fa_bwd_mfma.hip", "dkdv_kernelINS_4BF16ELi128ELb0E", 64, 6.0, 4),
    ("fa_bwd_mfma.hip", "dkdv_kernelINS_4BF16ELi64ELb0E", 32, 3.0, 4),
    ("fa_bwd_mfma.hip", "dkdv_kernelINS_4BF16ELi128ELb1E", 64, 6.0, 4),
    ("fa_bwd_mfma.hip", "dq_kernelINS_4BF16ELi128ELb0E", 96, 1.0, 32),
    ("fa_bwd_mfma.hip", "dq_kernelINS_4BF16ELi64ELb0E", 48, 1.0, 20),
    ("fa_fwd_mfma.hip", "fwd_mfma_kernelINS_4BF16ELi128ELb0ELb0ELb0E", 32, 6.0, 4),
    ("fa_fwd_mfma.hip", "fwd_mfma_kernelINS_4BF16ELi128ELb1ELb0ELb0E", 32, 6.0, 4),
    ("fa_fwd_mfma.hip", "fwd_mfma_kernelINS_4BF16ELi64ELb0ELb0ELb0E", 16, 3.0, 4),
    ("fa_fwd_mfma.hip", "fwd_mfma_kernelINS_4BF16ELi64ELb1ELb0ELb0E", 16, 3.0, 4),
]


@pytest.mark.parametrize("src,kernel,mfma,min_mean,max_after0", CASES, ids=[c[1] for c in CASES])
def test_full_tile_reads_run_ahead_of_the_products(assembly, src, kernel, mfma, min_mean, max_after0):
    # every copy of the full tile (the main loop unrolls it for each buffer
    # parity): one collapsed copy runs every other tile
    for k, block in enumerate(full_tile_blocks(assembly[src], kernel)):
        n, mean, after0 = read_ahead(block)
        assert n == mfma, f"{kernel} block {k}: {n} MFMAs, expected {mfma}"
        assert mean >= min_mean, f"{kernel} block {k}: LDS waits average lgkmcnt {mean:.1f} < {min_mean}"
        assert after0 <= max_after0, f"{kernel} block {k}: {after0} MFMAs follow a wait for every LDS read"
