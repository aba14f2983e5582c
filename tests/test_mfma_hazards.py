"""No path from a matrix-core product to the first read of its result has
fewer wait states than the compiler itself leaves on straight-line code.

The compiler inserts the wait states a product's result needs when producer
and reader sit in one straight run of code; a path that crosses a branch has
been seen to get fewer (a prefill variant whose first softmax read of a score
product could follow the product after a taken branch and two instructions;
its outputs then changed from run to run).  For each product opcode the
requirement is taken as the smallest distance the compiler uses on straight
paths, and every path through a branch must reach it.  CPU only: hipcc
writes the gfx950 assembly here.
"""
import collections
import os
import sys

import pytest

from asm_scan import device_asm, kernels, mfma_reads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.fixture(scope="module")
def scans():
    from concurrent.futures import ThreadPoolExecutor
    from paged_kv_cache_227_amd import build_lib
    srcs = [os.path.join(build_lib.CSRC, f) for f in ("prefill.hip", "decode.hip")]
    with ThreadPoolExecutor(2) as ex:
        asms = list(ex.map(lambda s: device_asm(s, build_lib.FLAGS, build_lib.HIPCC), srcs))
    out = {}
    for src, asm in zip(srcs, asms):
        for name, body in kernels(asm):
            if any(line.startswith("v_mfma") for line in body):
                out[(os.path.basename(src), name)] = mfma_reads(body)
    return out


def test_scan_sees_the_matrix_kernels(scans):
    """Every matrix kernel is scanned, and the scan finds product reads where
    they sit close to their products (the decode kernels: a read within the
    window shows the scan works).  The prefill kernels read their products'
    results only in the next phase, behind a workgroup barrier, so their
    scans find no read in the window at all, which is the strongest form of
    the property the next test checks."""
    files = collections.Counter(f for f, _ in scans)
    assert files["prefill.hip"] >= 8 and files["decode.hip"] >= 8, files
    near = collections.Counter()
    for (f, _), reads in scans.items():
        near[f] += len(reads)
    assert near["decode.hip"] >= 8, "product reads within the scan window: %s" % near


def test_no_branch_path_shorter_than_straight_code(scans):
    need = {}
    for reads in scans.values():
        for op, d, branched in reads:
            if not branched:
                need[op] = min(need.get(op, 1 << 30), d)
    short = []
    for (f, name), reads in scans.items():
        for op, d, branched in reads:
            if branched and op in need and d < need[op]:
                short.append((f, name[:90], op, d, need[op]))
    assert not short, "product results read too early after a branch: %s" % short[:5]
    # the compiler's straight-line distance for the 16x16x32 products these kernels use
    assert all(need[op] >= 4 for op in need), need


def test_scanner_flags_a_short_branch_path():
    """The scan itself: a product whose result is read two instructions after
    a taken branch (the shape the prefill kernel had) is reported as a branch
    path shorter than the straight one beside it."""
    body = [
        "v_mfma_f32_16x16x32_f16 v[64:67], v[98:101], v[54:57], v[64:67]",
        "s_cbranch_scc1 .LBB0_2",
        "v_mfma_f32_16x16x32_f16 v[60:63], v[100:103], v[54:57], v[60:63]",
        ".LBB0_2:",
        "s_setprio 0",
        "v_max3_f32 v86, v64, s9, v65",
        "v_max3_f32 v86, v86, v66, v67",
        "s_nop 5",
        "v_max3_f32 v86, v86, v60, v61",
        "s_endpgm",
    ]
    reads = mfma_reads(body)
    assert ("v_mfma_f32_16x16x32_f16", 2, True) in reads       # branch taken: s_cbranch, s_setprio
    assert ("v_mfma_f32_16x16x32_f16", 9, False) in reads      # straight on: s_setprio, 2 x v_max3, s_nop 5
