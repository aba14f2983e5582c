"""The decode kernels keep their prefetched tiles in flight (CPU only: hipcc
writes the gfx950 assembly here).

Vector loads are counted in issue order, and the compiler waits for a
register by count.  A table entry read with a vector load, a load issued on
one branch only, or a store among the loads made the wait for the tile being
computed also wait for every tile issued after it: in the kernels below no
wait then left more than half a tile's loads outstanding.  With the tiles kept
in flight, the steady-state wait leaves at least one whole tile's loads
(16: K and V of 16 rows at 512 bytes a row over 64 lanes; 8 for the
matrix-core engine's 256-byte rows) outstanding.
"""
import os
import re
import sys

import pytest

from asm_scan import device_asm, kernels

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

# (kernel name fragment, loads a wait must leave outstanding in the steady state)
CASES = {
    "flat, f16, head_dim 128, one query head per KV head (vector engine, two heads a wave)":
        (r"decode_flat_kernelINS_3F16ELi128ELi1ENS_4TuneILi4ELi16ELi1ELb1ELb0ELi2ELi1ELi1ELi1EEELb0E", 16),
    "flat with the append fused, f16, head_dim 128, one query head per KV head (vector engine)":
        (r"decode_flat_kernelINS_3F16ELi128ELi1ENS_4TuneILi4ELi16ELi1ELb1ELb0ELi2ELi1ELi1ELi1EEELb1E", 16),
    "flat, bf16, head_dim 128, four query heads per KV head (matrix-core engine)":
        (r"decode_flat_kernelINS_4BF16ELi128ELi4ENS_4TuneILi8ELi8ELi1ELb1ELb1ELi1ELi0ELi4ELi1EEELb0E", 8),
    "flat, bf16, head_dim 128, eight query heads per KV head (matrix-core engine)":
        (r"decode_flat_kernelINS_4BF16ELi128ELi8ENS_4TuneILi8ELi8ELi1ELb1ELb1ELi1ELi0ELi4ELi1EEELb0E", 8),
    "fixed partitions, bf16, head_dim 128, eight query heads per KV head (matrix-core engine)":
        (r"decode_partition_persistent_kernelINS_4BF16ELi128ELi8ENS_4TuneILi8ELi8ELi1ELb1ELb1ELi1ELi0ELi4ELi2E", 8),
}


@pytest.fixture(scope="module")
def bodies():
    from paged_kv_cache_227_amd import build_lib
    asm = device_asm(os.path.join(build_lib.CSRC, "decode.hip"), build_lib.FLAGS, build_lib.HIPCC)
    return kernels(asm)


@pytest.mark.parametrize("case", sorted(CASES))
def test_steady_state_wait_leaves_a_tile_in_flight(bodies, case):
    frag, need = CASES[case]
    found = [body for name, body in bodies if re.search(frag, name)]
    assert len(found) == 1, "kernel %s not found once in the assembly" % frag
    counts = [int(m.group(1)) for line in found[0] for m in [re.search(r"s_waitcnt\b.*\bvmcnt\((\d+)\)", line)] if m]
    assert counts, "no vmcnt waits in %s" % frag
    assert max(counts) >= need, "largest vmcnt wait %d < %d loads of a tile: the prefetch is drained" % (
        max(counts), need)
