"""moe_build_offsets_noalloc: moe_build_offsets with its scratch in the library's own
device array instead of a caller workspace (for callers that cannot allocate).

Its outputs are integers, so they must equal moe_build_offsets' bit for bit, and the
entries neither call writes (block-table rows past num_blocks) must stay as they were.
Two calls in a row on the same array, the second with a smaller input, check that a
call does not depend on what the previous one left there.
"""
import ctypes

import numpy as np
import pytest
import torch

from dropless_grouped_gemm_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _outputs(s, fill):
    E, M = s.E, s.T * s.k
    mb, rows = B.moe_max_blocks(s), B.moe_max_rows(s)
    i32 = lambda n: torch.full((max(n, 1),), fill, dtype=torch.int32, device=DEV)
    return dict(counts=i32(E), offsets=i32(E + 1), padded=i32(E + 1), meta=i32(3 * mb),
                nblk=i32(1), pos=i32(M), row_src=i32(rows), err=i32(1))


def _run(s, idx, noalloc):
    o = _outputs(s, -5)
    args = (o["counts"], o["offsets"], o["padded"], o["meta"], o["nblk"], o["pos"], o["row_src"],
            o["err"])
    if noalloc:
        B.moe_build_offsets_noalloc(s, idx, *args)
    else:
        B.moe_build_offsets(s, idx, *args, B.alloc_workspace(s))
    return o


CASES = [
    # (T, E, k, unpadded, id range): the first call of each pair is the larger one
    [(16384, 64, 6, False, 64), (300, 8, 2, False, 8)],
    [(8192, 256, 8, True, 256), (64, 256, 8, True, 256)],
    [(65536, 4, 8, False, 4), (1000, 5, 3, True, 6)],          # ids out of range in the second
]


@pytest.mark.parametrize("pair", CASES, ids=["padded", "unpadded", "ep-share-then-bad-ids"])
def test_noalloc_equals_workspace_entry_point_twice(pair):
    rng = np.random.default_rng(7)
    for T, E, k, unpadded, hi in pair:
        print(f"[no-alloc] T={T} E={E} k={k} unpadded={unpadded}", flush=True)
        s = B.make_shape(T=T, d=8, E=E, k=k, d_e=8, block_m=128, unpadded=unpadded)
        assert B.moe_build_offsets_scratch_bytes(s) <= B.moe_build_offsets_noalloc_capacity()
        idx = torch.from_numpy(rng.integers(0, hi, size=T * k).astype(np.int32)).to(DEV)
        got = _run(s, idx, True)
        want = _run(s, idx, False)
        torch.cuda.synchronize()
        for name in want:
            assert torch.equal(got[name], want[name]), name
        assert int(got["err"].item()) == (1 if hi > E else 0)


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    """A shape whose scratch exceeds the array: MOE_ENOTSUP before anything is launched."""
    L = B.lib()
    cap = B.moe_build_offsets_noalloc_capacity()
    s = B.make_shape(T=1 << 20, d=8, E=1024, k=8, d_e=8, block_m=128)
    assert B.moe_build_offsets_scratch_bytes(s) > cap
    fake = ctypes.c_void_p(0x10000)
    st = L.moe_build_offsets_noalloc(ctypes.byref(s), *([fake] * 9), None)
    assert st == B.MOE_ENOTSUP
