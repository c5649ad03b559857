"""The workgroup-to-XCD assignment the grid remaps rely on, read from the
hardware: on the MI355X (8 XCDs, each with its own L2) block b of a grid runs
on XCD b mod 8. The forward, dQ and dK/dV kernels remap block ids so that the
tiles of one head land on one XCD and share its L2 (and the causal grids rank
each XCD's tiles by length); if the assignment differed, results would not
change, but that L2 sharing and balance would be lost. The probe
(tests/hw/xcd_probe.hip) records HW_REG_XCC_ID in every workgroup of grids
of one, several and many rounds.
"""

import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw", "libfa_probe.so")


@pytest.mark.parametrize("n", [256, 1000, 4096])
def test_block_runs_on_xcd_b_mod_8(n):
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    lib.fa_probe_xcd_ids.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    lib.fa_probe_xcd_ids.restype = ctypes.c_int
    out = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    assert lib.fa_probe_xcd_ids(out.data_ptr(), n, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = out.cpu()
    want = torch.arange(n, dtype=torch.int32) % 8
    mism = int((got != want).sum())
    print(f"\n[xcd map] {n} workgroups: {n - mism} on XCD b mod 8; ids seen "
          f"{sorted(set(got.tolist()))}", flush=True)
    assert mism == 0
