"""The TurboQuant encoder's short norm sequences on the device, against the
IEEE results, for every input of their domains.

In the encoder's common case (every sum of squares of a wave's vectors in
[2^-96, 2^31)) the norm is RN(sqrt(S)) from the hardware square-root
estimate and one neighbour test each way, and its reciprocal is one Newton
step from the hardware reciprocal estimate (kvc_arch.h: sqrt_rn_normal,
recip_newton).  tests/fast_norm_check.c proves both on the CPU for every
start within one ulp, except one fixed point of the Newton step per binade;
this sweep runs the device's own estimates over all 1,065,353,216 square-root
inputs and all 536,870,912 reciprocal inputs, so that the fixed point (and
the estimates' accuracy) is settled on the hardware itself.  The reference
is the double-precision IEEE square root or quotient rounded to binary32.
"""
import ctypes
import os

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():      # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

from tests import build_test_kernels                     # noqa: E402

RANGES = {0: (0x0F800000, 0x4F000000),    # square root: S in [2^-96, 2^31)
          1: (0x27800000, 0x47800000)}    # reciprocal: n in [2^-48, 2^16)


def _lib():
    path = build_test_kernels.lib_path("norm_sweep.hip")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python -m tests.build_test_kernels)")
    L = ctypes.CDLL(path)
    L.kvc_test_norm_sweep.restype = ctypes.c_int
    L.kvc_test_norm_sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]
    return L


@pytest.mark.parametrize("which", [0, 1], ids=["sqrt", "reciprocal"])
def test_norm_sequences_every_input(which):
    lib = _lib()
    lo, hi = RANGES[which]
    print(f"[case] norm sweep {'sqrt' if which == 0 else 'reciprocal'} {hi - lo} inputs", flush=True)
    bad = torch.zeros(1, dtype=torch.int64, device="cuda")
    first_bad = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    assert lib.kvc_test_norm_sweep(lo, hi - lo, which, bad.data_ptr(), first_bad.data_ptr(), None) == 0
    torch.cuda.synchronize()
    nbad = int(bad.item())
    assert nbad == 0, f"{nbad} mismatches, first at bits {int(first_bad.item()) & 0xFFFFFFFF:#010x}"
