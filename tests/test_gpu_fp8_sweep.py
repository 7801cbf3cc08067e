"""The hardware E4M3FN conversion against the oracle on every binary32 value
in [-448, 448].

The scaled FP8 codecs convert arbitrary binary32 quotients (clipped to
+-448) with v_cvt_pk_fp8_f32 [knlp "Asymmetric KV: methods and results",
"Precision and scaling reference"].  A test-only kernel
(tests/fp8_cvt_sweep.hip) applies that instruction to every bit pattern of
the range -- 2 x 1,138,753,537 patterns, signed zeros included -- and each
chunk is compared with the oracle's conversion (the nearest E4M3FN value,
ties to even, written from the format's definition), run on host threads.
"""
import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():      # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

from oracle import kvc_oracle as O                       # noqa: E402
from tests import build_test_kernels                     # noqa: E402

CHUNK = 1 << 26                        # patterns per GPU launch and comparison
LAST_POS = 0x43E00000                  # 448.0


def _lib():
    path = build_test_kernels.lib_path("fp8_cvt_sweep.hip")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (python -m tests.build_test_kernels)")
    L = ctypes.CDLL(path)
    L.kvc_test_fp8_cvt_sweep.restype = ctypes.c_int
    L.kvc_test_fp8_cvt_sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    return L


def _oracle_codes(bits: np.ndarray, pool: ThreadPoolExecutor, parts: int) -> np.ndarray:
    x = bits.view(np.float32)
    pieces = np.array_split(x, parts)
    return np.concatenate(list(pool.map(O.f32_to_e4m3, pieces)))


def test_fp8_hardware_convert_every_binary32_in_range():
    lib = _lib()
    threads = max(1, min(16, os.cpu_count() or 1))
    out = torch.empty(CHUNK, dtype=torch.uint8, device="cuda")
    checked = 0
    with ThreadPoolExecutor(threads) as pool:
        for sign in (0, 0x80000000):
            first, last = sign, sign + LAST_POS
            print(f"[case] fp8 convert sweep sign={sign >> 31}", flush=True)
            start = first
            while start <= last:
                n = min(CHUNK, last - start + 1)
                groups = (n + 3) // 4
                rc = lib.kvc_test_fp8_cvt_sweep(start, groups, out.data_ptr(), None)
                assert rc == 0, f"launch failed: {rc}"
                torch.cuda.synchronize()
                gpu = out[:n].cpu().numpy()
                bits = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32)
                ora = _oracle_codes(bits, pool, threads)
                if not np.array_equal(gpu, ora):
                    i = int(np.nonzero(gpu != ora)[0][0])
                    raise AssertionError(f"pattern {int(bits[i]):#010x}: hardware {int(gpu[i]):#04x}, "
                                         f"oracle {int(ora[i]):#04x}")
                checked += n
                start += n
    assert checked == 2 * (LAST_POS + 1)
