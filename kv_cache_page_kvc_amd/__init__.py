"""Python binding of libkvc (include/kvc.h): argument marshalling only.

Every step of encode/decode runs in the HIP kernels of ``libkvc.so``; this
module converts Python/torch arguments into the C structures and calls the
entry points of the same names.  There is no fallback: if the library is
missing, importing the binding's functions raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# KVC_LIB: another build of the same sources (the host sanitizer build)
LIB_PATH = os.environ.get("KVC_LIB") or os.path.join(HERE, "libkvc.so")

KVC_ABI_VERSION = 2
KVC_SLOT_ALIGN = 256
KVC_HEADER_BYTES = 32
KVC_DEFAULT_WORKSPACE = 64 << 20

# kvc_status
KVC_OK, KVC_E_ARG, KVC_E_UNSUPPORTED, KVC_E_PAGE_RANGE, KVC_E_DUP_DST, KVC_E_CAPACITY, \
    KVC_E_BUDGET, KVC_E_HIP, KVC_E_NOMEM = range(9)
# kvc_dtype / kvc_layout_kind
KVC_BF16, KVC_FP16 = 1, 2
KVC_SEPARATE_NHD, KVC_PACKED_HT2D = 1, 2
# kvc_codec_id
KVC_RAW, KVC_FP8_DIRECT, KVC_FP8_FIXED, KVC_FP8_DYNAMIC, KVC_INT8, KVC_UNIFORM3, KVC_UNIFORM4, \
    KVC_TQ3, KVC_TQ4, KVC_INT8_ROWS, KVC_ANS16 = range(11)
CODECS = {"RAW": 0, "FP8_DIRECT": 1, "FP8_FIXED": 2, "FP8_DYNAMIC": 3, "INT8": 4,
          "UNIFORM3": 5, "UNIFORM4": 6, "TQ3": 7, "TQ4": 8, "INT8_ROWS": 9, "ANS16": 10}
# segment status / flags
KVC_SEG_ENCODED, KVC_SEG_RAW_POLICY, KVC_SEG_RAW_DATA, KVC_SEG_CAPACITY, KVC_SEG_GUARD = range(5)
KVC_FLAG_RAW_POLICY, KVC_FLAG_RAW_DATA, KVC_FLAG_CAPACITY, KVC_FLAG_CRC32, KVC_FLAG_HEAP = 1, 2, 4, 8, 16
# kvc_codec.flags
KVC_CODEC_CRC32 = 1
# decode seg_status values
DEC_OK, DEC_HEADER, DEC_GUARD, DEC_CRC = 0, 1, 2, 3


class KvcError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class kvc_layout(ctypes.Structure):
    _fields_ = [("abi", ctypes.c_uint32), ("kind", ctypes.c_uint32), ("dtype", ctypes.c_uint32),
                ("layers", ctypes.c_uint32), ("kv_heads", ctypes.c_uint32),
                ("head_dim", ctypes.c_uint32), ("tokens_per_page", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32), ("num_blocks", ctypes.c_uint64),
                ("stride_block", ctypes.c_int64), ("stride_token", ctypes.c_int64),
                ("stride_head", ctypes.c_int64),
                ("k_base", ctypes.POINTER(ctypes.c_void_p)),
                ("v_base", ctypes.POINTER(ctypes.c_void_p))]


class kvc_codec(ctypes.Structure):
    _fields_ = [("k", ctypes.c_uint32), ("v", ctypes.c_uint32), ("seed", ctypes.c_uint64),
                ("fixed_scales", ctypes.POINTER(ctypes.c_float)),
                ("protected_layers", ctypes.POINTER(ctypes.c_uint8)),
                ("flags", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class kvc_segment_desc(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("spill_offset", ctypes.c_uint64),
                ("stored_len", ctypes.c_uint32), ("original_len", ctypes.c_uint32),
                ("version", ctypes.c_uint8), ("format", ctypes.c_uint8),
                ("flags", ctypes.c_uint8), ("status", ctypes.c_uint8),
                ("crc32", ctypes.c_uint32)]


DESC_DTYPE = np.dtype([("offset", "<u8"), ("spill_offset", "<u8"), ("stored_len", "<u4"),
                       ("original_len", "<u4"), ("version", "u1"), ("format", "u1"),
                       ("flags", "u1"), ("status", "u1"), ("crc32", "<u4")])
assert DESC_DTYPE.itemsize == ctypes.sizeof(kvc_segment_desc) == 32

EXPORTS = ["kvc_create", "kvc_destroy", "kvc_plan", "kvc_validate_encode", "kvc_validate_decode",
           "kvc_encode_pages", "kvc_decode_pages", "kvc_decode_layers", "kvc_offload_pages",
           "kvc_restore_pages", "kvc_encode_pages_noalloc", "kvc_status_string"]

_lib = None


def lib():
    """Load libkvc.so (built by __graft_entry__.build()); raise if missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libkvc.so not built: {LIB_PATH} (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        st = ctypes.c_int
        L.kvc_create.restype = st
        L.kvc_create.argtypes = [ctypes.POINTER(P), ctypes.c_int, ctypes.c_size_t]
        L.kvc_destroy.restype = st
        L.kvc_destroy.argtypes = [P]
        L.kvc_plan.restype = st
        L.kvc_plan.argtypes = [ctypes.POINTER(kvc_layout), ctypes.POINTER(kvc_codec), ctypes.c_uint32,
                               ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t),
                               ctypes.POINTER(ctypes.c_size_t)]
        for name in ("kvc_validate_encode", "kvc_validate_decode"):
            getattr(L, name).restype = st
            getattr(L, name).argtypes = [ctypes.POINTER(kvc_layout), ctypes.POINTER(kvc_codec), P,
                                         ctypes.c_uint32, ctypes.c_size_t]
        L.kvc_encode_pages.restype = st
        L.kvc_encode_pages.argtypes = [P, ctypes.POINTER(kvc_layout), ctypes.POINTER(kvc_codec), P,
                                       ctypes.c_uint32, P, ctypes.c_size_t, P, P]
        L.kvc_decode_pages.restype = st
        L.kvc_decode_pages.argtypes = [P, ctypes.POINTER(kvc_layout), ctypes.POINTER(kvc_codec), P,
                                       ctypes.c_size_t, P, ctypes.c_uint32, P, P]
        L.kvc_decode_layers.restype = st
        L.kvc_decode_layers.argtypes = [P, ctypes.POINTER(kvc_layout), ctypes.POINTER(kvc_codec), P,
                                        ctypes.c_size_t, P, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                        P, P]
        L.kvc_offload_pages.restype = st
        L.kvc_offload_pages.argtypes = [P, ctypes.POINTER(kvc_layout), ctypes.POINTER(kvc_codec), P,
                                        ctypes.c_uint32, P, ctypes.c_size_t, P, ctypes.POINTER(ctypes.c_size_t), P]
        L.kvc_restore_pages.restype = st
        L.kvc_restore_pages.argtypes = [P, ctypes.POINTER(kvc_layout), ctypes.POINTER(kvc_codec), P,
                                        ctypes.c_size_t, P, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                        P, P, P]
        L.kvc_encode_pages_noalloc.restype = st
        L.kvc_encode_pages_noalloc.argtypes = [ctypes.POINTER(kvc_layout), ctypes.POINTER(kvc_codec), P,
                                               ctypes.c_uint32, P, ctypes.c_size_t, P, P]
        L.kvc_status_string.restype = ctypes.c_char_p
        L.kvc_status_string.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().kvc_status_string(int(s)).decode()


# --------------------------------------------------------------- marshalling
class Layout:
    """Owns a kvc_layout and the pointer arrays it references.

    k_ptrs / v_ptrs: device addresses (ints), one per layer; v_ptrs None for
    the packed layout.  Strides in elements.
    """

    def __init__(self, kind, dtype, layers, kv_heads, head_dim, tokens_per_page, num_blocks,
                 stride_block, stride_token, stride_head, k_ptrs, v_ptrs=None):
        self._k = (ctypes.c_void_p * layers)(*k_ptrs)
        self._v = (ctypes.c_void_p * layers)(*v_ptrs) if v_ptrs is not None else None
        self.c = kvc_layout(KVC_ABI_VERSION, kind, dtype, layers, kv_heads, head_dim, tokens_per_page,
                            0, num_blocks, stride_block, stride_token, stride_head,
                            ctypes.cast(self._k, ctypes.POINTER(ctypes.c_void_p)),
                            ctypes.cast(self._v, ctypes.POINTER(ctypes.c_void_p)) if self._v else None)

    @staticmethod
    def separate(k_layers, v_layers, kv_heads, head_dim, tokens_per_page):
        """From per-layer torch tensors [num_blocks, T, H, D] (K and V)."""
        t0 = k_layers[0]
        dtype = _dtype_code(t0)
        sb, st, sh, si = t0.stride()
        assert si == 1
        return Layout(KVC_SEPARATE_NHD, dtype, len(k_layers), kv_heads, head_dim, tokens_per_page,
                      t0.shape[0], sb, st, sh, [t.data_ptr() for t in k_layers],
                      [t.data_ptr() for t in v_layers])

    @staticmethod
    def packed(layers_t, kv_heads, head_dim, tokens_per_page):
        """From per-layer torch tensors [num_blocks, H, T, 2*D] (vLLM packed)."""
        t0 = layers_t[0]
        dtype = _dtype_code(t0)
        sb, sh, st, si = t0.stride()
        assert si == 1
        return Layout(KVC_PACKED_HT2D, dtype, len(layers_t), kv_heads, head_dim, tokens_per_page,
                      t0.shape[0], sb, st, sh, [t.data_ptr() for t in layers_t], None)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KVC_BF16
    if t.dtype == torch.float16:
        return KVC_FP16
    raise ValueError(f"unsupported KV dtype {t.dtype}")


class Codec:
    """Owns a kvc_codec and its host arrays."""

    def __init__(self, k, v, seed=0, fixed_scales=None, protected_layers=None, layers=None, crc=False):
        self._fs = None
        self._prot = None
        fs_ptr = None
        prot_ptr = None
        if fixed_scales is not None:
            self._fs = np.ascontiguousarray(np.asarray(fixed_scales, np.float32).reshape(-1))
            fs_ptr = self._fs.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
        if protected_layers is not None:
            n = layers if layers is not None else (max(protected_layers) + 1 if protected_layers else 1)
            bm = np.zeros((n + 7) // 8, np.uint8)
            for l in protected_layers:
                bm[l >> 3] |= 1 << (l & 7)
            self._prot = bm
            prot_ptr = bm.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))
        self.c = kvc_codec(CODECS[k] if isinstance(k, str) else k, CODECS[v] if isinstance(v, str) else v,
                           seed, fs_ptr, prot_ptr, KVC_CODEC_CRC32 if crc else 0, 0)


def _check(status, where):
    if status != KVC_OK:
        raise KvcError(status, where)


def _pages(ids):
    a = np.ascontiguousarray(np.asarray(ids, dtype=np.int32))
    return a, (a.ctypes.data_as(ctypes.c_void_p) if a.size else None)


def kvc_create(hip_device: int = 0, workspace_budget: int = 0):
    h = ctypes.c_void_p()
    _check(lib().kvc_create(ctypes.byref(h), hip_device, workspace_budget), "kvc_create")
    return h


def kvc_destroy(ctx):
    _check(lib().kvc_destroy(ctx), "kvc_destroy")


def kvc_plan(layout: Layout, codec: Codec, n_pages: int):
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().kvc_plan(ctypes.byref(layout.c), ctypes.byref(codec.c), n_pages,
                          ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)), "kvc_plan")
    return a.value, b.value, c.value


def kvc_validate_encode(layout: Layout, codec: Codec, page_ids, out_bytes: int) -> int:
    arr, ptr = _pages(page_ids)
    return lib().kvc_validate_encode(ctypes.byref(layout.c), ctypes.byref(codec.c), ptr, arr.size,
                                     out_bytes)


def kvc_validate_decode(layout: Layout, codec: Codec, dst_page_ids, in_bytes: int) -> int:
    arr, ptr = _pages(dst_page_ids)
    return lib().kvc_validate_decode(ctypes.byref(layout.c), ctypes.byref(codec.c), ptr, arr.size,
                                     in_bytes)


def kvc_encode_pages(ctx, layout: Layout, codec: Codec, page_ids, out_ptr: int, out_bytes: int,
                     desc_ptr: int, stream: int = 0):
    arr, ptr = _pages(page_ids)
    _check(lib().kvc_encode_pages(ctx, ctypes.byref(layout.c), ctypes.byref(codec.c), ptr, arr.size,
                                  out_ptr, out_bytes, desc_ptr, stream or None), "kvc_encode_pages")


def kvc_encode_pages_noalloc(layout: Layout, codec: Codec, page_ids, out_ptr: int, out_bytes: int,
                             desc_ptr: int, stream: int = 0):
    arr, ptr = _pages(page_ids)
    _check(lib().kvc_encode_pages_noalloc(ctypes.byref(layout.c), ctypes.byref(codec.c), ptr, arr.size,
                                          out_ptr, out_bytes, desc_ptr, stream or None),
           "kvc_encode_pages_noalloc")


def kvc_decode_pages(ctx, layout: Layout, codec: Codec, in_ptr: int, in_bytes: int, dst_page_ids,
                     seg_status_ptr: int = 0, stream: int = 0):
    arr, ptr = _pages(dst_page_ids)
    _check(lib().kvc_decode_pages(ctx, ctypes.byref(layout.c), ctypes.byref(codec.c), in_ptr, in_bytes,
                                  ptr, arr.size, seg_status_ptr or None, stream or None),
           "kvc_decode_pages")


def kvc_decode_layers(ctx, layout: Layout, codec: Codec, in_ptr: int, in_bytes: int, dst_page_ids,
                      layer_begin: int, layer_end: int, seg_status_ptr: int = 0, stream: int = 0):
    arr, ptr = _pages(dst_page_ids)
    _check(lib().kvc_decode_layers(ctx, ctypes.byref(layout.c), ctypes.byref(codec.c), in_ptr, in_bytes,
                                   ptr, arr.size, layer_begin, layer_end, seg_status_ptr or None,
                                   stream or None), "kvc_decode_layers")


def kvc_offload_pages(ctx, layout: Layout, codec: Codec, page_ids, host_ptr: int, host_bytes: int,
                      host_desc_ptr: int, stream: int = 0) -> int:
    """host_ptr / host_desc_ptr: pinned host memory (e.g. torch pin_memory
    tensors).  Returns the bytes of host_ptr that hold the encoding."""
    arr, ptr = _pages(page_ids)
    used = ctypes.c_size_t(0)
    _check(lib().kvc_offload_pages(ctx, ctypes.byref(layout.c), ctypes.byref(codec.c), ptr, arr.size,
                                   host_ptr, host_bytes, host_desc_ptr, ctypes.byref(used), stream or None),
           "kvc_offload_pages")
    return used.value


def kvc_restore_pages(ctx, layout: Layout, codec: Codec, host_ptr: int, host_bytes: int, dst_page_ids,
                      layer_begin: int, layer_end: int, seg_status_ptr: int = 0, layer_ready=None,
                      stream: int = 0):
    """layer_ready: None or a sequence of hipEvent_t handles (ints), one per
    restored layer (e.g. torch.cuda.Event(...).cuda_event after a first record)."""
    arr, ptr = _pages(dst_page_ids)
    evs = None
    if layer_ready is not None:
        evs = (ctypes.c_void_p * max(1, len(layer_ready)))(*[e or None for e in layer_ready])
    _check(lib().kvc_restore_pages(ctx, ctypes.byref(layout.c), ctypes.byref(codec.c), host_ptr, host_bytes,
                                   ptr, arr.size, layer_begin, layer_end, seg_status_ptr or None,
                                   ctypes.cast(evs, ctypes.c_void_p) if evs is not None else None,
                                   stream or None), "kvc_restore_pages")
