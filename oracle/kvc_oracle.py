"""ctypes front end of the CPU oracle (``libkvc_oracle.so``).

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module; the GPU library
and its Python binding never do.

All arithmetic lives in ``kvc_oracle.c``; this file only marshals arrays and
walks segments in the order the format defines (layer-major, then page, then
K before V).  The slot offsets are computed here from the format rules
(header 32 B, codes block, metadata block, or the INT8_ROWS token rows from
byte 128; 256-B alignment), independently of the GPU library's own plan.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
# KVC_ORACLE_LIB: another build of the same source (the sanitizer test)
_LIB = os.environ.get("KVC_ORACLE_LIB") or os.path.join(_HERE, "libkvc_oracle.so")

RAW, FP8_DIRECT, FP8_FIXED, FP8_DYNAMIC, INT8, UNIFORM3, UNIFORM4, TQ3, TQ4, INT8_ROWS, ANS16 = range(11)
CODEC_NAMES = ["RAW", "FP8_DIRECT", "FP8_FIXED", "FP8_DYNAMIC", "INT8",
               "UNIFORM3", "UNIFORM4", "TQ3", "TQ4", "INT8_ROWS", "ANS16"]
FLAG_HEAP = 16         # header flag: the stored bytes sit at spill_offset (ANS16)
ROWS_OFFSET = 128      # INT8_ROWS: token rows start 128 bytes into the slot
BF16, FP16 = 1, 2
SEG_ENCODED, SEG_RAW_POLICY, SEG_RAW_DATA = 0, 1, 2
HEADER_BYTES = 32
SLOT_ALIGN = 256


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE binary32, no contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
               "-fno-fast-math", "-shared", "-fPIC", "-o", _LIB, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            raise RuntimeError(f"oracle library missing: {_LIB} (run __graft_entry__.build())")
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.kvo_bf16_to_f32.restype = ctypes.c_float
        L.kvo_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.kvo_f16_to_f32.restype = ctypes.c_float
        L.kvo_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.kvo_f32_to_bf16.restype = ctypes.c_uint16
        L.kvo_f32_to_bf16.argtypes = [ctypes.c_float]
        L.kvo_f32_to_f16.restype = ctypes.c_uint16
        L.kvo_f32_to_f16.argtypes = [ctypes.c_float]
        L.kvo_f32_to_e4m3.restype = ctypes.c_uint8
        L.kvo_f32_to_e4m3.argtypes = [ctypes.c_float]
        L.kvo_e4m3_to_f32.restype = ctypes.c_float
        L.kvo_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.kvo_e4m3_nearest_search.restype = ctypes.c_uint8
        L.kvo_e4m3_nearest_search.argtypes = [ctypes.c_float]
        for name in ("kvo_f32_to_e4m3_n", "kvo_e4m3_nearest_search_n", "kvo_e4m3_to_f32_n",
                     "kvo_f32_to_bf16_n", "kvo_f32_to_f16_n", "kvo_f16_to_f32_n"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [P, P, ctypes.c_size_t]
        L.kvo_lloyd_max.restype = ctypes.c_int
        L.kvo_lloyd_max.argtypes = [ctypes.c_int, P, P]
        L.kvo_codebook_f32.restype = None
        L.kvo_codebook_f32.argtypes = [ctypes.c_int, P, P]
        L.kvo_signs.restype = None
        L.kvo_signs.argtypes = [ctypes.c_uint64, ctypes.c_int, P]
        L.kvo_splitmix64_next.restype = ctypes.c_uint64
        L.kvo_splitmix64_next.argtypes = [P]
        L.kvo_wht_f32.restype = None
        L.kvo_wht_f32.argtypes = [P, ctypes.c_int]
        L.kvo_sumsq_tree.restype = ctypes.c_float
        L.kvo_sumsq_tree.argtypes = [P, ctypes.c_int]
        L.kvo_code_bytes.restype = ctypes.c_int
        L.kvo_code_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        L.kvo_meta_bytes.restype = ctypes.c_int
        L.kvo_meta_bytes.argtypes = [ctypes.c_int]
        L.kvo_slot_bytes.restype = ctypes.c_size_t
        L.kvo_slot_bytes.argtypes = [ctypes.c_int] * 4
        L.kvo_row_bytes.restype = ctypes.c_size_t
        L.kvo_row_bytes.argtypes = [ctypes.c_int] * 2
        L.kvo_effective_codec.restype = ctypes.c_int
        L.kvo_effective_codec.argtypes = [ctypes.c_int] * 5
        L.kvo_encode_segment.restype = ctypes.c_int
        L.kvo_encode_segment.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_float, ctypes.c_uint64, P, P, ctypes.c_uint64,
                                         ctypes.c_int]
        L.kvo_ans_normalize.restype = None
        L.kvo_ans_normalize.argtypes = [P, ctypes.c_uint32, P]
        L.kvo_ans_encode_plane.restype = ctypes.c_size_t
        L.kvo_ans_encode_plane.argtypes = [P, ctypes.c_size_t, P]
        L.kvo_ans_coded_body.restype = ctypes.c_size_t
        L.kvo_ans_coded_body.argtypes = [P, ctypes.c_size_t]
        L.kvo_ans_decode_plane.restype = ctypes.c_size_t
        L.kvo_ans_decode_plane.argtypes = [P, ctypes.c_size_t, ctypes.c_size_t, P]
        L.kvo_crc32.restype = ctypes.c_uint32
        L.kvo_crc32.argtypes = [P, ctypes.c_size_t]
        L.kvo_decode_segment.restype = ctypes.c_int
        L.kvo_decode_segment.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_uint64, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------- conversions
def f32_to_e4m3(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().kvo_f32_to_e4m3_n(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_nearest_search(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().kvo_e4m3_nearest_search_n(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_to_f32(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().kvo_e4m3_to_f32_n(_ptr(c), _ptr(out), c.size)
    return out


def f32_to_bf16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().kvo_f32_to_bf16_n(_ptr(x), _ptr(out), x.size)
    return out


def f32_to_f16(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().kvo_f32_to_f16_n(_ptr(x), _ptr(out), x.size)
    return out


def f16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().kvo_f16_to_f32_n(_ptr(h), _ptr(out), h.size)
    return out


def bf16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def src_to_f32(bits, dtype) -> np.ndarray:
    return bf16_to_f32(bits) if dtype == BF16 else f16_to_f32(bits)


# ---------------------------------------------------------------- constants
def lloyd_max(bits: int):
    n = 1 << bits
    c = np.zeros(n, np.float64)
    t = np.zeros(n - 1, np.float64)
    it = lib().kvo_lloyd_max(bits, _ptr(c), _ptr(t))
    return c, t, it


def codebook_f32(bits: int):
    n = 1 << bits
    c = np.zeros(n, np.float32)
    t = np.zeros(n - 1, np.float32)
    lib().kvo_codebook_f32(bits, _ptr(c), _ptr(t))
    return c, t


def signs(seed: int, d: int) -> np.ndarray:
    s = np.zeros(d, np.int8)
    lib().kvo_signs(ctypes.c_uint64(seed), d, _ptr(s))
    return s


def splitmix64(seed: int, n: int):
    st = (ctypes.c_uint64 * 1)(seed)
    return [lib().kvo_splitmix64_next(st) for _ in range(n)]


def wht(v) -> np.ndarray:
    v = np.array(v, dtype=np.float32, copy=True)
    lib().kvo_wht_f32(_ptr(v), v.size)
    return v


def sumsq_tree(x) -> float:
    x = np.ascontiguousarray(x, dtype=np.float32)
    return float(lib().kvo_sumsq_tree(_ptr(x), x.size))


# ---------------------------------------------------------------- sizes
def code_bytes(codec, d):
    return lib().kvo_code_bytes(codec, d)


def meta_bytes(codec):
    return lib().kvo_meta_bytes(codec)


def slot_bytes(codec, d, n_vec, heads=1):
    """heads: vectors per token (only the INT8_ROWS layout depends on it)."""
    return lib().kvo_slot_bytes(codec, d, n_vec, heads)


def row_bytes(d, heads):
    return lib().kvo_row_bytes(d, heads)


def effective_codec(codec, d, n_vec, is_protected, heads=1):
    return lib().kvo_effective_codec(codec, d, n_vec, heads, int(bool(is_protected)))


# ---------------------------------------------------------------- segments
ENC_CRC32 = 1          # encode option: CRC32 of the stored bytes in the header
FLAG_CRC32 = 8         # header flag bit


class ChecksumError(ValueError):
    """A segment's stored bytes do not match its CRC32."""


def crc32(data) -> int:
    b = np.ascontiguousarray(np.frombuffer(bytes(data), np.uint8) if isinstance(data, (bytes, bytearray))
                             else data, dtype=np.uint8)
    return int(lib().kvo_crc32(_ptr(b), b.size))


def encode_segment(vec: np.ndarray, dtype: int, codec: int, component: int = 0,
                   is_protected: bool = False, fixed_scale: float = 1.0, seed: int = 0,
                   spill_offset: int = 0, crc: bool = False, heads: int = 1):
    """vec: uint16 [n_vec, D] source bits (v = t*heads + h).  Returns (slot
    uint8, status, spilled uint8|None): the spilled bytes are the raw source
    of a data-dependent raw segment, or an ANS16 segment's payload (header
    flag FLAG_HEAP).  crc: store the CRC32 of the stored bytes in the
    header."""
    vec = np.ascontiguousarray(vec, dtype=np.uint16)
    n_vec, d = vec.shape
    eff = effective_codec(codec, d, n_vec, is_protected, heads)
    slot = np.zeros(slot_bytes(eff, d, n_vec, heads), np.uint8)
    spill = np.zeros(n_vec * d * 2, np.uint8)
    st = lib().kvo_encode_segment(_ptr(vec), dtype, d, n_vec, heads, component, codec,
                                  int(bool(is_protected)), ctypes.c_float(fixed_scale),
                                  ctypes.c_uint64(seed), _ptr(slot), _ptr(spill),
                                  ctypes.c_uint64(spill_offset), ENC_CRC32 if crc else 0)
    if st < 0:
        raise ValueError("oracle encode failed")
    if st == SEG_RAW_DATA:
        return slot, st, spill
    if slot[2] & FLAG_HEAP:
        return slot, st, spill[:int(slot[12:16].view(np.uint32)[0])].copy()
    return slot, st, None


def decode_segment(slot: np.ndarray, buf_base, dtype: int, d: int, n_vec: int, seed: int = 0, heads: int = 1):
    slot = np.ascontiguousarray(slot, dtype=np.uint8)
    out = np.zeros((n_vec, d), np.uint16)
    base = _ptr(buf_base) if buf_base is not None else None
    rc = lib().kvo_decode_segment(_ptr(slot), base, dtype, d, n_vec, heads, ctypes.c_uint64(seed), _ptr(out))
    if rc == -2:
        raise ChecksumError("oracle decode: CRC32 mismatch")
    if rc != 0:
        raise ValueError("oracle decode: malformed segment header")
    return out


# ---------------------------------------------------------------- layouts
class HostLayout:
    """Host copy of one engine KV tensor set, addressed with element strides.

    ``k[l]`` / ``v[l]`` are flat uint16 arrays (the raw bits of layer l);
    element (block b, token t, head h, dim i) of component c sits at
    ``c_off + b*sb + t*st + h*sh + i`` of its array.  For the packed
    [block, head, token, 2*D] layout both components share one array and V
    starts at offset D.
    """

    def __init__(self, dtype, layers, heads, head_dim, tokens, num_blocks,
                 sb, st, sh, k, v=None):
        self.dtype, self.L, self.H, self.D, self.T = dtype, layers, heads, head_dim, tokens
        self.num_blocks, self.sb, self.st, self.sh = num_blocks, sb, st, sh
        self.k = k
        self.v = v
        self.packed = v is None

    def _arr(self, layer, comp):
        if self.packed:
            return self.k[layer], (self.D if comp == 1 else 0)
        return (self.k if comp == 0 else self.v)[layer], 0

    def _index(self, page, off):
        t = np.arange(self.T)[:, None, None]
        h = np.arange(self.H)[None, :, None]
        i = np.arange(self.D)[None, None, :]
        idx = off + page * self.sb + t * self.st + h * self.sh + i
        return idx.reshape(self.T * self.H, self.D)   # canonical order v = t*H + h

    def gather(self, layer, comp, page) -> np.ndarray:
        arr, off = self._arr(layer, comp)
        return arr[self._index(page, off)]

    def scatter(self, layer, comp, page, vecs):
        arr, off = self._arr(layer, comp)
        arr[self._index(page, off)] = vecs


def segment_list(layers, n_pages):
    """Segment order of the format: s = ((l * n_pages) + i) * 2 + c."""
    return [(l, i, c) for l in range(layers) for i in range(n_pages) for c in (0, 1)]


def plan(L, H, D, T, codec_k, codec_v, protected, n_pages):
    """Per-segment (offset, slot size, effective codec) and the slot-region size."""
    n_vec = T * H
    offs, sizes, effs = [], [], []
    off = 0
    for (l, i, c) in segment_list(L, n_pages):
        prot = bool(protected[l]) if protected is not None else False
        eff = effective_codec(codec_k if c == 0 else codec_v, D, n_vec, prot, H)
        sz = slot_bytes(eff, D, n_vec, H)
        offs.append(off)
        sizes.append(sz)
        effs.append(eff)
        off += sz
    return offs, sizes, effs, off


def encode_pages(lay: HostLayout, codec_k, codec_v, seed, page_ids, fixed_scales=None,
                 protected=None, segments=None, threads=1, crc=False):
    """Oracle encode of a whole call.

    Returns (buf, statuses, offsets, slot_region_bytes).  ``buf`` holds the
    slot region followed by a spill region in which data-dependent RAW
    segments are placed in segment order, each aligned to 256 B.  If
    ``segments`` is given (a list of segment indices) only those are encoded
    (the rest of ``buf`` stays zero, statuses -1).
    """
    n_pages = len(page_ids)
    offs, sizes, effs, total = plan(lay.L, lay.H, lay.D, lay.T, codec_k, codec_v,
                                    protected, n_pages)
    seglist = segment_list(lay.L, n_pages)
    todo = range(len(seglist)) if segments is None else segments
    n_vec = lay.T * lay.H
    raw_bytes = n_vec * lay.D * 2

    def work(s):
        l, i, c = seglist[s]
        prot = bool(protected[l]) if protected is not None else False
        fs = float(fixed_scales[l][c]) if fixed_scales is not None else 1.0
        vec = lay.gather(l, c, int(page_ids[i]))
        return encode_segment(vec, lay.dtype, codec_k if c == 0 else codec_v, c, prot, fs, seed, crc=crc,
                              heads=lay.H)

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(work, todo))
    else:
        results = [work(s) for s in todo]

    statuses = np.full(len(seglist), -1, np.int32)
    align = lambda n: (n + SLOT_ALIGN - 1) // SLOT_ALIGN * SLOT_ALIGN
    spilled = sum(align(r[2].size) for r in results if r[2] is not None)
    buf = np.zeros(total + spilled, np.uint8)
    spill_cur = total
    for s, (slot, st, extra) in zip(todo, results):
        statuses[s] = st
        buf[offs[s]:offs[s] + sizes[s]] = slot
        if extra is not None:              # raw source or ANS16 payload, in segment order
            buf[offs[s] + 16:offs[s] + 24] = np.frombuffer(np.uint64(spill_cur).tobytes(), np.uint8)
            buf[spill_cur:spill_cur + extra.size] = extra
            spill_cur += align(extra.size)
    return buf, statuses, offs, total


def decode_pages(buf: np.ndarray, out: HostLayout, codec_k, codec_v, seed, dst_page_ids,
                 protected=None, segments=None, threads=1):
    """Oracle decode of a whole call into the host layout ``out``."""
    n_pages = len(dst_page_ids)
    offs, sizes, effs, total = plan(out.L, out.H, out.D, out.T, codec_k, codec_v,
                                    protected, n_pages)
    seglist = segment_list(out.L, n_pages)
    todo = range(len(seglist)) if segments is None else segments
    n_vec = out.T * out.H

    def work(s):
        return decode_segment(buf[offs[s]:offs[s] + sizes[s]], buf, out.dtype, out.D, n_vec, seed, heads=out.H)

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            results = list(ex.map(work, todo))
    else:
        results = [work(s) for s in todo]
    for s, vecs in zip(todo, results):
        l, i, c = seglist[s]
        out.scatter(l, c, int(dst_page_ids[i]), vecs)


# ---------------------------------------------------------------- entropy stage
def ans_normalize(counts) -> np.ndarray:
    c = np.ascontiguousarray(counts, dtype=np.uint32)
    assert c.size == 256
    f = np.zeros(256, np.uint16)
    lib().kvo_ans_normalize(_ptr(c), int(c.sum()), _ptr(f))
    return f


def ans_encode_plane(sym) -> np.ndarray:
    sym = np.ascontiguousarray(sym, dtype=np.uint8)
    out = np.zeros(1024 + 2 * sym.size, np.uint8)
    n = lib().kvo_ans_encode_plane(_ptr(sym), sym.size, _ptr(out))
    return out[:n].copy()


def ans_coded_body(sym) -> int:
    """Bytes of the rANS body of a plane (bitmap on), coded or not."""
    sym = np.ascontiguousarray(sym, dtype=np.uint8)
    return int(lib().kvo_ans_coded_body(_ptr(sym), sym.size))


def ans_decode_plane(data, n):
    """Returns (symbols, bytes consumed); bytes consumed 0 means rejected."""
    data = np.ascontiguousarray(data, dtype=np.uint8)
    sym = np.zeros(n, np.uint8)
    used = lib().kvo_ans_decode_plane(_ptr(data), data.size, n, _ptr(sym))
    return sym, int(used)
