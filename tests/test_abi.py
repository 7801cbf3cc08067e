"""The C ABI without a GPU: the library loads and exports every entry point
include/kvc.h declares; kvc_plan agrees with the oracle's independent plan
and with the pages' payload sizes; host-side validation rejects bad
arguments before anything would be enqueued."""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_page_kvc_amd as kvc
from oracle import kvc_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "kvc.h")).read()
    declared = set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", hdr))
    assert declared == set(kvc.EXPORTS)
    L = kvc.lib()
    for name in declared:
        assert hasattr(L, name), name
    assert kvc.status_string(kvc.KVC_E_DUP_DST) == "duplicate destination page"


def test_struct_sizes():
    assert ctypes.sizeof(kvc.kvc_segment_desc) == 32
    assert ctypes.sizeof(kvc.kvc_layout) == 80
    assert ctypes.sizeof(kvc.kvc_codec) == 40
    assert kvc.kvc_codec.flags.offset == 32


def test_header_constants_match_binding():
    """The binding's ABI version and CRC flags are the header's."""
    hdr = open(os.path.join(ROOT, "include", "kvc.h")).read()
    assert int(re.search(r"#define KVC_ABI_VERSION (\d+)u", hdr).group(1)) == kvc.KVC_ABI_VERSION == 2
    assert int(re.search(r"#define KVC_CODEC_CRC32 (\d+)u", hdr).group(1)) == kvc.KVC_CODEC_CRC32
    assert int(re.search(r"KVC_FLAG_CRC32 = (\d+)", hdr).group(1)) == kvc.KVC_FLAG_CRC32 == O.FLAG_CRC32


def test_status_codes_match_header():
    """Every kvc_status value of the header is the binding's, with its own
    message; KVC_E_NOMEM is what a failed host allocation returns instead of
    an exception crossing the C ABI."""
    hdr = open(os.path.join(ROOT, "include", "kvc.h")).read()
    enum = hdr[hdr.index("typedef enum {\n  KVC_OK"):hdr.index("} kvc_status;")]
    values = {k: int(v) for k, v in re.findall(r"(KVC_[A-Z_]+) = (\d+)", enum)}
    assert values == {k: getattr(kvc, k) for k in values} and len(values) == 9
    msgs = {kvc.status_string(v) for v in values.values()}
    assert len(msgs) == 9 and "unknown status" not in msgs
    assert kvc.status_string(kvc.KVC_E_NOMEM) == "host memory exhausted"


FAKE = 1 << 40          # aligned fake device addresses: validation never dereferences them


def layout(kind=kvc.KVC_SEPARATE_NHD, dtype=kvc.KVC_BF16, L=4, H=8, D=128, T=16, nb=100, strides=None):
    if strides is None:
        strides = (T * H * D, H * D, D) if kind == kvc.KVC_SEPARATE_NHD else (H * T * 2 * D, 2 * D, T * 2 * D)
    k = [FAKE + l * (1 << 30) for l in range(L)]
    v = [FAKE + (1 << 38) + l * (1 << 30) for l in range(L)] if kind == kvc.KVC_SEPARATE_NHD else None
    return kvc.Layout(kind, dtype, L, H, D, T, nb, *strides, k, v)


@pytest.mark.parametrize("ck,cv", [("TQ4", "UNIFORM4"), ("TQ3", "UNIFORM3"), ("FP8_DYNAMIC", "INT8"),
                                   ("RAW", "FP8_FIXED"), ("FP8_DIRECT", "RAW"), ("INT8_ROWS", "TQ4")])
@pytest.mark.parametrize("D", [32, 64, 128, 256])
@pytest.mark.parametrize("H", [8, 3])
def test_plan_matches_oracle(ck, cv, D, H):
    L, T, n = 6, 16, 37
    prot = [0, 5]
    lay = layout(D=D, L=L, H=H, T=T)
    fixed = np.full((L, 2), 0.5, np.float32)
    codec = kvc.Codec(ck, cv, seed=1, fixed_scales=fixed, protected_layers=prot, layers=L)
    slot, spill, bpt = kvc.kvc_plan(lay, codec, n)
    offs, sizes, effs, total = O.plan(L, H, D, T, kvc.CODECS[ck], kvc.CODECS[cv],
                                      [1 if l in prot else 0 for l in range(L)], n)
    assert slot == total
    per_page = sum(sizes[:2 * L * n:2 * n]) + sum(sizes[1:2 * L * n:2 * n])
    assert bpt == -(-per_page // T)
    assert spill >= 256 * -(-H * T * D * 2 // 256)


def test_plan_pages_sizes_d128():
    """16 tokens x 8 heads x D128 per segment: 128 vectors at the pages'
    66/68 (4-bit) and 50/52 (3-bit) bytes plus the 32-byte header, rounded to
    256 bytes."""
    for ck, cv, kb, vb in (("TQ4", "UNIFORM4", 66, 68), ("TQ3", "UNIFORM3", 50, 52)):
        lay = layout(L=1)
        slot, _, bpt = kvc.kvc_plan(lay, kvc.Codec(ck, cv), 1)
        exp = sum(-(-(32 + 128 * b) // 256) * 256 for b in (kb, vb))
        assert slot == exp


def _st(fn, *a):
    return fn(*a)


def test_validation_errors():
    codec = kvc.Codec("TQ4", "UNIFORM4")
    ok = layout()
    ids = np.arange(10, dtype=np.int32)
    slot, _, _ = kvc.kvc_plan(ok, codec, 10)
    V = kvc.kvc_validate_encode
    assert V(ok, codec, ids, slot) == kvc.KVC_OK
    assert V(ok, codec, ids, slot - 1) == kvc.KVC_E_CAPACITY
    assert V(layout(D=96), codec, ids, slot) == kvc.KVC_E_UNSUPPORTED
    assert V(layout(D=512), codec, ids, slot) == kvc.KVC_E_UNSUPPORTED
    assert V(layout(dtype=3), codec, ids, slot) == kvc.KVC_E_UNSUPPORTED
    assert V(ok, codec, np.array([0, 100], np.int32), slot) == kvc.KVC_E_PAGE_RANGE
    assert V(ok, codec, np.array([-1], np.int32), slot) == kvc.KVC_E_PAGE_RANGE
    # strides must be positive multiples of 8 and non-overlapping for the kind
    assert V(layout(strides=(16 * 8 * 128, 8 * 128, 100)), codec, ids, slot) == kvc.KVC_E_ARG
    assert V(layout(strides=(16 * 8 * 128, 8 * 64, 128)), codec, ids, slot) == kvc.KVC_E_ARG
    assert V(layout(kind=kvc.KVC_PACKED_HT2D, strides=(8 * 16 * 128, 128, 16 * 128)), codec, ids,
             slot) == kvc.KVC_E_ARG
    # packed layout must not carry V pointers, separate must
    bad = layout()
    bad.c.v_base = None
    assert V(bad, codec, ids, slot) == kvc.KVC_E_ARG
    # unaligned base pointer
    lay = layout()
    lay._k[1] = FAKE + 8
    assert V(lay, codec, ids, slot) == kvc.KVC_E_ARG
    # FP8_FIXED needs sane scales
    assert V(ok, kvc.Codec("FP8_FIXED", "RAW"), ids, 1 << 40) == kvc.KVC_E_ARG
    for badscale in (0.0, -1.0, np.inf, np.nan, 1e-35):
        fs = np.full((4, 2), 1.0, np.float32)
        fs[2, 0] = badscale
        assert V(ok, kvc.Codec("FP8_FIXED", "RAW", fixed_scales=fs), ids, 1 << 40) == kvc.KVC_E_ARG
    assert V(ok, kvc.Codec(11, 0), ids, 1 << 40) == kvc.KVC_E_ARG
    # codec flags: only KVC_CODEC_CRC32 is defined; reserved must be 0
    assert V(ok, kvc.Codec("TQ4", "UNIFORM4", crc=True), ids, 1 << 40) == kvc.KVC_OK
    c = kvc.Codec("TQ4", "UNIFORM4")
    c.c.flags = 2
    assert V(ok, c, ids, 1 << 40) == kvc.KVC_E_ARG
    c.c.flags, c.c.reserved = kvc.KVC_CODEC_CRC32, 1
    assert V(ok, c, ids, 1 << 40) == kvc.KVC_E_ARG
    # the entropy stage needs the segment CRC32 (a corrupted stream shows only after decoding)
    for pair in (("ANS16", "INT8"), ("TQ4", "ANS16"), ("ANS16", "ANS16")):
        assert V(ok, kvc.Codec(*pair), ids, 1 << 40) == kvc.KVC_E_ARG
        assert V(ok, kvc.Codec(*pair, crc=True), ids, 1 << 40) == kvc.KVC_OK
        assert kvc.kvc_validate_decode(ok, kvc.Codec(*pair), ids, 1 << 40) == kvc.KVC_E_ARG
    lay_old = layout()
    lay_old.c.abi = 1                                   # callers built against the previous ABI
    assert V(lay_old, kvc.Codec("TQ4", "UNIFORM4"), ids, 1 << 40) == kvc.KVC_E_ARG


def test_decode_rejects_duplicate_destinations():
    codec = kvc.Codec("INT8", "INT8")
    ok = layout()
    slot, _, _ = kvc.kvc_plan(ok, codec, 3)
    assert kvc.kvc_validate_decode(ok, codec, np.array([3, 7, 9], np.int32), slot) == kvc.KVC_OK
    assert kvc.kvc_validate_decode(ok, codec, np.array([3, 7, 3], np.int32), slot) == kvc.KVC_E_DUP_DST
    # encode may read the same page twice
    assert kvc.kvc_validate_encode(ok, codec, np.array([3, 7, 3], np.int32), slot) == kvc.KVC_OK


def test_keep_rule_makes_tiny_segments_raw():
    # 1 token x 1 head x D32: a 256-B slot never saves 12.5% of 64 B -> raw slot
    lay = layout(H=1, T=1, D=32, L=1)
    slot, _, _ = kvc.kvc_plan(lay, kvc.Codec("INT8", "TQ4"), 1)
    assert slot == 2 * 256


def test_lane_and_layer_entry_points_validate_first():
    """kvc_decode_layers / kvc_offload_pages / kvc_restore_pages reject a
    missing context and bad layer ranges on the host, before any GPU call
    (the fake context below is never dereferenced)."""
    codec = kvc.Codec("INT8", "INT8")
    lay = layout(L=4)
    ids = np.arange(3, dtype=np.int32)
    idp = ids.ctypes.data_as(ctypes.c_void_p)
    slot, _, _ = kvc.kvc_plan(lay, codec, 3)
    L = kvc.lib()
    lc, cc = ctypes.byref(lay.c), ctypes.byref(codec.c)
    assert L.kvc_offload_pages(None, lc, cc, idp, 3, None, slot, None, None, None) == kvc.KVC_E_ARG
    assert L.kvc_restore_pages(None, lc, cc, None, slot, idp, 3, 0, 4, None, None, None) == kvc.KVC_E_ARG
    assert L.kvc_decode_layers(None, lc, cc, None, slot, idp, 3, 0, 4, None, None) == kvc.KVC_E_ARG
    fake = ctypes.c_void_p(16)
    for lb, le in ((3, 5), (2, 1), (0, 5)):
        assert L.kvc_decode_layers(fake, lc, cc, None, slot, idp, 3, lb, le, None, None) == kvc.KVC_E_ARG
        assert L.kvc_restore_pages(fake, lc, cc, None, slot, idp, 3, lb, le, None, None, None) == kvc.KVC_E_ARG
    # the usual validation comes first: capacity, duplicate destinations
    assert L.kvc_decode_layers(fake, lc, cc, None, slot - 1, idp, 3, 0, 1, None, None) == kvc.KVC_E_CAPACITY
    dup = np.array([1, 1, 2], np.int32)
    assert L.kvc_restore_pages(fake, lc, cc, None, slot, dup.ctypes.data_as(ctypes.c_void_p), 3, 0, 1, None,
                               None, None) == kvc.KVC_E_DUP_DST


def test_plan_int8_records_qwen3_row():
    """The INT8 record codec at 8 heads x D128: each token costs one
    1,152-byte row per component (the page's record), plus the slot's
    128-byte lead and its 256-byte rounding."""
    lay = layout(L=1, H=8, D=128, T=16)
    slot, _, bpt = kvc.kvc_plan(lay, kvc.Codec("INT8_ROWS", "INT8_ROWS"), 1)
    assert slot == 2 * ((128 + 16 * 1152 + 255) // 256 * 256)
    assert bpt == -(-slot // 16)


def test_create_checks_before_touching_a_device():
    """kvc_create rejects a missing out pointer and a workspace budget too
    small for its tables before any HIP call; kvc_destroy(NULL) is a no-op."""
    L = kvc.lib()
    h = ctypes.c_void_p(1)
    assert L.kvc_create(None, 0, 0) == kvc.KVC_E_ARG
    assert L.kvc_create(ctypes.byref(h), 0, 4096) == kvc.KVC_E_BUDGET
    assert h.value is None                              # *out cleared on failure
    assert L.kvc_destroy(None) == kvc.KVC_OK


def test_noalloc_encode_validates_before_the_device():
    """kvc_encode_pages_noalloc checks its arguments on the host like
    kvc_encode_pages, and rejects calls beyond its fixed scratch (more than
    256 layers or 65,536 pages) with KVC_E_BUDGET, before any GPU call (the
    fake tensor pointers below are never dereferenced)."""
    codec = kvc.Codec("TQ4", "UNIFORM4")
    L = kvc.lib()
    lay = layout()
    cc = ctypes.byref(codec.c)
    big = np.zeros(65537, np.int32)
    bp = big.ctypes.data_as(ctypes.c_void_p)
    assert L.kvc_encode_pages_noalloc(ctypes.byref(lay.c), cc, bp, 65537, None, 1 << 40, None, None) == \
        kvc.KVC_E_BUDGET
    deep = layout(L=257)
    ids = np.arange(3, dtype=np.int32)
    ip = ids.ctypes.data_as(ctypes.c_void_p)
    assert L.kvc_encode_pages_noalloc(ctypes.byref(deep.c), cc, ip, 3, None, 1 << 40, None, None) == \
        kvc.KVC_E_BUDGET
    slot, _, _ = kvc.kvc_plan(lay, codec, 3)
    assert L.kvc_encode_pages_noalloc(ctypes.byref(lay.c), cc, ip, 3, None, slot - 1, None, None) == \
        kvc.KVC_E_CAPACITY
    assert L.kvc_encode_pages_noalloc(ctypes.byref(layout(D=96).c), cc, ip, 3, None, slot, None, None) == \
        kvc.KVC_E_UNSUPPORTED
    bad = np.array([0, 100], np.int32)
    assert L.kvc_encode_pages_noalloc(ctypes.byref(lay.c), cc, bad.ctypes.data_as(ctypes.c_void_p), 2, None,
                                      1 << 40, None, None) == kvc.KVC_E_PAGE_RANGE
    # output and descriptor pointers are checked after the plan, still on the host
    assert L.kvc_encode_pages_noalloc(ctypes.byref(lay.c), cc, ip, 3, None, slot, None, None) == kvc.KVC_E_ARG
