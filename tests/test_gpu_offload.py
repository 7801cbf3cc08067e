"""GPU tests of the offload lane and the layer-range decode, through the C ABI.

kvc_offload_pages must leave in pinned host memory exactly the bytes the
oracle encodes; kvc_restore_pages and kvc_decode_layers must write exactly
the oracle's decode into the destination pages of the requested layers and
nothing else, in stream order, signalling each layer's event only after that
layer's pages are written.  Staging growth while earlier transfers are still
queued must not disturb them.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():      # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_page_kvc_amd as kvc                      # noqa: E402
from kv_cache_page_kvc_amd import inputs                 # noqa: E402
from oracle import kvc_oracle as O                       # noqa: E402
from tests import gpu_helpers as G                       # noqa: E402

TQ_TOL = 1e-3
POISON = 0x7FC1                                          # NaN bits: never a decode result here


@pytest.fixture(scope="module")
def ctx():
    c = kvc.kvc_create(0, 0)
    yield c
    kvc.kvc_destroy(c)


def pinned(nbytes):
    return torch.zeros(max(nbytes, 1), dtype=torch.uint8, pin_memory=True)


class Case:
    """A small call: workload, codec, page ids, and the oracle's encode (with
    a CRC32 per segment by default: the lane always stores one)."""

    def __init__(self, ck, cv, L=4, H=8, D=128, T=16, pool=40, n=13, seed=5, protected=None, crc=True,
                 inject=False, layout="separate", dtype="bf16"):
        self.wl = G.Workload(L, H, D, T, pool, dtype, layout, seed)
        self.ids = inputs.random_page_ids(pool, n, seed=seed + 1)
        if inject:
            inputs.inject_specials(self.wl.k, self.wl.v, self.ids, frac=0.2, seed=seed, controls=4)
        self.kc, self.vc = kvc.CODECS[ck], kvc.CODECS[cv]
        self.protected = protected
        self.seed = seed
        self.codec = kvc.Codec(ck, cv, seed=seed, protected_layers=protected, layers=L, crc=crc)
        self.crc = crc
        self.nseg = L * n * 2
        self.slot, spill, _ = kvc.kvc_plan(self.wl.layout, self.codec, n)
        if inject:                      # room to spill every segment: no CAPACITY statuses
            spill = self.nseg * ((T * H * D * 2 + 255) // 256 * 256)
        self.total = self.slot + spill
        self.ora_buf, self.ora_st, self.offs, ora_total = G.oracle_encode(
            self.wl, self.kc, self.vc, seed, self.ids, protected=protected, crc=crc)
        assert ora_total == self.slot

    def check_encoded(self, buf: np.ndarray, desc: np.ndarray):
        bad = G.compare_encoded(buf, desc, self.ora_buf, self.ora_st, self.offs, self.slot, range(self.nseg))
        assert not bad, f"encode mismatches (first 5 of {len(bad)}): {bad[:5]}"

    def check_decoded(self, dst, layers, dst_ids=None):
        """Restored layers equal the oracle decode; the others keep the poison."""
        dst_ids = self.ids if dst_ids is None else dst_ids
        segs = G.segments_of(self.wl.L, len(self.ids))
        want = [s for s in range(self.nseg) if segs[s][0] in layers]
        ora = G.oracle_decode_segments(self.ora_buf, self.wl, self.kc, self.vc, self.seed, len(self.ids),
                                       self.protected, want)
        for s in range(self.nseg):
            l, i, c = segs[s]
            got = G.gpu_segment_vectors(dst, l, c, int(dst_ids[i]))
            if l not in layers:
                assert np.all(got == POISON), f"layer {l} written outside the restored range"
                continue
            tq = (self.kc if c == 0 else self.vc) in (kvc.KVC_TQ3, kvc.KVC_TQ4) and self.ora_st[s] == 0
            if not tq:
                assert np.array_equal(got, ora[s]), f"segment {s} decode bits differ"
            else:
                a = G.bits_to_f32(got, self.wl.dt).astype(np.float64)
                b = G.bits_to_f32(ora[s], self.wl.dt).astype(np.float64)
                assert np.abs(a - b).max() <= TQ_TOL, f"segment {s} TurboQuant decode differs"


CASES = {
    "tq4-u4-prot": dict(ck="TQ4", cv="UNIFORM4", protected=[0]),
    "int8-fp8dyn-spill": dict(ck="INT8", cv="FP8_DYNAMIC", inject=True),
    "tq3-u3-d256-packed-fp16": dict(ck="TQ3", cv="UNIFORM3", D=256, H=4, layout="packed", dtype="fp16"),
    "int8rows-u4": dict(ck="INT8_ROWS", cv="UNIFORM4"),
    "ans16-fp8dyn": dict(ck="ANS16", cv="FP8_DYNAMIC"),
    "ans16-ans16-prot": dict(ck="ANS16", cv="ANS16", protected=[1]),
    "tq4-u4-nocrc-codec": dict(ck="TQ4", cv="UNIFORM4", crc=False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_offload_then_restore(ctx, name):
    """Offload to pinned host memory equals the oracle's encode with a CRC32
    per segment (the lane adds it to a codec without one); only the slot
    region and the spill bytes the encode used are copied -- the rest of
    the host buffer keeps its previous bytes -- and the size returned
    counts exactly those.  A restore of all layers from those bytes equals
    the oracle's decode, statuses 0."""
    print(f"[case] offload/restore {name}", flush=True)
    cs = Case(**CASES[name])
    if not cs.crc:                      # the lane's own CRC: compare with the oracle's CRC encode
        cs = Case(**dict(CASES[name], crc=True))
        codec = kvc.Codec(CASES[name]["ck"], CASES[name]["cv"], seed=cs.seed, protected_layers=cs.protected,
                          layers=cs.wl.L, crc=False)
    else:
        codec = cs.codec
    host = pinned(cs.total)
    host.fill_(0xA7)
    hdesc = pinned(cs.nseg * 32)
    used = kvc.kvc_offload_pages(ctx, cs.wl.layout, codec, cs.ids, host.data_ptr(), cs.total, hdesc.data_ptr())
    torch.cuda.synchronize()
    hb = host.numpy()
    d = hdesc.numpy().view(kvc.DESC_DTYPE)
    spilled = (d["flags"] & (kvc.KVC_FLAG_RAW_DATA | kvc.KVC_FLAG_HEAP)) != 0
    spilled &= d["status"] != kvc.KVC_SEG_CAPACITY
    expect = cs.slot + int(((d["stored_len"][spilled].astype(np.int64) + 255) // 256 * 256).sum())
    assert used == expect, (used, expect)
    assert np.all(hb[used:] == 0xA7), "bytes beyond the used spill region were copied"
    cs.check_encoded(hb, d)

    dst = cs.wl.empty_like(fill_bits=POISON)
    st = torch.full((cs.nseg,), 255, dtype=torch.uint8, device="cuda")
    kvc.kvc_restore_pages(ctx, dst.layout, codec, host.data_ptr(), used, cs.ids, 0, cs.wl.L, st.data_ptr())
    torch.cuda.synchronize()
    assert np.all(st.cpu().numpy() == 0)
    cs.check_decoded(dst, set(range(cs.wl.L)))


@pytest.mark.parametrize("pair", [("TQ4", "UNIFORM4"), ("ANS16", "ANS16")], ids=lambda p: f"{p[0]}-{p[1]}")
def test_restore_layer_ranges_signal_each_layer(ctx, pair):
    """Three restores over [0,1), [1,3), [3,4) into shuffled destination pages,
    each layer with its own event: a consumer stream that waits on a layer's
    event reads that layer fully restored; layers not yet restored keep the
    poison.  (ANS16 payloads sit in the spill region, which every restore
    copies before its first layer.)"""
    print(f"[case] restore by layer ranges {pair}", flush=True)
    cs = Case(pair[0], pair[1], L=4, n=11, seed=9, protected=[3])
    host = pinned(cs.total)
    hdesc = pinned(cs.nseg * 32)
    kvc.kvc_offload_pages(ctx, cs.wl.layout, cs.codec, cs.ids, host.data_ptr(), cs.total, hdesc.data_ptr())
    torch.cuda.synchronize()
    dst_ids = np.random.default_rng(3).permutation(cs.ids).astype(np.int32)
    dst = cs.wl.empty_like(fill_bits=POISON)
    st = torch.full((cs.nseg,), 255, dtype=torch.uint8, device="cuda")
    restore = torch.cuda.Stream()
    consumer = torch.cuda.Stream()
    events = [torch.cuda.Event() for _ in range(cs.wl.L)]
    for e in events:                    # create the HIP events (torch creates them on first record)
        e.record()
    torch.cuda.synchronize()
    done = []
    for lb, le in ((0, 1), (1, 3), (3, 4)):
        kvc.kvc_restore_pages(ctx, dst.layout, cs.codec, host.data_ptr(), cs.total, dst_ids, lb, le,
                              st.data_ptr(), [events[l].cuda_event for l in range(lb, le)],
                              restore.cuda_stream)
        copies = []
        with torch.cuda.stream(consumer):
            for l in range(lb, le):
                consumer.wait_event(events[l])
                copies.append((l, dst.k[l].clone(), dst.v[l].clone()))
        consumer.synchronize()
        restore.synchronize()
        done += list(range(lb, le))
        cs.check_decoded(dst, set(done), dst_ids)
        for l, kc_, vc_ in copies:      # what the consumer saw after waiting on the event
            assert torch.equal(kc_.view(torch.int16), dst.k[l].view(torch.int16))
            assert torch.equal(vc_.view(torch.int16), dst.v[l].view(torch.int16))
    assert np.all(st.cpu().numpy() == 0)


@pytest.mark.parametrize("pair", [("INT8", "FP8_DIRECT"), ("ANS16", "INT8")], ids=lambda p: f"{p[0]}-{p[1]}")
def test_decode_layers_device_buffer(ctx, pair):
    """kvc_decode_layers over a device buffer: only the requested layers are
    written, and their pages equal the oracle's decode."""
    print(f"[case] decode_layers {pair}", flush=True)
    cs = Case(pair[0], pair[1], L=5, n=9, seed=21)
    out, desc, slot, total = G.gpu_encode(ctx, cs.wl, cs.codec, cs.ids)
    torch.cuda.synchronize()
    cs.check_encoded(out.cpu().numpy(), G.desc_np(desc))
    dst = cs.wl.empty_like(fill_bits=POISON)
    st = torch.full((cs.nseg,), 255, dtype=torch.uint8, device="cuda")
    kvc.kvc_decode_layers(ctx, dst.layout, cs.codec, out.data_ptr(), total, cs.ids, 1, 4, st.data_ptr())
    torch.cuda.synchronize()
    cs.check_decoded(dst, {1, 2, 3})
    segs = G.segments_of(cs.wl.L, len(cs.ids))
    stn = st.cpu().numpy()
    for s in range(cs.nseg):
        assert stn[s] == (0 if segs[s][0] in (1, 2, 3) else 255)


def test_staging_grows_while_transfers_are_queued(ctx):
    """Offloads and restores of growing size on two streams, queued back to
    back without host synchronisation: every staging buffer replaced by a
    larger one stays valid until the work queued on it has finished, and
    the two directions never share bytes."""
    print("[case] staging growth", flush=True)
    sizes = [3, 9, 26]
    cases = [Case("TQ4", "UNIFORM4", L=3, pool=64, n=n, seed=30 + n) for n in sizes]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    hosts, hdescs = [], []
    for i, cs in enumerate(cases):
        host, hdesc = pinned(cs.total), pinned(cs.nseg * 32)
        kvc.kvc_offload_pages(ctx, cs.wl.layout, cs.codec, cs.ids, host.data_ptr(), cs.total, hdesc.data_ptr(),
                              (s1 if i % 2 == 0 else s2).cuda_stream)
        hosts.append(host)
        hdescs.append(hdesc)
    torch.cuda.synchronize()
    for cs, host, hdesc in zip(cases, hosts, hdescs):
        cs.check_encoded(host.numpy(), hdesc.numpy().view(kvc.DESC_DTYPE))
    # restores of growing size, alternating streams, while a new offload runs
    dsts, sts = [], []
    extra = Case("INT8", "FP8_DYNAMIC", L=3, pool=64, n=40, seed=77)
    xhost, xdesc = pinned(extra.total), pinned(extra.nseg * 32)
    for i, (cs, host) in enumerate(zip(cases, hosts)):
        dst = cs.wl.empty_like(fill_bits=POISON)
        st = torch.full((cs.nseg,), 255, dtype=torch.uint8, device="cuda")
        kvc.kvc_restore_pages(ctx, dst.layout, cs.codec, host.data_ptr(), cs.total, cs.ids, 0, cs.wl.L,
                              st.data_ptr(), None, (s2 if i % 2 == 0 else s1).cuda_stream)
        if i == 1:
            kvc.kvc_offload_pages(ctx, extra.wl.layout, extra.codec, extra.ids, xhost.data_ptr(), extra.total,
                                  xdesc.data_ptr(), s1.cuda_stream)
        dsts.append(dst)
        sts.append(st)
    torch.cuda.synchronize()
    for cs, dst, st in zip(cases, dsts, sts):
        assert np.all(st.cpu().numpy() == 0)
        cs.check_decoded(dst, set(range(cs.wl.L)))
    extra.check_encoded(xhost.numpy(), xdesc.numpy().view(kvc.DESC_DTYPE))


def test_lane_rejects_pageable_memory_and_bad_ranges(ctx):
    """Host buffers must be pinned; layer ranges must lie inside the layout.
    Errors come back before anything is enqueued."""
    cs = Case("INT8", "INT8", L=2, n=3, seed=2)
    pageable = np.zeros(cs.total, np.uint8)
    hdesc = pinned(cs.nseg * 32)
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_offload_pages(ctx, cs.wl.layout, cs.codec, cs.ids, pageable.ctypes.data, cs.total,
                              hdesc.data_ptr())
    assert e.value.status == kvc.KVC_E_ARG
    host = pinned(cs.total)
    with pytest.raises(kvc.KvcError) as e:
        kvc.kvc_restore_pages(ctx, cs.wl.layout, cs.codec, pageable.ctypes.data, cs.total, cs.ids, 0, 2)
    assert e.value.status == kvc.KVC_E_ARG
    for lb, le in ((1, 0), (0, 3)):
        with pytest.raises(kvc.KvcError) as e:
            kvc.kvc_restore_pages(ctx, cs.wl.layout, cs.codec, host.data_ptr(), cs.total, cs.ids, lb, le)
        assert e.value.status == kvc.KVC_E_ARG
    with pytest.raises(kvc.KvcError) as e:                # a pinned buffer smaller than the plan
        kvc.kvc_offload_pages(ctx, cs.wl.layout, cs.codec, cs.ids, host.data_ptr(), cs.slot - 1,
                              hdesc.data_ptr())
    assert e.value.status == kvc.KVC_E_CAPACITY
