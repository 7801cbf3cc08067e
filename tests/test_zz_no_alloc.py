"""kvc_encode_pages_noalloc against kvc_encode_pages through the C ABI.

The allocation-free entry point keeps its per-call tables and spill cursor
in a fixed device array per GPU; its output must be the existing entry
point's, byte for byte, on two calls in a row -- the second smaller, so
that a spill cursor or side table left over from the first call would show.
Data-raw and entropy-coded segments sit in the spill region in the order
their workgroups reached the cursor, which need not be the same between
two runs: for them the slot header is compared without its spill offset,
and the stored bytes at each side's own offset.
"""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():      # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_page_kvc_amd as kvc                      # noqa: E402
from kv_cache_page_kvc_amd import inputs                 # noqa: E402
from tests import gpu_helpers as G                       # noqa: E402


def _run(fn, wl, codec, ids, spill):
    slot, _, _ = kvc.kvc_plan(wl.layout, codec, len(ids))
    total = slot + spill
    out = torch.full((total,), 0xA5, dtype=torch.uint8, device="cuda")
    desc = torch.zeros(wl.L * len(ids) * 2 * 32, dtype=torch.uint8, device="cuda")
    fn(out, total, desc)
    torch.cuda.synchronize()
    return out.cpu().numpy(), G.desc_np(desc), slot, total


def _same(a, b, slot):
    (ga, da), (gb, db) = a, b
    assert len(da) == len(db)
    for s in range(len(da)):
        x, y = da[s], db[s]
        for f in ("offset", "stored_len", "original_len", "version", "format", "flags", "status", "crc32"):
            assert x[f] == y[f], (s, f, x[f], y[f])
        o = int(x["offset"])
        if int(x["flags"]) & (kvc.KVC_FLAG_RAW_DATA | kvc.KVC_FLAG_HEAP) and int(x["status"]) != kvc.KVC_SEG_CAPACITY:
            assert np.array_equal(ga[o:o + 16], gb[o:o + 16]) and np.array_equal(ga[o + 24:o + 32], gb[o + 24:o + 32])
            sa, sb = int(x["spill_offset"]), int(y["spill_offset"])
            assert sa >= slot and sb >= slot
            n = int(x["stored_len"])
            assert np.array_equal(ga[sa:sa + n], gb[sb:sb + n]), s
        else:
            assert x["spill_offset"] == y["spill_offset"], s
    # every slot byte outside the spill offsets of spilled segments
    mask = np.ones(slot, bool)
    for s in range(len(da)):
        if int(da[s]["flags"]) & (kvc.KVC_FLAG_RAW_DATA | kvc.KVC_FLAG_HEAP):
            o = int(da[s]["offset"])
            mask[o + 16:o + 24] = False
    assert np.array_equal(ga[:slot][mask], gb[:slot][mask])


@pytest.mark.parametrize("pair,crc", [(("TQ4", "UNIFORM4"), False), (("INT8", "FP8_DYNAMIC"), True),
                                      (("ANS16", "FP8_DIRECT"), True)], ids=lambda p: str(p))
def test_noalloc_encode_matches_encode(pair, crc):
    ctx = kvc.kvc_create(0, 0)
    try:
        for n_pages, seed in ((24, 1), (10, 2)):            # the second call is smaller
            print(f"[case] noalloc {pair} crc={crc} pages={n_pages}", flush=True)
            L, H, D, T, pool = 4, 8, 128, 16, 32
            wl = G.Workload(L, H, D, T, pool, "bf16", "separate", seed)
            ids = inputs.random_page_ids(pool, n_pages, seed=seed)
            inputs.inject_specials(wl.k, wl.v, ids, frac=0.1, seed=seed, controls=4)
            codec = kvc.Codec(pair[0], pair[1], seed=7 + seed, protected_layers=[3], layers=L, crc=crc)
            spill = L * n_pages * 2 * (H * T * D * 2)     # room for every segment
            ref = _run(lambda o, t, d: kvc.kvc_encode_pages(ctx, wl.layout, codec, ids, o.data_ptr(), t,
                                                            d.data_ptr()), wl, codec, ids, spill)
            got = _run(lambda o, t, d: kvc.kvc_encode_pages_noalloc(wl.layout, codec, ids, o.data_ptr(), t,
                                                                    d.data_ptr()), wl, codec, ids, spill)
            assert ref[2] == got[2]
            st = ref[1]["status"]
            assert (st == kvc.KVC_SEG_RAW_DATA).sum() > 0 or pair[0] == "ANS16"
            _same((got[0], got[1]), (ref[0], ref[1]), ref[2])
            # the spill cursor started at zero: spilled bytes are packed from the slot region's end
            d = got[1]
            sp = d[(d["flags"] & (kvc.KVC_FLAG_RAW_DATA | kvc.KVC_FLAG_HEAP)) != 0]
            used = int(((sp["stored_len"].astype(np.int64) + 255) // 256 * 256).sum())
            if len(sp):
                assert int(sp["spill_offset"].min()) == got[2]
                assert int((sp["spill_offset"].astype(np.int64) + sp["stored_len"]).max()) <= got[2] + used
    finally:
        kvc.kvc_destroy(ctx)
