"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: encoded bytes (codes, metadata, headers, padding) and segment statuses
bit-exact for every codec; decoded values bit-exact for FP8, INT8, uniform
and raw; TurboQuant decodes within 1e-3 absolute and bit-equal up to the
sign of zero.  Small cases cover every codec, head dim, dtype and
layout over several tiles and a ragged page count; the workload-sized cases
run at full size in the launch configuration the benchmark times, checked
on every segment (all layers, K and V) of sampled pages.
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


@pytest.fixture(scope="module")
def ctx():
    c = kvc.kvc_create(0, 0)
    yield c
    kvc.kvc_destroy(c)


def _codec_ids(ck, cv):
    return kvc.CODECS[ck], kvc.CODECS[cv]


def _fixed_scales(L, seed=0):
    rng = np.random.default_rng(seed)
    return (2.0 ** rng.uniform(-9, -2, (L, 2))).astype(np.float32)


def _check_decoded(dec_gpu: np.ndarray, dec_ora: np.ndarray, dt, lossy_tq: bool, where=""):
    if not lossy_tq:
        assert np.array_equal(dec_gpu, dec_ora), f"decode bits differ {where}"
        return
    # TurboQuant: within the 1e-3 bound, and bit-equal -- both sides fix the
    # same binary32 operation order -- except that a zero may carry either sign
    a = G.bits_to_f32(dec_gpu, dt).astype(np.float64)
    b = G.bits_to_f32(dec_ora, dt).astype(np.float64)
    err = np.abs(a - b).max()
    assert err <= TQ_TOL, f"TurboQuant decode error {err} {where}"
    same = (dec_gpu == dec_ora) | (((dec_gpu & 0x7FFF) == 0) & ((dec_ora & 0x7FFF) == 0))
    assert same.all(), f"TurboQuant decode bits differ at {int((~same).sum())} elements {where}"


def _roundtrip_case(ctx, wl, ck, cv, seed, page_ids, protected=None, fixed=None, segments=None,
                    dst_ids=None, decode_from_oracle=True, spill_bytes=None, crc=False):
    """Encode on GPU and oracle; compare.  Decode (a) the oracle's buffer on
    the GPU and (b) the GPU's buffer on the GPU; compare both with the
    oracle's decode of its own buffer."""
    n_pages = len(page_ids)
    kc, vc = _codec_ids(ck, cv)
    codec = kvc.Codec(kc, vc, seed=seed, fixed_scales=fixed, protected_layers=protected, layers=wl.L, crc=crc)
    out, desc, slot, total = G.gpu_encode(ctx, wl, codec, page_ids, spill_bytes=spill_bytes)
    torch.cuda.synchronize()
    nseg = wl.L * n_pages * 2
    segs = list(range(nseg)) if segments is None else segments
    ora_buf, ora_st, offs, ora_total = G.oracle_encode(wl, kc, vc, seed, page_ids, fixed, protected, segs, crc=crc)
    assert ora_total == slot
    gbuf = out.cpu().numpy()
    gdesc = G.desc_np(desc)
    bad = G.compare_encoded(gbuf, gdesc, ora_buf, ora_st, offs, ora_total, segs)
    assert not bad, f"encode mismatches (first 5 of {len(bad)}): {bad[:5]}"

    dst_ids = np.asarray(page_ids if dst_ids is None else dst_ids, np.int32)
    ora_dec = G.oracle_decode_segments(ora_buf, wl, kc, vc, seed, n_pages, protected, segs)
    seglist = G.segments_of(wl.L, n_pages)
    lossy = lambda s: (kc if seglist[s][2] == 0 else vc) in (kvc.KVC_TQ3, kvc.KVC_TQ4) and ora_st[s] == 0

    runs = [("gpu-encoded", out, total)]
    if decode_from_oracle:
        runs.append(("oracle-encoded", torch.from_numpy(ora_buf).cuda(), ora_buf.size))
    for name, buf, nbytes in runs:
        dst = wl.empty_like(fill_bits=0x7FC1)            # NaN sentinel poison
        st = G.gpu_decode(ctx, dst, codec, buf, nbytes, dst_ids)
        torch.cuda.synchronize()
        stn = st.cpu().numpy()
        for s in segs:
            l, i, c = seglist[s]
            assert stn[s] == 0, f"{name}: decode status {stn[s]} for segment {s}"
            got = G.gpu_segment_vectors(dst, l, c, int(dst_ids[i]))
            _check_decoded(got, ora_dec[s], wl.dt, lossy(s), f"{name} segment {s}")
    return ora_st, gdesc


# ----------------------------------------------------------------- small grid
PAIRS = [("FP8_DIRECT", "FP8_DYNAMIC"), ("FP8_FIXED", "INT8"), ("TQ4", "UNIFORM4"),
         ("TQ3", "UNIFORM3"), ("UNIFORM4", "TQ3"), ("INT8", "RAW"), ("INT8_ROWS", "TQ4"), ("ANS16", "FP8_DYNAMIC")]


@pytest.mark.parametrize("layout", ["separate", "packed"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("dim", [32, 64, 128, 256])
@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-{p[1]}")
def test_small_grid(ctx, pair, dim, dtype, layout):
    """3 layers (layer 1 protected), 2 heads, 16 tokens, 5 of 11 blocks in
    random order: every segment compared, both decode directions."""
    print(f"[case] small {pair} D={dim} {dtype} {layout}", flush=True)
    L, H, T, pool = 3, 2, 16, 11
    wl = G.Workload(L, H, dim, T, pool, dtype, layout, seed=dim + (7 if dtype == "fp16" else 0))
    ids = inputs.random_page_ids(pool, 5, seed=dim)
    fixed = _fixed_scales(L) if "FP8_FIXED" in pair else None
    dst = inputs.random_page_ids(pool, 5, seed=dim + 1)
    _roundtrip_case(ctx, wl, pair[0], pair[1], seed=1234 + dim, page_ids=ids, protected=[1], fixed=fixed,
                    dst_ids=dst, crc="ANS16" in pair)


@pytest.mark.parametrize("layout", ["separate", "packed"])
@pytest.mark.parametrize("dim", [32, 64, 128, 256])
@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-{p[1]}")
def test_wide_grid(ctx, pair, dim, layout):
    """Segments of 32 KiB (16 tokens x 16384/D/16 heads), so the 256-thread
    workgroups and LDS-staged slots run for every codec pair and head_dim:
    2 layers (layer 0 protected), 3 of 6 blocks, every segment compared."""
    dtype = "bf16" if layout == "separate" else "fp16"
    H = 16384 // dim // 16
    print(f"[case] wide {pair} D={dim} H={H} {dtype} {layout}", flush=True)
    wl = G.Workload(2, H, dim, 16, 6, dtype, layout, seed=3 * dim + 1)
    ids = inputs.random_page_ids(6, 3, seed=dim + 5)
    fixed = _fixed_scales(2) if "FP8_FIXED" in pair else None
    dst = inputs.random_page_ids(6, 3, seed=dim + 6)
    _roundtrip_case(ctx, wl, pair[0], pair[1], seed=99 + dim, page_ids=ids, protected=[0], fixed=fixed,
                    dst_ids=dst, crc="ANS16" in pair)


@pytest.mark.parametrize("heads", [3, 12, 40])
@pytest.mark.parametrize("pair", [("TQ4", "UNIFORM4"), ("INT8", "FP8_DYNAMIC"), ("UNIFORM3", "INT8_ROWS")],
                         ids=lambda p: f"{p[0]}-{p[1]}")
def test_odd_head_counts(ctx, pair, heads):
    """Head counts that do not divide the group count (the per-lane vector
    walk wraps across tokens): 3 heads (12 KiB segments, one-wave
    workgroups), 12 (48 KiB) and 40 (160 KiB, slots above the 32 KiB LDS
    stage, written directly), D=128, every segment compared."""
    print(f"[case] heads={heads} {pair}", flush=True)
    wl = G.Workload(2, heads, 128, 16, 5, "bf16", "separate", seed=heads)
    ids = inputs.random_page_ids(5, 3, seed=heads)
    _roundtrip_case(ctx, wl, pair[0], pair[1], seed=7 + heads, page_ids=ids, dst_ids=ids[::-1].copy())


@pytest.mark.parametrize("shape", [(1, 8), (3, 5), (5, 7), (2, 24)], ids=lambda s: f"H{s[0]}-T{s[1]}")
@pytest.mark.parametrize("dim", [32, 128])
@pytest.mark.parametrize("pair", [("TQ4", "UNIFORM4"), ("INT8", "FP8_DYNAMIC"), ("TQ3", "INT8_ROWS")],
                         ids=lambda p: f"{p[0]}-{p[1]}")
def test_ragged_vector_counts(ctx, pair, dim, shape):
    """Separate layouts whose heads x tokens is not a multiple of a
    workgroup's batch of vectors (the general loop with a ragged last batch)
    next to one that is (H2-T24 at D=32): every segment compared."""
    H, T = shape
    print(f"[case] ragged {pair} D={dim} H={H} T={T}", flush=True)
    wl = G.Workload(2, H, dim, T, 5, "bf16", "separate", seed=H * 100 + T)
    ids = inputs.random_page_ids(5, 3, seed=T)
    _roundtrip_case(ctx, wl, pair[0], pair[1], seed=5 + H + T, page_ids=ids, dst_ids=ids[::-1].copy())


def test_fp8_dynamic_small_full(ctx):
    """FP8 E4M3FN dynamic workload, 2 layers x 8 heads x D128 BF16, 64 pages:
    all 256 segments."""
    cfg = inputs.CONFIGS["fp8_dynamic_small"]
    print("[case] fp8_dynamic_small", flush=True)
    wl = G.Workload(cfg["layers"], cfg["heads"], cfg["dim"], cfg["tokens"], cfg["pool"], "bf16", "separate", 0)
    ids = np.arange(cfg["pages"], dtype=np.int32)
    _roundtrip_case(ctx, wl, "FP8_DYNAMIC", "FP8_DYNAMIC", 0, ids)


def test_fp8_direct_every_source_value(ctx):
    """Hardware E4M3FN conversion: every finite BF16 and FP16 pattern with
    |x| <= 448, packed into segments, must encode to the oracle's codes."""
    for dtype in ("bf16", "fp16"):
        print(f"[case] fp8 exhaustive {dtype}", flush=True)
        h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        x = O.src_to_f32(h, O.BF16 if dtype == "bf16" else O.FP16)
        vals = h[np.isfinite(x) & (np.abs(x) <= 448)]
        H, D, T = 8, 128, 16
        per_page = T * H * D
        n_pages = -(-vals.size // per_page)
        pool = np.resize(vals, n_pages * per_page).reshape(n_pages, T, H, D)
        wl = G.Workload(1, H, D, T, n_pages, dtype, "separate", 0)
        wl.k[0].view(torch.int16).copy_(torch.from_numpy(pool.view(np.int16)).cuda())
        wl.v[0].view(torch.int16).copy_(torch.from_numpy(pool[::-1].copy().view(np.int16)).cuda())
        ids = np.arange(n_pages, dtype=np.int32)
        _roundtrip_case(ctx, wl, "FP8_DIRECT", "FP8_DIRECT", 0, ids)


def test_fp8_scaled_quotients(ctx):
    """Scaled FP8 over many FP32 quotients: fixed scales spanning 2^-12..2^4
    (clipping included) and dynamic scales."""
    print("[case] fp8 scaled sweep", flush=True)
    L, H, D, T, pool = 4, 8, 128, 16, 24
    wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 5)
    fixed = (2.0 ** np.linspace(-12, 4, 2 * L)).reshape(L, 2).astype(np.float32) * 1.37
    ids = np.arange(pool, dtype=np.int32)
    _roundtrip_case(ctx, wl, "FP8_FIXED", "FP8_DYNAMIC", 0, ids, fixed=fixed)


def test_fp8_fixed_scales_around_the_division_shortcut(ctx):
    """FP8 fixed scales below, at and above the bounds of the encoder's
    division shortcut (2^-60 and 2^60; the IEEE division outside them), and
    the host's own bounds 2^-100 and 2^100.  Layers with a scale below 1 hold
    BF16 sources of about 64 times their scale, so their quotients span the
    E4M3 range (clipping included); larger scales see N(0,1)-sized sources.
    Slots bit-exact with the oracle's IEEE quotients, pages identical."""
    print("[case] fp8 fixed scales around 2^-60 and 2^60", flush=True)
    lo, hi = np.float32(2.0 ** -60), np.float32(2.0 ** 60)
    scales = np.array([2.0 ** -100, 2.0 ** -80, np.nextafter(lo, np.float32(0)), lo, np.nextafter(lo, np.float32(1)),
                       0.0123, np.nextafter(hi, np.float32(0)), hi, np.nextafter(hi, np.float32(np.inf)), 2.0 ** 100],
                      np.float32)
    L, H, D, T, pool = len(scales) // 2, 2, 128, 16, 12
    fixed = scales.reshape(L, 2)
    wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 41)
    for l in range(L):
        for comp, t in ((0, wl.k[l]), (1, wl.v[l])):
            s = float(fixed[l, comp])
            if s < 1.0:
                t.mul_(64.0 * s)
    ids = np.arange(pool, dtype=np.int32)
    _roundtrip_case(ctx, wl, "FP8_FIXED", "FP8_FIXED", 0, ids, fixed=fixed)


def test_zero_and_tiny_vectors(ctx):
    """All-zero vectors (INT8/FP8 floor, TurboQuant n = 0, uniform sigma = 0)
    and subnormal-scale vectors."""
    print("[case] zero/tiny", flush=True)
    for ck, cv in (("INT8", "FP8_DYNAMIC"), ("TQ4", "UNIFORM4"), ("TQ3", "UNIFORM3")):
        wl = G.Workload(2, 4, 64, 16, 6, "bf16", "separate", 9)
        for t in wl.k + wl.v:
            t[0].zero_()
            t[1].mul_(1e-30)
            t[2].fill_(3.0)
        ids = np.arange(6, dtype=np.int32)
        _roundtrip_case(ctx, wl, ck, cv, 77, ids)


def test_uniform_sigma_fp16_midpoint(ctx):
    """FP16 vectors with max = 8.5859375, min = 0.005615234375: the binary32
    scale RN(RN(max - min)/15) is exactly the FP16 midpoint 0.572021484375, so
    the stored FP16 scale must be its even neighbour 0.572265625 (0x3894), as
    in the oracle -- not a single rounding of an unrounded quotient."""
    print("[case] uniform sigma FP16 midpoint", flush=True)
    wl = G.Workload(1, 4, 32, 16, 2, "fp16", "separate", 3)
    for t in wl.k + wl.v:
        t[0].fill_(1.0)
        t[0][..., 0] = 8.5859375
        t[0][..., 1] = 0.005615234375
    ids = np.arange(2, dtype=np.int32)
    _roundtrip_case(ctx, wl, "UNIFORM4", "UNIFORM4", 0, ids)
    c = kvc.Codec("UNIFORM4", "UNIFORM4", seed=0, layers=1)
    out, desc, slot, total = G.gpu_encode(ctx, wl, c, np.zeros(1, np.int32))
    torch.cuda.synchronize()
    buf = out.cpu().numpy()
    n_vec = 4 * 16
    meta = buf[32 + n_vec * 16:32 + n_vec * 20].view(np.uint16).reshape(n_vec, 2)
    assert np.all(meta[:, 1] == 0x3894)


def test_uniform_signed_zero_extremes(ctx):
    """Vectors whose minimum (or, for all-zero vectors, both extremes) is a
    zero held as -0 and +0 in either order: the stored FP16 minimum and scale
    are the same as the oracle's (+0 for a zero extreme)."""
    print("[case] uniform signed zero extremes", flush=True)
    for bits in ("UNIFORM4", "UNIFORM3"):
        wl = G.Workload(1, 4, 64, 16, 4, "fp16", "separate", 5)
        for t in wl.k + wl.v:
            t[0].fill_(1.0)
            t[0].view(torch.int16)[..., 3] = -32768       # -0
            t[0].view(torch.int16)[..., 40] = 0           # +0
            t[1].fill_(2.0)
            t[1].view(torch.int16)[..., 3] = 0
            t[1].view(torch.int16)[..., 40] = -32768
            t[2].zero_()
            t[2].view(torch.int16)[::2, :, 1::3] = -32768
        ids = np.arange(4, dtype=np.int32)
        _roundtrip_case(ctx, wl, bits, bits, 0, ids)


def test_gate_small(ctx):
    """Injected NaN/Inf/|x|>448 values: the exact set of data-raw segments
    per codec, bit-exact raw round trip, +-448 controls stay encoded."""
    for ck, cv in (("INT8", "FP8_DIRECT"), ("FP8_DYNAMIC", "FP8_FIXED"), ("TQ4", "UNIFORM3")):
        print(f"[case] gate {ck}/{cv}", flush=True)
        L, H, D, T, pool = 4, 8, 128, 16, 40
        wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 11)
        ids = inputs.random_page_ids(pool, 32, seed=3)
        inj, ctl, kind = inputs.inject_specials(wl.k, wl.v, ids, frac=0.1, seed=4, controls=16)
        fixed = _fixed_scales(L) if "FP8_FIXED" in (ck, cv) else None
        # spill region large enough for every segment: no KVC_SEG_CAPACITY here
        ora_st, gdesc = _roundtrip_case(ctx, wl, ck, cv, 5, ids, fixed=fixed,
                                        dst_ids=inputs.permutation(pool, 1)[:32],
                                        spill_bytes=L * 32 * 2 * (H * T * D * 2))
        seglist = G.segments_of(L, 32)
        for s, (l, i, c) in enumerate(seglist):
            codec = ck if c == 0 else cv
            fp8 = codec.startswith("FP8")
            k = kind.get((l, i, c))
            expect_raw = k is not None and (fp8 or k in ("nan", "+inf", "-inf"))
            assert (gdesc[s]["status"] == kvc.KVC_SEG_RAW_DATA) == expect_raw, (s, codec, k)


def _bf16_row(vals):
    x = np.zeros(128, np.float32)
    x[:len(vals)] = vals
    return torch.from_numpy(O.f32_to_bf16(x).view(np.int16))


def test_fp16_metadata_overflow_goes_raw(ctx):
    """The FP16 metadata rule: a TurboQuant norm of exactly 65520 (FP16 inf)
    or above, a uniform minimum of -65536 or a uniform scale >= 65520 sends
    the segment raw; norms of 65519.996 and 65519.8, a minimum of -65280 and a
    scale of 64989.9 stay coded.  The exact set of data-raw segments, every
    slot byte and a bit-exact raw round trip against the oracle."""
    print("[case] FP16 metadata overflow", flush=True)
    L, H, D, T, pool = 2, 8, 128, 16, 10
    for ck, cv in (("TQ4", "UNIFORM4"), ("TQ3", "UNIFORM4")):
        wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 31)
        k_cases = [([65280.0, 5600.0, 160.0, 80.0], True), ([65280.0, 5600.0, 160.0, 64.0, 32.0, 32.0], False),
                   ([65280.0, 5632.0], True), ([65280.0, 5600.0], False)]
        v_cases = [({3: -65280.0}, False), ({3: -65536.0}, True), ({100: 974848.0}, False),
                   ({100: 983040.0}, True)]
        expect = {}
        for j, (vals, raw) in enumerate(k_cases):
            wl.k[j % L][j + 1, 5, 3] = _bf16_row(vals).cuda().view(torch.bfloat16)
            expect[(j % L, j + 1, 0)] = raw
        for j, (pos, raw) in enumerate(v_cases):
            row = O.src_to_f32(G.u16(wl.v[j % L][j + 5, 9, 1]), O.BF16).copy()
            for i, val in pos.items():
                row[i] = val
            wl.v[j % L][j + 5, 9, 1] = torch.from_numpy(O.f32_to_bf16(row).view(np.int16)).cuda().view(torch.bfloat16)
            expect[(j % L, j + 5, 1)] = raw
        ids = np.arange(pool, dtype=np.int32)
        ora_st, gdesc = _roundtrip_case(ctx, wl, ck, cv, 3, ids, dst_ids=inputs.permutation(pool, 2),
                                        spill_bytes=L * pool * 2 * (H * T * D * 2))
        for s, (l, i, c) in enumerate(G.segments_of(L, pool)):
            raw = expect.get((l, int(ids[i]), c), False)
            assert (gdesc[s]["status"] == kvc.KVC_SEG_RAW_DATA) == raw, (s, l, i, c)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_uniform_quotient_ties(ctx, dtype):
    """Uniform codes at the tie points of the quotient rule: vectors with
    minimum 0 and maximum 3 * (2^b - 1) (sigma_h = 3) whose elements are the
    half-integer multiples 1.5, 4.5, ... of the scale and their neighbours,
    so that the quotient RN(d / sigma_h) decides each code (the rounded
    reciprocal would give other codes); every slot byte against the oracle."""
    print(f"[case] uniform quotient ties {dtype}", flush=True)
    L, H, D, T, pool = 1, 4, 32, 16, 4
    for bits in (3, 4):
        codec = "UNIFORM3" if bits == 3 else "UNIFORM4"
        top = (1 << bits) - 1
        wl = G.Workload(L, H, D, T, pool, dtype, "separate", 40 + bits)
        conv = O.f32_to_bf16 if dtype == "bf16" else O.f32_to_f16
        dt = O.BF16 if dtype == "bf16" else O.FP16
        for b in range(pool):
            x = np.zeros((T, H, D), np.float32)
            x[..., 1] = 3.0 * top
            ties = np.array([1.5 + 3.0 * k for k in range(top)], np.float32)
            tb = conv(ties).astype(np.int32)
            step = (0, 1, -1, 2)[b]                       # units in the last place off the ties
            x[..., 2:2 + top] = O.src_to_f32((tb + step).astype(np.uint16), dt)
            for t in (wl.k[0], wl.v[0]):
                t[b] = torch.from_numpy(conv(x.ravel()).view(np.int16).reshape(T, H, D)).cuda().view(t.dtype)
        ids = np.arange(pool, dtype=np.int32)
        _roundtrip_case(ctx, wl, codec, codec, 0, ids)


def test_raw_data_unstaged_slot(ctx):
    """Segments of 40 heads (160 KiB, slots written straight to memory, not
    staged in LDS) that fall back to raw: the slot keeps only its header and
    is zero after it, the bytes go to the spill region, as in the oracle."""
    print("[case] raw data unstaged slot", flush=True)
    L, H, D, T, pool = 2, 40, 128, 16, 4
    wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 17)
    wl.k[0][1, 3, 7, 9] = float("nan")
    wl.v[1][2, 15, 39, 127] = float("inf")
    wl.v[0][3, 0, 0, 0] = 1000.0
    ids = np.arange(pool, dtype=np.int32)
    for ck, cv in (("TQ4", "UNIFORM4"), ("INT8", "FP8_DYNAMIC")):
        ora_st, gdesc = _roundtrip_case(ctx, wl, ck, cv, 5, ids, spill_bytes=4 * (H * T * D * 2))
        raw = {(0, 1, 0), (1, 2, 1)} | ({(0, 3, 1)} if cv == "FP8_DYNAMIC" else set())
        for s, (l, i, c) in enumerate(G.segments_of(L, pool)):
            assert (gdesc[s]["status"] == kvc.KVC_SEG_RAW_DATA) == ((l, i, c) in raw), (s, l, i, c)


def test_small_call_spill_cursor_slots_wrap():
    """Small encode calls take their spill cursor from a pool of 65,536 slots
    that are never cleared: each call's first reservation must start at
    offset 0 whatever an earlier call left in its slot.  65,539 calls in a
    row on one context (every slot used once, then three slots again), each
    with one data-raw segment: the raw bytes always land at the start of the
    spill region, and the last call's output equals the oracle's."""
    print("[case] small-call cursor slots wrap", flush=True)
    ctx = kvc.kvc_create(0, 0)
    try:
        L, H, D, T, pool = 1, 1, 128, 16, 4
        wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 23)
        wl.k[0][1, 5, 0, 7] = float("nan")
        ids = np.array([1, 3], np.int32)
        codec = kvc.Codec("INT8", "INT8", seed=0, layers=L)
        slot, _, _ = kvc.kvc_plan(wl.layout, codec, len(ids))
        spill = 2 * H * T * D * 2
        total = slot + spill
        out = torch.zeros(total, dtype=torch.uint8, device="cuda")
        desc = torch.zeros(L * len(ids) * 2 * 32, dtype=torch.uint8, device="cuda")
        firsts = []
        for k in range(65536 + 3):
            kvc.kvc_encode_pages(ctx, wl.layout, codec, ids, out.data_ptr(), total, desc.data_ptr())
            if k in (0, 1, 65535, 65536, 65537, 65538):
                torch.cuda.synchronize()
                d = G.desc_np(desc)
                assert int(d[0]["status"]) == kvc.KVC_SEG_RAW_DATA and int(d[0]["spill_offset"]) == slot, (k, d[0])
                firsts.append(k)
        torch.cuda.synchronize()
        assert len(firsts) == 6
        ora_buf, ora_st, offs, ora_total = G.oracle_encode(wl, kvc.KVC_INT8, kvc.KVC_INT8, 0, ids)
        bad = G.compare_encoded(out.cpu().numpy(), G.desc_np(desc), ora_buf, ora_st, offs, ora_total,
                                range(L * len(ids) * 2))
        assert not bad, bad[:5]
    finally:
        kvc.kvc_destroy(ctx)


def test_spill_capacity_exhausted(ctx):
    """A spill region for only two raw segments: later raw segments report
    KVC_SEG_CAPACITY; their destination pages are left untouched and the
    decode status says so; every other segment decodes."""
    print("[case] spill capacity", flush=True)
    L, H, D, T, pool = 2, 8, 128, 16, 16
    wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 12)
    ids = np.arange(pool, dtype=np.int32)
    inj = inputs.inject_specials(wl.k, wl.v, ids, frac=0.2, seed=6, controls=0)
    codec = kvc.Codec(kvc.KVC_INT8, kvc.KVC_INT8, seed=0)
    out, desc, slot, total = G.gpu_encode(ctx, wl, codec, ids, spill_bytes=2 * (32768 + 0))
    torch.cuda.synchronize()
    d = G.desc_np(desc)
    st = d["status"]
    _, _, kinds = inj
    n_inj = len([1 for k in kinds.values() if k in ("nan", "+inf", "-inf")])
    assert n_inj > 2
    assert (st == kvc.KVC_SEG_RAW_DATA).sum() == 2
    assert (st == kvc.KVC_SEG_CAPACITY).sum() == n_inj - 2
    dst = wl.empty_like(fill_bits=0x1234)
    dec = G.gpu_decode(ctx, dst, codec, out, total, ids)
    torch.cuda.synchronize()
    decn = dec.cpu().numpy()
    seglist = G.segments_of(L, pool)
    for s, (l, i, c) in enumerate(seglist):
        got = G.gpu_segment_vectors(dst, l, c, int(ids[i]))
        if st[s] == kvc.KVC_SEG_CAPACITY:
            assert decn[s] == 1 and np.all(got == 0x1234)
        else:
            assert decn[s] == 0 and not np.all(got == 0x1234)


def test_stream_ordered_and_untouched_pages(ctx):
    """Encode then decode on a side stream with no host sync in between;
    pages not named in the decode stay bit-identical."""
    print("[case] stream order", flush=True)
    L, H, D, T, pool = 3, 8, 128, 16, 20
    wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 13)
    ids = inputs.random_page_ids(pool, 8, seed=8)
    codec = kvc.Codec(kvc.KVC_TQ4, kvc.KVC_UNIFORM4, seed=42)
    s = torch.cuda.Stream()
    dst = wl.empty_like(fill_bits=0x4321)
    with torch.cuda.stream(s):
        out, desc, slot, total = G.gpu_encode(ctx, wl, codec, ids, stream=s.cuda_stream)
        st = G.gpu_decode(ctx, dst, codec, out, total, ids[::-1].copy(), stream=s.cuda_stream)
    s.synchronize()
    assert np.all(st.cpu().numpy() == 0)
    untouched = sorted(set(range(pool)) - set(int(x) for x in ids))
    for l in range(L):
        for c, tl in ((0, dst.k), (1, dst.v)):
            for b in untouched:
                assert np.all(G.u16(tl[l][b]) == 0x4321)


# ----------------------------------------------------------------- workload-sized
def _sample_segments(L, n_pages, count, seed, layers=None):
    rng = np.random.default_rng(seed)
    nseg = L * n_pages * 2
    segs = set(int(x) for x in rng.choice(nseg, size=count, replace=False))
    if layers:
        for l in layers:                                   # make sure policy-raw layers are covered
            segs.add((l * n_pages + int(rng.integers(n_pages))) * 2)
    return sorted(segs)


def _sample_pages(L, n_pages, count, seed):
    """Every segment (all layers, K and V) of `count` sampled positions in
    the call's page list: the oracle then copies only those pages."""
    rng = np.random.default_rng(seed)
    pos = rng.choice(n_pages, size=count, replace=False)
    return sorted(int((l * n_pages + int(i)) * 2 + c) for i in pos for l in range(L) for c in (0, 1))


@pytest.mark.parametrize("heads,codec_pair,raw", [(32, ("TQ4", "FP8_DYNAMIC"), False), (40, ("INT8", "UNIFORM4"), True)],
                         ids=["16MiB-coded", "20MiB-raw"])
def test_segment_size_limit(ctx, heads, codec_pair, raw):
    """Segments at the size limit: 1024 tokens x `heads` heads x D256 BF16 is
    16 MiB at 32 heads -- still coded, each in one workgroup writing its
    codes straight out (the slot exceeds the LDS staging limit) -- and 20 MiB
    at 40 heads, above the 16 MiB cap: stored raw by policy.  Every segment
    compared with the oracle, both directions."""
    print(f"[case] segment size limit heads={heads} {codec_pair}", flush=True)
    wl = G.Workload(1, heads, 256, 1024, 3, "bf16", "separate", seed=heads)
    ids = np.array([2, 0], np.int32)
    ora_st, gdesc = _roundtrip_case(ctx, wl, codec_pair[0], codec_pair[1], 5, ids, dst_ids=np.array([1, 2], np.int32))
    want = O.SEG_RAW_POLICY if raw else O.SEG_ENCODED
    assert all(int(v) == want for v in ora_st) and all(int(v) == want for v in gdesc["status"])


def test_tq4_u4_llama3_full_size(ctx):
    """TurboQuant-4 K + uniform-4 V, 32 layers x 8 heads x D128 BF16, 4096 of
    8192 blocks in random order, protected layers 0, 1, 30, 31: one full-size
    launch each way (as timed by the benchmark); every segment of 64 sampled
    pages (4096 segments, all layers) checked."""
    cfg = inputs.CONFIGS["tq4_u4_llama3"]
    print("[case] tq4_u4_llama3 full size", flush=True)
    wl = G.Workload(cfg["layers"], cfg["heads"], cfg["dim"], cfg["tokens"], cfg["pool"], "bf16", "separate", 0)
    ids = inputs.random_page_ids(cfg["pool"], cfg["pages"], seed=0)
    segs = _sample_pages(cfg["layers"], cfg["pages"], 64, 1)
    _roundtrip_case(ctx, wl, "TQ4", "UNIFORM4", 0, ids, protected=list(cfg["protected"]), segments=segs,
                    decode_from_oracle=False)


def test_tq4_u4_llama3_tp8_full_size(ctx):
    """One 8-way tensor-parallel shard of the TurboQuant-4 / uniform-4
    workload: 1 KV head, 4 KiB segments (one-wave workgroups), 4096 of 8192
    blocks, protected layers 0, 1, 30, 31; full-size launch, every segment
    of 128 sampled pages (8192 segments)."""
    cfg = inputs.CONFIGS["tq4_u4_llama3_tp8"]
    print("[case] tq4_u4_llama3 tp8 shard full size", flush=True)
    wl = G.Workload(cfg["layers"], cfg["heads"], cfg["dim"], cfg["tokens"], cfg["pool"], "bf16", "separate", 0)
    ids = inputs.random_page_ids(cfg["pool"], cfg["pages"], seed=0)
    segs = _sample_pages(cfg["layers"], cfg["pages"], 128, 4)
    _roundtrip_case(ctx, wl, "TQ4", "UNIFORM4", 0, ids, protected=list(cfg["protected"]), segments=segs,
                    decode_from_oracle=False)


@pytest.mark.parametrize("dim", [32, 64, 256])
def test_tq3_u3_dsweep_full_size(ctx, dim):
    """TurboQuant-3 K (outlier channels) + uniform-3 V, 28 layers x 4 heads,
    2048 pages: full-size launch, every segment of 32 sampled pages, 3-bit
    sizes."""
    cfg = inputs.CONFIGS["tq3_u3_dsweep"]
    print(f"[case] tq3_u3 D={dim} full size", flush=True)
    wl = G.Workload(cfg["layers"], cfg["heads"], dim, cfg["tokens"], cfg["pool"], "bf16", "separate", 0,
                    k_kind="outliers")
    ids = np.arange(cfg["pages"], dtype=np.int32)
    segs = _sample_pages(cfg["layers"], cfg["pages"], 32, dim)
    ora_st, gdesc = _roundtrip_case(ctx, wl, "TQ3", "UNIFORM3", 0, ids, segments=segs, decode_from_oracle=False)
    n_vec = cfg["heads"] * cfg["tokens"]
    assert set(gdesc["stored_len"][0::2]) == {n_vec * (3 * dim // 8 + 2)}
    assert set(gdesc["stored_len"][1::2]) == {n_vec * (3 * dim // 8 + 4)}


@pytest.mark.parametrize("vcodec", ["FP8_FIXED", "FP8_DYNAMIC"])
def test_k16v8_packed_full_size(ctx, vcodec):
    """vLLM packed FP16 [2048 blocks, 8 heads, 16 tokens, 256], 36 layers,
    K raw, V FP8 with a fixed per-layer scale (calibrated on sequence 0's V)
    or per-vector scales: full-size launch, every segment of 16 sampled pages."""
    cfg = inputs.CONFIGS["k16v8_packed"]
    print(f"[case] k16v8 packed {vcodec}", flush=True)
    wl = G.Workload(cfg["layers"], cfg["heads"], cfg["dim"], cfg["tokens"], cfg["pool"], "fp16", "packed", 0)
    fixed = None
    if vcodec == "FP8_FIXED":
        amax = np.array([float(t[:512, :, :, cfg["dim"]:].abs().max()) for t in wl.k])
        fixed = np.stack([np.ones(cfg["layers"]), amax / 448.0], 1).astype(np.float32)
    ids = np.arange(cfg["pages"], dtype=np.int32)
    segs = _sample_pages(cfg["layers"], cfg["pages"], 16, 3)
    _roundtrip_case(ctx, wl, "RAW", vcodec, 0, ids, fixed=fixed, segments=segs, decode_from_oracle=False)


def test_int8_records_qwen3_full_size(ctx):
    """INT8 host-pool records on the Qwen3-8B shape, 36 layers x 8 heads x
    D128 BF16, 3392 of 4096 blocks in random order: one full-size launch
    each way, every segment of 16 sampled pages checked bit-exactly (codes, BF16 scales, row
    padding, decode)."""
    cfg = inputs.CONFIGS["int8_records_qwen3"]
    print("[case] int8 records qwen3", flush=True)
    wl = G.Workload(cfg["layers"], cfg["heads"], cfg["dim"], cfg["tokens"], cfg["pool"], "bf16", "separate", 0)
    ids = inputs.random_page_ids(cfg["pool"], cfg["pages"], seed=0)
    segs = _sample_pages(cfg["layers"], cfg["pages"], 16, 11)
    _roundtrip_case(ctx, wl, "INT8_ROWS", "INT8_ROWS", 0, ids, segments=segs, decode_from_oracle=False)


def test_ans16_llama3_full_size(ctx):
    """The lossless entropy stage on the Llama-3-8B shape, 32 layers x 8 heads
    x D128 BF16, 4096 of 8192 blocks in random order: one full-size launch
    each way; the headers and payloads of every segment of 16 sampled pages equal the oracle's and
    every sampled page decodes bit-exactly."""
    cfg = inputs.CONFIGS["ans16_llama3"]
    print("[case] ans16 llama3", flush=True)
    wl = G.Workload(cfg["layers"], cfg["heads"], cfg["dim"], cfg["tokens"], cfg["pool"], "bf16", "separate", 0)
    ids = inputs.random_page_ids(cfg["pool"], cfg["pages"], seed=0)
    segs = _sample_pages(cfg["layers"], cfg["pages"], 16, 13)
    ora_st, gdesc = _roundtrip_case(ctx, wl, "ANS16", "ANS16", 0, ids, segments=segs, decode_from_oracle=False,
                                    crc=True)
    assert all(int(ora_st[s]) == O.SEG_ENCODED for s in segs)


def _bf16_planes(hi, lo):
    """BF16 tensor from byte planes (int64 tensors of the same shape)."""
    b = (hi << 8) | lo
    return (b - (b >= 32768).to(b.dtype) * 65536).to(torch.int16).view(torch.bfloat16)


def test_ans16_plane_modes(ctx):
    """ANS16 with each kind of payload the decoder distinguishes, 8 heads x
    D128 BF16 (32 KiB segments), 2 layers x 4 of 9 blocks: both byte planes
    coded (small integers), only the low plane coded (random high bytes,
    low bytes from 4 values), only the high plane coded (Gaussian data), and
    neither (uniform bits: stored raw).  The plane modes are checked on the
    oracle's own coding of the planes; every segment is compared."""
    print("[case] ans16 plane modes", flush=True)
    wl = G.Workload(2, 8, 128, 16, 9, "bf16", "separate", seed=21)
    g = torch.Generator(device="cuda").manual_seed(77)
    shape = wl.k[0].shape
    wl.k[0].copy_((torch.randn(shape, generator=g, device="cuda") * 3).round().clamp(-8, 8).to(torch.bfloat16))

    def finite_hi():                                      # high bytes except 0x7F and 0xFF (Inf/NaN exponents)
        r = torch.randint(0, 254, shape, generator=g, device="cuda")
        return r + (r >= 127).to(r.dtype)

    wl.k[1].copy_(_bf16_planes(finite_hi(), torch.randint(0, 4, shape, generator=g, device="cuda") * 64))
    wl.v[1].copy_(_bf16_planes(finite_hi(), torch.randint(0, 256, shape, generator=g, device="cuda")))
    ids = inputs.random_page_ids(9, 4, seed=3)
    expect = {(0, 0): (1, 1), (0, 1): (0, 1), (1, 0): (1, 0)}       # (layer, comp) -> (low, high) plane mode
    for (l, c), modes in expect.items():
        t = (wl.k if c == 0 else wl.v)[l][int(ids[0])]
        bits = t.contiguous().view(torch.int16).cpu().numpy().astype(np.uint16).reshape(-1)
        got = tuple(int(O.ans_encode_plane((bits >> (8 * pl)) & 0xFF)[0]) for pl in (0, 1))
        assert got == modes, f"layer {l} comp {c}: plane modes {got}"
    ora_st, _ = _roundtrip_case(ctx, wl, "ANS16", "ANS16", 0, ids, dst_ids=inputs.random_page_ids(9, 4, seed=4),
                                crc=True)
    seglist = G.segments_of(wl.L, len(ids))
    for sidx, (l, i, c) in enumerate(seglist):
        want = O.SEG_RAW_DATA if (l, c) == (1, 1) else O.SEG_ENCODED
        assert int(ora_st[sidx]) == want, f"segment {sidx}: status {ora_st[sidx]}"


def test_ans16_two_raw_planes_payload(ctx):
    """A payload whose two byte planes are both stored raw (mode 0, 2n + 32
    bytes) is valid for the format though the encoder never writes one (its
    keep rule stores such a segment as raw data): written by hand over a
    GPU-encoded segment, it decodes on the GPU to the oracle's decode of the
    same buffer, the source values; the other segments are unaffected."""
    print("[case] ans16 two raw planes", flush=True)
    wl = G.Workload(1, 8, 128, 16, 4, "bf16", "separate", seed=5)
    ids = np.array([2, 0], np.int32)
    kc = vc = kvc.CODECS["ANS16"]
    codec = kvc.Codec(kc, vc, seed=0, layers=wl.L, crc=True)
    out, desc, slot, total = G.gpu_encode(ctx, wl, codec, ids)
    torch.cuda.synchronize()
    gdesc = G.desc_np(desc)
    assert all(int(d["status"]) == O.SEG_ENCODED for d in gdesc)
    buf = out.cpu().numpy()
    src = G.gpu_segment_vectors(wl, 0, 0, int(ids[0])).reshape(-1)      # segment 0: layer 0, page ids[0], K
    n = src.size
    payload = np.zeros(2 * n + 32, np.uint8)
    payload[16:16 + n] = (src & 0xFF).astype(np.uint8)
    payload[32 + n:] = (src >> 8).astype(np.uint8)
    at = (buf.size + 255) // 256 * 256
    crafted = np.zeros(at + payload.size, np.uint8)
    crafted[:buf.size] = buf
    crafted[at:] = payload
    so = int(gdesc[0]["offset"])
    crafted[so + 12:so + 16] = np.array([payload.size], np.uint32).view(np.uint8)    # stored_len
    crafted[so + 16:so + 24] = np.array([at], np.uint64).view(np.uint8)              # spill offset
    crafted[so + 24:so + 28] = np.array([O.crc32(payload)], np.uint32).view(np.uint8)  # its CRC32
    ora = G.oracle_decode_segments(crafted, wl, kc, vc, 0, len(ids), None, [0, 1, 2, 3])
    assert np.array_equal(ora[0].reshape(-1), src)
    dst = wl.empty_like(fill_bits=0x7FC1)
    st = G.gpu_decode(ctx, dst, codec, torch.from_numpy(crafted).cuda(), crafted.size, ids)
    torch.cuda.synchronize()
    assert st.cpu().numpy().tolist() == [0, 0, 0, 0]
    for sidx, (l, i, c) in enumerate(G.segments_of(wl.L, len(ids))):
        got = G.gpu_segment_vectors(dst, l, c, int(ids[i]))
        assert np.array_equal(got, ora[sidx]), f"segment {sidx}"


def test_k8v8_packed_full_size(ctx):
    """K8/V8 with per-token/head FP8 scales on the vLLM packed FP16 Qwen3-8B
    layout [2048 blocks, 8 heads, 16 tokens, 256], 36 layers: full-size
    launch, every segment of 16 sampled pages."""
    cfg = inputs.CONFIGS["k8v8_packed"]
    print("[case] k8v8 packed", flush=True)
    wl = G.Workload(cfg["layers"], cfg["heads"], cfg["dim"], cfg["tokens"], cfg["pool"], "fp16", "packed", 0)
    ids = np.arange(cfg["pages"], dtype=np.int32)
    segs = _sample_pages(cfg["layers"], cfg["pages"], 16, 5)
    _roundtrip_case(ctx, wl, "FP8_DYNAMIC", "FP8_DYNAMIC", 0, ids, segments=segs, decode_from_oracle=False)


@pytest.mark.parametrize("codec", ["INT8", "FP8_DYNAMIC", "FP8_DIRECT"])
def test_int8_fp8_stress_full_size(ctx, codec):
    """32 layers x 8 heads x D128 BF16, 8192 pages (128K tokens), 1% of the
    524,288 segments injected with NaN/Inf/+-450/+-1000 (plus +-448
    controls), decoded into a shuffled destination pool: exact raw set over
    all segments; sampled parity; every raw segment round-trips bit-exactly."""
    cfg = inputs.CONFIGS["int8_fp8_stress"]
    print(f"[case] stress {codec}", flush=True)
    L, n = cfg["layers"], cfg["pages"]
    wl = G.Workload(L, cfg["heads"], cfg["dim"], cfg["tokens"], cfg["pool"], "bf16", "separate", 0)
    ids = np.arange(n, dtype=np.int32)
    inj, ctl, kind = inputs.inject_specials(wl.k, wl.v, ids, frac=cfg["inject"], seed=0)
    kc = vc = kvc.CODECS[codec]
    c = kvc.Codec(kc, vc, seed=0)
    out, desc, slot, total = G.gpu_encode(ctx, wl, c, ids)
    torch.cuda.synchronize()
    d = G.desc_np(desc)
    fp8 = codec.startswith("FP8")
    expect = np.zeros(L * n * 2, bool)
    for (l, i, cc), k in kind.items():
        if fp8 or k in ("nan", "+inf", "-inf"):
            expect[(l * n + i) * 2 + cc] = True
    assert np.array_equal(d["status"] == kvc.KVC_SEG_RAW_DATA, expect)
    assert not np.any(d["status"] == kvc.KVC_SEG_CAPACITY)
    # decode into a shuffled destination pool
    perm = inputs.permutation(n, 0)
    dst = wl.empty_like(fill_bits=0x7FC1)
    st = G.gpu_decode(ctx, dst, c, out, total, perm)
    torch.cuda.synchronize()
    assert np.all(st.cpu().numpy() == 0)
    raw_segs = np.nonzero(expect)[0]
    rng = np.random.default_rng(5)
    seglist = G.segments_of(L, n)
    for s in rng.choice(raw_segs, size=min(200, raw_segs.size), replace=False):
        l, i, cc = seglist[int(s)]
        src = G.gpu_segment_vectors(wl, l, cc, int(ids[i]))
        got = G.gpu_segment_vectors(dst, l, cc, int(perm[i]))
        assert np.array_equal(src, got)
    # sampled parity against the oracle (encode bytes + decode values)
    segs = _sample_segments(L, n, 48, 9) + [int(x) for x in raw_segs[:16]]
    segs = sorted(set(segs))
    ora_buf, ora_st, offs, ora_total = G.oracle_encode(wl, kc, vc, 0, ids, segments=segs)
    bad = G.compare_encoded(out.cpu().numpy(), d, ora_buf, ora_st, offs, ora_total, segs)
    assert not bad, bad[:5]
    ora_dec = G.oracle_decode_segments(ora_buf, wl, kc, vc, 0, n, None, segs)
    for s in segs:
        l, i, cc = seglist[s]
        got = G.gpu_segment_vectors(dst, l, cc, int(perm[i]))
        assert np.array_equal(got, ora_dec[s]), s


# ----------------------------------------------------------------- CRC32 per segment
CRC_SHAPES = {
    # name: (layers, heads, tokens, pool, pages); layer 1 protected (raw by policy)
    "n15": (3, 3, 5, 9, 4),        # 15 vectors: payloads end mid-unit (ragged CRC tail), 64-thread groups
    "n231": (2, 7, 33, 6, 3),      # 231 vectors: 256-thread groups; D=256 slots exceed the LDS stage
}


@pytest.mark.parametrize("shape", sorted(CRC_SHAPES))
@pytest.mark.parametrize("dim", [32, 64, 128, 256])
@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0]}-{p[1]}")
def test_crc_roundtrip(ctx, pair, dim, shape):
    """KVC_CODEC_CRC32: every encoded slot (header CRC included) bit-exact
    with the oracle's, descriptors carry the header's CRC, and both buffers
    decode with status 0 to the oracle's values."""
    L, H, T, pool, n = CRC_SHAPES[shape]
    layout = "packed" if (dim // 32) % 2 else "separate"
    print(f"[case] crc {pair} D={dim} {shape} {layout}", flush=True)
    wl = G.Workload(L, H, dim, T, pool, "bf16", layout, seed=dim + 3)
    ids = inputs.random_page_ids(pool, n, seed=dim + 5)
    fixed = _fixed_scales(L) if "FP8_FIXED" in pair else None
    ora_st, gdesc = _roundtrip_case(ctx, wl, pair[0], pair[1], seed=77 + dim, page_ids=ids, protected=[1],
                                    fixed=fixed, dst_ids=inputs.random_page_ids(pool, n, seed=dim + 6), crc=True)
    assert np.all(gdesc["flags"] & kvc.KVC_FLAG_CRC32)


def _flip_stored_byte(buf: np.ndarray, d, s):
    """Flip one bit of one stored byte of segment s (first, last or middle
    byte, by segment) in a host copy of an encoded buffer."""
    base = int(d["spill_offset"]) if d["status"] == kvc.KVC_SEG_RAW_DATA else int(d["offset"]) + 32
    n = int(d["stored_len"])
    at = (0, n - 1, n // 2)[s % 3]
    buf[base + at] ^= np.uint8(1 << (s % 8))


def test_crc_detects_corruption(ctx):
    """One flipped bit in the stored bytes (coded payload, raw slot body or
    spilled raw bytes) of every third segment: decode reports 3 for exactly
    those and leaves their pages untouched, decodes the rest; the oracle
    rejects the same segments."""
    print("[case] crc corruption", flush=True)
    L, H, D, T, pool, n = 3, 8, 128, 16, 24, 12
    wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 21)
    ids = inputs.random_page_ids(pool, n, seed=21)
    inputs.inject_specials(wl.k, wl.v, ids, frac=0.15, seed=22, controls=0)
    kc, vc = kvc.KVC_TQ4, kvc.KVC_FP8_DYNAMIC
    codec = kvc.Codec(kc, vc, seed=9, protected_layers=[1], layers=L, crc=True)
    out, desc, slot, total = G.gpu_encode(ctx, wl, codec, ids, spill_bytes=L * n * 2 * (H * T * D * 2))
    torch.cuda.synchronize()
    d = G.desc_np(desc)
    assert {int(x) for x in d["status"]} >= {kvc.KVC_SEG_ENCODED, kvc.KVC_SEG_RAW_POLICY, kvc.KVC_SEG_RAW_DATA}
    nseg = L * n * 2
    flipped = set(range(0, nseg, 3))
    buf = out.cpu().numpy().copy()
    for s in flipped:
        _flip_stored_byte(buf, d[s], s)
    dst = wl.empty_like(fill_bits=0x2468)
    dst_ids = inputs.random_page_ids(pool, n, seed=23)
    st = G.gpu_decode(ctx, dst, codec, torch.from_numpy(buf).cuda(), total, dst_ids).cpu().numpy()
    torch.cuda.synchronize()
    segs = list(range(nseg))
    ora_buf, ora_st, offs, _ = G.oracle_encode(wl, kc, vc, 9, ids, None, [1], segs, crc=True)
    ora_dec = G.oracle_decode_segments(ora_buf, wl, kc, vc, 9, n, [1], segs)
    seglist = G.segments_of(L, n)
    for s, (l, i, c) in enumerate(seglist):
        got = G.gpu_segment_vectors(dst, l, c, int(dst_ids[i]))
        if s in flipped:
            assert st[s] == 3, (s, st[s])
            assert np.all(got == 0x2468), s
        else:
            assert st[s] == 0, (s, st[s])
            _check_decoded(got, ora_dec[s], wl.dt, c == 0 and ora_st[s] == 0, f"segment {s}")
    # the oracle refuses the same corruption in its own buffer
    for s in sorted(flipped)[:12]:
        bad = ora_buf.copy()
        ds = {"status": ora_st[s], "offset": offs[s], "stored_len": int(ora_buf[offs[s] + 12:offs[s] + 16].view(np.uint32)[0]),
              "spill_offset": int(ora_buf[offs[s] + 16:offs[s] + 24].view(np.uint64)[0])}
        _flip_stored_byte(bad, ds, s)
        size = (offs[s + 1] if s + 1 < len(offs) else slot) - offs[s]
        with pytest.raises(O.ChecksumError):
            O.decode_segment(bad[offs[s]:offs[s] + size], bad, wl.dt, D, H * T, 9)


def test_crc_option_must_match(ctx):
    """A buffer written with the CRC option decodes only with it, and one
    written without only without: otherwise every segment reports 1 and no
    page is written."""
    print("[case] crc option mismatch", flush=True)
    L, H, D, T, pool, n = 2, 4, 64, 16, 8, 4
    wl = G.Workload(L, H, D, T, pool, "fp16", "packed", 31)
    ids = inputs.random_page_ids(pool, n, seed=31)
    for enc_crc in (True, False):
        c_enc = kvc.Codec(kvc.KVC_TQ3, kvc.KVC_UNIFORM3, seed=1, protected_layers=[0], layers=L, crc=enc_crc)
        c_dec = kvc.Codec(kvc.KVC_TQ3, kvc.KVC_UNIFORM3, seed=1, protected_layers=[0], layers=L, crc=not enc_crc)
        out, desc, slot, total = G.gpu_encode(ctx, wl, c_enc, ids)
        dst = wl.empty_like(fill_bits=0x1357)
        st = G.gpu_decode(ctx, dst, c_dec, out, total, ids).cpu().numpy()
        torch.cuda.synchronize()
        assert np.all(st == 1), st
        for l in range(L):
            assert np.all(G.u16(dst.k[l]) == 0x1357)


def test_crc_spill_capacity(ctx):
    """With the CRC option and a spill region for two raw segments: stored
    raw segments carry the CRC of their spilled bytes and decode; segments
    that were not stored carry none and report 1."""
    print("[case] crc spill capacity", flush=True)
    L, H, D, T, pool = 2, 8, 128, 16, 16
    wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 12)
    ids = np.arange(pool, dtype=np.int32)
    inputs.inject_specials(wl.k, wl.v, ids, frac=0.2, seed=6, controls=0)
    codec = kvc.Codec(kvc.KVC_INT8, kvc.KVC_INT8, seed=0, crc=True)
    out, desc, slot, total = G.gpu_encode(ctx, wl, codec, ids, spill_bytes=2 * 32768)
    torch.cuda.synchronize()
    d = G.desc_np(desc)
    buf = out.cpu().numpy()
    raw = np.nonzero(d["status"] == kvc.KVC_SEG_RAW_DATA)[0]
    cap = np.nonzero(d["status"] == kvc.KVC_SEG_CAPACITY)[0]
    assert len(raw) == 2 and len(cap) > 0
    for s in raw:
        so, nb = int(d[s]["spill_offset"]), int(d[s]["stored_len"])
        assert d[s]["flags"] & kvc.KVC_FLAG_CRC32 and int(d[s]["crc32"]) == O.crc32(buf[so:so + nb])
    for s in cap:
        assert not d[s]["flags"] & kvc.KVC_FLAG_CRC32 and int(d[s]["crc32"]) == 0
    dst = wl.empty_like(fill_bits=0x1234)
    st = G.gpu_decode(ctx, dst, codec, out, total, ids).cpu().numpy()
    torch.cuda.synchronize()
    assert np.all(st[cap] == 1) and np.all(np.delete(st, cap) == 0)


def test_ans16_corrupted_payloads_match_oracle(ctx):
    """Bytes of an ANS16 payload changed at random (plane headers, bitmap,
    frequencies, stream lengths, streams, padding).  As stored, every such
    payload fails its CRC32: status 3, the page untouched, as the oracle
    rejects it.  With the header's CRC32 recomputed over the changed bytes,
    the structural checks decide: the GPU accepts exactly the payloads the
    oracle accepts (status 0 or 1) and then decodes the same values.  200
    trials over the 4 segments of a small call."""
    print("[case] ans16 corrupted payloads", flush=True)
    wl = G.Workload(1, 8, 128, 16, 3, "bf16", "separate", seed=41)
    ids = np.array([2, 0], np.int32)
    kc = vc = kvc.CODECS["ANS16"]
    codec = kvc.Codec(kc, vc, seed=0, layers=wl.L, crc=True)
    out, desc, slot, total = G.gpu_encode(ctx, wl, codec, ids)
    torch.cuda.synchronize()
    gdesc = G.desc_np(desc)
    assert all(int(d["status"]) == O.SEG_ENCODED for d in gdesc)
    buf = out.cpu().numpy()
    rng = np.random.default_rng(42)
    dev = torch.empty(total, dtype=torch.uint8, device="cuda")
    seglist = G.segments_of(wl.L, len(ids))
    accepted = 0
    for trial in range(200):
        s_ = int(rng.integers(4))
        so, nb, off = int(gdesc[s_]["spill_offset"]), int(gdesc[s_]["stored_len"]), int(gdesc[s_]["offset"])
        bad = buf.copy()
        flips = set()
        for _ in range(int(rng.integers(1, 4))):
            if rng.random() < 0.5:                          # the plane headers, bitmap, frequencies and lengths
                pos = so + int(rng.integers(min(nb, 800)))
            else:
                pos = so + int(rng.integers(nb))
            flips.add((pos, int(rng.integers(8))))         # distinct bits: the bytes always change
        for pos, bit in flips:
            bad[pos] ^= np.uint8(1 << bit)
        l, i, c = seglist[s_]
        for patched in (False, True):
            if patched:
                bad[off + 24:off + 28] = np.array([O.crc32(bad[so:so + nb])], np.uint32).view(np.uint8)
            try:
                ora = G.oracle_decode_segments(bad, wl, kc, vc, 0, len(ids), None, [s_])[s_]
                ora_st = 0
            except O.ChecksumError:
                ora, ora_st = None, 3
            except ValueError:
                ora, ora_st = None, 1
            dev.copy_(torch.from_numpy(bad))
            dst = wl.empty_like(fill_bits=0x7FC1)
            st = G.gpu_decode(ctx, dst, codec, dev, total, ids).cpu().numpy()
            torch.cuda.synchronize()
            assert int(st[s_]) == ora_st, f"trial {trial} patched={patched}: segment {s_} status {st[s_]}"
            assert patched or ora_st == 3
            assert all(int(st[t]) == 0 for t in range(4) if t != s_)
            got = G.gpu_segment_vectors(dst, l, c, int(ids[i]))
            if ora is not None:
                accepted += 1
                assert np.array_equal(got, ora), f"trial {trial}"
            elif ora_st == 3:
                assert np.all(got == 0x7FC1), f"trial {trial}: a page written despite a CRC mismatch"
    assert accepted < 200


def test_ans16_spill_capacity(ctx):
    """ANS16 payloads live in the spill region: sized for about ten of the
    32 payloads, the segments that found room hold the oracle's payload bytes
    and decode losslessly; the others report KVC_SEG_CAPACITY, are not
    stored, decode with status 1 and leave their pages untouched."""
    print("[case] ans16 spill capacity", flush=True)
    L, H, D, T, pool = 2, 8, 128, 16, 8
    wl = G.Workload(L, H, D, T, pool, "bf16", "separate", 14)
    ids = np.arange(pool, dtype=np.int32)
    codec = kvc.Codec(kvc.KVC_ANS16, kvc.KVC_ANS16, seed=0, layers=L, crc=True)
    out, desc, slot, total = G.gpu_encode(ctx, wl, codec, ids, spill_bytes=10 * 24 * 1024)
    torch.cuda.synchronize()
    d = G.desc_np(desc)
    buf = out.cpu().numpy()
    enc = np.nonzero(d["status"] == kvc.KVC_SEG_ENCODED)[0]
    cap = np.nonzero(d["status"] == kvc.KVC_SEG_CAPACITY)[0]
    assert len(enc) + len(cap) == L * pool * 2 and 8 <= len(enc) <= 10 and len(cap) > 0
    seglist = G.segments_of(L, pool)
    for sidx in enc:
        l, i, c = seglist[sidx]
        src = G.gpu_segment_vectors(wl, l, c, int(ids[i]))
        _, ost, payload = O.encode_segment(src, wl.dt, kvc.KVC_ANS16, component=c, heads=H, crc=True)
        so, nb = int(d[sidx]["spill_offset"]), int(d[sidx]["stored_len"])
        assert ost == O.SEG_ENCODED and nb == payload.size and slot <= so and so + nb <= total
        assert np.array_equal(buf[so:so + nb], payload), f"segment {sidx}: payload differs"
    dst = wl.empty_like(fill_bits=0x1234)
    st = G.gpu_decode(ctx, dst, codec, out, total, ids).cpu().numpy()
    torch.cuda.synchronize()
    assert np.all(st[cap] == 1) and np.all(st[enc] == 0)
    for sidx, (l, i, c) in enumerate(seglist):
        got = G.gpu_segment_vectors(dst, l, c, int(ids[i]))
        want = G.gpu_segment_vectors(wl, l, c, int(ids[i])) if sidx in enc else np.full_like(got, 0x1234)
        assert np.array_equal(got, want), f"segment {sidx}"


@pytest.mark.parametrize("crc", [False, True])
def test_fp8_large_call_one_wave_encode(ctx, crc):
    """A call of raw/FP8-direct/FP8-dynamic components with at least 32 x 256
    segments encodes one wave per 32 KiB segment without CRC32 (two waves
    with it): 2 layers x 2048 pages x 8 heads x D128 BF16 (8192 segments), K
    FP8 dynamic, V FP8 direct, layer 1 protected, 1% of segments injected
    with values the FP8 gate keeps raw; with and without CRC, sampled
    segments compared both ways."""
    print(f"[case] fp8 large call one-wave encode crc={crc}", flush=True)
    L, pages = 2, 2048
    wl = G.Workload(L, 8, 128, 16, pages, "bf16", "separate", seed=31)
    ids = inputs.random_page_ids(pages, pages, seed=32)
    inputs.inject_specials(wl.k, wl.v, ids, frac=0.01, seed=33)
    segs = _sample_segments(L, pages, 96, 34, layers=[1])
    spill = L * pages * 2 // 20 * 32768                  # room for the injected segments
    _roundtrip_case(ctx, wl, "FP8_DYNAMIC", "FP8_DIRECT", 0, ids, protected=[1], segments=segs,
                    decode_from_oracle=False, crc=crc, spill_bytes=spill)


def test_tq4_u4_llama3_full_size_crc(ctx):
    """The TurboQuant-4 / uniform-4 Llama-3-8B workload with the CRC option:
    one full-size launch each way, every segment of 32 sampled pages bit-exact (CRCs
    included) and decoded with status 0 after the CRC check."""
    cfg = inputs.CONFIGS["tq4_u4_llama3"]
    print("[case] tq4_u4_llama3 full size crc", flush=True)
    wl = G.Workload(cfg["layers"], cfg["heads"], cfg["dim"], cfg["tokens"], cfg["pool"], "bf16", "separate", 0)
    ids = inputs.random_page_ids(cfg["pool"], cfg["pages"], seed=0)
    segs = _sample_pages(cfg["layers"], cfg["pages"], 32, 2)
    _roundtrip_case(ctx, wl, "TQ4", "UNIFORM4", 0, ids, protected=list(cfg["protected"]), segments=segs,
                    decode_from_oracle=False, crc=True)
