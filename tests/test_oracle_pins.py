"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/*.json, each with its citation), library routines
(torch/numpy dtype casts, scipy's Hadamard matrix, numerical integration),
closed forms, invariants and brute force on tiny inputs.  No GPU needed.
"""
import json
import math
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32bits(x):
    return int(np.float32(x).view(np.uint32))


# ------------------------------------------------------------------ E4M3FN
def _all_bf16_finite_inrange():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = (h.astype(np.uint32) << 16).view(np.float32)
    m = np.isfinite(x) & (np.abs(x) <= 448)
    return x[m]


def _all_f16_finite_inrange():
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    m = np.isfinite(x) & (np.abs(x) <= 448)
    return x[m]


@pytest.mark.parametrize("src", ["bf16", "f16"])
def test_e4m3_exhaustive_vs_nearest_search(oracle, src):
    """Every finite in-range BF16/FP16 source value: the arithmetic RNE
    conversion equals a brute-force nearest-value search (ties to the even
    code) over the 254 finite E4M3FN values."""
    x = _all_bf16_finite_inrange() if src == "bf16" else _all_f16_finite_inrange()
    assert x.size == (34754 if src == "bf16" else 48642)
    np.testing.assert_array_equal(oracle.f32_to_e4m3(x), oracle.e4m3_nearest_search(x))


@pytest.mark.parametrize("src", ["bf16", "f16"])
def test_e4m3_exhaustive_vs_torch(oracle, src):
    """Library routine: torch's CPU float8_e4m3fn cast (RNE, OCP E4M3FN)."""
    torch = pytest.importorskip("torch")
    x = _all_bf16_finite_inrange() if src == "bf16" else _all_f16_finite_inrange()
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.f32_to_e4m3(x), ref)


def test_e4m3_f32_sweep_vs_torch(oracle):
    """Random binary32 values in [-448, 448] plus +-4 ulp around every
    rounding midpoint between neighbouring E4M3FN values."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    lim = f32bits(448.0)
    bits = rng.integers(0, lim + 1, 400000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32) * np.where(rng.random(bits.size) < 0.5, -1, 1).astype(np.float32)
    vals = np.sort(oracle.e4m3_to_f32(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = ((vals[1:].astype(np.float64) + vals[:-1]) / 2).astype(np.float32)
    near = (mids.view(np.uint32)[:, None].astype(np.int64) + np.arange(-4, 5)[None, :]).ravel()
    near = near[(near >= 0) & (near <= lim)].astype(np.uint32).view(np.float32)
    x = np.concatenate([x, near, -near])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.f32_to_e4m3(x), ref)


def test_e4m3_special_values(oracle):
    for name, val, code in golden("e4m3fn_special_values.json")["cases"]:
        got = int(oracle.f32_to_e4m3(np.array([val], np.float32))[0])
        assert got == int(code, 16), name


def test_e4m3_decode_table(oracle):
    codes = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_to_f32(codes)
    fin = np.isfinite(v)
    assert fin.sum() == 254 and set(np.nonzero(~fin)[0]) == {0x7F, 0xFF}
    assert v[fin].max() == 448.0 and v[0x01] == 2.0 ** -9 and v[0x08] == 2.0 ** -6
    # decode then encode is the identity on every finite code (incl. -0)
    np.testing.assert_array_equal(oracle.f32_to_e4m3(v[fin]), codes[fin])


# ------------------------------------------------------------ BF16 / FP16
def test_f16_conversion_vs_numpy(oracle):
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(1000.0),
        (rng.integers(0, 2 ** 32, 200000, dtype=np.uint64).astype(np.uint32)).view(np.float32),
        np.array([65504, 65519.99, 65520, 1e-8, 2 ** -25, 2 ** -24 * 1.5, -0.0], np.float32)])
    x = x[~np.isnan(x)]
    np.testing.assert_array_equal(oracle.f32_to_f16(x), x.astype(np.float16).view(np.uint16))
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = oracle.f16_to_f32(h)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))


def test_bf16_conversion_vs_torch(oracle):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = (rng.integers(0, 2 ** 32, 500000, dtype=np.uint64).astype(np.uint32)).view(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_bf16(x), ref)


# ------------------------------------------------------------ Lloyd-Max
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_vs_table(oracle, bits):
    g = golden("lloyd_max_gaussian.json")
    ref = g["levels"][str(bits)]
    c, t, _ = oracle.lloyd_max(bits)
    n = 1 << bits
    np.testing.assert_allclose(c[n // 2:], ref["centroids"], atol=g["tolerance"])
    np.testing.assert_allclose(t[n // 2 - 1:], ref["thresholds"], atol=g["tolerance"])
    np.testing.assert_array_equal(c, -c[::-1])
    assert t[n // 2 - 1] == 0.0
    # distortion by numerical integration of (x - Q(x))^2 phi(x)
    from scipy import integrate
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    edges = [-math.inf] + list(t) + [math.inf]
    mse = sum(integrate.quad(lambda x, ck=ck: (x - ck) ** 2 * pdf(x), edges[k], edges[k + 1],
                             epsabs=1e-13)[0] for k, ck in enumerate(c))
    assert abs(mse - ref["mse"]) < 2e-5 * max(1.0, ref["mse"] * 100)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_max_optimality_conditions(oracle, bits):
    """Independent check of the fixed point: each centroid equals the
    conditional mean of its cell computed by numerical integration, and each
    threshold is the midpoint of its neighbours."""
    from scipy import integrate
    c, t, _ = oracle.lloyd_max(bits)
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    edges = [-math.inf] + list(t) + [math.inf]
    for k in range(len(c)):
        m1 = integrate.quad(lambda x: x * pdf(x), edges[k], edges[k + 1], epsabs=1e-14)[0]
        m0 = integrate.quad(pdf, edges[k], edges[k + 1], epsabs=1e-14)[0]
        assert abs(m1 / m0 - c[k]) < 1e-9
    np.testing.assert_allclose(t, (c[1:] + c[:-1]) / 2, rtol=0, atol=1e-15)


def test_codebook_f32_rounding(oracle):
    for bits in (3, 4):
        c, t, _ = oracle.lloyd_max(bits)
        cf, tf = oracle.codebook_f32(bits)
        np.testing.assert_array_equal(cf, c.astype(np.float32))
        np.testing.assert_array_equal(tf, t.astype(np.float32))
        assert np.all(np.diff(tf) > 0) and np.array_equal(tf, -tf[::-1])


# ------------------------------------------------------------ signs
def test_splitmix64_published_vector(oracle):
    g = golden("splitmix64_seed0.json")
    assert oracle.splitmix64(g["seed"], 3) == [int(v, 16) for v in g["outputs"]]


def test_signs_from_bit63(oracle):
    outs = oracle.splitmix64(12345, 256)
    exp = np.array([-1 if (o >> 63) else 1 for o in outs], np.int8)
    np.testing.assert_array_equal(oracle.signs(12345, 256), exp)
    s = oracle.signs(0, 256)
    assert 96 < int((s < 0).sum()) < 160          # roughly balanced
    assert np.array_equal(oracle.signs(7, 64), oracle.signs(7, 128)[:64])


# ------------------------------------------------------------ WHT
@pytest.mark.parametrize("d", [2, 4, 8, 32, 64, 128, 256])
def test_wht_equals_hadamard_matrix(oracle, d):
    """On small integers every FP32 sum is exact, so the fast transform must
    equal scipy's Sylvester-ordered Hadamard matrix times the vector."""
    from scipy.linalg import hadamard
    rng = np.random.default_rng(d)
    v = rng.integers(-1000, 1000, d).astype(np.float32)
    ref = hadamard(d).astype(np.float64) @ v.astype(np.float64)
    np.testing.assert_array_equal(oracle.wht(v), ref.astype(np.float32))


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_wht_involution_and_orthonormality(oracle, d):
    rng = np.random.default_rng(100 + d)
    v = rng.integers(-1000, 1000, d).astype(np.float32)
    np.testing.assert_array_equal(oracle.wht(oracle.wht(v)), v * d)   # H H = D I, exact
    x = rng.standard_normal(d).astype(np.float32)
    z = oracle.wht(x).astype(np.float64) / math.sqrt(d)               # orthonormal version
    gamma = d * 2.0 ** -24 / (1 - d * 2.0 ** -24)
    assert abs(np.linalg.norm(z) - np.linalg.norm(x.astype(np.float64))) <= \
        4 * math.log2(d) * gamma * np.linalg.norm(x)


def test_sumsq_tree(oracle):
    rng = np.random.default_rng(5)
    v = rng.integers(-300, 300, 128).astype(np.float32)
    assert oracle.sumsq_tree(v) == float((v.astype(np.int64) ** 2).sum())    # exact
    x = rng.standard_normal(256).astype(np.float32)
    ref = math.fsum(float(a) * float(a) for a in x)
    assert abs(oracle.sumsq_tree(x) - ref) <= 9 * 2.0 ** -24 * ref


# ------------------------------------------------------------ sizes / rules
def test_payload_sizes(oracle):
    g = golden("payload_sizes.json")
    d = g["head_dim"]
    per = lambda c: oracle.code_bytes(c, d) + oracle.meta_bytes(c)
    assert per(oracle.TQ4) == g["tq4_k"] and per(oracle.UNIFORM4) == g["uniform4_v"]
    assert per(oracle.TQ3) == g["tq3_k"] and per(oracle.UNIFORM3) == g["uniform3_v"]
    assert per(oracle.RAW) == g["original"]
    assert [per(oracle.TQ3) for d in (32,)] and \
        [oracle.code_bytes(oracle.TQ3, dd) + 2 for dd in (32, 64, 256)] == [14, 26, 98]
    assert [oracle.code_bytes(oracle.UNIFORM3, dd) + 4 for dd in (32, 64, 256)] == [16, 28, 100]


def test_slot_and_keep_rules(oracle):
    # 16 tokens x 8 heads x 128: slot = align256(32 + 128*66) = 8704 B
    assert oracle.slot_bytes(oracle.TQ4, 128, 128) == 8704
    assert oracle.slot_bytes(oracle.RAW, 128, 128) == 32768 + 256
    assert oracle.effective_codec(oracle.TQ4, 128, 128, False) == oracle.TQ4
    assert oracle.effective_codec(oracle.TQ4, 128, 128, True) == oracle.RAW
    # a single 32-dim vector: 256-B slot saves nothing -> raw (12.5% rule)
    assert oracle.effective_codec(oracle.INT8, 32, 1, False) == oracle.RAW
    # > 16 MiB source segment -> raw
    assert oracle.effective_codec(oracle.FP8_DIRECT, 256, 32769, False) == oracle.RAW
    assert oracle.effective_codec(oracle.FP8_DIRECT, 256, 32768, False) == oracle.FP8_DIRECT


# ------------------------------------------------------------ INT8
def _bits(vals, dtype):
    import oracle.kvc_oracle as O
    vals = np.asarray(vals, np.float32)
    return O.f32_to_bf16(vals) if dtype == 1 else O.f32_to_f16(vals)


def test_int8_worked_example(oracle):
    g = golden("int8_worked_example.json")
    vec = np.zeros((16, 128), np.uint16)
    vec[0, :4] = _bits(g["values"], oracle.BF16)
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.INT8)
    assert st == oracle.SEG_ENCODED and slot[1] == oracle.INT8
    assert list(slot[32:36].view(np.int8)) == g["codes"]
    # all-zero vectors: zero codes, restore to exactly zero
    assert not slot[32 + 128:32 + 16 * 128].any()
    out = oracle.decode_segment(slot, None, oracle.BF16, 128, 16)
    assert not out[1:].any()


def test_int8_error_bound(oracle):
    """|x - x_hat| <= s/2 + 2*127*s*2^-24 + half an output ulp."""
    rng = np.random.default_rng(6)
    for dtype in (oracle.BF16, oracle.FP16):
        x = (rng.standard_normal((64, 128)) * np.exp(rng.standard_normal((64, 1)))).astype(np.float32)
        vec = _bits(x, dtype)
        xs = oracle.src_to_f32(vec, dtype)
        slot, st, _ = oracle.encode_segment(vec, dtype, oracle.INT8)
        s = slot[32 + 64 * 128:32 + 64 * 132].view(np.float32)
        # scale rule: s = RN(max(amax, 1e-12) / 127)
        amax = np.abs(xs).max(axis=1)
        np.testing.assert_array_equal(s, (np.maximum(amax, np.float32(1e-12)) / np.float32(127)))
        out = oracle.src_to_f32(oracle.decode_segment(slot, None, dtype, 128, 64), dtype)
        ulp = np.spacing(np.abs(out)).astype(np.float64) * (2 ** 16 if dtype == oracle.BF16 else 2 ** 13)
        bound = s[:, None] * (0.5 + 254 * 2.0 ** -24) + ulp / 2 + 1e-30
        assert np.all(np.abs(out.astype(np.float64) - xs) <= bound)


# ------------------------------------------------------------ FP8
def test_fp8_scale_rule_constants():
    g = golden("fp8_scale_rule.json")
    assert hex(f32bits(np.float32(1) / np.float32(448))) == g["recip_448_bits"]
    assert hex(f32bits(g["amax_floor"])) == g["amax_floor_bits"]
    assert float(np.float32(1) / np.float32(448)) > 1 / 448  # rounded up: s*448 >= amax


def test_fp8_dynamic_invariants(oracle):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((128, 128)) * np.exp(rng.standard_normal((1, 128)))).astype(np.float32)
    vec = _bits(x, oracle.BF16)
    xs = oracle.src_to_f32(vec, oracle.BF16)
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.FP8_DYNAMIC)
    assert st == oracle.SEG_ENCODED
    codes = slot[32:32 + 128 * 128].reshape(128, 128)
    s = slot[32 + 128 * 128:32 + 128 * 132].view(np.float32)
    r = np.float32(1) / np.float32(448)
    np.testing.assert_array_equal(s, np.abs(xs).max(1) * r)
    am = np.abs(xs).argmax(1)
    picked = codes[np.arange(128), am]
    assert set(picked.tolist()) <= {0x7E, 0xFE}               # amax element -> +-448
    np.testing.assert_array_equal(picked >> 7, (xs[np.arange(128), am] < 0).astype(np.uint8))
    # decode error: half an E4M3 step (relative 2^-4) of the scaled value
    out = oracle.src_to_f32(oracle.decode_segment(slot, None, oracle.BF16, 128, 128), oracle.BF16)
    err = np.abs(out - xs)
    assert np.all(err <= np.maximum(np.abs(xs) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * 1.02 +
                  np.abs(out) * 2.0 ** -8)


@pytest.mark.parametrize("codec", ["FP8_DIRECT", "FP8_FIXED", "FP8_DYNAMIC", "INT8", "UNIFORM4", "TQ4"])
def test_segment_gate(oracle, codec):
    c = getattr(oracle, codec)
    fp8 = codec.startswith("FP8")
    base = np.full((16, 128), 0x3F80, np.uint16)          # bf16 1.0
    cases = {0x7FC0: True, 0x7F80: True, 0xFF80: True,    # NaN, +Inf, -Inf
             0x43E1: fp8, 0xC3E1: fp8, 0x447A: fp8,       # +-450 (next bf16 above 448), 1000
             0x43E0: False, 0xC3E0: False}                # +-448 exactly: never raw
    for bits, raw in cases.items():
        v = base.copy()
        v[5, 17] = bits
        slot, st, spill = oracle.encode_segment(v, oracle.BF16, c, fixed_scale=0.25,
                                                spill_offset=1 << 20)
        assert (st == oracle.SEG_RAW_DATA) == raw, hex(bits)
        if raw:
            assert slot[1] == oracle.RAW and slot[2] == 2
            assert slot[16:24].view(np.uint64)[0] == 1 << 20
            np.testing.assert_array_equal(spill.view(np.uint16), v.ravel())   # bit-exact
            buf = np.zeros((1 << 20) + spill.size, np.uint8)
            buf[1 << 20:] = spill
            np.testing.assert_array_equal(oracle.decode_segment(slot, buf, oracle.BF16, 128, 16), v)


# The FP16 metadata rule [OKV-SF "FP8 and TurboQuant": the TurboQuant norm,
# the uniform minimum and the uniform scale are stored as FP16;
# "Ownership, storage and GDS": a segment the codec cannot represent stays
# raw]: a norm, minimum or scale that rounds past the FP16 range (|v| >=
# 65520 rounds to infinity) sends the segment raw, bit-exactly.
# BF16 vectors with exactly computed squared norms: every square and partial
# sum below is a multiple of 256 under 2^32, so any summation order is exact.
OVERFLOW_TQ_BF16 = {
    # squared norm 65520^2: RN(sqrt) = 65520, FP16 -> inf: raw
    "norm_65520": ([65280.0, 5600.0, 160.0, 80.0], True),
    # 65520^2 - 256: sqrt = 65519.99805 rounds (just below the binary32
    # midpoint) to 65519.996, FP16 65504: coded
    "norm_65520_minus_256": ([65280.0, 5600.0, 160.0, 64.0, 32.0, 32.0], False),
    # a norm of about 65522.5: raw; about 65519.8: coded
    "norm_65522": ([65280.0, 5632.0], True),
    "norm_65519": ([65280.0, 5600.0], False),
}


def _raw_roundtrip(oracle, vec, dtype, codec, raw):
    n_vec, d = vec.shape
    slot, st, spill = oracle.encode_segment(vec, dtype, codec, spill_offset=1 << 16)
    assert (st == oracle.SEG_RAW_DATA) == raw
    if raw:
        assert slot[1] == oracle.RAW and slot[2] == 2
        np.testing.assert_array_equal(spill.view(np.uint16), vec.ravel())
        buf = np.zeros((1 << 16) + spill.size, np.uint8)
        buf[1 << 16:] = spill
        np.testing.assert_array_equal(oracle.decode_segment(slot, buf, dtype, d, n_vec), vec)
    return slot


@pytest.mark.parametrize("case", sorted(OVERFLOW_TQ_BF16))
@pytest.mark.parametrize("codec", ["TQ3", "TQ4"])
def test_tq_norm_fp16_overflow_goes_raw(oracle, case, codec):
    vals, raw = OVERFLOW_TQ_BF16[case]
    vec = np.zeros((16, 128), np.uint16)
    vec[7, :len(vals)] = _bits(vals, oracle.BF16)
    slot = _raw_roundtrip(oracle, vec, oracle.BF16, getattr(oracle, codec), raw)
    if not raw:
        bits = 3 if codec == "TQ3" else 4
        meta = slot[32 + 16 * bits * 16:32 + 16 * (bits * 16 + 2)].view(np.uint16)
        assert meta[7] == 0x7BFF                         # FP16 65504


def test_tq_norm_fp16_overflow_fp16_source(oracle):
    """Two FP16 maxima give a norm of 92,636: raw; one gives 65,504: coded."""
    vec = np.zeros((16, 64), np.uint16)
    vec[3, 5] = 0x7BFF
    _raw_roundtrip(oracle, vec, oracle.FP16, oracle.TQ4, False)
    vec[3, 9] = 0xFBFF
    _raw_roundtrip(oracle, vec, oracle.FP16, oracle.TQ4, True)


@pytest.mark.parametrize("codec", ["UNIFORM3", "UNIFORM4"])
def test_uniform_fp16_metadata_overflow_goes_raw(oracle, codec):
    """BF16 sources: a minimum of -65536 (FP16 -inf) or a scale of
    983040/(2^b - 1) >= 65520 sends the segment raw; a minimum of -65280 and
    a scale of 974848/15 = 64989.9 (FP16 64992) stay coded.  The scale case
    applies to 4-bit codes: 3-bit ones divide by 7, so both spans overflow."""
    c = getattr(oracle, codec)
    top = 7 if codec == "UNIFORM3" else 15
    base = np.zeros((16, 32), np.uint16)
    for lo, raw in ((-65280.0, False), (-65536.0, True)):
        vec = base.copy()
        vec[2, 3] = _bits([lo], oracle.BF16)[0]
        _raw_roundtrip(oracle, vec, oracle.BF16, c, raw)
    for hi in (974848.0, 983040.0):
        vec = base.copy()
        vec[9, 30] = _bits([hi], oracle.BF16)[0]
        raw = float(np.float32(hi) / np.float32(top)) >= 65520
        assert raw == (hi == 983040.0 or top == 7)
        slot = _raw_roundtrip(oracle, vec, oracle.BF16, c, raw)
        if not raw:
            meta = slot[32 + 16 * 16:32 + 16 * 20].view(np.uint16).reshape(16, 2)
            assert meta[9, 1] == np.float16(64992.0).view(np.uint16)


def test_fp8_direct_roundtrip_exact_on_representable(oracle):
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_to_f32(codes)
    vals = vals[np.isfinite(vals)]
    vec = np.resize(oracle.f32_to_bf16(vals), (16, 128)).astype(np.uint16)
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.FP8_DIRECT)
    out = oracle.decode_segment(slot, None, oracle.BF16, 128, 16)
    np.testing.assert_array_equal(out, vec)


# ------------------------------------------------------------ uniform
def _rn32(q):
    """binary32 round-to-nearest-even of a rational (exact; no overflow)."""
    from fractions import Fraction
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1                                   # now 2^e <= a < 2^(e+1)
    ulp = Fraction(2) ** (max(e, -126) - 23)
    n, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and n % 2 == 1):
        n += 1
    return (n * ulp) if q > 0 else -(n * ulp)


def _rne_int(q):
    """nearest integer to a rational, ties to even"""
    import math as _m
    n = _m.floor(q)
    r = q - n
    return n + 1 if r * 2 > 1 or (r * 2 == 1 and n % 2 == 1) else n


def _uniform_reference_codes(xs, bits):
    """The uniform codec's codes written from its definition with exact
    rationals: m = min, M = max (values, a zero extreme +0),
    sigma = RN(RN(M - m) / (2^b - 1)), m_h = FP16(m), sigma_h = FP16(sigma),
    code = clamp(RNE(RN(RN(x - m_h) / sigma_h)), 0, 2^b - 1)."""
    from fractions import Fraction
    top = (1 << bits) - 1
    m, M = Fraction(float(xs.min())), Fraction(float(xs.max()))
    sigma = _rn32(_rn32(M - m) / top)
    mh = Fraction(float(np.float16(float(m))))             # numpy: RNE to FP16
    sh = Fraction(float(np.float16(float(sigma))))
    codes = []
    for x in xs:
        if sh == 0:
            codes.append(0)
            continue
        d = _rn32(Fraction(float(x)) - mh)
        codes.append(min(max(_rne_int(_rn32(d / sh)), 0), top))
    return codes, mh, sh


def _uniform_slot_codes(slot, v, d, bits, n_vec):
    cb = bits * d // 8
    blk = slot[32 + v * cb:32 + (v + 1) * cb]
    stream = np.unpackbits(blk, bitorder="little")
    return [int(sum(int(stream[bits * i + k]) << k for k in range(bits))) for i in range(d)]


@pytest.mark.parametrize("bits", [3, 4])
def test_uniform_codes_are_the_rounded_quotient(oracle, bits):
    """Every code against the definition built with exact rationals: the
    FP16 minimum and scale, the binary32 quotient RN(RN(x - m_h)/sigma_h)
    and its nearest integer, ties to even; the decode lies within half a step
    of the source."""
    rng = np.random.default_rng(8)
    codec = oracle.UNIFORM3 if bits == 3 else oracle.UNIFORM4
    top = (1 << bits) - 1
    x = rng.standard_normal((16, 32)).astype(np.float32) * 3
    vec = _bits(x, oracle.BF16)
    xs = oracle.src_to_f32(vec, oracle.BF16)
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, codec)
    assert st == oracle.SEG_ENCODED
    cb = bits * 32 // 8
    meta = slot[32 + 16 * cb:32 + 16 * (cb + 4)].view(np.uint16).reshape(16, 2)
    for v in range(16):
        ref, mh, sh = _uniform_reference_codes(xs[v], bits)
        assert float(np.ravel(oracle.f16_to_f32(meta[v, 0]))[0]) == float(mh)
        assert float(np.ravel(oracle.f16_to_f32(meta[v, 1]))[0]) == float(sh)
        assert _uniform_slot_codes(slot, v, 32, bits, 16) == ref
        dec = oracle.src_to_f32(oracle.decode_segment(slot, None, oracle.BF16, 32, 16)[v], oracle.BF16)
        assert np.all(np.abs(dec - xs[v]) <= float(sh) / 2 * 1.001 + abs(float(mh) - xs[v].min()) +
                      np.abs(dec) * 2.0 ** -8)
    assert top in (7, 15)


@pytest.mark.parametrize("bits", [3, 4])
def test_uniform_quotient_ties_go_to_even(oracle, bits):
    """Half-integer quotients decide the tie rule and the division: with
    minimum 0 and maximum 3*(2^b - 1), sigma_h = 3, and x = 1.5, 4.5, 7.5, ...
    give the exact quotients 0.5, 1.5, 2.5, ..., whose codes are the even
    neighbours 0, 2, 2, 4, 4, ...  Multiplying by the rounded reciprocal
    RN(1/3) > 1/3 instead would push every such quotient above the tie
    (codes 1, 2, 3, 4, 5, ...).  Both orders of x near the ties are also
    checked against the exact-rational definition."""
    codec = oracle.UNIFORM3 if bits == 3 else oracle.UNIFORM4
    top = (1 << bits) - 1
    xs = np.zeros(32, np.float32)
    xs[1] = 3.0 * top
    ties = [1.5 + 3.0 * k for k in range(top)]
    xs[2:2 + top] = ties
    # neighbours of the ties, one BF16 step either side
    nb = []
    for t in ties[:7]:
        b = int(np.float32(t).view(np.uint32)) >> 16
        nb += [float(np.uint32((b + 1) << 16).view(np.float32)), float(np.uint32((b - 1) << 16).view(np.float32))]
    xs[2 + top:2 + top + len(nb)] = nb[:32 - 2 - top]
    vec = np.tile(_bits(xs[None, :], oracle.BF16), (16, 1))
    xs = oracle.src_to_f32(vec, oracle.BF16)[0]
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, codec)
    assert st == oracle.SEG_ENCODED
    codes = _uniform_slot_codes(slot, 0, 32, bits, 16)
    ref, mh, sh = _uniform_reference_codes(xs, bits)
    assert float(mh) == 0.0 and float(sh) == 3.0
    assert codes == ref
    assert codes[2:2 + top] == [k + (k & 1) for k in range(top)]   # 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, ...


@pytest.mark.parametrize("bits", [3, 4])
def test_uniform_codes_random_scales_near_ties(oracle, bits):
    """FP16 vectors over many scales whose elements include every source
    value (up to a cap) at which the quotient rule differs from the two
    reciprocal readings -- RNE(RN(d * RN(1/sigma_h))) and the exact product
    d * RN(1/sigma_h) rounded once -- plus values next to the tie points
    m_h + (k + 1/2) sigma_h: every code against the exact-rational
    definition."""
    rng = np.random.default_rng(21)
    codec = oracle.UNIFORM3 if bits == 3 else oracle.UNIFORM4
    top = (1 << bits) - 1
    all_h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    all_h = np.concatenate([-all_h[1:], all_h])
    vecs, separating = [], 0
    for v in range(16):
        lo = np.float32(np.float16(rng.uniform(-4, 4)))
        hi = np.float32(np.float16(lo + rng.uniform(0.05, 60)))
        mh = np.float32(np.float16(lo))
        sig = np.float32(np.float16((hi - lo) / np.float32(top)))
        y = np.float32(1) / sig
        xs = all_h[(all_h > lo) & (all_h < hi)]
        d = (xs - mh).astype(np.float32)
        q = np.rint(d / sig)
        other = (q != np.rint((d * y).astype(np.float32))) | (q != np.rint(d.astype(np.float64) * float(y)))
        pick = list(xs[other][:40])
        separating += len(pick)
        while len(pick) < 62:
            k = int(rng.integers(0, top))
            t = np.float16(mh + (k + 0.5) * sig)
            pick.append(np.float32(np.uint16(int(t.view(np.uint16)) + int(rng.integers(-2, 3))).view(np.float16)))
        vecs.append(np.clip(np.array([lo, hi] + pick[:62], np.float32), lo, hi))
    assert separating >= 8                       # the readings are told apart
    vec = np.stack(vecs).astype(np.float16).view(np.uint16)
    xs = oracle.src_to_f32(vec, oracle.FP16)
    slot, st, _ = oracle.encode_segment(vec, oracle.FP16, codec)
    assert st == oracle.SEG_ENCODED
    for v in range(16):
        ref, _, _ = _uniform_reference_codes(xs[v], bits)
        assert _uniform_slot_codes(slot, v, 64, bits, 16) == ref


def test_uniform_sigma_rounds_to_binary32_then_fp16(oracle):
    """sigma is a binary32 value, RN(RN(max - min) / 15), that is then
    rounded to FP16.  With max = 8.5859375 and min = 0.005615234375 (FP16
    values), max - min = 15 * 0.572021484375 exactly, so sigma is exactly the
    FP16 midpoint 0.572021484375 and the stored scale is its even neighbour
    0.572265625 (0x3894).  A single rounding of a slightly different
    quotient (e.g. an FMA residual step rounded straight to FP16) can land on
    the odd neighbour 0.57177734375 (0x3893) instead."""
    from fractions import Fraction
    hi, lo = np.float16(8.5859375), np.float16(0.005615234375)
    assert float(hi) == 8.5859375 and float(lo) == 0.005615234375
    vec = np.full((16, 32), np.float16(1.0)).view(np.uint16)
    vec[:, 0] = hi.view(np.uint16)
    vec[:, 1] = lo.view(np.uint16)
    a = np.float32(hi) - np.float32(lo)
    assert Fraction(float(a)) == 15 * Fraction(0.572021484375)
    assert float(a / np.float32(15)) == 0.572021484375
    slot, st, _ = oracle.encode_segment(vec, oracle.FP16, oracle.UNIFORM4)
    assert st == oracle.SEG_ENCODED
    meta = slot[32 + 16 * 16:32 + 16 * 20].view(np.uint16).reshape(16, 2)
    assert np.all(meta[:, 1] == np.float16(0.572265625).view(np.uint16))
    assert np.all(meta[:, 0] == lo.view(np.uint16))


def test_uniform_zero_extremes_are_plus_zero(oracle):
    """A zero minimum or maximum is stored as +0 whichever signed zeros the
    vector holds and in whatever order (min and max are values)."""
    for first, second in ((0x8000, 0x0000), (0x0000, 0x8000), (0x8000, 0x8000)):
        vec = np.full((16, 32), np.float16(1.0)).view(np.uint16)
        vec[:, 3], vec[:, 7] = first, second
        slot, st, _ = oracle.encode_segment(vec, oracle.FP16, oracle.UNIFORM4)
        meta = slot[32 + 16 * 16:32 + 16 * 20].view(np.uint16).reshape(16, 2)
        assert np.all(meta[:, 0] == 0x0000)
        assert np.all(meta[:, 1] == np.float16(np.float32(1.0) / np.float32(15)).view(np.uint16))
        zero = np.zeros((16, 32), np.uint16)
        zero[:, 5] = first
        zero[:, 9] = second
        slot, st, _ = oracle.encode_segment(zero, oracle.FP16, oracle.UNIFORM4)
        meta = slot[32 + 16 * 16:32 + 16 * 20].view(np.uint16).reshape(16, 2)
        assert np.all(meta == 0)


def test_uniform_constant_vector(oracle):
    vec = np.full((16, 64), 0x4040, np.uint16)            # bf16 3.0
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.UNIFORM4)
    assert st == oracle.SEG_ENCODED and not slot[32:32 + 16 * 32].any()
    np.testing.assert_array_equal(oracle.decode_segment(slot, None, oracle.BF16, 64, 16), vec)


# ------------------------------------------------------------ TurboQuant
def _tq_codes(slot, n_vec, d, bits):
    cb = bits * d // 8
    out = np.zeros((n_vec, d), np.int64)
    for v in range(n_vec):
        stream = np.unpackbits(slot[32 + v * cb:32 + (v + 1) * cb], bitorder="little")
        out[v] = stream.reshape(d, bits) @ (1 << np.arange(bits))
    return out


@pytest.mark.parametrize("bits", [3, 4])
def test_tq_closed_form_basis_vector(oracle, bits):
    """x = sigma (.) H_j (a signed Hadamard row, D = 64, |x_i| = 1): n = 8,
    u = x/8 exactly, v = H_j / 8, z = H v = 8 e_j exactly.  So every code is
    the code of 0 (2^(b-1) - 1) except position j, which takes the top code."""
    from scipy.linalg import hadamard
    d, seed = 64, 99
    sig = oracle.signs(seed, d).astype(np.float32)
    H = hadamard(d).astype(np.float32)
    vecs = np.stack([sig * H[j] for j in range(16)])
    slot, st, _ = oracle.encode_segment(_bits(vecs, oracle.BF16), oracle.BF16,
                                        oracle.TQ3 if bits == 3 else oracle.TQ4, seed=seed)
    assert st == oracle.SEG_ENCODED
    codes = _tq_codes(slot, 16, d, bits)
    exp = np.full((16, d), (1 << (bits - 1)) - 1)
    exp[np.arange(16), np.arange(16)] = (1 << bits) - 1
    np.testing.assert_array_equal(codes, exp)
    norms = slot[32 + 16 * bits * 8:32 + 16 * bits * 8 + 32].view(np.uint16)
    assert np.all(norms == 0x4800)                           # FP16 8.0


@pytest.mark.parametrize("bits", [3, 4])
def test_tq_bucketize_is_nearest_centroid(oracle, bits):
    """Brute force over a segment: each code is the index of the nearest
    FP32 centroid to z = WHT(sigma * RN(x * RN(1/n)))."""
    rng = np.random.default_rng(9)
    d, seed = 32, 5
    x = rng.standard_normal((16, d)).astype(np.float32)
    vec = _bits(x, oracle.BF16)
    xs = oracle.src_to_f32(vec, oracle.BF16)
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.TQ3 if bits == 3 else oracle.TQ4,
                                        seed=seed)
    codes = _tq_codes(slot, 16, d, bits)
    cent, _ = oracle.codebook_f32(bits)
    sig = oracle.signs(seed, d).astype(np.float32)
    for v in range(16):
        n = np.float32(math.sqrt(oracle.sumsq_tree(xs[v])))
        u = xs[v] * (np.float32(1) / n)
        z = oracle.wht(sig * u)
        dist = np.abs(z[:, None].astype(np.float64) - cent[None, :])
        np.testing.assert_array_equal(codes[v], dist.argmin(1))


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_tq_scale_invariance_and_norm(oracle, d):
    """Scaling x by a power of two leaves every code unchanged (u is exactly
    the same); the restored vector has the stored FP16 norm."""
    rng = np.random.default_rng(10 + d)
    x = rng.standard_normal((16, d)).astype(np.float32)
    a, st, _ = oracle.encode_segment(_bits(x, oracle.BF16), oracle.BF16, oracle.TQ4, seed=3)
    b, st2, _ = oracle.encode_segment(_bits(x * 8, oracle.BF16), oracle.BF16, oracle.TQ4, seed=3)
    cb = d // 2
    np.testing.assert_array_equal(a[32:32 + 16 * cb], b[32:32 + 16 * cb])
    nh = oracle.f16_to_f32(a[32 + 16 * cb:32 + 16 * cb + 32].view(np.uint16))
    out = oracle.src_to_f32(oracle.decode_segment(a, None, oracle.BF16, d, 16, seed=3), oracle.BF16)
    np.testing.assert_allclose(np.linalg.norm(out.astype(np.float64), axis=1), nh, rtol=2 ** -7)


def test_tq_distortion_matches_lloyd_max(oracle):
    """Statistical: for Gaussian vectors the relative reconstruction error
    ||x - x_hat||^2 / ||x||^2 is close to the per-coordinate Lloyd-Max
    distortion (norm correction adds a little)."""
    g = golden("lloyd_max_gaussian.json")
    rng = np.random.default_rng(11)
    x = rng.standard_normal((128, 128)).astype(np.float32)
    for bits, codec in ((3, oracle.TQ3), (4, oracle.TQ4)):
        vec = _bits(x, oracle.FP16)
        xs = oracle.src_to_f32(vec, oracle.FP16)
        slot, st, _ = oracle.encode_segment(vec, oracle.FP16, codec, seed=1)
        out = oracle.src_to_f32(oracle.decode_segment(slot, None, oracle.FP16, 128, 128, seed=1),
                                oracle.FP16)
        rel = ((out - xs) ** 2).sum() / (xs ** 2).sum()
        mse = g["levels"][str(bits)]["mse"]
        assert 0.7 * mse < rel < 1.3 * mse


def test_raw_policy_roundtrip_bit_exact(oracle):
    rng = np.random.default_rng(12)
    vec = rng.integers(0, 65536, (128, 128), dtype=np.uint64).astype(np.uint16)   # incl. NaNs
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.TQ4, is_protected=True)
    assert st == oracle.SEG_RAW_POLICY and slot[1] == oracle.RAW and slot[2] == 1
    np.testing.assert_array_equal(oracle.decode_segment(slot, None, oracle.BF16, 128, 128), vec)


def test_header_fields(oracle):
    rng = np.random.default_rng(13)
    vec = _bits(rng.standard_normal((128, 128)), oracle.FP16)
    slot, st, _ = oracle.encode_segment(vec, oracle.FP16, oracle.FP8_FIXED, component=1,
                                        fixed_scale=0.5)
    h = slot[:32]
    assert h[0] == 1 and h[1] == oracle.FP8_FIXED and h[2] == 0 and h[3] == (2 | 1 << 4)
    assert h[4:6].view(np.uint16)[0] == 128 and h[6:8].view(np.uint16)[0] == 128
    assert h[8:12].view(np.uint32)[0] == 32768 and h[12:16].view(np.uint32)[0] == 128 * 128
    assert h[28:32].view(np.float32)[0] == 0.5
    assert len(slot) == 16640 and not slot[32 + 16384:].any()   # zero padding


def test_int8_round_half_to_even(oracle):
    """The page's codec rounds the FP32 quotient with torch's round(), which
    is half-to-even.  With amax = 127 the scale is exactly 1.0, so x itself is
    the quotient: 62.5 -> 62, 63.5 -> 64, -62.5 -> -62, 0.5 -> 0, 2.5 -> 2."""
    vals = [127.0, 62.5, 63.5, -62.5, 0.5, 1.5, 2.5, -0.5]
    vec = np.zeros((16, 32), np.uint16)
    vec[0, :len(vals)] = _bits(vals, oracle.BF16)
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.INT8)
    assert st == oracle.SEG_ENCODED
    assert list(slot[32:32 + len(vals)].view(np.int8)) == [127, 62, 64, -62, 0, 2, 2, 0]
    assert slot[32 + 16 * 32:36 + 16 * 32].view(np.float32)[0] == 1.0


# ------------------------------------------------------------ CRC32
def test_crc32_check_value(oracle):
    g = json.load(open(os.path.join(GOLDEN, "crc32_check.json")))
    assert oracle.crc32(g["input_ascii"].encode()) == int(g["crc32"], 16)


def test_crc32_matches_zlib(oracle):
    """The library routine zlib.crc32 computes the same CRC-32."""
    import zlib
    rng = np.random.default_rng(12)
    for n in (0, 1, 2, 3, 15, 16, 17, 255, 4096, 8480, 33000):
        b = rng.integers(0, 256, n, dtype=np.uint8)
        assert oracle.crc32(b) == zlib.crc32(b.tobytes())


@pytest.mark.parametrize("codec", ["TQ4", "UNIFORM3", "INT8", "FP8_DYNAMIC", "RAW"])
def test_segment_crc32(oracle, codec):
    """With the CRC option the header carries flag 8 and the CRC32 of the
    stored bytes (payload, raw slot body, or spilled raw bytes); a flipped
    stored byte makes decode fail; without it the field stays 0."""
    import zlib
    c = getattr(oracle, codec if codec != "RAW" else "RAW")
    rng = np.random.default_rng(5)
    vec = _bits(rng.standard_normal((16, 64)).astype(np.float32), oracle.BF16)
    slot, st, raw = oracle.encode_segment(vec, oracle.BF16, c, crc=True)
    stored = int(slot[12:16].view(np.uint32)[0])
    assert slot[2] & oracle.FLAG_CRC32
    assert int(slot[24:28].view(np.uint32)[0]) == zlib.crc32(slot[32:32 + stored].tobytes())
    out = oracle.decode_segment(slot, None, oracle.BF16, 64, 16)
    bad = slot.copy()
    bad[32 + stored // 2] ^= 0x10
    with pytest.raises(oracle.ChecksumError):
        oracle.decode_segment(bad, None, oracle.BF16, 64, 16)
    plain, st2, _ = oracle.encode_segment(vec, oracle.BF16, c)
    assert not (plain[2] & oracle.FLAG_CRC32) and not plain[24:28].any()
    np.testing.assert_array_equal(out, oracle.decode_segment(plain, None, oracle.BF16, 64, 16))


def test_segment_crc32_spilled(oracle):
    """A segment raw because of its data: the CRC covers the spilled bytes."""
    import zlib
    vec = np.full((16, 32), 0x3F80, np.uint16)
    vec[3, 4] = 0x7FC0                                    # NaN
    slot, st, raw = oracle.encode_segment(vec, oracle.BF16, oracle.TQ4, crc=True)
    assert st == oracle.SEG_RAW_DATA and slot[2] & oracle.FLAG_CRC32
    assert int(slot[24:28].view(np.uint32)[0]) == zlib.crc32(raw.tobytes())
    buf = np.concatenate([slot, raw])
    slot2 = slot.copy()
    slot2[16:24] = np.frombuffer(np.uint64(slot.size).tobytes(), np.uint8)
    np.testing.assert_array_equal(oracle.decode_segment(slot2, buf, oracle.BF16, 32, 16), vec)
    buf[slot.size + 7] ^= 1
    with pytest.raises(oracle.ChecksumError):
        oracle.decode_segment(slot2, buf, oracle.BF16, 32, 16)


# ------------------------------------------------------------ INT8 record codec
def _rows_segment(oracle, values_at, T=4, H=8, D=128, seed=0, dtype=1):
    """A segment of T tokens x H heads: N(0,1) values, with given vectors
    overwritten ({(t, h): values})."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T * H, D)).astype(np.float32)
    for (t, h), vals in values_at.items():
        x[t * H + h] = 0.0
        x[t * H + h, :len(vals)] = vals
    return _bits(x, dtype), x


def test_int8_record_sizes(oracle):
    """Row and record sizes are the page's: 1,040 data bytes padded to 1,152
    (9 x 128) at 8 heads x 128; 43.75% less than a 2,048-byte BF16 row,
    about 1.78x the tokens per budget."""
    g = golden("int8_record_sizes.json")
    H, D = g["kv_heads"], g["head_dim"]
    assert H * D == g["int8_bytes"] and 2 * H == g["scale_bytes"]
    assert g["int8_bytes"] + g["scale_bytes"] == g["raw_record"]
    assert oracle.row_bytes(D, H) == g["record"] == 9 * 128
    assert 1 - g["record"] / g["bf16_row"] == g["saving"]
    assert round(g["bf16_row"] / g["record"], 2) == g["capacity_ratio_rounded"]
    # slot: 32-byte header, rows from byte 128, 256-byte alignment
    T = 16
    assert oracle.slot_bytes(oracle.INT8_ROWS, D, T * H, H) == (128 + T * 1152 + 255) // 256 * 256
    for D2, H2 in ((32, 1), (64, 3), (256, 40)):
        assert oracle.row_bytes(D2, H2) % 128 == 0 and 0 <= oracle.row_bytes(D2, H2) - (H2 * D2 + 2 * H2) < 128


def test_int8_record_worked_example_and_layout(oracle):
    """The page's worked example (1.0, 0.5, -0.2, 0.0 -> 127, 64, -25, 0)
    planted in token 1, head 5: its codes sit at byte 128 + 1*1152 + 5*128
    of the slot, its BF16 scale after the row's 8 code blocks, the row
    padding and an all-zero head are zero, and the zero head restores to
    exactly zero."""
    g = golden("int8_worked_example.json")
    vec, _ = _rows_segment(oracle, {(1, 5): g["values"], (2, 3): [0.0]})
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.INT8_ROWS, heads=8)
    assert st == oracle.SEG_ENCODED and slot[1] == oracle.INT8_ROWS
    R = 1152
    row1 = slot[128 + R:128 + 2 * R]
    assert list(row1[5 * 128:5 * 128 + 4].view(np.int8)) == g["codes"]
    assert not row1[5 * 128 + 4:6 * 128].any()
    assert int(slot[12:16].view(np.uint32)[0]) == 4 * R                 # stored length: the rows
    assert not slot[32:128].any()                                        # gap before the rows
    for t in range(4):
        assert not slot[128 + t * R + 1040:128 + (t + 1) * R].any()      # row padding
    row2 = slot[128 + 2 * R:128 + 3 * R]
    assert not row2[3 * 128:4 * 128].any()                               # zero head: zero codes
    out = oracle.decode_segment(slot, None, oracle.BF16, 128, 32, heads=8)
    assert not out[2 * 8 + 3].any()                                      # ... restored to exact +0


def test_int8_record_power_of_two_amax_closed_form(oracle):
    """amax = 2^k: amax/127 = 2^(k-7) * 1.00787..., whose BF16 rounding is
    2^(k-7) * 129/128; x = 2^(k-1) then quotes 63.5039 -> code 64, and the
    amax element restores to 127*129*2^(k-14) = 2^k * 16383/16384, which
    rounds to 2^k in BF16 (hand-derived; k from -39 to 60, above the 1e-12
    floor).  Below the floor (2^-60) the scale is the floor's, and every
    code is 0."""
    vec, _ = _rows_segment(oracle, {(0, 0): [2.0 ** -60, -(2.0 ** -61)]}, T=16, H=8, D=32)
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.INT8_ROWS, heads=8)
    assert st == oracle.SEG_ENCODED and not slot[128:128 + 32].any()
    for k in range(-39, 61, 7):
        a = np.float32(2.0) ** k
        vec, _ = _rows_segment(oracle, {(0, 0): [a, a / 2, -a, a / 4]}, T=16, H=8, D=32, seed=k + 100)
        slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.INT8_ROWS, heads=8)
        assert st == oracle.SEG_ENCODED and slot[1] == oracle.INT8_ROWS
        R = oracle.row_bytes(32, 8)
        row = slot[128:128 + R]
        codes = list(row[:4].view(np.int8))
        assert codes == [127, 64, -127, 32], (k, codes)
        s = float(oracle.bf16_to_f32(row[256:258].view(np.uint16))[0])
        assert s == float(a) * 129.0 / 16384.0
        out = oracle.src_to_f32(oracle.decode_segment(slot, None, oracle.BF16, 32, 128, heads=8)[0, :3],
                                oracle.BF16)
        assert list(out) == [float(a), float(a) * 64 * 129 / 16384, -float(a)]


def test_int8_record_amax_codes_127_over_bf16_values(oracle):
    """Every third BF16 magnitude from 2^-39 (above the 1e-12 floor) to 2^100
    as a vector's amax encodes to code 127: the BF16-rounded scale is within
    2^-9 of amax/127, which keeps the quotient within (126.5, 127.5)."""
    mags = np.arange(0x2C00, 0x7180, 3, dtype=np.uint32)                 # BF16 bit patterns
    vals = (mags << 16).view(np.float32)
    H, D, T = 8, 32, 16
    per = T * H
    for i in range(0, len(vals), per):
        chunk = vals[i:i + per]
        x = np.zeros((per, D), np.float32)
        x[:len(chunk), 0] = chunk
        x[:len(chunk), 1] = -chunk / 3
        slot, st, _ = oracle.encode_segment(_bits(x, oracle.BF16), oracle.BF16, oracle.INT8_ROWS, heads=H)
        assert st == oracle.SEG_ENCODED
        R = oracle.row_bytes(D, H)
        for v in range(len(chunk)):
            t, h = divmod(v, H)
            assert np.int8(slot[128 + t * R + h * D]) == 127


def test_int8_record_error_bound(oracle):
    """|x - x_hat| <= s/2 (rounding to the code) + 127*s*2^-24 (FP32
    quotient) + half an output ulp, with s the stored BF16 scale; BF16 and
    FP16 outputs."""
    rng = np.random.default_rng(12)
    H, D, T = 4, 64, 16
    for dtype in (oracle.BF16, oracle.FP16):
        x = (rng.standard_normal((T * H, D)) * np.exp(rng.standard_normal((T * H, 1)) * 2)).astype(np.float32)
        bits = _bits(x, dtype)
        xs = oracle.src_to_f32(bits, dtype).astype(np.float64)
        slot, st, _ = oracle.encode_segment(bits, dtype, oracle.INT8_ROWS, heads=H)
        assert st == oracle.SEG_ENCODED
        out = oracle.src_to_f32(oracle.decode_segment(slot, None, dtype, D, T * H, heads=H), dtype).astype(np.float64)
        R = oracle.row_bytes(D, H)
        for v in range(T * H):
            t, h = divmod(v, H)
            s = float(oracle.bf16_to_f32(slot[128 + t * R + H * D + 2 * h:128 + t * R + H * D + 2 * h + 2]
                                         .view(np.uint16))[0])
            ulp = np.spacing(np.abs(out[v]).astype(np.float32 if dtype == oracle.BF16 else np.float16))
            half = ulp.astype(np.float64) * (2 ** 16 if dtype == oracle.BF16 else 1) / 2
            bound = s / 2 + 127 * s * 2.0 ** -24 + half
            assert np.all(np.abs(xs[v] - out[v]) <= bound + 1e-30), v


def test_int8_record_nonfinite_raw_and_crc(oracle):
    """A nonfinite value keeps the segment raw (spilled bit-exactly); with the
    CRC option the checksum covers the rows -- padding included -- and a
    flipped padding byte is caught."""
    vec, _ = _rows_segment(oracle, {(0, 1): [np.inf]}, T=16, H=4, D=64)
    slot, st, raw = oracle.encode_segment(vec, oracle.BF16, oracle.INT8_ROWS, heads=4)
    assert st == oracle.SEG_RAW_DATA and np.array_equal(raw.view(np.uint16).reshape(vec.shape), vec)
    vec, _ = _rows_segment(oracle, {}, T=16, H=4, D=64)
    slot, st, _ = oracle.encode_segment(vec, oracle.BF16, oracle.INT8_ROWS, heads=4, crc=True)
    assert st == oracle.SEG_ENCODED
    R = oracle.row_bytes(64, 4)
    assert slot[2] & oracle.FLAG_CRC32
    assert int(slot[24:28].view(np.uint32)[0]) == oracle.crc32(slot[128:128 + 16 * R])
    oracle.decode_segment(slot, None, oracle.BF16, 64, 64, heads=4)
    bad = slot.copy()
    bad[128 + R - 1] ^= 1                                                # padding of row 0
    with pytest.raises(oracle.ChecksumError):
        oracle.decode_segment(bad, None, oracle.BF16, 64, 64, heads=4)


# ------------------------------------------------------------ lossless entropy stage (rANS)
def _plane(kind, n, rng):
    if kind == "uniform":
        return rng.integers(0, 256, n).astype(np.uint8)
    if kind == "geometric":
        return np.minimum(rng.geometric(0.3, n) - 1, 255).astype(np.uint8)
    if kind == "constant":
        return np.full(n, 77, np.uint8)
    if kind == "two":
        return rng.choice(np.array([3, 200], np.uint8), n, p=[0.9, 0.1])
    raise ValueError(kind)


def test_ans_normalize_invariants(oracle):
    """Frequencies sum to 4096, a symbol gets a frequency iff it occurs, each
    present symbol gets at least 1 + floor(count * (4096 - K) / n), and only
    the most frequent symbol (lowest on ties) gets the remainder."""
    rng = np.random.default_rng(30)
    cases = [np.bincount(_plane(k, n, rng), minlength=256) for k in ("uniform", "geometric", "two", "constant")
             for n in (1, 8, 2048, 16384)]
    cases.append(np.arange(256))
    cases.append(np.r_[np.full(255, 1), 100000])
    for c in cases:
        c = c.astype(np.uint32)
        n, K = int(c.sum()), int((c > 0).sum())
        f = oracle.ans_normalize(c).astype(np.int64)
        if n == 0:
            continue
        assert f.sum() == 4096 and np.array_equal(f > 0, c > 0)
        base = np.where(c > 0, 1 + (c.astype(np.int64) * (4096 - K)) // n, 0)
        extra = f - base
        assert np.all(extra >= 0) and np.count_nonzero(extra) <= 1
        if extra.any():
            assert int(np.argmax(extra)) == int(np.argmax(c))


@pytest.mark.parametrize("kind", ["uniform", "geometric", "two", "constant"])
@pytest.mark.parametrize("n", [8, 2000, 2048, 16384, 16392])
def test_ans_plane_round_trip(oracle, kind, n):
    """decode(encode(plane)) is the plane, consuming exactly the encoded
    bytes, for several symbol distributions and lengths (streams of unequal
    length when n is not a multiple of 2048)."""
    sym = _plane(kind, n, np.random.default_rng(n))
    enc = oracle.ans_encode_plane(sym)
    dec, used = oracle.ans_decode_plane(enc, n)
    assert used == enc.size and np.array_equal(dec, sym)


def test_ans_constant_plane_closed_form(oracle):
    """A plane of one repeated symbol has probability 1: every stream is just
    the untouched initial state L = 2^23 (bytes 00 00 80 00).  The plane is
    the 16-byte header (mode 1, K = 1), the bitmap with only that symbol, its
    frequency 4096, 64 stream lengths of 4, 64 copies of L, padded to a
    multiple of 16."""
    enc = oracle.ans_encode_plane(np.full(16384, 9, np.uint8))
    want = [1, 0, 1, 0] + [0] * 12 + [0] * 32 + [0x00, 0x10] + [4, 0] * 64 + [0x00, 0x00, 0x80, 0x00] * 64
    want[16 + 1] = 0x02                                             # symbol 9: byte 1, bit 1
    want += [0] * (-len(want) % 16)
    assert list(enc) == want and enc.size % 16 == 0


def test_ans_raw_plane_when_coding_does_not_shrink(oracle):
    """Uniform random bytes do not compress: the plane is stored raw (a zero
    16-byte header, the bytes, zero padding to 16) and still round-trips."""
    sym = _plane("uniform", 16383, np.random.default_rng(4))
    enc = oracle.ans_encode_plane(sym)
    assert not enc[:16].any() and np.array_equal(enc[16:16 + sym.size], sym)
    assert enc.size == 16 + 16384 and enc[-1] == 0
    dec, used = oracle.ans_decode_plane(enc, sym.size)
    assert used == enc.size and np.array_equal(dec, sym)


def _rans_layout(enc):
    """(K, offset of the stream lengths, offset of the first stream) of a mode-1 plane."""
    k = int(enc[2:4].view(np.uint16)[0])
    lens = 16 + 32 + 2 * k
    return k, lens, lens + 128


@pytest.mark.parametrize("kind", ["geometric", "two"])
def test_ans_size_tracks_model_entropy(oracle, kind):
    """The streams of a coded plane hold its cross-entropy under the quantised
    model, sum of log2(4096 / f(s)) over the symbols: each stream adds its
    31-bit final state, and rANS with a 2^23..2^31 state loses well under
    1e-5 bits per symbol, so the renormalisation bytes lie between
    bits/8 - 4 per stream and bits/8 + 1 per stream."""
    n = 16384
    sym = _plane(kind, n, np.random.default_rng(7))
    enc = oracle.ans_encode_plane(sym)
    assert enc[0] == 1
    k, lens, first = _rans_layout(enc)
    f = oracle.ans_normalize(np.bincount(sym, minlength=256)).astype(np.float64)
    bits = np.log2(4096.0 / f[sym]).sum()
    renorm = int(enc[lens:lens + 128].view(np.uint16).astype(np.int64).sum()) - 4 * 64
    assert bits / 8 - 4 * 64 <= renorm <= bits / 8 * (1 + 1e-5) + 64


def test_ans_coded_size_lower_bound(oracle):
    """A coding step from a state in [2^23, 2^31) that emits b bytes leaves a
    state above x 2^(-8b) (4096 / f) (1 - 2^-11)^2, so a plane's 64 streams
    emit more than (H - 512 - 0.00141 n) / 8 renormalisation bytes, H the
    sum of log2(4096 / f(s)) over its symbols; its body is then at least
    416 + 2K + that.  The encoder skips the sizing pass of a plane whose
    bound reaches n.  Checked against the coded size on planes from uniform
    to skewed, including the low bytes of BF16 Gaussian data, which the
    bound declares raw."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal(16384).astype(np.float32)
    bf_lo = (_bits(x, oracle.BF16) & 0xFF).astype(np.uint8)
    planes = [_plane(k, n, rng) for k in ("uniform", "geometric", "two") for n in (2048, 8192, 16384)]
    planes += [bf_lo, (_bits(x, oracle.FP16) & 0xFF).astype(np.uint8), rng.integers(0, 200, 16384).astype(np.uint8)]
    for sym in planes:
        n = sym.size
        f = oracle.ans_normalize(np.bincount(sym, minlength=256)).astype(np.float64)
        k = int((f > 0).sum())
        h = np.log2(4096.0 / f[sym]).sum()
        body = oracle.ans_coded_body(sym)
        assert body >= 416 + 2 * k + (h - 512 - 0.00141 * n) / 8
    f = oracle.ans_normalize(np.bincount(bf_lo, minlength=256)).astype(np.float64)
    h = np.log2(4096.0 / f[bf_lo]).sum()
    assert 416 + 2 * int((f > 0).sum()) + (h * (1 - 2.0 ** -10) - 512 - 0.002 * 16384) / 8 >= 16384 + 1


def test_ans_exact_length_check(oracle):
    """A stream that ends early, runs long, or is corrupted is rejected, as is
    a frequency table that does not sum to 4096: the decoder must consume
    each stream to exactly its recorded length and end in the encoder's
    initial state."""
    rng = np.random.default_rng(3)
    sym = _plane("geometric", 16384, rng)
    enc = oracle.ans_encode_plane(sym)
    n = sym.size
    k, lens, first = _rans_layout(enc)
    assert oracle.ans_decode_plane(enc, n)[1] == enc.size
    short = enc.copy()
    short[lens:lens + 2] = (short[lens:lens + 2].view(np.uint16) - 1).view(np.uint8)   # stream 0 one byte shorter
    assert oracle.ans_decode_plane(short, n)[1] == 0
    longer = np.r_[enc[:first + 4], np.uint8(0), enc[first + 4:]]
    longer[lens:lens + 2] = (longer[lens:lens + 2].view(np.uint16) + 1).view(np.uint8)  # one byte longer
    assert oracle.ans_decode_plane(longer, n)[1] == 0
    rejected = 0
    for pos in rng.choice(np.arange(first, enc.size - 4), 40, replace=False):
        bad = enc.copy()
        bad[pos] ^= 1 << int(rng.integers(8))
        dec, used = oracle.ans_decode_plane(bad, n)
        assert used == 0 or not np.array_equal(dec, sym)     # never silently accepted as the original
        rejected += used == 0
    assert rejected >= 36                                     # the final-state check catches nearly all
    table = enc.copy()
    table[48:50] = (table[48:50].view(np.uint16) + 1).view(np.uint8)                    # frequencies sum to 4097
    assert oracle.ans_decode_plane(table, n)[1] == 0
    # a starting state outside the state interval [2^23, 2^31) is malformed
    for state in (0, (1 << 23) - 1, 1 << 31, 0xFFFFFFFF):
        st = enc.copy()
        st[first:first + 4] = np.array([state], np.uint32).view(np.uint8)
        assert oracle.ans_decode_plane(st, n)[1] == 0


def _kv_bits(rng, n_vec, d, dtype, scale=None):
    x = rng.standard_normal((n_vec, d)).astype(np.float32)
    if scale is not None:
        x *= scale
    return _bits(x, dtype)


def test_ans16_segment_lossless_and_compressing(oracle):
    """BF16 and FP16 KV segments (N(0,1) with lognormal channel scales, and
    with NaN, Inf and signed zeros planted) round-trip bit-exactly.  BF16:
    the payload sits in the spill region behind a header-only slot and the
    sign/exponent plane compresses the segment to about 71%; FP16 saves less
    than 12.5% and is stored raw."""
    rng = np.random.default_rng(8)
    for dtype in (oracle.BF16, oracle.FP16):
        vec = _kv_bits(rng, 128, 128, dtype, np.exp(rng.standard_normal(128)).astype(np.float32))
        vec[3, 5], vec[9, 0], vec[100, 127] = 0x7FC0 if dtype == oracle.BF16 else 0x7E00, 0x8000, \
            0x7F80 if dtype == oracle.BF16 else 0x7C00
        slot, st, pay = oracle.encode_segment(vec, dtype, oracle.ANS16)
        assert slot.size == 256
        if dtype == oracle.BF16:      # sign + 7 exponent bits: the high plane codes to ~3.3 bits
            assert st == oracle.SEG_ENCODED and slot[1] == oracle.ANS16
            assert slot[2] & oracle.FLAG_HEAP and int(slot[12:16].view(np.uint32)[0]) == pay.size
            assert pay.size < 0.72 * vec.nbytes
        else:                         # FP16 keeps 2 mantissa bits in the high byte: under 12.5% saved
            assert st == oracle.SEG_RAW_DATA and slot[1] == oracle.RAW
        buf = np.zeros(4096 + pay.size, np.uint8)
        buf[4096:] = pay
        slot[16:24] = np.frombuffer(np.uint64(4096).tobytes(), np.uint8)
        out = oracle.decode_segment(slot, buf, dtype, 128, 128)
        assert np.array_equal(out, vec)


def test_ans16_incompressible_size_and_crc(oracle):
    """Uniformly random 16-bit patterns do not compress: the segment is stored
    raw (data-dependent).  Sources below 4 KiB or above 32 KiB are raw by
    policy.  With the CRC option the checksum covers the payload."""
    rng = np.random.default_rng(9)
    vec = rng.integers(0, 1 << 16, (128, 128)).astype(np.uint16)
    slot, st, raw = oracle.encode_segment(vec, oracle.BF16, oracle.ANS16)
    assert st == oracle.SEG_RAW_DATA and np.array_equal(raw.view(np.uint16).reshape(vec.shape), vec)
    for n_vec, d in ((15, 64), (129, 128)):                  # 1,920 B and 33,024 B of source
        assert oracle.effective_codec(oracle.ANS16, d, n_vec, False) == oracle.RAW
    assert oracle.effective_codec(oracle.ANS16, 128, 16, False) == oracle.ANS16   # 4 KiB
    vec = _kv_bits(rng, 64, 64, oracle.BF16)
    slot, st, pay = oracle.encode_segment(vec, oracle.BF16, oracle.ANS16, crc=True)
    assert st == oracle.SEG_ENCODED and slot[2] & oracle.FLAG_CRC32
    assert int(slot[24:28].view(np.uint32)[0]) == oracle.crc32(pay)
    buf = np.r_[np.zeros(256, np.uint8), pay]
    slot[16:24] = np.frombuffer(np.uint64(256).tobytes(), np.uint8)
    assert np.array_equal(oracle.decode_segment(slot, buf, oracle.BF16, 64, 64), vec)
    buf[256 + pay.size // 2] ^= 0x10
    with pytest.raises(oracle.ChecksumError):
        oracle.decode_segment(slot, buf, oracle.BF16, 64, 64)
