"""Pins of the fp8 (E4M3) cache oracle against the format's definition and
the mathematics of the quantiser, independent of the oracle's own code paths."""
import math

import numpy as np

import oracle
from oracle import fp8_cache as f8

TABLE = f8.E4M3_TABLE


def test_e4m3_constants_of_the_format():
    # OCP E4M3: largest finite 448 (S.1111.110), smallest normal 2^-6,
    # smallest subnormal 2^-9, one = exponent 7 (bias 7), two NaN codes, no inf
    assert TABLE[0x7E] == 448.0 and TABLE[0xFE] == -448.0
    assert TABLE[0x08] == 2.0 ** -6 and TABLE[0x01] == 2.0 ** -9 and TABLE[0x07] == 7 * 2.0 ** -9
    assert TABLE[0x38] == 1.0 and TABLE[0x40] == 2.0 and TABLE[0x30] == 0.5
    assert math.isnan(TABLE[0x7F]) and math.isnan(TABLE[0xFF])
    assert np.isfinite(TABLE).sum() == 254 and not np.isinf(TABLE).any()
    pos = TABLE[:0x7F]
    assert (np.diff(pos) > 0).all()  # codes 0..0x7E increase
    # spacing: 2^-9 up to the first binade, then 2^(e-10) inside binade e
    assert np.allclose(np.diff(pos[:16]), 2.0 ** -9)
    assert np.diff(pos[0x70:0x78]).tolist() == [16.0] * 7 and np.diff(pos[0x78:0x7F]).tolist() == [32.0] * 6


def test_encode_round_trip_and_ties():
    finite = [c for c in range(256) if np.isfinite(TABLE[c])]
    vals = np.array([TABLE[c] for c in finite], dtype=np.float32)
    assert f8.e4m3_encode(vals).tolist() == finite  # every code round-trips (0x80 is -0.0)
    for c in range(0x7E):  # the midpoint of two neighbours goes to the even code
        mid = np.float32((TABLE[c] + TABLE[c + 1]) / 2)  # exact in float32
        want = c if c % 2 == 0 else c + 1
        assert f8.e4m3_encode(mid) == want and f8.e4m3_encode(-mid) == want | 0x80
        lo, hi = np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(1e9))
        assert f8.e4m3_encode(lo) == c and f8.e4m3_encode(hi) == c + 1


def test_quantize_row_pins():
    rng = np.random.default_rng(8)
    for _ in range(50):
        x = (rng.standard_normal(128) * rng.uniform(1e-3, 1e3)).astype(np.float32)
        codes, scale = f8.quantize_row(x)
        i = int(np.argmax(np.abs(x)))
        assert codes[i] == (0xFE if x[i] < 0 else 0x7E)  # the largest magnitude becomes 448
        assert scale == np.float32(np.float32(np.abs(x).max()) / np.float32(448))
        # error bound: half an ulp of 3 mantissa bits, or half the subnormal step
        err = np.abs(TABLE[codes] * float(scale) - x.astype(np.float64))
        bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * float(scale) + 2.0 ** -20 * np.abs(x)
        assert (err <= bound).all()
        # powers of two commute with the quantiser: same codes, scale times 2^k
        for k in (-5, 3):
            c2, s2 = f8.quantize_row(x * np.float32(2.0 ** k))
            assert np.array_equal(c2, codes) and s2 == np.float32(scale * 2.0 ** k)
    codes, scale = f8.quantize_row(np.zeros(64, np.float32))
    assert scale == 0 and not codes.any()


def test_write_fp8_places_rows_and_skips():
    rng = np.random.default_rng(9)
    nb, hkv, d = 4, 2, 64
    kc = np.full((nb, hkv, 16, d), 0x7F, np.uint8)
    vc = kc.copy()
    ks = np.full((nb, hkv, 16), np.nan, np.float32)
    vs = ks.copy()
    nk = rng.standard_normal((3, hkv, d)).astype(np.float32)
    nv = rng.standard_normal((3, hkv, d)).astype(np.float32)
    slots = np.array([5, -1, 63], np.int32)
    k2, v2, ks2, vs2 = f8.kv_write_fp8(kc, vc, ks, vs, nk, nv, slots, "f32")
    for i, s in ((0, 5), (2, 63)):
        b, o = divmod(s, 16)
        for g in range(hkv):
            c, sc = f8.quantize_row(nk[i, g])
            assert np.array_equal(k2[b, g, o], c) and ks2[b, g, o] == sc
            c, sc = f8.quantize_row(nv[i, g])
            assert np.array_equal(v2[b, g, o], c) and vs2[b, g, o] == sc
    touched = np.zeros((nb, 16), bool)
    touched[0, 5] = touched[3, 15] = True
    assert (k2.transpose(0, 2, 1, 3)[~touched] == 0x7F).all() and np.isnan(ks2.transpose(0, 2, 1)[~touched]).all()
    assert (v2.transpose(0, 2, 1, 3)[~touched] == 0x7F).all() and np.isnan(vs2.transpose(0, 2, 1)[~touched]).all()


def test_decode_fp8_special_cases():
    rng = np.random.default_rng(10)
    hq, hkv, d = 8, 2, 64
    kc = rng.integers(0, 0x7F, size=(6, hkv, 16, d)).astype(np.uint8)
    vc = rng.integers(0, 0x7F, size=(6, hkv, 16, d)).astype(np.uint8) | (rng.integers(0, 2, (6, hkv, 16, d)) << 7).astype(np.uint8)
    ks = rng.uniform(1e-3, 1e-2, size=(6, hkv, 16)).astype(np.float32)
    vs = rng.uniform(1e-3, 1e-2, size=(6, hkv, 16)).astype(np.float32)
    q = rng.standard_normal((2, hq, d)).astype(np.float32)
    tables = np.array([[4, 1], [2, 0]], np.int32)
    # one token: the output is that token's dequantised V row
    out = f8.decode_fp8(q, kc, vc, ks, vs, tables, [1, 1], 0.125, "f32")
    for s in range(2):
        b = tables[s, 0]
        for h in range(hq):
            g = h // (hq // hkv)
            assert np.array_equal(out[s, h], TABLE[vc[b, g, 0]] * float(vs[b, g, 0]))
    # identical keys everywhere: the mean of the dequantised V rows (20 tokens)
    kc2 = np.full_like(kc, 0x38)
    ks2 = np.ones_like(ks)
    out = f8.decode_fp8(q, kc2, vc, ks2, vs, tables, [20, 20], 0.3, "f32")
    V = f8.dequantize(vc, vs)
    for s in range(2):
        rows = [V[tables[s, t // 16], :, t % 16] for t in range(20)]
        mean = np.mean(rows, axis=0)  # [hkv, d]
        for h in range(hq):
            assert np.allclose(out[s, h], mean[h // (hq // hkv)], rtol=1e-12, atol=1e-15)


def test_decode_fp8_close_to_unquantised():
    """Quantising K and V moves the attention output by about the codes' relative
    precision (2^-4), not more: a dropped scale or a wrong code table would not."""
    w_rng = np.random.default_rng(11)
    hq, hkv, d, L = 8, 2, 128, 200
    nb = -(-L // 16)
    x_k = w_rng.standard_normal((nb, hkv, 16, d)).astype(np.float32)
    x_v = w_rng.standard_normal((nb, hkv, 16, d)).astype(np.float32)
    q = w_rng.standard_normal((1, hq, d)).astype(np.float32)
    kc = np.zeros((nb, hkv, 16, d), np.uint8)
    vc = kc.copy()
    ks = np.zeros((nb, hkv, 16), np.float32)
    vs = ks.copy()
    for b in range(nb):
        for g in range(hkv):
            for o in range(16):
                kc[b, g, o], ks[b, g, o] = f8.quantize_row(x_k[b, g, o])
                vc[b, g, o], vs[b, g, o] = f8.quantize_row(x_v[b, g, o])
    table = np.arange(nb, dtype=np.int32)[None]
    got = f8.decode_fp8(q, kc, vc, ks, vs, table, [L], 1 / np.sqrt(d), "f32")
    ref = oracle.decode(q, x_k, x_v, table, [L], 1 / np.sqrt(d), "f32")
    rel = oracle.max_rownorm_rel_err(got, ref)
    assert 1e-4 < rel < 0.1, rel
