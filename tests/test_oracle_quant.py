"""Pins of the quantization references: OCP E4M3 code table, exhaustive
round trips and ties; int8 hand values, ties and error bound."""
import math

import numpy as np

from oracle import quant as Q


def test_e4m3_table_values():
    # Values from the OCP OFP8 E4M3 definition (bias 7, subnormal m * 2^-9).
    assert Q.e4m3_decode(0x00) == 0.0
    assert Q.e4m3_decode(0x01) == 2.0 ** -9
    assert Q.e4m3_decode(0x07) == 7 * 2.0 ** -9
    assert Q.e4m3_decode(0x08) == 2.0 ** -6
    assert Q.e4m3_decode(0x38) == 1.0
    assert Q.e4m3_decode(0x39) == 1.125
    assert Q.e4m3_decode(0x7E) == 448.0
    assert Q.e4m3_decode(0xFE) == -448.0
    assert Q.e4m3_decode(0x77) == 240.0
    assert math.isnan(Q.e4m3_decode(0x7F)) and math.isnan(Q.e4m3_decode(0xFF))
    vals = [Q.e4m3_decode(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:]))


def test_e4m3_round_trip_all_codes():
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = np.array([Q.e4m3_decode(c) for c in codes])
    vals[codes.index(0x80)] = -0.0
    enc = Q.e4m3_encode(vals)
    assert list(enc) == codes


def test_e4m3_ties_and_saturation():
    cases = {
        1.0625: 0x38,          # midpoint of 1.0 (0x38) and 1.125 (0x39) -> even 0x38
        1.1875: 0x3A,          # midpoint of 1.125 and 1.25 -> even 0x3A
        1.0624999: 0x38,
        1.0625001: 0x39,
        2.0 ** -10: 0x00,      # half the smallest subnormal -> 0 (even)
        3 * 2.0 ** -10: 0x02,  # midpoint of codes 1 and 2 -> 2
        432.0: 0x7E,           # midpoint of 416 (0x7D) and 448 (0x7E) -> even 0x7E
        424.0: 0x7D,
        449.0: 0x7E, 500.0: 0x7E, 1e6: 0x7E,
        -1.0625: 0xB8, -500.0: 0xFE,
    }
    for x, c in cases.items():
        assert int(Q.e4m3_encode(np.array([x]))[0]) == c, (x, hex(c))


def test_int8_hand_values():
    x = np.zeros((1, 1, 4, 8), np.float32)
    x[0, 0, 0, :] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, 63.4, -127.0]
    codes, scales = Q.quantize_int8_blocks(x, block=128)
    assert scales[0, 0, 0] == np.float32(1.0)
    assert list(codes[0, 0, 0]) == [127, 0, 2, 2, 0, -2, 63, -127]
    z = np.zeros((1, 1, 130, 4), np.float32)
    c, s = Q.quantize_int8_blocks(z)
    assert s.shape == (1, 1, 2) and not s.any() and not c.any()


def test_int8_ragged_blocks_and_error_bound():
    r = np.random.default_rng(0)
    x = r.standard_normal((2, 3, 300, 16)).astype(np.float32)
    codes, scales = Q.quantize_int8_blocks(x)
    assert scales.shape == (2, 3, 3)
    for i in range(3):
        blk = x[:, :, 128 * i:128 * (i + 1)]
        np.testing.assert_array_equal(scales[:, :, i], (np.abs(blk).max(axis=(2, 3)) / np.float32(127)).astype(np.float32))
    deq = Q.dequantize_int8(codes, scales)
    bound = np.repeat(scales, 128, axis=2)[:, :, :300, None] * 0.5 * (1 + 1e-6)
    assert np.all(np.abs(deq - x) <= bound)
    assert np.abs(codes).max() == 127


def test_fp8_channels_scale_and_bound():
    r = np.random.default_rng(1)
    x = (r.standard_normal((1, 2, 257, 8)) * r.uniform(0.5, 2, (1, 2, 1, 8))).astype(np.float32)
    codes, scales = Q.quantize_fp8_channels(x)
    np.testing.assert_array_equal(scales, (np.abs(x).max(axis=2) / np.float32(448)).astype(np.float32))
    deq = Q.dequantize_fp8(codes, scales)
    # E4M3 has 3 mantissa bits: relative error <= 2^-4 for normals, plus the
    # subnormal absolute step 2^-10 (half of 2^-9) in scaled units.
    err = np.abs(deq - x)
    bound = np.abs(x) * 2.0 ** -4 + scales[:, :, None, :] * 2.0 ** -10 + 1e-12
    assert np.all(err <= bound)
    # The absmax entry of every channel encodes to +-448 exactly.
    dec = Q.e4m3_decode_array(codes)
    assert np.allclose(np.abs(dec).max(axis=2), 448.0)


def test_int8_block32_hand_values():
    # Two 32-row blocks with different magnitudes: each block gets its own amax / 127.
    x = np.zeros((1, 1, 64, 4), np.float32)
    x[0, 0, 3, 1] = 2.54     # block 0 amax
    x[0, 0, 10, 2] = -1.0
    x[0, 0, 40, 0] = 0.127   # block 1 amax
    x[0, 0, 50, 3] = 0.0635
    codes, scales = Q.quantize_int8_blocks(x, block=32)
    assert scales.shape == (1, 1, 2)
    assert scales[0, 0, 0] == np.float32(np.float32(2.54) / np.float32(127.0))
    assert scales[0, 0, 1] == np.float32(np.float32(0.127) / np.float32(127.0))
    assert codes[0, 0, 3, 1] == 127 and codes[0, 0, 40, 0] == 127
    assert codes[0, 0, 10, 2] == -50                        # -1 / 0.02 = -50
    assert codes[0, 0, 50, 3] == 64                         # 0.0635 / 0.001 = 63.5 -> ties to even 64
    # The coarse block takes the larger magnitude for both halves.
    c128, s128 = Q.quantize_int8_blocks(x, block=128)
    assert s128[0, 0, 0] == scales[0, 0, 0] and c128[0, 0, 40, 0] == 6   # 0.127 / 0.02 = 6.35 -> 6


def test_centering_keeps_output_and_shifts_lse():
    """Closed form: attention(q, k - mu, v) = attention(q, k, v) and lse moves by
    sm_scale * q . mu (pinned against the separately pinned attention oracle)."""
    from oracle import attention as A
    rng = np.random.default_rng(3)
    B, Hq, Hkv, L, D = 2, 4, 2, 37, 16
    q = rng.standard_normal((B, Hq, L, D)).astype(np.float32)
    k = (rng.standard_normal((B, Hkv, L, D)) + 3.0 * rng.standard_normal((1, Hkv, 1, D))).astype(np.float32)
    v = rng.standard_normal((B, Hkv, L, D)).astype(np.float32)
    mu = Q.k_channel_mean(k)
    np.testing.assert_allclose(mu, k.astype(np.float64).mean(axis=2), rtol=0, atol=1e-6)
    kc = Q.center_k(k, mu)
    o1, l1 = A.attention(q, k, v, {})
    o2, l2 = A.attention(q, kc, v, {})
    delta = Q.q_dot_mean(q, mu)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-5)
    np.testing.assert_allclose(l2 + delta / np.sqrt(D), l1, rtol=0, atol=1e-4)
    assert np.abs(kc.astype(np.float64).mean(axis=2)).max() < 1e-5


def test_k_mean_is_exactly_rounded():
    # Values whose float32 running sum loses bits: the fsum-based mean is exact.
    k = np.zeros((1, 1, 4, 1), np.float32)
    k[0, 0, :, 0] = [1e8, 1.0, -1e8, 1.0]
    assert Q.k_channel_mean(k)[0, 0, 0] == np.float32(0.5)


def test_attention_dequantized_without_rounding_is_attention_on_dequantized_inputs():
    """With round_p=False the diagnostic is plain attention on the dequantized tensors, so it must
    equal the (separately pinned) attention oracle run on dequantize_int8 / dequantize_fp8 outputs."""
    from oracle import attention as A
    rng = np.random.default_rng(11)
    B, H, L, D = 2, 3, 150, 16
    q = rng.standard_normal((B, H, L, D)).astype(np.float32)
    k = rng.standard_normal((B, H, L, D)).astype(np.float32)
    v = (rng.standard_normal((B, H, L, D)) * rng.uniform(0.5, 2, (1, H, 1, D))).astype(np.float32)
    q8, sq = Q.quantize_int8_blocks(q)
    k8, sk = Q.quantize_int8_blocks(k)
    v8, sv = Q.quantize_fp8_channels(v)
    qd, kd, vd = Q.dequantize_int8(q8, sq), Q.dequantize_int8(k8, sk), Q.dequantize_fp8(v8, sv)
    o_ref, _ = A.attention(qd, kd, vd, {})
    for b, h in ((0, 0), (1, 2)):
        rows = np.arange(L)
        got = Q.attention_dequantized(q8, sq, k8, sk, v8, sv, rows, b, h, round_p=False)
        np.testing.assert_allclose(got, o_ref[b, h], rtol=0, atol=1e-12)
    # An explicit scale is the attention oracle's sm_scale.
    o_ref2, _ = A.attention(qd, kd, vd, {"sm_scale": 0.3})
    got = Q.attention_dequantized(q8, sq, k8, sk, v8, sv, np.arange(L), 1, 1, sm_scale=0.3, round_p=False)
    np.testing.assert_allclose(got, o_ref2[1, 1], rtol=0, atol=1e-12)


def test_attention_dequantized_p_rounding_hand_case():
    """Two keys worked by hand (tests/golden/quant_p_tie.json): 448 P lands exactly on the midpoint of
    the E4M3 values 160 and 176 and must round to the even code (160); the row sum must use the
    unrounded P."""
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quant_p_tie.json")))
    s = -float(np.log(g["p_key1"]))
    while np.exp(-s) != g["p_key1"]:  # the precondition of the derivation: exp(-s) is exactly 0.375
        s = float(np.nextafter(s, 0.0))
    q8 = np.array(g["q_codes"], np.int8).reshape(1, 1, 1, 4)
    k8 = np.array(g["k_codes"], np.int8).reshape(1, 1, 2, 4)
    v8 = np.array(g["v_codes"], np.uint8).reshape(1, 1, 2, 4)
    one = np.ones((1, 1, 1), np.float32)
    sv = np.array(g["v_scales"], np.float32).reshape(1, 1, 4)
    want_r = np.array([n / d for n, d in g["out_round_p"]])
    want_x = np.array([n / d for n, d in g["out_exact_p"]])
    got_r = Q.attention_dequantized(q8, one, k8, one, v8, sv, [0], 0, 0, sm_scale=s, round_p=True)[0]
    got_x = Q.attention_dequantized(q8, one, k8, one, v8, sv, [0], 0, 0, sm_scale=s, round_p=False)[0]
    np.testing.assert_allclose(got_r, want_r, rtol=0, atol=1e-15)
    np.testing.assert_allclose(got_x, want_x, rtol=0, atol=1e-15)
    # The plausible wrong readings give different values (the pin can tell them apart).
    v0 = np.array([1.0, 1.0, -2.0, 0.5])
    v1 = np.array([2.0, -0.5, 8.0, 1.0])
    assert np.abs(got_r - (28 * v0 + 11 * v1) / 38.5).max() > 1e-3   # tie rounded up to 176
    assert np.abs(got_r - (14 * v0 + 5 * v1) / 19.0).max() > 1e-3    # row sum of the rounded P
