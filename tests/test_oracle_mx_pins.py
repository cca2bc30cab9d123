"""Pins of the oracle's MXFP8 functions against the format definitions and an
independent implementation (torch's float8_e4m3fn cast), and of the MXFP8
layer against the BF16 layer within the format's error bound."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as orc


def _all_finite_codes():
    return np.array([c for c in range(256) if c not in (0x7F, 0xFF)])


def test_e4m3_table_from_its_definition():
    v = orc.e4m3_decode(np.arange(256))
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.sum(np.isnan(v)) == 2
    pos = v[:127]
    assert np.all(np.diff(pos) > 0)                  # code order is value order
    assert pos[0] == 0 and pos[1] == 2.0 ** -9       # smallest subnormal
    assert pos[8] == 2.0 ** -6                       # smallest normal
    assert pos[126] == 448.0 == orc.E4M3_MAX         # largest normal 1.75 * 2^8
    assert pos[56] == 1.0                            # exponent field 7 = bias
    np.testing.assert_array_equal(v[128:255], -v[:127])
    # spacing: 8 values per binade, step 2^(e-3) in binade 2^e (e >= -6)
    for e in range(-6, 9):
        b = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(b) == (8 if e < 8 else 7)
        np.testing.assert_allclose(np.diff(b), 2.0 ** (e - 3))


def test_e4m3_round_trip_and_ties():
    codes = _all_finite_codes()
    np.testing.assert_array_equal(orc.e4m3_encode(orc.e4m3_decode(codes)), codes)
    pos = orc.e4m3_decode(np.arange(127))
    mid = (pos[:-1] + pos[1:]) / 2
    got = orc.e4m3_encode(mid)
    lo = np.arange(126)
    expect = np.where(lo % 2 == 0, lo, lo + 1)       # ties go to the even code
    np.testing.assert_array_equal(got, expect)
    eps = np.diff(pos) * 1e-3
    np.testing.assert_array_equal(orc.e4m3_encode(mid - eps), lo)
    np.testing.assert_array_equal(orc.e4m3_encode(mid + eps), lo + 1)


def test_e4m3_saturates_and_keeps_the_sign():
    assert orc.e4m3_encode(np.array([449.0, 464.0, 479.9, 1e6]))[0] == 0x7E
    np.testing.assert_array_equal(orc.e4m3_encode(np.array([479.9, 1e6, -1e6])),
                                  [0x7E, 0x7E, 0xFE])
    np.testing.assert_array_equal(orc.e4m3_encode(np.array([-0.0, -1e-9, 0.0, 1e-9])),
                                  [0x80, 0x80, 0x00, 0x00])


def test_e4m3_matches_torch_cast_in_range():
    """torch's float8_e4m3fn cast rounds to nearest even and turns overflow
    into NaN; below 464 (the tie above 448) the two must agree."""
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-463.9, 463.9, 20000),
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000),        # subnormal range
                        np.ldexp(rng.uniform(0.5, 1, 5000), rng.integers(-12, 9, 5000))])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(orc.e4m3_encode(v32.astype(np.float64)), ref)


def test_mx_scale_is_the_smallest_that_fits():
    """Brute force: the shared exponent is floor(log2 amax) - 8, i.e. the one
    that puts amax / X in [256, 512)."""
    rng = np.random.default_rng(1)
    v = np.ldexp(rng.standard_normal((64, 32 * 4)), rng.integers(-30, 30, (64, 1)))
    q, s = orc.mx_quantize(v)
    for r in range(64):
        for b in range(4):
            amax = np.max(np.abs(v[r, 32 * b:32 * b + 32]))
            k = -200
            while amax / 2.0 ** k >= 512:
                k += 1
            while amax / 2.0 ** k < 256:
                k -= 1
            assert s[r, b] == k + 127
            assert 256 <= amax / 2.0 ** k < 512


def test_mx_zero_block_power_of_two_invariance_and_error_bound():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((16, 96))
    v[3, 32:64] = 0.0
    q, s = orc.mx_quantize(v)
    assert s[3, 1] == 0 and np.all(q[3, 32:64] == 0)
    q2, s2 = orc.mx_quantize(v * 2.0 ** 13)
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2[s > 0].astype(int), s[s > 0].astype(int) + 13)
    # each element within half an E4M3 step of its value (relative to the block
    # scale X: half a step is 2^(e-4) X for a scaled magnitude in [2^e, 2^(e+1)),
    # 2^-10 X in the subnormal range), except saturated ones (scaled value > 448)
    deq = orc.mx_dequantize(q, s)
    X = np.repeat(orc.e8m0_decode(s), 32, axis=1)
    a = np.abs(v) / X
    half = np.where(a >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(a, 1e-300))) - 4), 2.0 ** -10)
    sat = a > 448
    assert np.all(np.abs(deq - v)[~sat] <= (half * X)[~sat] * (1 + 1e-12))
    assert np.all(np.abs(deq[sat]) == 448 * X[sat])


def test_mx_layer_tracks_the_bf16_layer():
    """The MXFP8 layer equals the BF16 layer up to MXFP8 quantization error.
    E4M3 keeps 3 mantissa bits: a value is moved by at most 2^-4 of itself,
    about 2.4% RMS; four quantized operands (x, W_gu, H, W_d) compound to a
    few percent to ~10% per output row on random data. A scale applied along
    the wrong dimension or to the wrong block would be off by orders of
    magnitude."""
    rng = np.random.default_rng(3)
    T, d, N, K, F, C = 96, 64, 8, 2, 96, 40
    logits = rng.standard_normal((T, N)).astype(np.float32)
    x = orc.round_bf16(rng.standard_normal((T, d)) * np.exp2(rng.integers(-3, 4, (T, 1))))
    w_gu = orc.round_bf16(rng.standard_normal((N, 2 * F, d)) * 0.05)
    w_d = orc.round_bf16(rng.standard_normal((N, d, F)) * 0.05)
    ref = orc.moe_layer(logits, x, w_gu, w_d, K, C, 1, 0, "f64")
    mx = orc.moe_layer_mx(logits, x, w_gu, w_d, K, C, 1, 0)
    err = np.linalg.norm(mx["out"] - ref["out"], axis=1) / np.linalg.norm(ref["out"], axis=1)
    assert err.max() < 0.25 and np.median(err) < 0.12, (err.max(), np.median(err))
    # qdata / scales rows follow the route map: every written row is its token's
    q, s = orc.mx_quantize(x)
    for t in range(T):
        for k in range(K):
            r = mx["dest_row"][t, k]
            if r >= 0:
                np.testing.assert_array_equal(mx["qbuf"][r], q[t])
                np.testing.assert_array_equal(mx["sbuf"][r], s[t])
    n = int(mx["offsets"][0, -1])
    assert mx["written"][:n].all() and not mx["written"][n:].any()


def test_mx_expert_ffn_against_the_bf16_ffn_on_dequantized_operands():
    """On the dequantized operands, the MXFP8 expert's H before quantization is
    bit for bit the BF16 expert's H (expert_ffn_rows, pinned separately), its
    qdata/scales are that H quantized, and Y is torch's dense product of the
    dequantized H and W_d rounded to bf16."""
    rng = np.random.default_rng(4)
    n, d, F = 40, 96, 64
    X = rng.standard_normal((n, d)) * np.exp2(rng.integers(-4, 4, (n, 1)))
    Wgu = rng.standard_normal((2 * F, d)) * 0.05
    Wd = rng.standard_normal((d, F)) * 0.05
    Xq, Xs = orc.mx_quantize(X)
    gq, gs = orc.mx_quantize(Wgu)
    dq, ds = orc.mx_quantize(Wd)
    Hq, Hs, Y = orc.expert_ffn_mx_rows(Xq, Xs, gq, gs, dq, ds)
    H_bf16, _ = orc.expert_ffn_rows(orc.mx_dequantize(Xq, Xs), orc.mx_dequantize(gq, gs),
                                    orc.mx_dequantize(dq, ds), "bf16")
    q2, s2 = orc.mx_quantize(H_bf16)
    np.testing.assert_array_equal(Hq, q2)
    np.testing.assert_array_equal(Hs, s2)
    Yt = torch.nn.functional.linear(torch.from_numpy(orc.mx_dequantize(Hq, Hs)),
                                    torch.from_numpy(orc.mx_dequantize(dq, ds)))
    np.testing.assert_array_equal(Y, orc.round_bf16(Yt.numpy()))
