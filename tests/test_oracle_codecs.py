"""Pins of the oracle's codecs against definitions, library routines and hand-derived bytes."""
import os

import numpy as np
import pytest
import torch

from oracle import codecs as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- FP8 E4M3
def _known_e4m3():
    out = []
    for line in open(os.path.join(GOLDEN, "e4m3_known_values.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        out.append((int(code, 16), float(val)))
    return out


def test_e4m3_known_values_from_spec():
    for code, val in _known_e4m3():
        got = C.e4m3_decode(np.uint8(code))
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e4m3_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = C.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.array_equal(np.isnan(ref), np.isnan(ours))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], ours[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(ours[fin]))


def _torch_e4m3(x32):
    return torch.from_numpy(x32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_on_values_midpoints_and_random():
    vals = np.sort(C.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    mids = (vals[1:] + vals[:-1]) / 2.0                      # exact ties
    near = np.concatenate([np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(1e9))])
    rng = np.random.default_rng(7)
    rand = rng.uniform(-448, 448, 200000).astype(np.float32)
    small = (rng.standard_normal(50000) * 0.01).astype(np.float32)
    x = np.concatenate([vals, -vals, mids, -mids, near, -near, rand, small]).astype(np.float32)
    assert np.array_equal(C.e4m3_encode(x), _torch_e4m3(x))


def test_e4m3_encode_saturates_where_torch_gives_nan():
    x = np.array([448, 449, 463.99, 464, 465, 1e6, 3.4e38, -465, -1e30], np.float32)
    ours = C.e4m3_encode(x)
    ref = _torch_e4m3(np.clip(x, -448, 448).astype(np.float32))
    assert np.array_equal(ours, ref)
    assert list(ours[:6]) == [0x7E] * 6 and ours[-1] == 0xFE


def test_e4m3_round_trip_all_finite_codes_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = C.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(C.e4m3_encode(vals), codes)
    # 2^-10 is the midpoint of 0 and 2^-9: ties to the even code 0x00.
    assert C.e4m3_encode(np.float32(2.0 ** -10)) == 0x00
    # 3 * 2^-11 lies nearer 2^-9 (code 0x01).
    assert C.e4m3_encode(np.float32(3 * 2.0 ** -11)) == 0x01
    # 1 + 1/16 is the midpoint of 1 (0x38) and 1.125 (0x39): ties to even 0x38.
    assert C.e4m3_encode(np.float32(1.0625)) == 0x38
    assert C.e4m3_encode(np.float32(1.1875)) == 0x3A


# ------------------------------------------------------------------- fp16/bf16
def test_tq3_scale_matches_torch_half_rounding():
    rng = np.random.default_rng(3)
    a = np.concatenate([rng.uniform(0, 10, 100000), rng.uniform(0, 1e-4, 10000),
                        rng.uniform(1e4, 3e5, 10000)]).astype(np.float32)
    q = (a / np.float32(3.5)).astype(np.float32)
    ref = torch.from_numpy(np.minimum(q, np.float32(65504))).to(torch.float16).numpy()
    assert np.array_equal(C.tq3_scale(a).view(np.uint16), ref.view(np.uint16))


def test_tq3_scale_closed_forms():
    assert C.tq3_scale(np.float32(3.5)) == np.float16(1.0)
    assert C.tq3_scale(np.float32(0.0)) == np.float16(0.0)
    assert C.tq3_scale(np.float32(3.5 * 65504 * 4)) == np.float16(65504.0)
    assert C.tq3_scale(np.float32(3.5 * 2.0 ** -24)) == np.float16(2.0 ** -24)


def test_bf16_bits():
    x = torch.tensor([1.0, -2.5, 3.140625, 1e-20], dtype=torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(C.bf16_bits_to_value(bits), x.to(torch.float64).numpy())


# -------------------------------------------------------------------- TQ3 pack
def _kats():
    out = []
    for line in open(os.path.join(GOLDEN, "tq3_pack_kat.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, codes, hexbytes = [p.strip() for p in line.split(";")]
        out.append((name, np.array([int(c) for c in codes.split(",")], np.uint8),
                    bytes.fromhex(hexbytes)))
    return out


@pytest.mark.parametrize("name,codes,expect", _kats(), ids=[k[0] for k in _kats()])
def test_tq3_pack_known_answers(name, codes, expect):
    got = C.tq3_pack_row(codes).tobytes()
    assert got == expect
    assert np.array_equal(C.tq3_unpack_row(np.frombuffer(expect, np.uint8), 32), codes)


def test_tq3_pack_unpack_round_trip_rows():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 8, (50, 256)).astype(np.uint8)
    packed = C.tq3_pack_row(codes)
    assert packed.shape == (50, 96)
    assert np.array_equal(C.tq3_unpack_row(packed, 256), codes)
    # groups of one row concatenate: group g's 12 bytes equal the group packed alone
    for g in range(8):
        assert np.array_equal(packed[:, 12 * g:12 * g + 12], C.tq3_pack_row(codes[:, 32 * g:32 * g + 32]))


# ------------------------------------------------------------------ TQ3 encode
def _rand_fp16_scales(rng, n):
    bits = rng.integers(0x0001, 0x7BFF, n).astype(np.uint16)      # finite positive fp16
    return bits.view(np.float16)


def test_tq3_exact_round_trip_of_representable_groups():
    rng = np.random.default_rng(5)
    n = 20000
    s = _rand_fp16_scales(rng, n)
    codes = rng.integers(0, 8, (n, 32)).astype(np.uint8)
    codes[np.arange(n), rng.integers(0, 32, n)] = rng.choice([0, 7], n)   # amax = 3.5 s
    x = ((codes.astype(np.float64) - 3.5) * s.astype(np.float64)[:, None]).astype(np.float32)
    assert np.array_equal(x.astype(np.float64),
                          (codes.astype(np.float64) - 3.5) * s.astype(np.float64)[:, None])
    got_c, got_s = C.tq3_encode_groups(x)
    assert np.array_equal(got_s.view(np.uint16), s.view(np.uint16))
    assert np.array_equal(got_c, codes)
    assert np.array_equal(C.tq3_decode(got_c, got_s), x.astype(np.float64))


def test_tq3_threshold_ties_go_up_and_neighbours_go_down():
    rng = np.random.default_rng(9)
    s = _rand_fp16_scales(rng, 2000).astype(np.float16)
    for b in range(-3, 4):
        tie = (b * s.astype(np.float64)).astype(np.float32)
        assert np.array_equal(tie.astype(np.float64), b * s.astype(np.float64))
        assert np.all(C.tq3_codes(tie, s) == b + 4)
        below = np.nextafter(tie, np.float32(-np.inf))
        assert np.all(C.tq3_codes(below, s) == b + 3)


def test_tq3_codes_are_nearest_level_by_brute_force():
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((3000, 32)) * rng.uniform(0.01, 50, (3000, 1))).astype(np.float32)
    c, s = C.tq3_encode_groups(x)
    levels = (np.arange(8)[None, None, :] - 3.5) * s.astype(np.float64)[:, None, None]
    dist = np.abs(x.astype(np.float64)[..., None] - levels)             # [n][32][8]
    best = dist.min(axis=-1)
    # chosen level is a nearest one; among equals the upper level is chosen
    chosen = np.take_along_axis(dist, c[..., None].astype(np.int64), -1)[..., 0]
    assert np.array_equal(chosen, best)
    upper = 7 - np.argmin(dist[..., ::-1], axis=-1)
    assert np.array_equal(c, upper.astype(np.uint8))


def test_tq3_zero_scale_and_zero_group():
    x = np.full((2, 32), 1e-30, np.float32)
    x[1] = 0.0
    c, s = C.tq3_encode_groups(x)
    assert np.all(s == 0) and np.all(c == 4)
    assert np.all(C.tq3_decode(c, s) == 0.0)


def test_tq3_zero_element_maps_to_code_4():
    x = np.zeros(32, np.float32)
    x[0] = 3.5
    c, s = C.tq3_encode_groups(x)
    assert s == np.float16(1.0) and c[0] == 7 and np.all(c[1:] == 4)


# ----------------------------------------------------------------- bf16 encode
@pytest.mark.parametrize("x, bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                 # exact tie, kept part even: down
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # exact tie, kept part odd: up to even
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above the tie: up
    (1.0 + 2.0 ** -8 - 2.0 ** -20, 0x3F80),    # just below the tie: down
    (-(1.0 + 3 * 2.0 ** -8), 0xBF82),          # sign-magnitude: same rounding
    (2.0 - 2.0 ** -23, 0x4000),                # carry out of the significand into the exponent
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (3.0, 0x4040),
])
def test_bf16_encode_hand_values(x, bits):
    assert int(C.bf16_encode(np.float32(x))) == bits


def test_bf16_encode_is_nearest_with_ties_to_even():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(20000) * 10.0 ** rng.integers(-20, 20, 20000)).astype(np.float32)
    enc = C.bf16_encode(x).astype(np.int64)
    r = C.bf16_bits_to_value(enc)
    lo = C.bf16_bits_to_value(enc - 1)        # neighbours in the same binade direction
    hi = C.bf16_bits_to_value(enc + 1)
    xd = x.astype(np.float64)
    assert np.all(np.abs(xd - r) <= np.abs(xd - lo)) and np.all(np.abs(xd - r) <= np.abs(xd - hi))
    tie = (np.abs(xd - r) == np.abs(xd - lo)) | (np.abs(xd - r) == np.abs(xd - hi))
    assert np.all(enc[tie] % 2 == 0)


def test_bf16_encode_matches_torch_bfloat16():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal(50000) * 10.0 ** rng.integers(-35, 35, 50000)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(C.bf16_encode(x), ref)
