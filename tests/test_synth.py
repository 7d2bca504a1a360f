"""The seeded input generator: Philox known answers, random access, moments,
bf16 rounding and the DHSA chunk-length recipe."""
import math

import numpy as np

import synth


def test_philox_known_answers():
    # Known-answer vectors of Philox4x32-10 published with the SC'11 paper's
    # reference implementation (Random123 kat_vectors).
    assert synth.philox_block([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C,
                                                         0x9B00DBD8]
    assert synth.philox_block([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E,
                                                                       0xA20BC7C6, 0x6D5451FD]
    assert synth.philox_block([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344],
                              [0xA4093822, 0x299F31D0]) == [0xD16CFE09, 0x94FDCCEB, 0x5001E420,
                                                            0x24126EA1]


def test_own_log_and_sincos_match_libm():
    rng = np.random.default_rng(1)
    for x in list(rng.random(2000) * 0.9999 + 1e-10) + [2.0 ** -33, 0.5, 1.0 - 2.0 ** -33]:
        assert abs(synth.log_(x) - math.log(x)) <= 4e-16 * abs(math.log(x)) + 1e-300
    for a in np.linspace(0.0, math.pi / 2, 4001)[:-1]:
        s, c = synth.sincos_quarter(a)
        assert abs(s - math.sin(a)) < 5e-16 and abs(c - math.cos(a)) < 5e-16


def test_random_access_equals_sequential():
    full = synth.normal((4099,), synth.F64, 11, synth.TID_K)
    for first, n in [(0, 5), (1, 7), (3, 1), (1001, 999), (4095, 4)]:
        part = synth.normal((n,), synth.F64, 11, synth.TID_K, first=first)
        assert np.array_equal(part, full[first:first + n])


def test_determinism_and_independence():
    a = synth.normal((1000,), synth.F32, 5, synth.TID_Q)
    b = synth.normal((1000,), synth.F32, 5, synth.TID_Q)
    c = synth.normal((1000,), synth.F32, 6, synth.TID_Q)
    d = synth.normal((1000,), synth.F32, 5, synth.TID_K)
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c) and not np.array_equal(a, d)


def test_normal_moments():
    z = synth.normal((1 << 22,), synth.F64, 3, synth.TID_V)
    n = z.size
    assert abs(z.mean()) < 5 / math.sqrt(n)
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / n)
    assert abs((z ** 3).mean()) < 5 * math.sqrt(15 / n)
    assert abs((z ** 4).mean() - 3) < 5 * math.sqrt(96 / n)
    # tail mass beyond 3 sigma: 0.0027
    assert abs((np.abs(z) > 3).mean() - 0.0026998) < 5 * math.sqrt(0.0027 / n)


def test_scale_and_dtypes():
    z = synth.normal((512,), synth.F64, 9, synth.TID_Q)
    f = synth.normal((512,), synth.F32, 9, synth.TID_Q, scale=0.5)
    h = synth.normal((512,), synth.BF16, 9, synth.TID_Q, scale=0.5)
    assert np.array_equal(f, (0.5 * z).astype(np.float32))
    assert np.array_equal(h, synth.f32_to_bf16(f))


def test_bf16_round_to_nearest_even():
    cases = {
        1.0: 0x3F80,
        -2.0: 0xC000,
        # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to even -> 1.0
        1.0 + 2.0 ** -8: 0x3F80,
        # 1 + 3*2^-8 halfway between 1+2^-7 and 1+2^-6: ties to even (up)
        1.0 + 3 * 2.0 ** -8: 0x3F82,
        1.0 + 2.0 ** -8 + 2.0 ** -20: 0x3F81,
        3.3895313892515355e38: 0x7F7F,  # largest bf16 value is exact
        1e-40: 0x0001,  # fp32 subnormal rounds to the nearest bf16 subnormal
        0.0: 0x0000,
    }
    for x, bits in cases.items():
        assert int(synth.f32_to_bf16(np.float32(x))) == bits, x
    back = synth.bf16_to_f32(np.array([0x3F80, 0xC000, 0x3F81], np.uint16))
    assert list(back) == [1.0, -2.0, 1.0078125]


def test_chunk_offsets_recipe():
    offs = synth.chunk_offsets(16384, 16, 128, seed=5)
    lens = np.diff(offs)
    assert offs[0] == 0 and offs[-1] == 16384
    assert (lens >= 1).all() and (lens[:-1] >= 16).all() and (lens <= 128).all()
    assert 180 < len(lens) < 300
    assert np.array_equal(offs, synth.chunk_offsets(16384, 16, 128, seed=5))
    # the mean of U{16..128} is 72
    big = np.diff(synth.chunk_offsets(2_000_000, 16, 128, seed=7))[:-1]
    assert abs(big.mean() - 72) < 0.5
    assert big.min() == 16 and big.max() == 128


def test_needle_key_direction():
    q = synth.normal((4, 128), synth.BF16, 4, synth.TID_QDEC)
    k = synth.bf16_to_f32(synth.needle_key(q, True)).astype(np.float64)
    u = synth.bf16_to_f32(q).astype(np.float64).sum(0)
    cos = k @ u / np.linalg.norm(k) / np.linalg.norm(u)
    assert cos > 0.9999 and abs(np.linalg.norm(k) - 3) < 0.02
