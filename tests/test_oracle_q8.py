"""Pins of the oracle's low-bit latent rows (CPU only).

Section 8 ("Compositionality") stacks quantisation on the loop axis; the oracle stores a latent row
as E4M3 codes with one float32 scale. Pinned to torch's float8_e4m3fn conversion (a library
routine), to the exhaustive list of E4M3 values, and to the rounding-error bound of the format.
"""
import numpy as np
import torch

from oracle import lla_oracle as O


def _all_e4m3_values():
    out = []
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e, m = (c >> 3) & 0xF, c & 7
        if e == 15 and m == 7:
            continue  # NaN
        out.append(s * (m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)))
    return np.array(out)


def test_every_e4m3_value_rounds_to_itself():
    v = _all_e4m3_values()
    assert v.size == 254
    np.testing.assert_array_equal(O.e4m3_round(v), v)


def test_rounding_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(7)
    v = _all_e4m3_values()
    pos = np.sort(v[v > 0])
    mids = (pos[:-1] + pos[1:]) / 2  # exact ties
    x = np.concatenate([
        mids, -mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf),
        rng.standard_normal(100000) * 10.0 ** rng.uniform(-4, 2.6, 100000),
        [0.0, -0.0, 447.9, 448.0, 455.0, 463.9, 464.0, 470.0, 1e4, 2.0 ** -10, 3 * 2.0 ** -11],
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_round(x.astype(np.float64))
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), x[~same][:10]


def test_quantized_rows_bound_and_extremes():
    rng = np.random.default_rng(8)
    z = (rng.standard_normal((64, 24)) * 10.0 ** rng.uniform(-3, 3, (64, 1))).astype(np.float32)
    z[3] = 0.0
    codes, s = O.quantize_latent_rows(z)
    assert s[3] == 0 and np.all(codes[3] == 0)
    live = s > 0
    # the largest magnitude of each row lands on +-448 exactly
    np.testing.assert_array_equal(np.max(np.abs(codes[live]), axis=1), 448.0)
    # scales are float32 values
    np.testing.assert_array_equal(s, s.astype(np.float32).astype(np.float64))
    # round-to-nearest error bound: half a step, 2^-4 relative for normals, s * 2^-10 below 2^-6 s
    zq = O.dequantize_latent_rows(codes, s)
    err = np.abs(zq - z)
    bound = np.maximum(np.abs(z) * 2.0 ** -4, s[:, None] * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    # and every code is an E4M3 value
    assert np.isin(codes, _all_e4m3_values()).all()


# --------------------------------------------------------------------------------------------
# integer rows: symmetric int8 codes with one float32 scale per row
# --------------------------------------------------------------------------------------------

def test_int8_rows_extremes_bound_and_symmetry():
    rng = np.random.default_rng(18)
    z = (rng.standard_normal((64, 24)) * 10.0 ** rng.uniform(-3, 3, (64, 1))).astype(np.float32)
    z[5] = 0.0
    codes, s = O.quantize_latent_rows_int8(z)
    assert s[5] == 0 and np.all(codes[5] == 0)
    live = s > 0
    # integer codes in [-127, 127]; the largest magnitude of each row lands on +-127 exactly
    np.testing.assert_array_equal(codes, np.round(codes))
    assert np.max(np.abs(codes)) <= 127
    np.testing.assert_array_equal(np.max(np.abs(codes[live]), axis=1), 127.0)
    np.testing.assert_array_equal(np.sign(codes[live][np.abs(codes[live]) == 127]),
                                  np.sign(z[live][np.abs(codes[live]) == 127]))
    # scales are float32 values equal to max|z| / 127 rounded to float32
    np.testing.assert_array_equal(s, (np.max(np.abs(z), axis=1) / np.float32(127)).astype(np.float32))
    # round to nearest: at most half a step from the value
    err = np.abs(O.dequantize_latent_rows(codes, s) - z)
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    # odd symmetry
    cn, sn = O.quantize_latent_rows_int8(-z)
    np.testing.assert_array_equal(sn, s)
    np.testing.assert_array_equal(cn, -codes)


def test_int8_integer_rows_and_ties_to_even():
    # a row of integers whose largest magnitude is 127 has scale 1 and reproduces itself
    z = np.array([[127, -3, 0, 64, -127, 1, 2, -100]], np.float32)
    codes, s = O.quantize_latent_rows_int8(z)
    assert s[0] == 1.0
    np.testing.assert_array_equal(codes, z)
    # scale 2 (max 254): z / s = k + 1/2 exactly, ties go to the even neighbour
    z = np.array([[254, 1, 3, 5, -1, -3, -5, 7]], np.float32)
    codes, s = O.quantize_latent_rows_int8(z)
    assert s[0] == 2.0
    np.testing.assert_array_equal(codes, [[127, 0, 2, 2, -0, -2, -2, 4]])
