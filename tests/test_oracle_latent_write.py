"""Pins of the oracle's cache writer and FP8 encoder against things other than
themselves.

Page citation: [decode_k] "metrale_model_arch/glm5next_dsa/layer/decode_k.rs"
(the latent_write launch: kv_a row, kv_a_layernorm weight, pool, slot,
rms_eps, 1/kv_scale; the slot of a position is physical page * block_size +
position mod block_size).

What pins what:
  * FP8 encode: every finite code survives decode -> encode; torch's
    float32 -> float8_e4m3fn cast (round to nearest even) on random values in
    range; hand-placed midpoints; saturation beyond 448.
  * RMSNorm: closed forms (a constant row normalises to its sign; a one-hot
    row to sqrt(D) at the hot position; a zero row with eps > 0 to zero), and
    invariance of the codes to scaling the row by a power of two (eps = 0).
  * Where eps sits: rows whose mean square is comparable to eps, with closed
    forms (eps = c^2 on a constant row c gives 1/sqrt(2); eps = 3 * mean
    square gives exactly half of each entry over the rms). eps added after
    the root, or scaled by D, fails both.
  * Addressing: a pool pre-filled with a sentinel, rows written to hand-placed
    slots, every other byte untouched; negative slots write nothing.
"""
import math

import numpy as np
import pytest
import torch


def bf16_bits(x) -> np.ndarray:
    t = torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def torch_encode(x: np.ndarray) -> np.ndarray:
    """Library FP8 encode (torch), round to nearest even, no saturation."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_encode_inverts_decode_on_every_finite_code(oracle_mod):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = oracle_mod.fp8_e4m3fn(codes)
    back = oracle_mod.fp8_e4m3fn_encode(vals)
    np.testing.assert_array_equal(back, codes)


def test_encode_matches_torch_cast_in_range(oracle_mod):
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.uniform(-448, 448, 3000),
        rng.normal(0, 1, 3000),
        rng.normal(0, 1e-2, 2000),  # subnormal range
        np.exp2(rng.uniform(-12, 8.8, 2000)) * rng.choice([-1, 1], 2000),
    ]).astype(np.float32)  # torch casts from float32: compare on float32 inputs
    x = x[np.abs(x) < 448]
    np.testing.assert_array_equal(oracle_mod.fp8_e4m3fn_encode(x.astype(np.float64)),
                                  torch_encode(x))


@pytest.mark.parametrize("value,code", [
    (1.0625, 0x38),      # midpoint of 1.0 (m=0) and 1.125 (m=1): even m
    (1.1875, 0x3A),      # midpoint of 1.125 (m=1) and 1.25 (m=2): even m
    (1.9375, 0x40),      # midpoint of 1.875 (e=7, m=7) and 2.0 (e=8, m=0)
    (2.0 ** -10, 0x00),  # midpoint of 0 and the smallest subnormal
    (3 * 2.0 ** -10, 0x02),
    (464.0, 0x7E),       # past 448: saturates (a NaN code is never produced)
    (1e30, 0x7E),
    (-1e30, 0xFE),
    (-0.0, 0x80),
])
def test_encode_landmarks(oracle_mod, value, code):
    assert int(oracle_mod.fp8_e4m3fn_encode([value])[0]) == code


def _write(oracle_mod, rows, w, slots, *, D, B=16, pages=8, stride=0, eps=0.0, inv=1.0):
    stride_b = stride or B * D
    pool = np.full(pages * stride_b, 0xA5, dtype=np.uint8)
    vals = oracle_mod.latent_write(bf16_bits(rows), bf16_bits(w), np.asarray(slots, np.int64),
                                   pool, block_size=B, cache_stride_bytes=stride,
                                   eps=eps, inv_kv_scale=inv)
    return pool, vals


def test_constant_row_normalises_to_its_sign(oracle_mod):
    D = 64
    rows = np.stack([np.full(D, 3.0), np.full(D, -0.25)])
    w = np.linspace(0.5, 2.0, D)
    pool, vals = _write(oracle_mod, rows, w, [0, 1], D=D, inv=4.0)
    wb = oracle_mod.bf16(bf16_bits(w))
    np.testing.assert_allclose(vals[0], wb * 4.0, rtol=1e-15)
    np.testing.assert_allclose(vals[1], -wb * 4.0, rtol=1e-15)


def test_one_hot_row_normalises_to_sqrt_d(oracle_mod):
    D = 128
    row = np.zeros(D)
    row[37] = -5.0
    pool, vals = _write(oracle_mod, row[None], np.ones(D), [5], D=D)
    want = np.zeros(D)
    want[37] = -math.sqrt(D)
    np.testing.assert_allclose(vals[0], want, rtol=1e-15, atol=0)
    got = oracle_mod.fp8_e4m3fn(pool[5 * D:6 * D])
    np.testing.assert_array_equal(got, oracle_mod.fp8_e4m3fn(oracle_mod.fp8_e4m3fn_encode(want)))


def test_zero_row_with_eps_is_zero(oracle_mod):
    D = 64
    pool, vals = _write(oracle_mod, np.zeros((1, D)), np.ones(D), [2], D=D, eps=1e-6)
    assert np.all(vals == 0.0)
    assert np.all(pool[2 * D:3 * D] == 0)


def test_codes_invariant_to_power_of_two_scaling(oracle_mod):
    rng = np.random.default_rng(3)
    D = 256
    row = rng.normal(0, 1, D)
    w = rng.uniform(0.5, 1.5, D)
    p1, _ = _write(oracle_mod, row[None], w, [0], D=D, inv=10.0)
    p2, _ = _write(oracle_mod, (row * 64.0)[None], w, [0], D=D, inv=10.0)
    np.testing.assert_array_equal(p1[:D], p2[:D])


def test_rows_land_in_their_slots_and_nowhere_else(oracle_mod):
    rng = np.random.default_rng(5)
    D, B, pages = 64, 16, 8
    stride = B * D + 256  # pages further apart than their rows
    slots = [0, 17, 3 * B + 15, -1, 7 * B]
    rows = rng.normal(0, 1, (len(slots), D))
    pool, vals = _write(oracle_mod, rows, np.ones(D), slots, D=D, B=B, pages=pages,
                        stride=stride, inv=3.0)
    touched = np.zeros(pool.size, dtype=bool)
    for i, s in enumerate(slots):
        if s < 0:
            assert np.all(vals[i] == 0)
            continue
        off = (s // B) * stride + (s % B) * D
        np.testing.assert_array_equal(pool[off:off + D], oracle_mod.fp8_e4m3fn_encode(vals[i]))
        touched[off:off + D] = True
    assert np.all(pool[~touched] == 0xA5)


def test_writer_rejects_bad_arguments(oracle_mod):
    D = 64
    with pytest.raises(ValueError):
        _write(oracle_mod, np.ones((1, D)), np.ones(D), [8 * 16], D=D)  # past the pool
    with pytest.raises(ValueError):
        _write(oracle_mod, np.ones((1, D)), np.ones(D), [0], D=D, eps=-1.0)


def test_eps_sits_inside_the_root_constant_row(oracle_mod):
    # A constant row c with eps = c^2: the mean square is c^2, so the row
    # normalises to c / sqrt(2 c^2) = 1/sqrt(2) (times weight and 1/kv_scale).
    # eps added after the root (c / (|c| + eps)) gives ~1, a scaled eps
    # (D * eps, eps / D) gives 1/sqrt(D + 1) or ~1: all fail.
    D = 64
    c = 2.0 ** -10
    w = np.linspace(0.5, 2.0, D)
    pool, vals = _write(oracle_mod, np.full((1, D), c), w, [0], D=D, eps=c * c, inv=4.0)
    wb = oracle_mod.bf16(bf16_bits(w))
    np.testing.assert_allclose(vals[0], wb * 4.0 / math.sqrt(2.0), rtol=1e-15)
    np.testing.assert_array_equal(pool[:D], oracle_mod.fp8_e4m3fn_encode(vals[0]))


def test_eps_three_times_the_mean_square_halves_the_row(oracle_mod):
    # Entries +-2^-8 (mean square 2^-16) with eps = 3 * 2^-16: the root is
    # sqrt(4 * 2^-16) = 2^-7, so every entry maps to +-1/2 exactly.
    D = 128
    sign = np.where(np.arange(D) % 3 == 0, -1.0, 1.0)
    row = sign * 2.0 ** -8
    pool, vals = _write(oracle_mod, row[None], np.ones(D), [1], D=D,
                        eps=3.0 * 2.0 ** -16, inv=1.0)
    np.testing.assert_array_equal(vals[0], sign * 0.5)
    # 0.5 is an FP8 code: 0x30 (e = 6, m = 0), with the sign bit for -0.5
    want = np.where(sign < 0, 0xB0, 0x30).astype(np.uint8)
    np.testing.assert_array_equal(pool[D:2 * D], want)
