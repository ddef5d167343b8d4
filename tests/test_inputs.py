"""The seeded input generators (CPU only)."""
import numpy as np
import pytest

import fa_inputs
from oracle import fa_back_oracle as O


def test_q8_0_encoding_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 128), dtype=np.float32)
    x[0, 0, :32] = 0.0                                   # an all-zero block
    enc = fa_inputs.encode_q8_0(x)
    assert enc.shape == (3, 5, 4 * 34) and enc.dtype == np.uint8
    dec = O.widen(enc, "q8_0", 128)
    blk = x.reshape(3, 5, 4, 32).astype(np.float64)
    step = np.abs(blk).max(-1, keepdims=True) / 127.0
    err = np.abs(dec.reshape(blk.shape) - blk)
    # |x - s*q| <= s/2 from the rounding, plus the fp16 rounding of s times |q| <= 127
    assert np.all(err <= step * (0.5 + 127 * 2.0 ** -11) + 1e-12)
    assert np.all(dec[0, 0, :32] == 0.0)
    assert np.all(enc[0, 0, :34] == 0)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -9], dtype=np.float32)
    got = O.widen(fa_inputs.to_bf16_bits(x), "bf16")
    np.testing.assert_array_equal(got, [1.0, 1.0, 1.0 + 2.0 ** -6, -2.5, 1.0])


def test_seeded_and_reproducible():
    a = fa_inputs.make("c1")
    b = fa_inputs.make("c1")
    for f in ("q", "k", "v", "d"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    c = fa_inputs.make("c1", seed=1)
    assert not np.array_equal(a.q, c.q)


def test_causal_tail_mask_structure():
    m = fa_inputs.causal_tail_mask(4, 10, Hm=1, typ="f32")
    for i in range(4):
        for j in range(10):
            assert (m[0, i, j] == 0.0) == (j <= 10 - 4 + i)
            assert m[0, i, j] in (0.0, -np.inf)


def test_config0_has_one_fully_masked_row():
    p = fa_inputs.make("c0")
    assert p.Hm == 2 and p.mask.shape == (2, 16, 64)
    dead = ~np.isfinite(p.mask).any(axis=2)
    assert dead.sum() == 1 and dead[1, 0]
    np.testing.assert_array_equal(p.mask[0, 1:], p.mask[1, 1:])


def test_strided_view_shares_values_with_contiguous():
    a = fa_inputs.make("c1")
    s = fa_inputs.make("c1_strided")
    np.testing.assert_array_equal(np.asarray(a.k), np.asarray(s.k))
    assert s.k.strides[1] == a.Hkv * s.k.shape[2] and s.k.strides[0] == s.k.shape[2]


def test_visible_pairs_and_flops():
    p = fa_inputs.make("c0")
    V = fa_inputs.visible_pairs(p)
    # head 0: sum_i (M-N+i+1) = 16*49 + 120 = 904 ; head 1 loses row 0 (49 keys)
    assert V == 904 + 904 - 49
    f = fa_inputs.flop_count(p)
    assert f["full"] == 2 * V * 9 * 64 and f["five"] == 2 * V * 5 * 64


def test_near_constant_v_is_bf16_rounded():
    p = fa_inputs.make_custom("nc", D=32, N=8, M=16, v_offset=1.0, v_spread=1e-3, v_type="bf16")
    vals = np.unique(O.widen(p.v, "bf16"))
    assert set(vals.tolist()) <= {1.0 - 2.0 ** -8, 1.0, 1.0 + 2.0 ** -7}


def test_q4_0_encoding_round_trip_error():
    # every code in [0, 15]; the decoded values within one step of the drawn ones (the value of
    # largest magnitude maps to code 0, so the other side clips at code 15 = +7 steps)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 5, 64)).astype(np.float32)
    x[0, 0, :32] = 0.0                                  # an all-zero block
    raw = fa_inputs.encode_q4_0(x)
    assert raw.shape == (3, 5, 36) and raw.dtype == np.uint8
    blocks = raw.reshape(3, 5, 2, 18)
    step = blocks[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
    codes = np.concatenate([blocks[..., 2:] & 15, blocks[..., 2:] >> 4], axis=-1).astype(np.float64)
    dec = step[..., None] * (codes - 8.0)
    err = np.abs(dec - x.reshape(3, 5, 2, 32).astype(np.float64))
    assert np.all(err <= np.abs(step)[..., None] * (1 + 1e-3) + 1e-6)
    assert np.all(dec[0, 0, 0] == 0.0)


@pytest.mark.parametrize("typ,nbytes", [("q4_1", 20), ("q5_0", 22), ("q5_1", 24)])
def test_other_block_encodings_round_trip_error(typ, nbytes):
    # the decoded values lie within one step of the drawn ones (half a step where no code clips),
    # and a constant block (zero for q5_0) decodes exactly
    rng = np.random.default_rng(12)
    x = rng.standard_normal((3, 5, 64)).astype(np.float32)
    x[0, 0, :32] = 0.0 if typ == "q5_0" else 0.75
    raw = fa_inputs.encode(x, typ)
    assert raw.shape == (3, 5, 2 * nbytes) and raw.dtype == np.uint8
    dec = O.widen(raw, typ, 64).reshape(3, 5, 2, 32)
    step = np.abs(raw.reshape(3, 5, 2, nbytes)[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64))
    err = np.abs(dec - x.reshape(3, 5, 2, 32).astype(np.float64))
    assert np.all(err <= step[..., None] * (1 + 2e-3) + 2e-3)
    assert np.all(dec[0, 0, 0] == x[0, 0, 0])
