"""The seeded input generators (gqa_inputs): the same seed gives the same
bytes whatever the thread count, bf16 inputs are float32 draws rounded to
nearest with ties to even, rows past each length hold the requested filler,
and the ragged lengths stay in [1, 32768]."""
import numpy as np
import pytest

import gqa_inputs as gi


def _bits(a):
    return a.view(np.uint8).tobytes()


def test_same_seed_same_bytes_and_other_seeds_differ():
    a = gi.decode_case(3, 8, 2, 64, 40, [40, 7, 0], "bf16", q_seed=1, kv_seed=2)
    b = gi.decode_case(3, 8, 2, 64, 40, [40, 7, 0], "bf16", q_seed=1, kv_seed=2)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert _bits(x) == _bits(y)
    c = gi.decode_case(3, 8, 2, 64, 40, [40, 7, 0], "bf16", q_seed=1, kv_seed=3)
    assert _bits(a.q) == _bits(c.q) and _bits(a.k[0]) != _bits(c.k[0])
    p1 = gi.prefill_case(1, 33, 4, 2, 64, "bf16", seed=5)
    p2 = gi.prefill_case(1, 33, 4, 2, 64, "bf16", seed=5)
    assert _bits(p1.q) == _bits(p2.q) and _bits(p1.k) == _bits(p2.k) and _bits(p1.v) == _bits(p2.v)


def test_rows_do_not_depend_on_the_thread_count(monkeypatch):
    lens = [50, 3, 17, 0, 64]
    monkeypatch.setattr(gi, "_threads", lambda: 1)
    one = gi.decode_case(5, 4, 2, 64, 64, lens, "f32", q_seed=7, kv_seed=8, invalid="zero")
    monkeypatch.setattr(gi, "_threads", lambda: 4)
    four = gi.decode_case(5, 4, 2, 64, 64, lens, "f32", q_seed=7, kv_seed=8, invalid="zero")
    assert _bits(one.k) == _bits(four.k) and _bits(one.v) == _bits(four.v)
    # sequence b's rows come from its own stream: a longer batch leaves them alone
    more = gi.decode_case(6, 4, 2, 64, 64, lens + [9], "f32", q_seed=7, kv_seed=8, invalid="zero")
    assert _bits(more.k[:5]) == _bits(one.k) and _bits(more.v[:5]) == _bits(one.v)


@pytest.mark.parametrize("f32,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                  # halfway, even neighbour below
    (1.0 + 3 * 2.0 ** -8, 0x3F82),              # halfway, even neighbour above
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),     # just above halfway
    (-2.5, 0xC020),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (3.3895313892515355e38, 0x7F7F),            # the largest bf16 stays finite
])
def test_bf16_rounding_is_nearest_even(f32, bits):
    assert int(gi.bf16_bits_from_f32(np.array([f32], np.float32))[0]) == bits


def test_filler_of_rows_past_each_length():
    c = gi.decode_case(2, 4, 2, 64, 10, [10, 4], "bf16", q_seed=1, kv_seed=2, invalid="nan")
    assert np.all(c.k[1, 4:] == gi.NAN_BF16) and np.all(c.v[1, 4:] == gi.NAN_BF16)
    assert not np.any(c.k[1, :4] == gi.NAN_BF16)
    f = gi.decode_case(2, 4, 2, 64, 10, [10, 4], "f32", q_seed=1, kv_seed=2, invalid="nan")
    assert np.all(np.isnan(f.k[1, 4:])) and np.all(np.isfinite(f.k[1, :4]))
    z = gi.decode_case(2, 4, 2, 64, 10, [10, 4], "f32", q_seed=1, kv_seed=2, invalid="zero")
    assert not np.any(z.k[1, 4:]) and _bits(z.k[1, :4]) == _bits(f.k[1, :4])


def test_ragged_lengths():
    lens = gi.ragged_seqlens()
    assert lens.shape == (64,) and lens.dtype == np.int32
    assert lens.min() >= 1 and lens.max() <= 32768
    assert len(set(lens.tolist())) > 50                  # drawn, not constant
    assert np.array_equal(lens, gi.ragged_seqlens())
