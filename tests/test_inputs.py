"""The seeded input recipe (CPU only): bf16 rounding is one round-to-nearest-
even step from the float64 draw, bf16 scan inputs are rounded once (not via
fp32), and every stream depends only on (seed, tag, channel), so a subset of
channels draws the same values as the full array."""
import numpy as np

from linear_recurrence_scan_diagonal_amd import inputs as I


def test_bf16_rounding_nearest_even():
    # bf16 has 8 significant bits: spacing 2^-7 in [1, 2)
    ulp = 2.0 ** -7
    cases = {
        1.0: 1.0,
        1.0 + ulp / 2: 1.0,                        # tie, rounds to even (1.0)
        1.0 + 3 * ulp / 2: 1.0 + 2 * ulp,          # tie, rounds to even (1 + 2 ulp)
        1.0 + ulp / 2 + 2.0 ** -40: 1.0 + ulp,     # just above the tie
        1.0 + ulp / 2 - 2.0 ** -40: 1.0,           # just below the tie
        -(1.0 + 3 * ulp / 2): -(1.0 + 2 * ulp),
        0.0: 0.0,
        2.0 ** 100 * (1.0 + 5 * ulp / 2): 2.0 ** 100 * (1.0 + 2 * ulp),  # tie at a large exponent
    }
    x = np.array(list(cases), dtype=np.float64)
    got = I.bf16_bits_to_f64(I.to_bf16_bits(x))
    assert np.array_equal(got, np.array(list(cases.values()), dtype=np.float64))


def test_bf16_single_rounding_differs_from_double():
    """A float64 just above a bf16 tie that rounds to the tie in fp32: one
    rounding goes up, rounding via fp32 lands on the tie and then goes to even."""
    ulp = 2.0 ** -7
    x = np.array([1.0 + ulp / 2 + 2.0 ** -30])     # below fp32 resolution at 1.0 (2^-23)
    assert np.float32(x[0]) == np.float32(1.0 + ulp / 2)
    one = I.bf16_bits_to_f64(I.to_bf16_bits(x))[0]
    via_f32 = I.bf16_bits_to_f64(I.to_bf16_bits(x.astype(np.float32)))[0]
    assert one == 1.0 + ulp and via_f32 == 1.0


def test_scan_inputs_bf16_one_rounding_and_channel_subsets():
    w = I.scaled(I.WORKLOADS["scan_fwd_bwd_bf16"], B=2, D=9, T=513)
    x = I.scan_inputs_bf16(w, batch=4)
    for k in ("a", "b", "g"):
        ref = I.to_bf16_bits(I.series(w.seed, k, w.dists[k], np.arange(w.C), w.T))
        assert x[k].dtype == np.uint16 and np.array_equal(x[k], ref), k
    sub = np.array([3, 0, 17])
    y = I.scan_inputs_bf16(w, channels=sub)
    for k in ("a", "b", "g"):
        assert np.array_equal(y[k], x[k][sub]), k
    assert np.array_equal(y["h0"], x["h0"][sub])
    # the fp32 recipe draws the same streams, rounded to fp32 instead
    f = I.scan_inputs(w)
    assert np.all(np.abs(I.bf16_bits_to_f64(x["a"]) - f["a"]) <= 2.0 ** -8 * np.abs(f["a"]))
    # a in U(0.8, 0.999): every bf16 value stays in [0.8, 1] after rounding
    a = I.bf16_bits_to_f64(x["a"])
    assert a.min() >= 0.796875 and a.max() <= 1.0
