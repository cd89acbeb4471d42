"""Host logic of the seeded input generators (CPU only)."""
import numpy as np

import synthetic


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)           # bf16 spacing at 1.0
    x = np.array([1.0,
                  1.0 + 2.0 ** -8,        # exactly half an ulp above 1: tie -> even (1.0)
                  1.0 + 3 * 2.0 ** -8,    # tie between 1+ulp (odd) and 1+2ulp (even) -> up
                  1.0 + 2.0 ** -8 + 2.0 ** -20,  # just above the tie -> up
                  -2.5, 3.0e-3], dtype=np.float32)
    b = synthetic.bf16_bits_from_f32(x)
    back = synthetic.f32_from_bf16_bits(b)
    assert back[0] == one
    assert back[1] == one
    assert back[2] == one + 2 * ulp
    assert back[3] == one + ulp
    assert back[4] == np.float32(-2.5)
    assert abs(back[5] - 3.0e-3) <= 3.0e-3 * 2.0 ** -8
    # widening is exact: re-rounding a bf16 value is the identity
    assert np.array_equal(synthetic.bf16_bits_from_f32(back), b)


def test_f16_round_to_nearest_even():
    ulp = 2.0 ** -10                      # binary16 spacing at 1.0
    x = np.array([1.0 + 2.0 ** -11,       # tie -> even (1.0)
                  1.0 + 3 * 2.0 ** -11,   # tie between 1+ulp (odd) and 1+2ulp (even) -> up
                  1.0 + 2.0 ** -11 + 2.0 ** -20,
                  -2.5, 65504.0, 2.0 ** -24], dtype=np.float32)
    b = synthetic.f16_bits_from_f32(x)
    assert b.dtype == np.uint16
    assert b[3] == 0xC100 and b[4] == 0x7BFF and b[5] == 0x0001   # -2.5, max normal, min subnormal
    back = synthetic.f32_from_f16_bits(b)
    assert back.tolist() == [1.0, 1.0 + 2 * ulp, 1.0 + ulp, -2.5, 65504.0, 2.0 ** -24]
    assert np.array_equal(synthetic.storage_values(b, "f16"), back.astype(np.float64))
    assert np.array_equal(synthetic.f16_bits_from_f32(back), b)


def test_seeded_lengths_of_the_packed_workload():
    w = synthetic.WORKLOADS[synthetic.METRIC_WORKLOAD]
    rng = np.random.default_rng(0)
    lengths = synthetic.draw_lengths(rng, w["B"], w["len_lo"], w["len_hi"])
    assert lengths.tolist() == [3485, 2609, 2094, 1106, 1261, 168, 309, 68, 718, 3332, 2661,
                                3739, 2063, 2485, 3977, 2989]
    assert synthetic.cumulative_ends(lengths)[-1] == 33064


def test_csr_band_random_pattern():
    rng = np.random.default_rng(0)
    S, band, nr = 300, 16, 8
    off, col = synthetic.csr_band_random(rng, S, band, nr)
    assert off[0] == 0 and off[-1] == len(col) and np.all(np.diff(off) > 0)
    for i in range(S):
        row = col[off[i]:off[i + 1]]
        assert np.all(np.diff(row) > 0)                # sorted, distinct
        assert np.all(row <= i) and np.all(row >= 0)   # causal
        lo = max(0, i - band + 1)
        assert set(range(lo, i + 1)) <= set(row.tolist())
        assert len(row) == (i + 1 - lo) + min(nr, max(0, i - band + 1))


def test_full_size_csr_nnz():
    """Band 128 + 64 random earlier columns over S = 4096: 516,160 + 251,936 entries."""
    rng = np.random.default_rng(0)
    off, col = synthetic.csr_band_random(rng, 4096, 128, 64)
    assert len(col) == 768096


def test_layout_views_round_trip():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 3, 5, 4))
    for lay in synthetic.LAYOUTS:
        st = synthetic.from_bnsd(x, lay)
        assert st.shape == synthetic.storage_shape(lay, 2, 3, 5, 4)
        assert np.array_equal(synthetic.to_bnsd(st, lay, 3), x)
