"""The seeded input generators (CPU only): the FP8 test-cache quantiser."""
import numpy as np

from synth import gen


def test_fast_e4m3_quantiser_matches_table_search():
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.standard_normal(200_000).astype(np.float32) * s for s in (1e-3, 0.02, 1, 30, 300)])
    edges = np.array([448, -448, 500, -1e9, 2 ** -10, 3 * 2 ** -10, 2 ** -6, 0.0, -0.0, 1.0625, 1.1875,
                      15 * 2 ** -10, 2 ** -9 * 8.5, 240, 464, 0.0009765625], np.float32)
    y = np.concatenate([y, edges])
    assert np.array_equal(gen.quantize_e4m3(y), gen.quantize_e4m3_reference(y))


def test_e4m3_round_trip_and_ties():
    vals = gen._e4m3_positive_values()
    codes = np.arange(0x7F, dtype=np.uint8)
    assert np.array_equal(gen.quantize_e4m3(vals.astype(np.float32)), codes)       # exact values round-trip
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)                          # exact midpoints (fp32)
    got = gen.quantize_e4m3(mids)
    assert np.all(got % 2 == 0) and np.all((got == codes[:-1]) | (got == codes[1:]))   # ties to the even code
